// internal.hpp -- shared declarations of the gfx950 KV-retention library.
//
// Nothing here is part of the C ABI (include/hubkv.h); these are the launch
// helpers and device utilities the kernels share.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hubkv {

constexpr int kMaxSeqs = 64;

// Per-call sequence table, passed to kernels by value (kernel-argument
// memory, no device allocation).  `tile_off[b]` is the first tile index of
// sequence b when every sequence is cut into `tile`-token tiles; tile_off[B]
// is the total tile count.
struct SeqTable {
  int B;
  int tile;
  int64_t N[kMaxSeqs];
  int64_t cu[kMaxSeqs];  // first packed token of each sequence
  int64_t ko[kMaxSeqs];  // first kept row of each sequence (sum of kept before b)
  int64_t kept[kMaxSeqs];
  int32_t tile_off[kMaxSeqs + 1];
};

// Sequence owning tile `x` (linear scan; B <= 64).
__device__ __forceinline__ int seq_of_tile(const SeqTable& st, int x) {
  int b = 0;
  while (b + 1 < st.B && st.tile_off[b + 1] <= x) ++b;
  return b;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---- score -----------------------------------------------------------------
// Keys per work-group chunk: a multiple of this on the MFMA path (sized so
// the grid holds about kScoreGroups work-groups), fixed on the fp32 VALU path.
constexpr int kScoreChunkMfma = 1024;
constexpr int kScoreChunkF32 = 256;
constexpr int64_t kScoreGroups = 256;     // MI355X compute units
constexpr int64_t kScoreStartKeys = 2048;  // per-work-group start-up, in keys streamed

struct ScoreGeom {
  int M;       // G * W query rows per KV head
  int Mpad;    // rows rounded up to 64
  int chunk;   // keys per work-group task
  int nchunk;  // chunks over all sequences of one (layer, KV head)
  size_t off_part1, off_rowstat, off_part2, off_ctl, bytes;  // rowstat: fp32 path only
};

// Chunk size the score path uses for these sequence lengths, `units` (layers
// x KV heads) independent score problems and `rows` (G * W) query rows each.
int score_chunk(int B, const int64_t* seqlens, int64_t units, int rows, int dtype);

ScoreGeom score_geometry(const SeqTable& st, int L, int Hq, int Hkv, int W, int d, int dtype);

// Element strides of the score operands; the d axis is always contiguous.
// Q row (layer l, query head h, sequence b, window row w) starts at
// l*q_l + h*q_h + (b*W + w)*q_r; key token t of (layer l, KV head g) at
// l*k_l + g*k_h + t*k_t, t counted over the packed sequences.
struct ScoreStrides {
  int64_t q_l, q_h, q_r, k_l, k_h, k_t;
};

// Score scratch the library holds itself, for callers that cannot allocate:
// one fixed array per device (a file-scope __device__ array in score.hip).
constexpr size_t kScoreScratchBytes = (size_t)16 << 20;

// Device address of that array on the device `stream` runs on (the current
// device for the null stream), looked up once per device.
hipError_t score_scratch(hipStream_t stream, char** ptr);

hipError_t launch_score(const void* q, const void* k, int dtype, const SeqTable& st, int L, int Hq,
                        int Hkv, int W, int d, const ScoreStrides& sd, float scale, int causal,
                        float* s, double* head_stats, char* ws, const ScoreGeom& geo,
                        hipStream_t stream);

// ---- refine / select ---------------------------------------------------------
constexpr int kRefineTile = 1024;

struct RefineGeom {
  int nchunk;
  size_t off_part, off_stats, bytes;
};

RefineGeom refine_geometry(const SeqTable& st, int L, int Hkv);

hipError_t launch_head_stats(const float* s, const SeqTable& st, int L, int Hkv, double* part,
                             double* stats, hipStream_t stream);

hipError_t launch_refine(const float* s, const SeqTable& st, int L, int Hkv,
                         const double* head_stats, const float* beta_in, int pool, float gamma,
                         float beta_lo, float beta_hi, float r2, float* z, float* beta_out,
                         hipStream_t stream);

hipError_t launch_select(const float* z, const SeqTable& st, int L, int Hkv, int n_sink,
                         int n_recent, int32_t* idx, hipStream_t stream);

// ---- protected Top-K over many work-groups per unit ---------------------------
constexpr int kMsSlice = 4096;       // positions per work-group (the table's tile)
constexpr int kMsMaxSlices = 1024;   // slices per sequence: sequences up to 4M positions

struct MselGeomDev {
  size_t off_head, off_pre, off_sorted;
};
struct MselGeom {
  MselGeomDev d;
  size_t bytes;
};

// Kernel-argument block of the many-work-group select (and its fused
// refinement); st is cut into kMsSlice-position tiles and carries kept/ko.
struct MselArgs {
  SeqTable st;
  int Hkv, n_sink, n_recent, nslice;
  int max_nsl;  // slices of the longest sequence
  int64_t T, Ktot;
  MselGeomDev g;
  int half;
  float gamma, r2, beta_lo, beta_hi;
  const float* beta_in;
  const double* stats;
  float* beta_out;
};

struct RefineParams {
  int pool;
  float gamma, r2, beta_lo, beta_hi;
  const float* beta_in;
  const double* stats;
  float* beta_out;
};

MselGeom msel_geometry(const SeqTable& st, int L, int Hkv);

// Select on z (refine = false: src is z), or refine s into z and select
// (refine = true: src is s, z receives the refined scores).
hipError_t launch_msel(const float* src, bool refine, float* z, const SeqTable& st, int L,
                       int Hkv, int n_sink, int n_recent, const RefineParams& rp, int32_t* idx,
                       char* ws, const MselGeom& geo, hipStream_t stream);

// ---- layer-wide budget --------------------------------------------------------------
constexpr int kMaxLayerSegs = 256;  // (layer, sequence) pairs per call
constexpr int kLselChunk = 4096;    // positions per work-group

// Kernel-argument table of a layer-wide selection (no device allocation).
struct LselArgs {
  int B, L, Hkv, n_sink, n_recent;
  int nchunk;                       // chunks of one (layer, head) over all sequences
  int64_t T;                        // packed tokens
  int32_t N[kMaxSeqs];
  int64_t cu[kMaxSeqs];
  int32_t f[kMaxSeqs];              // per-head floor of each sequence
  int32_t ch_off[kMaxSeqs + 1];     // first chunk of each sequence
  int32_t budget[kMaxLayerSegs];    // kept total per (layer, sequence), row-major
};

struct LselGeom {
  size_t off_hs, off_ss, off_hh, off_hg, off_ch, off_cg, off_ec, bytes;
};

LselGeom lsel_geometry(const LselArgs& a);

hipError_t launch_select_layer(const float* z, const LselArgs& a, const LselGeom& g, char* ws,
                               int32_t* idx, int32_t* head_kept, hipStream_t stream);

hipError_t launch_compact_layer(const void* k_in, const void* v_in, int elem_bytes,
                                const int32_t* idx, const int32_t* head_kept, const LselArgs& a,
                                int d, void* k_out, void* v_out, hipStream_t stream);

// ---- NestedKV key-only score ----------------------------------------------------------
constexpr int kNkvTile = 1024;    // keys per sum tile (sum tiles never straddle a block)
constexpr int kNkvAnTile = 2048;  // keys per anomaly tile

struct NkvArgs {
  int B, L, Hkv, d;
  int ntile;       // tiles of one (layer, head) over all sequences
  int nblk_total;  // blocks of one (layer, head) over all sequences
  int nat;         // anomaly tiles of one (layer, head) over all sequences
  int64_t T;
  float theta;
  float prior[3];
  int32_t N[kMaxSeqs];
  int64_t cu[kMaxSeqs];
  int32_t bs[kMaxSeqs];    // block length of each sequence
  int32_t nblk[kMaxSeqs];  // blocks of each sequence
  int32_t tpb[kMaxSeqs];   // tiles per block
  int32_t tile_off[kMaxSeqs + 1];
  int32_t blk_off[kMaxSeqs + 1];
  int32_t at_off[kMaxSeqs + 1];  // first anomaly tile of each sequence
};

struct NkvGeom {
  size_t off_part, off_bsum, off_bnorm, off_mm, off_an, off_inv, bytes;
};

NkvGeom nkv_geometry(const NkvArgs& a);

hipError_t launch_nestedkv(const void* k, int dtype, const NkvArgs& a, const NkvGeom& g, char* ws,
                           float* anomalies, float* s, float* weights, hipStream_t stream);

// ---- compaction ------------------------------------------------------------------
// Strides of a compaction in 16-byte units (the d axis contiguous): row t of
// (layer l, KV head h) starts at l*s_l + h*s_h + t*s_t, t counted over the
// packed sequences (the input) or the packed kept rows (the output).
struct RowStrides {
  int64_t s_l, s_h, s_t;
};

hipError_t launch_compact(const void* k_in, const void* v_in, int elem_bytes, const int32_t* idx,
                          const SeqTable& st, int L, int Hkv, int d, const RowStrides& ki,
                          const RowStrides& vi, const RowStrides& ko, const RowStrides& vo,
                          void* k_out, void* v_out, hipStream_t stream);

// ---- streaming H2O step ------------------------------------------------------------
struct H2OArgs {
  int B, Hq, Hkv, d, C, n_sink, n_recent, include_self;
  int ring;  // 0: fixed slots; 1: heavy slots [0, C - n_recent) + a ring of n_recent slots
  float scale;
  int64_t t[kMaxSeqs];
};

hipError_t launch_h2o_step(const void* q, const void* k_new, const void* v_new, int dtype,
                           void* k_cache, void* v_cache, float* acc, int32_t* pos,
                           const H2OArgs& a, int32_t* evicted, float* probs, float* out,
                           hipStream_t stream);

}  // namespace hubkv
