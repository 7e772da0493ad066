// abi.cpp -- the C ABI declared in include/hubkv.h: host-side validation,
// workspace sizing and dispatch to the gfx950 kernels.
//
// Every entry point validates all of its arguments with plain host code
// before it makes any HIP call, so a rejected call enqueues nothing and
// leaves the outputs untouched.
#include <math.h>
#include <string.h>

#include "../../include/hubkv.h"
#include "internal.hpp"

using namespace hubkv;

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return HUBKV_OK;
  g_last_hip_error = (int)e;
  return HUBKV_EHIP;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int64_t kMaxGridY = 65535;
constexpr int64_t kMaxTokens = (int64_t)1 << 31;  // positions are int32
// Longest sequence: kernels do their position arithmetic in int32, including
// rounding a length up to a whole number of tiles or select rounds (at most
// 2^20 positions), so every sequence stays below 2^30.
constexpr int64_t kMaxSeqLen = (int64_t)1 << 30;

static_assert(kScoreScratchBytes == (size_t)HUBKV_SCORE_NOALLOC_BYTES,
              "the header states the fixed score scratch size");

// Validate the sequence table and fill it; tile size `tile` sets tile_off.
int make_table(SeqTable& st, int B, const int64_t* seqlens, int tile) {
  if (B < 1 || B > kMaxSeqs || !seqlens) return HUBKV_EINVAL;
  memset(&st, 0, sizeof(st));
  st.B = B;
  st.tile = tile;
  int64_t cu = 0, tiles = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t n = seqlens[b];
    if (n < 1 || n >= kMaxSeqLen) return HUBKV_EINVAL;
    st.N[b] = n;
    st.cu[b] = cu;
    st.tile_off[b] = (int32_t)tiles;
    cu += n;
    tiles += (n + tile - 1) / tile;
    if (cu >= ((int64_t)1 << 40) || tiles >= ((int64_t)1 << 30)) return HUBKV_EINVAL;
  }
  st.tile_off[B] = (int32_t)tiles;
  return HUBKV_OK;
}

int check_kept(SeqTable& st, const int64_t* kept, int n_sink, int n_recent, bool need_protected) {
  if (!kept || n_sink < 0 || n_recent < 0) return HUBKV_EINVAL;
  int64_t ko = 0;
  for (int b = 0; b < st.B; ++b) {
    const int64_t P = need_protected ? hubkv_protected_count(st.N[b], n_sink, n_recent) : 0;
    if (kept[b] < P || kept[b] > st.N[b]) return HUBKV_EINVAL;
    st.ko[b] = ko;
    st.kept[b] = kept[b];
    ko += kept[b];
  }
  if (ko >= kMaxTokens) return HUBKV_EINVAL;
  return HUBKV_OK;
}

// Rows kept over all sequences (after check_kept).  A call that keeps none
// writes no row, so its row outputs may be null.
int64_t kept_total(const SeqTable& st) {
  int64_t K = 0;
  for (int b = 0; b < st.B; ++b) K += st.kept[b];
  return K;
}

int check_dtype_d(int dtype, int d) {
  if (dtype != HUBKV_F32 && dtype != HUBKV_BF16) return HUBKV_EDTYPE;
  if (d != 64 && d != 128) return HUBKV_EDTYPE;
  return HUBKV_OK;
}

int check_score_shape(int L, int Hq, int Hkv, int W, const SeqTable& st) {
  if (L < 1 || Hq < 1 || Hkv < 1 || W < 1 || Hq % Hkv) return HUBKV_EINVAL;
  if ((int64_t)L * Hkv > kMaxGridY) return HUBKV_EINVAL;
  if ((int64_t)(Hq / Hkv) * W > 512) return HUBKV_EINVAL;
  for (int b = 0; b < st.B; ++b)
    if (st.N[b] < W) return HUBKV_EINVAL;
  return HUBKV_OK;
}

// Validate the element strides (layer, head, row) of an operand whose rows
// hold `row` contiguous elements of `esize` bytes, with `ext` layers, heads
// and rows: every stride a non-negative multiple of 16 bytes, every offset
// below 2^60 bytes and, for an output, distinct (layer, head, row) triples on
// disjoint bytes.
int check_strides(const int64_t* sd, const int64_t ext[3], int esize, int64_t row, bool output) {
  if (!sd) return HUBKV_EINVAL;
  for (int i = 0; i < 3; ++i) {
    if (sd[i] < 0 || sd[i] > ((int64_t)1 << 50)) return HUBKV_EINVAL;
    if ((sd[i] * esize) % 16) return HUBKV_EALIGN;
  }
  if (ext[0] < 1 || ext[1] < 1 || ext[2] < 1) return HUBKV_OK;  // nothing addressed
  int64_t last = row;
  for (int i = 0; i < 3; ++i) {
    int64_t t;
    if (__builtin_mul_overflow(sd[i], ext[i] - 1, &t) || __builtin_add_overflow(last, t, &last))
      return HUBKV_EINVAL;
  }
  if (last > ((int64_t)1 << 60) / esize) return HUBKV_EINVAL;
  if (!output) return HUBKV_OK;
  int o[3] = {0, 1, 2};  // dimensions by ascending stride
  for (int i = 1; i < 3; ++i)
    for (int j = i; j > 0 && sd[o[j]] < sd[o[j - 1]]; --j) {
      const int x = o[j];
      o[j] = o[j - 1];
      o[j - 1] = x;
    }
  int64_t span = row;  // elements covered by the dimensions placed so far
  for (int i = 0; i < 3; ++i) {
    const int64_t n = ext[o[i]], st = sd[o[i]];
    if (n <= 1) continue;
    if (st < span) return HUBKV_EINVAL;
    span = st * (n - 1) + span;
  }
  return HUBKV_OK;
}

// Fill the layer-wide selection table; validates shapes and budgets.
int make_lsel(LselArgs& a, int B, const int64_t* seqlens, int L, int Hkv, const int64_t* layer_kept,
              int n_sink, int n_recent, int floor_min) {
  if (B < 1 || B > kMaxSeqs || !seqlens || !layer_kept) return HUBKV_EINVAL;
  if (L < 1 || Hkv < 1 || Hkv > 1024 || (int64_t)L * Hkv > kMaxGridY) return HUBKV_EINVAL;
  if ((int64_t)L * B > kMaxLayerSegs || n_sink < 0 || n_recent < 0 || floor_min < 0)
    return HUBKV_EINVAL;
  memset(&a, 0, sizeof(a));
  a.B = B;
  a.L = L;
  a.Hkv = Hkv;
  a.n_sink = n_sink;
  a.n_recent = n_recent;
  int64_t cu = 0, ch = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t n = seqlens[b];
    if (n < 1 || n >= kMaxSeqLen) return HUBKV_EINVAL;
    const int64_t P = hubkv_protected_count(n, n_sink, n_recent);
    a.N[b] = (int32_t)n;
    a.cu[b] = cu;
    a.f[b] = (int32_t)(floor_min < n - P ? floor_min : n - P);
    a.ch_off[b] = (int32_t)ch;
    cu += n;
    ch += (n + kLselChunk - 1) / kLselChunk;
  }
  if (cu >= ((int64_t)1 << 40) || ch > 65535) return HUBKV_EINVAL;
  a.ch_off[B] = (int32_t)ch;
  a.nchunk = (int)ch;
  a.T = cu;
  int64_t tot = 0;
  for (int l = 0; l < L; ++l)
    for (int b = 0; b < B; ++b) {
      const int64_t n = a.N[b];
      const int64_t P = hubkv_protected_count(n, n_sink, n_recent);
      const int64_t k = layer_kept[(int64_t)l * B + b];
      if (k < (int64_t)Hkv * (P + a.f[b]) || k > (int64_t)Hkv * n) return HUBKV_EINVAL;
      a.budget[l * B + b] = (int32_t)(k < kMaxTokens ? k : 0);
      tot += k;
      if (tot >= kMaxTokens) return HUBKV_EINVAL;
    }
  return HUBKV_OK;
}

// Fill the NestedKV table: blocks of ceil(N / nblocks) keys, tiles of at most
// kNkvTile keys inside each block.
int make_nkv(NkvArgs& a, int B, const int64_t* seqlens, int L, int Hkv, int d, int nblocks) {
  if (B < 1 || B > kMaxSeqs || !seqlens || L < 1 || Hkv < 1) return HUBKV_EINVAL;
  if ((int64_t)L * Hkv > kMaxGridY || nblocks < 1 || nblocks > 4096) return HUBKV_EINVAL;
  memset(&a, 0, sizeof(a));
  a.B = B;
  a.L = L;
  a.Hkv = Hkv;
  a.d = d;
  int64_t cu = 0, tiles = 0, blks = 0, ats = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t n = seqlens[b];
    if (n < 1 || n >= kMaxSeqLen) return HUBKV_EINVAL;
    a.at_off[b] = (int32_t)ats;
    ats += (n + kNkvAnTile - 1) / kNkvAnTile;
    const int64_t bs = (n + nblocks - 1) / nblocks;
    const int64_t nb = (n + bs - 1) / bs;
    const int64_t tpb = (bs + kNkvTile - 1) / kNkvTile;
    a.N[b] = (int32_t)n;
    a.cu[b] = cu;
    a.bs[b] = (int32_t)bs;
    a.nblk[b] = (int32_t)nb;
    a.tpb[b] = (int32_t)tpb;
    a.tile_off[b] = (int32_t)tiles;
    a.blk_off[b] = (int32_t)blks;
    cu += n;
    tiles += nb * tpb;
    blks += nb;
  }
  if (cu >= ((int64_t)1 << 40) || tiles > 65535 || blks > 65535 || ats > 65535) return HUBKV_EINVAL;
  a.at_off[B] = (int32_t)ats;
  a.nat = (int)ats;
  a.tile_off[B] = (int32_t)tiles;
  a.blk_off[B] = (int32_t)blks;
  a.ntile = (int)tiles;
  a.nblk_total = (int)blks;
  a.T = cu;
  return HUBKV_OK;
}

}  // namespace

namespace {

// Shared body of h2o_step (ring = 0) and h2o_step_ring (ring = 1).
int h2o_impl(const void* q, const void* k_new, const void* v_new, int dtype, void* k_cache,
             void* v_cache, float* acc, int32_t* pos, const int64_t* t, int B, int Hq, int Hkv,
             int d, int C, int n_sink, int n_recent, float scale, int include_self,
             int32_t* evicted, float* probs, float* out, void* stream, int ring) {
  int rc = check_dtype_d(dtype, d);
  if (rc) return rc;
  if (B < 1 || B > kMaxSeqs || Hq < 1 || Hkv < 1 || Hq % Hkv || !t) return HUBKV_EINVAL;
  const int G = Hq / Hkv;
  if (G > 16 || C < 1 || (int64_t)(G + 1) * C > 16384) return HUBKV_EINVAL;
  if (n_sink < 0 || n_recent < 0 || (int64_t)n_sink + n_recent > C) return HUBKV_EINVAL;
  if (ring && (n_recent < 1 || n_recent >= C)) return HUBKV_EINVAL;  // a ring and a heavy slot
  if ((int64_t)B * Hkv > ((int64_t)1 << 30) || !isfinite(scale)) return HUBKV_EINVAL;
  H2OArgs a;
  memset(&a, 0, sizeof(a));
  for (int b = 0; b < B; ++b) {
    if (t[b] < 0 || t[b] >= kMaxTokens - 1) return HUBKV_EINVAL;
    a.t[b] = t[b];
  }
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !acc || !pos) return HUBKV_EALIGN;
  if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(acc, 4) || !aligned(pos, 4))
    return HUBKV_EALIGN;
  if ((evicted && !aligned(evicted, 4)) || (probs && !aligned(probs, 4)) ||
      (out && !aligned(out, 4)))
    return HUBKV_EALIGN;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.C = C;
  a.n_sink = n_sink;
  a.n_recent = n_recent;
  a.include_self = include_self ? 1 : 0;
  a.ring = ring;
  a.scale = scale;
  return hip_status(launch_h2o_step(q, k_new, v_new, dtype, k_cache, v_cache, acc, pos, a, evicted,
                                    probs, out, (hipStream_t)stream));
}

// Validation and launch of the score, on a caller's workspace or (noalloc)
// on the library's fixed per-device scratch.
int score_impl(const void* q, const int64_t* q_strides, const void* k, const int64_t* k_strides,
               int dtype, int B, const int64_t* seqlens, int L, int Hq, int Hkv, int W, int d,
               float scale, int causal, float* s, double* head_stats, void* workspace,
               size_t workspace_bytes, void* stream, bool noalloc) {
  int rc = check_dtype_d(dtype, d);
  if (rc) return rc;
  SeqTable st;
  if (B < 1 || B > kMaxSeqs || !seqlens) return HUBKV_EINVAL;
  const int chunk = score_chunk(B, seqlens, (int64_t)L * Hkv, Hkv > 0 ? (Hq / Hkv) * W : 0, dtype);
  if ((rc = make_table(st, B, seqlens, chunk))) return rc;
  if ((rc = check_score_shape(L, Hq, Hkv, W, st))) return rc;
  if (!isfinite(scale)) return HUBKV_EINVAL;
  int64_t T = 0;
  for (int b = 0; b < B; ++b) T += st.N[b];
  const int esize = dtype == HUBKV_BF16 ? 2 : 4;
  const int64_t qext[3] = {L, Hq, (int64_t)B * W}, kext[3] = {L, Hkv, T};
  if ((rc = check_strides(q_strides, qext, esize, d, false))) return rc;
  if ((rc = check_strides(k_strides, kext, esize, d, false))) return rc;
  if (!q || !k || !s || !aligned(q, 16) || !aligned(k, 16) || !aligned(s, 4)) return HUBKV_EALIGN;
  if (head_stats && !aligned(head_stats, 8)) return HUBKV_EALIGN;
  const ScoreGeom geo = score_geometry(st, L, Hq, Hkv, W, d, dtype);
  char* ws = (char*)workspace;
  if (noalloc) {
    if (geo.bytes > kScoreScratchBytes) return HUBKV_ESCRATCH;
    if ((rc = hip_status(score_scratch((hipStream_t)stream, &ws)))) return rc;
  } else {
    if (!workspace || workspace_bytes < geo.bytes) return HUBKV_EWORKSPACE;
    if (!aligned(workspace, 256)) return HUBKV_EALIGN;
  }
  const ScoreStrides sd{q_strides[0], q_strides[1], q_strides[2],
                        k_strides[0], k_strides[1], k_strides[2]};
  return hip_status(launch_score(q, k, dtype, st, L, Hq, Hkv, W, d, sd, scale, causal, s,
                                 head_stats, ws, geo, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int64_t hubkv_protected_count(int64_t N, int n_sink, int n_recent) {
  if (N <= 0) return 0;
  const int64_t a = n_sink < N ? (n_sink > 0 ? n_sink : 0) : N;
  int64_t c = N - (n_recent > 0 ? n_recent : 0);
  if (c < 0) c = 0;
  if (c <= a) return N;
  return a + (N - c);
}

const char* hubkv_strerror(int status) {
  switch (status) {
    case HUBKV_OK: return "success";
    case HUBKV_EINVAL: return "invalid size, count or parameter";
    case HUBKV_EDTYPE: return "unsupported element type or head dimension";
    case HUBKV_EALIGN: return "null or misaligned pointer";
    case HUBKV_EWORKSPACE: return "workspace missing or too small";
    case HUBKV_EHIP: return "HIP launch failure";
    case HUBKV_ESCRATCH: return "problem needs more scratch than the library's fixed array holds";
    default: return "unknown status";
  }
}

int hubkv_last_hip_error(void) { return g_last_hip_error; }

int hubkv_version(void) { return 100; }

size_t hubkv_score_workspace(int B, const int64_t* seqlens, int L, int Hq, int Hkv, int W, int d,
                             int dtype) {
  if (check_dtype_d(dtype, d) != HUBKV_OK) return 0;
  SeqTable st;
  if (B < 1 || B > kMaxSeqs || !seqlens) return 0;
  const int chunk = score_chunk(B, seqlens, (int64_t)L * Hkv, Hkv > 0 ? (Hq / Hkv) * W : 0, dtype);
  if (make_table(st, B, seqlens, chunk) != HUBKV_OK) return 0;
  if (check_score_shape(L, Hq, Hkv, W, st) != HUBKV_OK) return 0;
  return score_geometry(st, L, Hq, Hkv, W, d, dtype).bytes;
}

int hubkv_score_strided(const void* q, const int64_t* q_strides, const void* k,
                        const int64_t* k_strides, int dtype, int B, const int64_t* seqlens, int L,
                        int Hq, int Hkv, int W, int d, float scale, int causal, float* s,
                        double* head_stats, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return score_impl(q, q_strides, k, k_strides, dtype, B, seqlens, L, Hq, Hkv, W, d, scale, causal,
                    s, head_stats, workspace, workspace_bytes, stream, false);
}

// Packed strides of Q [L][Hq][B*W][d] and K [L][Hkv][T][d]; validates what
// they are computed from so they cannot overflow.
static int packed_score_strides(int B, const int64_t* seqlens, int L, int Hq, int Hkv, int W,
                                int d, int64_t qs[3], int64_t ks[3]) {
  if (B < 1 || B > kMaxSeqs || !seqlens) return HUBKV_EINVAL;
  int64_t T = 0;
  for (int b = 0; b < B; ++b) {
    if (seqlens[b] < 1 || seqlens[b] >= kMaxSeqLen) return HUBKV_EINVAL;
    T += seqlens[b];
  }
  // Bounds that check_score_shape implies, so the packed strides cannot overflow.
  if (L < 1 || Hq < 1 || Hkv < 1 || W < 1 || W > 512 || Hkv > kMaxGridY || Hq > 512 * kMaxGridY)
    return HUBKV_EINVAL;
  qs[0] = (int64_t)Hq * B * W * d;
  qs[1] = (int64_t)B * W * d;
  qs[2] = d;
  ks[0] = (int64_t)Hkv * T * d;
  ks[1] = T * d;
  ks[2] = d;
  return HUBKV_OK;
}

int hubkv_score(const void* q, const void* k, int dtype, int B, const int64_t* seqlens, int L,
                int Hq, int Hkv, int W, int d, float scale, int causal, float* s,
                double* head_stats, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_dtype_d(dtype, d);
  if (rc) return rc;
  int64_t qs[3], ks[3];
  if ((rc = packed_score_strides(B, seqlens, L, Hq, Hkv, W, d, qs, ks))) return rc;
  return score_impl(q, qs, k, ks, dtype, B, seqlens, L, Hq, Hkv, W, d, scale, causal, s,
                    head_stats, workspace, workspace_bytes, stream, false);
}

int hubkv_score_noalloc(const void* q, const void* k, int dtype, int B, const int64_t* seqlens,
                        int L, int Hq, int Hkv, int W, int d, float scale, int causal, float* s,
                        double* head_stats, void* stream) {
  int rc = check_dtype_d(dtype, d);
  if (rc) return rc;
  int64_t qs[3], ks[3];
  if ((rc = packed_score_strides(B, seqlens, L, Hq, Hkv, W, d, qs, ks))) return rc;
  return score_impl(q, qs, k, ks, dtype, B, seqlens, L, Hq, Hkv, W, d, scale, causal, s,
                    head_stats, nullptr, 0, stream, true);
}

size_t hubkv_refine_workspace(int B, const int64_t* seqlens, int L, int Hkv) {
  SeqTable st;
  if (make_table(st, B, seqlens, kRefineTile) != HUBKV_OK) return 0;
  if (L < 1 || Hkv < 1 || Hkv > 1024 || (int64_t)L * Hkv > kMaxGridY) return 0;
  return refine_geometry(st, L, Hkv).bytes;
}

int hubkv_refine(const float* s, int B, const int64_t* seqlens, int L, int Hkv,
                 const double* head_stats, const float* beta_in, int pool, float gamma,
                 float beta_lo, float beta_hi, float r, float* z, float* beta_out, void* workspace,
                 size_t workspace_bytes, void* stream) {
  SeqTable st;
  int rc = make_table(st, B, seqlens, kRefineTile);
  if (rc) return rc;
  if (L < 1 || Hkv < 1 || Hkv > 1024 || (int64_t)L * Hkv > kMaxGridY) return HUBKV_EINVAL;
  if (pool < 1 || pool % 2 == 0 || pool > 63) return HUBKV_EINVAL;
  if (!(gamma > 0.f && gamma <= 1.f)) return HUBKV_EINVAL;
  if (!(isfinite(beta_lo) && isfinite(beta_hi) && beta_lo <= beta_hi)) return HUBKV_EINVAL;
  if (!(r >= 0.f && r <= 1.f)) return HUBKV_EINVAL;
  if (!s || !z || !aligned(s, 4) || !aligned(z, 4)) return HUBKV_EALIGN;
  if ((head_stats && !aligned(head_stats, 8)) || (beta_in && !aligned(beta_in, 4)) ||
      (beta_out && !aligned(beta_out, 4)))
    return HUBKV_EALIGN;
  int64_t T = 0;
  for (int b = 0; b < B; ++b) T += st.N[b];
  const uintptr_t n = (uintptr_t)((int64_t)L * Hkv * T) * sizeof(float);
  if ((uintptr_t)s < (uintptr_t)z + n && (uintptr_t)z < (uintptr_t)s + n) return HUBKV_EINVAL;
  const RefineGeom geo = refine_geometry(st, L, Hkv);
  if (!workspace || workspace_bytes < geo.bytes) return HUBKV_EWORKSPACE;
  if (!aligned(workspace, 256)) return HUBKV_EALIGN;
  char* ws = (char*)workspace;
  hipStream_t strm = (hipStream_t)stream;
  const double* stats = head_stats;
  if (!beta_in && !stats) {
    double* st_ws = (double*)(ws + geo.off_stats);
    rc = hip_status(launch_head_stats(s, st, L, Hkv, (double*)(ws + geo.off_part), st_ws, strm));
    if (rc) return rc;
    stats = st_ws;
  }
  const float r2 = r * r;  // fp32 product, as the gate formula is evaluated in fp32
  return hip_status(launch_refine(s, st, L, Hkv, stats, beta_in, pool, gamma, beta_lo, beta_hi, r2,
                                  z, beta_out, strm));
}

// Which select a call runs.  The many-work-group select covers sequences of
// up to kMsSlice x kMsMaxSlices positions; a call with a longer sequence uses
// the one-work-group select for all of its units.  So does a call whose
// units alone fill the chip (one work-group per unit on each of the 256
// CUs): slicing then adds no parallelism, only the bin data the sliced
// select writes and reads back (on 32 layers x 8 KV heads x 131072
// positions: 266 us against 190 us for refine then the one-work-group select).
constexpr int64_t kFullChipUnits = 256;

static bool msel_fits(const SeqTable& st, int L, int Hkv) {
  if ((int64_t)L * Hkv * st.B >= kFullChipUnits) return false;
  for (int b = 0; b < st.B; ++b)
    if (st.N[b] > (int64_t)kMsSlice * kMsMaxSlices) return false;
  return true;
}

size_t hubkv_select_workspace(int B, const int64_t* seqlens, int L, int Hkv) {
  SeqTable st;
  if (make_table(st, B, seqlens, kMsSlice) != HUBKV_OK) return 0;
  if (L < 1 || Hkv < 1 || (int64_t)L * Hkv > kMaxGridY) return 0;
  if (!msel_fits(st, L, Hkv)) return 256;  // the one-work-group select needs no workspace
  return msel_geometry(st, L, Hkv).bytes;
}

int hubkv_select(const float* z, int B, const int64_t* seqlens, int L, int Hkv,
                 const int64_t* kept, int n_sink, int n_recent, int32_t* idx, void* workspace,
                 size_t workspace_bytes, void* stream) {
  SeqTable st;
  int rc = make_table(st, B, seqlens, kMsSlice);
  if (rc) return rc;
  if (L < 1 || Hkv < 1 || (int64_t)L * Hkv > kMaxGridY) return HUBKV_EINVAL;
  if ((rc = check_kept(st, kept, n_sink, n_recent, true))) return rc;
  const int64_t K = kept_total(st);
  if (!z || !aligned(z, 4) || (K > 0 && (!idx || !aligned(idx, 4)))) return HUBKV_EALIGN;
  if (K == 0) return HUBKV_OK;  // nothing kept: no row to write
  if (!msel_fits(st, L, Hkv))
    return hip_status(launch_select(z, st, L, Hkv, n_sink, n_recent, idx, (hipStream_t)stream));
  const MselGeom geo = msel_geometry(st, L, Hkv);
  if (!workspace || workspace_bytes < geo.bytes) return HUBKV_EWORKSPACE;
  if (!aligned(workspace, 256)) return HUBKV_EALIGN;
  const RefineParams rp{};
  return hip_status(launch_msel(z, false, nullptr, st, L, Hkv, n_sink, n_recent, rp, idx,
                                (char*)workspace, geo, (hipStream_t)stream));
}

size_t hubkv_refine_select_workspace(int B, const int64_t* seqlens, int L, int Hkv) {
  const size_t r = hubkv_refine_workspace(B, seqlens, L, Hkv);
  const size_t q = hubkv_select_workspace(B, seqlens, L, Hkv);
  if (!r || !q) return 0;
  return ((r + 255) & ~(size_t)255) + q;
}

int hubkv_refine_select(const float* s, int B, const int64_t* seqlens, int L, int Hkv,
                        const double* head_stats, const float* beta_in, int pool, float gamma,
                        float beta_lo, float beta_hi, float r, float* z, float* beta_out,
                        const int64_t* kept, int n_sink, int n_recent, int32_t* idx,
                        void* workspace, size_t workspace_bytes, void* stream) {
  SeqTable rt, st;
  int rc = make_table(rt, B, seqlens, kRefineTile);
  if (rc) return rc;
  if ((rc = make_table(st, B, seqlens, kMsSlice))) return rc;
  if (L < 1 || Hkv < 1 || Hkv > 1024 || (int64_t)L * Hkv > kMaxGridY) return HUBKV_EINVAL;
  if (pool < 1 || pool % 2 == 0 || pool > 63) return HUBKV_EINVAL;
  if (!(gamma > 0.f && gamma <= 1.f)) return HUBKV_EINVAL;
  if (!(isfinite(beta_lo) && isfinite(beta_hi) && beta_lo <= beta_hi)) return HUBKV_EINVAL;
  if (!(r >= 0.f && r <= 1.f)) return HUBKV_EINVAL;
  if ((rc = check_kept(st, kept, n_sink, n_recent, true))) return rc;
  const int64_t K = kept_total(st);
  if (!s || !z || !aligned(s, 4) || !aligned(z, 4) || (K > 0 && (!idx || !aligned(idx, 4))))
    return HUBKV_EALIGN;
  if ((head_stats && !aligned(head_stats, 8)) || (beta_in && !aligned(beta_in, 4)) ||
      (beta_out && !aligned(beta_out, 4)))
    return HUBKV_EALIGN;
  int64_t T = 0;
  for (int b = 0; b < B; ++b) T += st.N[b];
  const uintptr_t n = (uintptr_t)((int64_t)L * Hkv * T) * sizeof(float);
  if ((uintptr_t)s < (uintptr_t)z + n && (uintptr_t)z < (uintptr_t)s + n) return HUBKV_EINVAL;
  const RefineGeom rg = refine_geometry(rt, L, Hkv);
  const size_t roff = (rg.bytes + 255) & ~(size_t)255;
  const bool many = K > 0 && msel_fits(st, L, Hkv);
  const MselGeom geo = many ? msel_geometry(st, L, Hkv) : MselGeom{};
  if (!workspace || workspace_bytes < roff + (many ? geo.bytes : 256)) return HUBKV_EWORKSPACE;
  if (!aligned(workspace, 256)) return HUBKV_EALIGN;
  char* ws = (char*)workspace;
  hipStream_t strm = (hipStream_t)stream;
  const double* stats = head_stats;
  if (!beta_in && !stats) {
    double* st_ws = (double*)(ws + rg.off_stats);
    rc = hip_status(launch_head_stats(s, rt, L, Hkv, (double*)(ws + rg.off_part), st_ws, strm));
    if (rc) return rc;
    stats = st_ws;
  }
  const float r2 = r * r;  // fp32 product, as the gate formula is evaluated in fp32
  if (!many) {
    rc = hip_status(launch_refine(s, rt, L, Hkv, stats, beta_in, pool, gamma, beta_lo, beta_hi,
                                  r2, z, beta_out, strm));
    if (rc || K == 0) return rc;  // nothing kept: z is the whole result
    return hip_status(launch_select(z, st, L, Hkv, n_sink, n_recent, idx, strm));
  }
  const RefineParams rp{pool, gamma, r2, beta_lo, beta_hi, beta_in, stats, beta_out};
  return hip_status(launch_msel(s, true, z, st, L, Hkv, n_sink, n_recent, rp, idx, ws + roff, geo,
                                strm));
}

int hubkv_compact_strided(const void* k_in, const int64_t* k_in_strides, const void* v_in,
                          const int64_t* v_in_strides, int dtype, const int32_t* idx, int B,
                          const int64_t* seqlens, const int64_t* kept, int L, int Hkv, int d,
                          void* k_out, const int64_t* k_out_strides, void* v_out,
                          const int64_t* v_out_strides, void* stream) {
  int rc = check_dtype_d(dtype, d);
  if (rc) return rc;
  SeqTable st;
  if ((rc = make_table(st, B, seqlens, kRefineTile))) return rc;
  if (L < 1 || Hkv < 1 || (int64_t)L * Hkv > kMaxGridY) return HUBKV_EINVAL;
  if ((rc = check_kept(st, kept, 0, 0, false))) return rc;
  int64_t T = 0, K = 0;
  for (int b = 0; b < B; ++b) {
    T += st.N[b];
    K += st.kept[b];
  }
  const int esize = dtype == HUBKV_BF16 ? 2 : 4;
  const int64_t in_ext[3] = {L, Hkv, T}, out_ext[3] = {L, Hkv, K};
  if ((rc = check_strides(k_in_strides, in_ext, esize, d, false))) return rc;
  if ((rc = check_strides(v_in_strides, in_ext, esize, d, false))) return rc;
  if ((rc = check_strides(k_out_strides, out_ext, esize, d, true))) return rc;
  if ((rc = check_strides(v_out_strides, out_ext, esize, d, true))) return rc;
  if (K == 0) return HUBKV_OK;  // nothing kept: no row to move
  if (!k_in || !v_in || !k_out || !v_out || !idx) return HUBKV_EALIGN;
  if (!aligned(k_in, 16) || !aligned(v_in, 16) || !aligned(k_out, 16) || !aligned(v_out, 16) ||
      !aligned(idx, 4))
    return HUBKV_EALIGN;
  const int per = 16 / esize;  // elements per 16-byte unit
  auto rows = [per](const int64_t* x) { return RowStrides{x[0] / per, x[1] / per, x[2] / per}; };
  return hip_status(launch_compact(k_in, v_in, esize, idx, st, L, Hkv, d, rows(k_in_strides),
                                   rows(v_in_strides), rows(k_out_strides), rows(v_out_strides),
                                   k_out, v_out, (hipStream_t)stream));
}

int hubkv_compact(const void* k_in, const void* v_in, int dtype, const int32_t* idx, int B,
                  const int64_t* seqlens, const int64_t* kept, int L, int Hkv, int d, void* k_out,
                  void* v_out, void* stream) {
  int rc = check_dtype_d(dtype, d);
  if (rc) return rc;
  if (B < 1 || B > kMaxSeqs || !seqlens || !kept) return HUBKV_EINVAL;
  if (L < 1 || Hkv < 1 || (int64_t)L * Hkv > kMaxGridY) return HUBKV_EINVAL;
  int64_t T = 0, K = 0;
  for (int b = 0; b < B; ++b) {
    if (seqlens[b] < 1 || seqlens[b] >= kMaxSeqLen || kept[b] < 0 || kept[b] > seqlens[b])
      return HUBKV_EINVAL;
    T += seqlens[b];
    K += kept[b];
  }
  const int64_t is[3] = {(int64_t)Hkv * T * d, T * d, d};
  const int64_t os[3] = {(int64_t)Hkv * K * d, K * d, d};
  return hubkv_compact_strided(k_in, is, v_in, is, dtype, idx, B, seqlens, kept, L, Hkv, d, k_out,
                               os, v_out, os, stream);
}

size_t hubkv_select_layer_workspace(int B, const int64_t* seqlens, int L, int Hkv) {
  if (B < 1 || B > kMaxSeqs || !seqlens || L < 1 || Hkv < 1 || Hkv > 1024) return 0;
  if ((int64_t)L * B > kMaxLayerSegs || (int64_t)L * Hkv > kMaxGridY) return 0;
  LselArgs a;
  memset(&a, 0, sizeof(a));
  a.B = B;
  a.L = L;
  a.Hkv = Hkv;
  int64_t ch = 0;
  for (int b = 0; b < B; ++b) {
    if (seqlens[b] < 1 || seqlens[b] >= kMaxSeqLen) return 0;
    ch += (seqlens[b] + kLselChunk - 1) / kLselChunk;
  }
  if (ch > 65535) return 0;
  a.nchunk = (int)ch;
  return lsel_geometry(a).bytes;
}

int hubkv_select_layer(const float* z, int B, const int64_t* seqlens, int L, int Hkv,
                       const int64_t* layer_kept, int n_sink, int n_recent, int floor_min,
                       int32_t* idx, int32_t* head_kept, void* workspace, size_t workspace_bytes,
                       void* stream) {
  LselArgs a;
  int rc = make_lsel(a, B, seqlens, L, Hkv, layer_kept, n_sink, n_recent, floor_min);
  if (rc) return rc;
  int64_t K = 0;
  for (int i = 0; i < L * B; ++i) K += layer_kept[i];
  if (!z || !head_kept || !workspace || (K > 0 && !idx)) return HUBKV_EALIGN;
  if (!aligned(z, 4) || (idx && !aligned(idx, 4)) || !aligned(head_kept, 4) ||
      !aligned(workspace, 256))
    return HUBKV_EALIGN;
  const LselGeom g = lsel_geometry(a);
  if (workspace_bytes < g.bytes) return HUBKV_EWORKSPACE;
  return hip_status(launch_select_layer(z, a, g, (char*)workspace, idx, head_kept,
                                        (hipStream_t)stream));
}

int hubkv_compact_layer(const void* k_in, const void* v_in, int dtype, const int32_t* idx,
                        const int32_t* head_kept, int B, const int64_t* seqlens, int L, int Hkv,
                        const int64_t* layer_kept, int d, void* k_out, void* v_out, void* stream) {
  int rc = check_dtype_d(dtype, d);
  if (rc) return rc;
  LselArgs a;
  // the budgets only set the row offsets here: no floor or window bound applies
  if ((rc = make_lsel(a, B, seqlens, L, Hkv, layer_kept, 0, 0, 0))) return rc;
  int64_t K = 0;
  for (int i = 0; i < L * B; ++i) K += layer_kept[i];
  if (K == 0) return HUBKV_OK;  // nothing kept: no row to move
  if (!k_in || !v_in || !k_out || !v_out || !idx || !head_kept) return HUBKV_EALIGN;
  if (!aligned(k_in, 16) || !aligned(v_in, 16) || !aligned(k_out, 16) || !aligned(v_out, 16) ||
      !aligned(idx, 4) || !aligned(head_kept, 4))
    return HUBKV_EALIGN;
  return hip_status(launch_compact_layer(k_in, v_in, dtype == HUBKV_BF16 ? 2 : 4, idx, head_kept,
                                         a, d, k_out, v_out, (hipStream_t)stream));
}

size_t hubkv_nestedkv_workspace(int B, const int64_t* seqlens, int L, int Hkv, int d, int nblocks) {
  if (d != 64 && d != 128) return 0;
  NkvArgs a;
  if (make_nkv(a, B, seqlens, L, Hkv, d, nblocks) != HUBKV_OK) return 0;
  return nkv_geometry(a).bytes;
}

int hubkv_nestedkv(const void* k, int dtype, int B, const int64_t* seqlens, int L, int Hkv, int d,
                   int nblocks, int window, const float* log_prior, float theta, float* s,
                   float* anomalies, float* weights, void* workspace, size_t workspace_bytes,
                   void* stream) {
  int rc = check_dtype_d(dtype, d);
  if (rc) return rc;
  NkvArgs a;
  if ((rc = make_nkv(a, B, seqlens, L, Hkv, d, nblocks))) return rc;
  if (window != 64 || !isfinite(theta)) return HUBKV_EINVAL;
  for (int x = 0; x < 3; ++x) {
    a.prior[x] = log_prior ? log_prior[x] : 0.f;
    if (!isfinite(a.prior[x])) return HUBKV_EINVAL;
  }
  a.theta = theta;
  if (!k || !s || !workspace) return HUBKV_EALIGN;
  if (!aligned(k, 16) || !aligned(s, 4) || !aligned(workspace, 256) ||
      (anomalies && !aligned(anomalies, 4)) || (weights && !aligned(weights, 4)))
    return HUBKV_EALIGN;
  const NkvGeom g = nkv_geometry(a);
  if (workspace_bytes < g.bytes) return HUBKV_EWORKSPACE;
  return hip_status(launch_nestedkv(k, dtype, a, g, (char*)workspace, anomalies, s, weights,
                                    (hipStream_t)stream));
}


int h2o_step(const void* q, const void* k_new, const void* v_new, int dtype, void* k_cache,
             void* v_cache, float* acc, int32_t* pos, const int64_t* t, int B, int Hq, int Hkv,
             int d, int C, int n_sink, int n_recent, float scale, int include_self,
             int32_t* evicted, float* probs, float* out, void* stream) {
  return h2o_impl(q, k_new, v_new, dtype, k_cache, v_cache, acc, pos, t, B, Hq, Hkv, d, C, n_sink,
                  n_recent, scale, include_self, evicted, probs, out, stream, 0);
}

int h2o_step_ring(const void* q, const void* k_new, const void* v_new, int dtype, void* k_cache,
                  void* v_cache, float* acc, int32_t* pos, const int64_t* t, int B, int Hq,
                  int Hkv, int d, int C, int n_sink, int n_recent, float scale, int include_self,
                  int32_t* evicted, float* probs, float* out, void* stream) {
  return h2o_impl(q, k_new, v_new, dtype, k_cache, v_cache, acc, pos, t, B, Hq, Hkv, d, C, n_sink,
                  n_recent, scale, include_self, evicted, probs, out, stream, 1);
}

}  // extern "C"
