// score.hip -- base retention score: attention mass of an observation window.
//
// For every (layer l, sequence b, KV head g) and every key i of the sequence:
//   s_i = sum over the G query heads of the group and the W window rows w of
//         softmax_i(scale * q_{h,w} . k_i)      (keys i <= N - W + w if causal)
// H2O breakdown page, "Observation 2" (accumulated attention probability of a
// token over query positions); KV-cache survey page, section 1.1 (the softmax
// of q K^T / sqrt(d_head)) and section 3.3 (GQA: the heads of a group share a
// KV head, so their probabilities add up on it).
//
// Column sums need each row's softmax normaliser, which depends on every key
// of the row, so the keys are swept twice and nothing of size rows x keys is
// ever stored:
//   pass 1  per work-group chunk of keys and per query row, the running
//           maximum m and sum l of exp2(x - m), x the logit in log2 units;
//   fold    per row, the chunk partials become M = m + log2(l);
//   pass 2  the logits are recomputed and p = exp2(x - M) is summed down each
//           key column; per-chunk {sum s, sum s ln s} give the head weight.
// bf16 inputs use MFMA (v_mfma_f32_32x32x16_bf16): each wave keeps 64 query
// rows of Q in registers and streams 32-key tiles of K straight from global
// memory, the next tile in flight while the current one is reduced.  Pass 1
// puts keys on the MFMA rows (row statistics become lane-local), pass 2 puts
// queries on the rows (column sums become lane-local).  fp32 inputs use a
// plain VALU path.
#include <mutex>

#include "internal.hpp"

namespace hubkv {

namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kMinit = -1.0e30f;   // finite "no key yet" reference

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  l = l * fast_exp2(m - mn) + l2 * fast_exp2(m2 - mn);
  m = mn;
}

struct ScoreArgs {
  int L, Hq, Hkv, G, W, M, Mpad, chunk, nchunk, causal;
  int64_t T;
  int64_t qsl, qsh, qsr;  // Q element strides: layer, query head, window row
  int64_t ksl, ksh, kst;  // K element strides: layer, KV head, token
  float c2;  // scale * log2(e)
};

}  // namespace

// --------------------------------------------------------------------------
// Geometry
// --------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int score_chunk(int B, const int64_t* seqlens, int64_t units, int rows, int dtype) {
  if (dtype != 1) return kScoreChunkF32;
  // Chunks in multiples of 1024 keys, chosen to minimise the makespan
  // (rounds of kScoreGroups work-groups) x (chunk + a fixed start-up cost of
  // kScoreStartKeys keys): long runs of K tiles per wave, about one
  // work-group per compute unit, no straggling second round.  On the
  // Llama-2-7B-shaped layer 4096-key chunks (256 work-groups) measured
  // 102 us for the score op against 131 us with 1024-key chunks.
  int64_t mx = 0;
  for (int b = 0; b < B; ++b) mx = seqlens[b] > mx ? seqlens[b] : mx;
  if (units < 1) units = 1;
  // work-groups of several 64-row groups are MFMA-heavy and want two waves
  // per SIMD: a round then holds as many of them as fit two per SIMD
  const int nrg = (rows + 63) / 64;
  const int64_t per_round = nrg >= 2 ? kScoreGroups * (8 / nrg > 1 ? 8 / nrg : 1) : kScoreGroups;
  const int64_t top = (mx + kScoreChunkMfma - 1) / kScoreChunkMfma;
  int64_t best_c = kScoreChunkMfma, best_cost = INT64_MAX;
  for (int64_t m = 1; m <= top && m <= ((int64_t)1 << 20); ++m) {
    const int64_t c = m * kScoreChunkMfma;
    int64_t groups = 0;
    for (int b = 0; b < B; ++b) groups += (seqlens[b] + c - 1) / c;
    groups *= units;
    const int64_t rounds = (groups + per_round - 1) / per_round;
    const int64_t cost = rounds * (c + kScoreStartKeys);
    if (cost < best_cost) {
      best_cost = cost;
      best_c = c;
    }
  }
  return (int)best_c;
}

ScoreGeom score_geometry(const SeqTable& st, int L, int Hq, int Hkv, int W, int d, int dtype) {
  (void)d;
  (void)dtype;
  ScoreGeom g{};
  g.M = (Hq / Hkv) * W;
  g.Mpad = ((g.M + 63) / 64) * 64;
  g.chunk = st.tile;
  g.nchunk = st.tile_off[st.B];
  const size_t LH = (size_t)L * Hkv;
  const size_t U = LH * st.B;
  g.off_part1 = 0;
  g.off_rowstat = align256(LH * g.nchunk * g.Mpad * sizeof(float2));
  g.off_part2 = g.off_rowstat + align256(U * g.Mpad * sizeof(float));
  g.off_ctl = g.off_part2 + align256(LH * g.nchunk * 2 * sizeof(double));
  g.bytes = g.off_ctl + align256(U * sizeof(int));
  return g;
}

namespace {

// Row r (head-local index h_local * W + w) of query group g, sequence b.
__device__ __forceinline__ const void* q_row_ptr(const void* Q, int esize, const ScoreArgs& a,
                                                 int l, int g, int b, int r) {
  const int hl = r / a.W, w = r - hl * a.W;
  const int h = g * a.G + hl;
  const int64_t off = (int64_t)l * a.qsl + (int64_t)h * a.qsh + ((int64_t)b * a.W + w) * a.qsr;
  return (const char*)Q + off * esize;
}

// First token of sequence b of KV head lh (= l * Hkv + g); token i at + i * kst.
template <typename T>
__device__ __forceinline__ const T* k_head(const T* K, const ScoreArgs& a, const SeqTable& st,
                                           int lh, int b) {
  const int l = lh / a.Hkv, g = lh - l * a.Hkv;
  return K + (int64_t)l * a.ksl + (int64_t)g * a.ksh + st.cu[b] * a.kst;
}

// --------------------------------------------------------------------------
// bf16 MFMA path: two launches over (chunk, layer-head) grids.
//   pass 1: each work-group reduces its chunk to per-row partials (m, l); the
//           unit's (layer-head, sequence) first chunk clears the unit's
//           pass-2 counter.
//   pass 2: each work-group first folds its unit's partials into the row
//           normalisers M = m + log2(l) (every work-group of a unit computes
//           the same values), then recomputes its chunk's logits, sums
//           p = exp2(x - M) down every key column, writes s and its chunk's
//           {sum s, sum s ln s}, and counts itself in; the last one of a unit
//           to count in adds the unit's chunks up in chunk order.
// Nobody waits for anybody (the last one to arrive does the fold), so no
// schedule can deadlock, and no separate clearing launch is needed.  The
// chunk statistics read by the folding work-group go through agent-scope
// coherent accesses, and a counter is bumped only after the writer's stores
// completed (s_waitcnt vmcnt(0)), so no cache write-back or invalidation is
// needed.
// --------------------------------------------------------------------------
__device__ __forceinline__ void st_agent(float2* p, float2 v) {
  __hip_atomic_store((unsigned long long*)p, __builtin_bit_cast(unsigned long long, v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_agent(const float2* p) {
  return __builtin_bit_cast(float2, __hip_atomic_load((const unsigned long long*)p,
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void st_agent(double* p, double v) {
  __hip_atomic_store((unsigned long long*)p, __builtin_bit_cast(unsigned long long, v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double ld_agent(const double* p) {
  return __builtin_bit_cast(double, __hip_atomic_load((const unsigned long long*)p,
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ int bump_agent(int* p) {
  return __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Query fragments of the wave's 64 rows [64 rg, 64 rg + 64): two 32-row tiles
// x D/16 k-steps of v_mfma_f32_32x32x16_bf16.  Lane l holds row l % 32 of the
// tile, head-dimension elements 16 kk + 8 (l / 32) + [0, 8).  The same
// registers serve as the B operand (pass 1, queries as columns) and as the A
// operand (pass 2, queries as rows).
template <int D>
__device__ __forceinline__ void load_q_frags(bf16x8 (&qf)[2][D / 16], const __bf16* Q,
                                             const ScoreArgs& a, const SeqTable& st, int l, int g,
                                             int b, int rg, int lane) {
  const int col8 = (lane >> 5) * 8;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int r = rg * 64 + qt * 32 + (lane & 31);
    if (r < a.M) {
      const __bf16* qr = (const __bf16*)q_row_ptr(Q, 2, a, l, g, b, r);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) qf[qt][kk] = *(const bf16x8*)(qr + kk * 16 + col8);
    } else {
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        bf16x8 z;
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.0f;
        qf[qt][kk] = z;
      }
    }
  }
}

// Last visible key (inclusive) of query row r, clamped to `last`.  Padding
// rows (zero Q, ignored statistics, +inf normaliser) count as fully visible
// so they do not defeat the full-tile fast path.
__device__ __forceinline__ int row_limit(const ScoreArgs& a, int N, int r, int last) {
  if (r >= a.M) return last;
  const int v = a.causal ? (N - a.W + r % a.W) : (N - 1);
  return v < last ? v : last;
}

// Smallest row limit of the wave's 64 rows: tiles ending at or before it need
// no masking.  Uniform, so callers branch on it with scalar control.
__device__ __forceinline__ int wave_min_limit(const ScoreArgs& a, int N, int rg, int lane,
                                              int last) {
  int v = row_limit(a, N, rg * 64 + lane, last);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off));
  return __builtin_amdgcn_readfirstlane(v);
}

// Key fragments of a 32-key tile: lane l holds key `key` = key0 + l % 32,
// elements 16 kk + 8 (l / 32) + [0, 8).  Keys at or past key_end load the
// last valid key instead (always in bounds, no per-lane branch); callers
// mask them.
template <int D>
__device__ __forceinline__ void load_k_frags(bf16x8 (&kf)[D / 16], const __bf16* Kh, int64_t kst,
                                             int64_t key, int64_t key_end, int lane) {
  const int col8 = (lane >> 5) * 8;
  const int64_t row = key < key_end ? key : key_end - 1;
  const __bf16* kr = Kh + row * kst;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) kf[kk] = *(const bf16x8*)(kr + kk * 16 + col8);
}

// Output element j of a 32x32 tile sits at row 8 (j / 4) + 4 (lane / 32) +
// (j % 4) and column lane % 32.
__device__ __forceinline__ int c_row(int j, int lane) {
  return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
}

// Column sums of one 32-key tile over the wave's 64 query rows: logits of
// both 32-row query tiles on v_mfma_f32_32x32x16_bf16 (queries as rows, this
// lane's key as the column), then sum over the lane's 32 rows of
// p = exp2(x c2 - M_row); when MASK, rows whose last visible key (rl, from
// LDS) is below this lane's key are dropped, and so is a key past `last`.
// The lane's rows of a tile are 4 runs of 4 consecutive rows, read from LDS
// as broadcast float4s / int4s.  The two MFMA chains are independent: the second one
// is interleaved with the first one's exponentials, and four partial sums
// keep the exp / add dependency chains short.
template <int D, bool MASK>
__device__ __forceinline__ float tile_col_sums(const bf16x8 (&qf)[2][D / 16],
                                               const bf16x8 (&kf)[D / 16], const float* mr,
                                               const int* rl, float c2, int lane, int key,
                                               int last) {
  constexpr int KS = D / 16;
  f32x16 acc[2] = {{}, {}};
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[0][kk], kf[kk], acc[0], 0, 0, 0);
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[1][kk], kf[kk], acc[1], 0, 0, 0);
  float ps[4];
  // re-read the normalisers every tile rather than holding 32 of them in
  // registers across the loop (the opaque offset keeps them from being hoisted)
  int moff = 4 * (lane >> 5);
  asm volatile("" : "+v"(moff));
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float Mr[16];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4 v = *(const f32x4*)&mr[qt * 32 + 8 * jj + moff];
      Mr[4 * jj] = v[0];
      Mr[4 * jj + 1] = v[1];
      Mr[4 * jj + 2] = v[2];
      Mr[4 * jj + 3] = v[3];
    }
    int Lr[16];
    if constexpr (MASK) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int4 v = *(const int4*)&rl[qt * 32 + 8 * jj + moff];
        Lr[4 * jj] = v.x;
        Lr[4 * jj + 1] = v.y;
        Lr[4 * jj + 2] = v.z;
        Lr[4 * jj + 3] = v.w;
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float p = fast_exp2(fmaf(acc[qt][j], c2, -Mr[j]));
      if constexpr (MASK) p = key <= Lr[j] ? p : 0.f;
      ps[j & 3] = (qt == 0 && j < 4) ? p : ps[j & 3] + p;
    }
  }
  // MFMA(acc1) k-steps interleaved with the VALU work on acc0
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
  }
  const float sum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
  return (!MASK || key <= last) ? sum : 0.f;
}

// Row statistics of one 32-key tile for the wave's 64 query rows: logits on
// v_mfma_f32_32x32x16_bf16 with keys as rows, so lane l holds 16 keys of
// query row l % 32 of each 32-row tile; the lane's running maximum m and sum
// s of exp2(x c2 - m) absorb them (keys past the row's limit lim masked when
// MASK).  As in the column sums, the second MFMA chain is interleaved with
// the first one's VALU work and partial sums keep dependency chains short.
template <int D, bool MASK>
__device__ __forceinline__ void tile_row_stats(const bf16x8 (&qf)[2][D / 16],
                                               const bf16x8 (&kf)[D / 16], float c2, int key0,
                                               const int (&lim)[2], int lane, float (&m)[2],
                                               float (&s)[2]) {
  constexpr int KS = D / 16;
  f32x16 acc[2] = {{}, {}};
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[0][kk], acc[0], 0, 0, 0);
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[1][kk], acc[1], 0, 0, 0);
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    if constexpr (MASK) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (key0 + c_row(j, lane) > lim[qt]) acc[qt][j] = -INFINITY;
    }
    // IEEE maximum (v_maximum3_f32) needs no canonicalising of the MFMA
    // results, unlike fmaxf; logits are finite or -inf here
    float tmax = acc[qt][0];
#pragma unroll
    for (int j = 1; j < 16; ++j) tmax = __builtin_elementwise_maximum(tmax, acc[qt][j]);
    const float mn = fmaxf(m[qt], tmax * c2);
    const float mref = fmaxf(mn, -1.0e30f);  // all keys masked so far: stay at zero
    float ps[4];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float p = fast_exp2(fmaf(acc[qt][j], c2, -mref));
      ps[j & 3] = j < 4 ? p : ps[j & 3] + p;
    }
    s[qt] = fmaf(s[qt], fast_exp2(m[qt] - mref), (ps[0] + ps[1]) + (ps[2] + ps[3]));
    m[qt] = mn;
  }
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
  }
}

// Sweep the 32-key tiles [first, end) with stride STEP, software-pipelined:
// the next tile's loads are issued before the current tile is reduced, so a
// wave keeps HBM requests in flight while it computes.  Every path issues the
// same loads (past-the-end ones are clamped) so the compiler's wait counts
// stay exact; scheduling barriers keep the loads ahead of the arithmetic.
// The tile count is uniform, so the loop runs on scalar control.
template <int D, int STEP, typename F>
__device__ __forceinline__ void sweep_tiles(const __bf16* Kh, int64_t kst, int64_t first,
                                            int64_t end, int lane, F&& body) {
  const int ntile = __builtin_amdgcn_readfirstlane(
      first < end ? (int)((end - first + STEP - 1) / STEP) : 0);
  if (ntile == 0) return;
  bf16x8 ka[D / 16], kb[D / 16];
  load_k_frags<D>(ka, Kh, kst, first + (lane & 31), end, lane);
  for (int it = 0; it < ntile; it += 2) {
    const int64_t key0 = first + (int64_t)it * STEP;
    load_k_frags<D>(kb, Kh, kst, key0 + STEP + (lane & 31), end, lane);
    __builtin_amdgcn_sched_barrier(0);
    body(ka, key0);
    load_k_frags<D>(ka, Kh, kst, key0 + 2 * STEP + (lane & 31), end, lane);
    __builtin_amdgcn_sched_barrier(0);
    if (it + 1 < ntile) body(kb, key0 + STEP);
  }
}

// Pass-2 prologue: fold every chunk's pass-1 partials of the unit into the
// row normalisers M = m + log2(l), in chunk order (every work-group of the
// unit computes the same values), and the last visible key of every row
// (the whole sequence for padding rows), both into LDS.
__device__ __forceinline__ void fold_row_norms(const float2* __restrict__ part1, const ScoreArgs& a,
                                               const SeqTable& st, int lh, int b, int nch, int N,
                                               int tid, int nthreads, float* mrow, int* rlim) {
  const float2* pp = part1 + ((int64_t)lh * a.nchunk + st.tile_off[b]) * a.Mpad;
  for (int r = tid; r < a.Mpad; r += nthreads) {
    float mm = kMinit, ss = 0.f;
    for (int cc = 0; cc < nch; cc += 8) {
      float2 pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pv[e] = cc + e < nch ? pp[(int64_t)(cc + e) * a.Mpad + r] : make_float2(kMinit, 0.f);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (pv[e].y > 0.f) merge_ml(mm, ss, pv[e].x, pv[e].y);
    }
    mrow[r] = (r < a.M && ss > 0.f) ? mm + __builtin_amdgcn_logf(ss) : INFINITY;
    rlim[r] = row_limit(a, N, r, N - 1);
  }
}

// Pass-2 epilogue: the work-group's {sum s, sum s ln s} (per-thread doubles)
// are reduced, published for its chunk, and the unit's last chunk to count
// in adds all chunks up in chunk order into the head statistics.
template <int WAVES>
__device__ __forceinline__ void finish_chunk_stats(double hs, double ha, double2* hred,
                                                   double2* __restrict__ part2, int* done,
                                                   const ScoreArgs& a, const SeqTable& st, int lh,
                                                   int chunk_g, int b, int nch, int l, int g,
                                                   double* __restrict__ stats, int tid, int lane,
                                                   int wave) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    hs += __shfl_xor(hs, off);
    ha += __shfl_xor(ha, off);
  }
  if (lane == 0) hred[wave] = make_double2(hs, ha);
  __syncthreads();
  if (tid == 0) {
    double S = 0.0, A = 0.0;
    for (int w = 0; w < WAVES; ++w) {
      S += hred[w].x;
      A += hred[w].y;
    }
    double* p2w = (double*)&part2[(int64_t)lh * a.nchunk + chunk_g];
    st_agent(p2w, S);
    st_agent(p2w + 1, A);
    wait_stores();
    if (bump_agent(done) == nch - 1 && stats) {
      // the unit's last chunk: head statistics, chunks added in order
      double S2 = 0.0, A2 = 0.0;
      const double* p2 = (const double*)(part2 + (int64_t)lh * a.nchunk + st.tile_off[b]);
      // eight chunks' loads in flight at a time (clamped, always in bounds),
      // then added in chunk order
      for (int c0 = 0; c0 < nch; c0 += 8) {
        double sv[8], av[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int cc = c0 + e < nch ? c0 + e : nch - 1;
          sv[e] = ld_agent(p2 + 2 * cc);
          av[e] = ld_agent(p2 + 2 * cc + 1);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (c0 + e < nch) {
            S2 += sv[e];
            A2 += av[e];
          }
        }
      }
      const int64_t su = (((int64_t)l * st.B + b) * a.Hkv + g) * 2;
      stats[su] = S2;
      stats[su + 1] = A2;
    }
  }
}

template <int D, int NRG, int NKG, int PHASE>
__global__ __launch_bounds__(64 * NRG * NKG, 2) void score_pass_mfma(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, SeqTable st, ScoreArgs a,
    int* __restrict__ ctl, float2* __restrict__ part1, double2* __restrict__ part2,
    float* __restrict__ s_out, double* __restrict__ stats) {
  constexpr int TH = 64 * NRG * NKG;
  constexpr int WAVES = NRG * NKG;
  constexpr int STEP = 32 * NKG;
  constexpr int KS = D / 16;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int rg = wave % NRG, kg = wave / NRG;
  const int lh = blockIdx.y, chunk_g = blockIdx.x;
  const int b = seq_of_tile(st, chunk_g);
  const int c = chunk_g - st.tile_off[b];
  const int u = lh * st.B + b;
  const int l = lh / a.Hkv, g = lh - l * a.Hkv;
  const int nch = st.tile_off[b + 1] - st.tile_off[b];
  const int N = (int)st.N[b];
  const int64_t key_begin = (int64_t)c * a.chunk;
  const int64_t key_end = key_begin + a.chunk < N ? key_begin + a.chunk : N;
  const __bf16* Kh = k_head(K, a, st, lh, b);

  static_assert(NRG == 1, "several row groups use score_pass_shared");

  bf16x8 qf[2][KS];
  load_q_frags<D>(qf, Q, a, st, l, g, b, rg, lane);

  if constexpr (PHASE == 1) {
    // ---- pass 1: keys as MFMA rows, queries as columns: lane l owns query
    // row 64 rg + 32 qt + l % 32 and 16 of the tile's keys, so the running
    // row maximum and sum are lane-local.
    __shared__ float2 red[NKG][64 * NRG];
    const int last = (int)key_end - 1;
    const int minlim = wave_min_limit(a, N, rg, lane, last);
    int lim[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) lim[qt] = row_limit(a, N, rg * 64 + qt * 32 + (lane & 31), last);
    float m[2] = {-INFINITY, -INFINITY}, s[2] = {0.f, 0.f};
    auto body1 = [&](const bf16x8 (&kf)[KS], int64_t key0) {
      // fully visible tiles (nearly all) and masked ones get separate
      // straight-line copies
      if ((int)key0 + 31 <= minlim)
        tile_row_stats<D, false>(qf, kf, a.c2, (int)key0, lim, lane, m, s);
      else
        tile_row_stats<D, true>(qf, kf, a.c2, (int)key0, lim, lane, m, s);
    };
    sweep_tiles<D, STEP>(Kh, a.kst, key_begin + kg * 32, key_end, lane, body1);
    // lanes l and l + 32 hold the same rows over different keys
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float m2 = __shfl_xor(m[qt], 32), s2 = __shfl_xor(s[qt], 32);
      const float mn = fmaxf(m[qt], m2);
      const float mref = fmaxf(mn, -1.0e30f);
      s[qt] = s[qt] * fast_exp2(m[qt] - mref) + s2 * fast_exp2(m2 - mref);
      m[qt] = mn;
      if (lane < 32) red[kg][rg * 64 + qt * 32 + lane] = make_float2(fmaxf(m[qt], kMinit), s[qt]);
    }
    __syncthreads();
    // wave 0 publishes the chunk's partials (read by pass 2, after this
    // launch); the unit's first chunk also clears the unit's pass-2 counter
    if (wave == 0) {
      for (int rl = lane; rl < a.Mpad; rl += 64) {
        float mm = red[0][rl].x, ss = red[0][rl].y;
#pragma unroll
        for (int q = 1; q < NKG; ++q) merge_ml(mm, ss, red[q][rl].x, red[q][rl].y);
        part1[((int64_t)lh * a.nchunk + chunk_g) * a.Mpad + rl] = make_float2(mm, ss);
      }
      if (c == 0 && lane == 0) ctl[u] = 0;
    }
  } else {
    // ---- pass 2: queries as MFMA rows, keys as columns: lane l owns key
    // key0 + l % 32 and 16 rows of each query tile, so a column sum is a
    // lane-local sum plus one exchange between the two half-waves.  With one
    // row group that sum is final: the low half-wave stores it at once and
    // keeps its chunk statistics in registers (no LDS pass, no barrier).
    __shared__ double2 hred[WAVES];
    // row normalisers in LDS: a lane's 16 rows of a query tile are 4 runs of
    // 4 consecutive rows, the same for every lane of a half-wave, so they are
    // read as broadcast float4s instead of being held in 32 registers
    __shared__ __attribute__((aligned(16))) float mrow[64 * NRG];
    // last visible key of every row (the whole sequence for padding rows)
    __shared__ __attribute__((aligned(16))) int rlim[64 * NRG];
    fold_row_norms(part1, a, st, lh, b, nch, N, tid, TH, mrow, rlim);
    __syncthreads();
    double hs = 0.0, ha = 0.0;
    float* so = s_out + (int64_t)lh * a.T + st.cu[b];
    const int last = (int)key_end - 1;
    const int minlim = wave_min_limit(a, N, rg, lane, last);
    auto body2 = [&](const bf16x8 (&kf)[KS], int64_t key0) {
      const int key = (int)key0 + (lane & 31);
      // fully visible tiles (nearly all) and masked ones get separate
      // straight-line copies, so the scheduler can overlap the second MFMA
      // chain with the first chain's exponentials
      float cv;
      if ((int)key0 + 31 <= minlim)
        cv = tile_col_sums<D, false>(qf, kf, mrow + rg * 64, rlim + rg * 64, a.c2, lane, key,
                                     last);
      else
        cv = tile_col_sums<D, true>(qf, kf, mrow + rg * 64, rlim + rg * 64, a.c2, lane, key,
                                    last);
      cv += __shfl_xor(cv, 32);
      if (lane < 32 && key <= last) {
        so[key] = cv;
        hs += (double)cv;
        if (cv > 0.f) ha += (double)cv * (double)(__builtin_amdgcn_logf(cv) * kLn2);
      }
    };
    sweep_tiles<D, STEP>(Kh, a.kst, key_begin + kg * 32, key_end, lane, body2);
    finish_chunk_stats<WAVES>(hs, ha, hred, part2, ctl + u, a, st, lh, chunk_g, b, nch, l, g,
                              stats, tid, lane, wave);
  }
}

// --------------------------------------------------------------------------
// Several 64-row query groups (G * W > 64): the work-group's NRG waves (one
// per row group) share every K tile.  Keys are processed in stages of 32
// NRG; wave w brings tile w of the next stage straight from global memory
// into LDS (global_load_lds_dwordx4: 16 bytes per lane, 1 KiB per
// instruction, no staging registers) while all waves reduce the current
// stage's tiles for their own rows, reading MFMA fragments from LDS.  Stages
// are double-buffered, one barrier per stage.  Within a tile's LDS image,
// 16-byte piece p of key row r sits at slot p ^ (r mod pieces-per-row), so
// the 32 lanes that read the same piece of 32 rows spread over the banks.
// Pass 2 writes each stage's per-row-group column sums to LDS (also double
// buffered) and reduces them after the stage barrier.
// --------------------------------------------------------------------------
typedef const __attribute__((address_space(1))) void* gvoid_p;
typedef __attribute__((address_space(3))) void* lvoid_p;

template <int D, int NRG, int PHASE>
__global__ __launch_bounds__(64 * NRG, 2) void score_pass_shared(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, SeqTable st, ScoreArgs a,
    int* __restrict__ ctl, float2* __restrict__ part1, double2* __restrict__ part2,
    float* __restrict__ s_out, double* __restrict__ stats) {
  constexpr int TH = 64 * NRG;
  constexpr int KS = D / 16;
  constexpr int PPR = 2 * D / 16;  // 16-byte pieces per key row
  constexpr int RB = 2 * D;        // key row bytes
  constexpr int TILEB = 32 * RB;   // one 32-key tile
  constexpr int RPI = 64 / PPR;    // key rows per DMA instruction
  constexpr int NI = 32 / RPI;     // DMA instructions per tile
  constexpr int SK = 32 * NRG;     // keys per stage
  __shared__ __attribute__((aligned(1024))) char kbuf[2][NRG * TILEB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave;
  const int lh = blockIdx.y, chunk_g = blockIdx.x;
  const int b = seq_of_tile(st, chunk_g);
  const int c = chunk_g - st.tile_off[b];
  const int u = lh * st.B + b;
  const int l = lh / a.Hkv, g = lh - l * a.Hkv;
  const int nch = st.tile_off[b + 1] - st.tile_off[b];
  const int N = (int)st.N[b];
  const int64_t key_begin = (int64_t)c * a.chunk;
  const int64_t key_end = key_begin + a.chunk < N ? key_begin + a.chunk : N;
  const __bf16* Kh = k_head(K, a, st, lh, b);
  const int nst = __builtin_amdgcn_readfirstlane((int)((key_end - key_begin + SK - 1) / SK));

  // wave w's tile of the stage at s0 into buffer `buf`; rows past the end
  // load the last key (always in bounds) and are masked by the callers
  const int drow = lane / PPR, dslot = lane % PPR;
  auto dma = [&](int64_t s0, int buf) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = RPI * i + drow;
      const int piece = dslot ^ (r & (PPR - 1));
      int64_t key = s0 + 32 * wave + r;
      key = key < key_end ? key : key_end - 1;
      __builtin_amdgcn_global_load_lds((gvoid_p)(Kh + key * a.kst + piece * 8),
                                       (lvoid_p)(kbuf[buf] + wave * TILEB + i * 1024), 16, 0,
                                       0);
    }
  };
  // MFMA fragments of tile t: lane l takes row l % 32, pieces 2 kk + l / 32
  auto frags = [&](int buf, int t, bf16x8 (&kf)[KS]) {
    const int r = lane & 31;
    const char* row = kbuf[buf] + t * TILEB + r * RB;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int piece = 2 * kk + (lane >> 5);
      kf[kk] = *(const bf16x8*)(row + 16 * (piece ^ (r & (PPR - 1))));
    }
  };

  if (nst > 0) dma(key_begin, 0);
  bf16x8 qf[2][KS];
  load_q_frags<D>(qf, Q, a, st, l, g, b, rg, lane);
  const int last = (int)key_end - 1;
  const int minlim = wave_min_limit(a, N, rg, lane, last);

  if constexpr (PHASE == 1) {
    __shared__ float2 red[64 * NRG];
    int lim[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) lim[qt] = row_limit(a, N, rg * 64 + qt * 32 + (lane & 31), last);
    float m[2] = {-INFINITY, -INFINITY}, sm[2] = {0.f, 0.f};
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int si = 0; si < nst; ++si) {
      const int buf = si & 1;
      const int64_t s0 = key_begin + (int64_t)si * SK;
      if (si + 1 < nst) dma(s0 + SK, buf ^ 1);
      // unrolled: each tile's LDS offset becomes an instruction immediate
#pragma unroll
      for (int t = 0; t < NRG; ++t) {
        const int64_t key0 = s0 + 32 * t;
        if (key0 >= key_end) break;
        bf16x8 kf[KS];
        frags(buf, t, kf);
        if ((int)key0 + 31 <= minlim)
          tile_row_stats<D, false>(qf, kf, a.c2, (int)key0, lim, lane, m, sm);
        else
          tile_row_stats<D, true>(qf, kf, a.c2, (int)key0, lim, lane, m, sm);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    // lanes l and l + 32 hold the same rows over different keys
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float m2 = __shfl_xor(m[qt], 32), s2 = __shfl_xor(sm[qt], 32);
      const float mn = fmaxf(m[qt], m2);
      const float mref = fmaxf(mn, -1.0e30f);
      sm[qt] = sm[qt] * fast_exp2(m[qt] - mref) + s2 * fast_exp2(m2 - mref);
      m[qt] = mn;
      if (lane < 32) red[rg * 64 + qt * 32 + lane] = make_float2(fmaxf(m[qt], kMinit), sm[qt]);
    }
    __syncthreads();
    for (int rl = tid; rl < a.Mpad; rl += TH)
      part1[((int64_t)lh * a.nchunk + chunk_g) * a.Mpad + rl] = red[rl];
    if (c == 0 && tid == 0) ctl[u] = 0;
  } else {
    __shared__ float csb[2][NRG][SK];
    __shared__ double2 hred[NRG];
    __shared__ __attribute__((aligned(16))) float mrow[64 * NRG];
    __shared__ __attribute__((aligned(16))) int rlim[64 * NRG];
    fold_row_norms(part1, a, st, lh, b, nch, N, tid, TH, mrow, rlim);
    double hs = 0.0, ha = 0.0;
    float* so = s_out + (int64_t)lh * a.T + st.cu[b];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int si = 0; si < nst; ++si) {
      const int buf = si & 1;
      const int64_t s0 = key_begin + (int64_t)si * SK;
      if (si + 1 < nst) dma(s0 + SK, buf ^ 1);
      // unrolled: each tile's LDS offset becomes an instruction immediate
#pragma unroll
      for (int t = 0; t < NRG; ++t) {
        const int64_t key0 = s0 + 32 * t;
        if (key0 >= key_end) break;
        bf16x8 kf[KS];
        frags(buf, t, kf);
        const int key = (int)key0 + (lane & 31);
        float cv;
        if ((int)key0 + 31 <= minlim)
          cv = tile_col_sums<D, false>(qf, kf, mrow + rg * 64, rlim + rg * 64, a.c2, lane, key,
                                       last);
        else
          cv = tile_col_sums<D, true>(qf, kf, mrow + rg * 64, rlim + rg * 64, a.c2, lane, key,
                                      last);
        cv += __shfl_xor(cv, 32);
        if (lane < 32) csb[buf][rg][32 * t + lane] = cv;
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      // this stage's column sums over the row groups (csb[buf] is written
      // again two stages on, after another barrier)
      for (int i = tid; i < SK; i += TH) {
        if (s0 + i >= key_end) break;
        float v = csb[buf][0][i];
#pragma unroll
        for (int q = 1; q < NRG; ++q) v += csb[buf][q][i];
        so[s0 + i] = v;
        hs += (double)v;
        if (v > 0.f) ha += (double)v * (double)(__builtin_amdgcn_logf(v) * kLn2);
      }
    }
    finish_chunk_stats<NRG>(hs, ha, hred, part2, ctl + u, a, st, lh, chunk_g, b, nch, l, g, stats,
                            tid, lane, wave);
  }
}

// --------------------------------------------------------------------------
// fp32 VALU path: one key per thread, query rows staged through LDS in
// groups of 16.
// --------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void score_stats_f32(const float* __restrict__ Q,
                                                       const float* __restrict__ K, SeqTable st,
                                                       ScoreArgs a, float2* __restrict__ part1) {
  __shared__ float qs[16][D];
  __shared__ float red[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lh = blockIdx.y, l = lh / a.Hkv, g = lh % a.Hkv;
  const int chunk_g = blockIdx.x;
  const int b = seq_of_tile(st, chunk_g);
  const int64_t N = st.N[b];
  const int64_t key_begin = (int64_t)(chunk_g - st.tile_off[b]) * a.chunk;
  const int64_t key = key_begin + tid;
  const int64_t key_end = key_begin + a.chunk < N ? key_begin + a.chunk : N;
  const bool have = key < key_end;
  float kr[D];
  const float* kp = k_head(K, a, st, lh, b) + (have ? key : key_begin) * a.kst;
#pragma unroll
  for (int e = 0; e < D; ++e) kr[e] = kp[e];
  for (int r0 = 0; r0 < a.M; r0 += 16) {
    __syncthreads();
    for (int i = tid; i < 16 * D; i += 256) {
      const int rr = r0 + i / D;
      qs[i / D][i % D] =
          rr < a.M ? ((const float*)q_row_ptr(Q, 4, a, l, g, b, rr))[i % D] : 0.f;
    }
    __syncthreads();
    const int rend = min(16, a.M - r0);
    for (int rr = 0; rr < rend; ++rr) {
      const int r = r0 + rr;
      const int w = r % a.W;
      const int64_t lim = a.causal ? (N - a.W + w) : (N - 1);
      const bool vis = have && key <= lim;
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) dot = fmaf(qs[rr][e], kr[e], dot);
      const float x = vis ? dot * a.c2 : -INFINITY;
      float mx = x;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      if (lane == 0) red[0][wave] = mx;
      __syncthreads();
      mx = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
      float e = (vis && mx > -INFINITY) ? fast_exp2(x - mx) : 0.f;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) e += __shfl_xor(e, off);
      if (lane == 0) red[1][wave] = e;
      __syncthreads();
      if (tid == 0) {
        const float sum = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
        part1[((int64_t)lh * a.nchunk + chunk_g) * a.Mpad + r] =
            make_float2(mx > -INFINITY ? mx : kMinit, sum);
      }
      __syncthreads();
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void score_probs_f32(const float* __restrict__ Q,
                                                       const float* __restrict__ K, SeqTable st,
                                                       ScoreArgs a,
                                                       const float* __restrict__ rowstat,
                                                       float* __restrict__ s_out,
                                                       double2* __restrict__ part2) {
  __shared__ float qs[16][D];
  __shared__ float ms[16];
  __shared__ double2 hred[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lh = blockIdx.y, l = lh / a.Hkv, g = lh % a.Hkv;
  const int chunk_g = blockIdx.x;
  const int b = seq_of_tile(st, chunk_g);
  const int64_t N = st.N[b];
  const int64_t key_begin = (int64_t)(chunk_g - st.tile_off[b]) * a.chunk;
  const int64_t key = key_begin + tid;
  const int64_t key_end = key_begin + a.chunk < N ? key_begin + a.chunk : N;
  const bool have = key < key_end;
  float kr[D];
  const float* kp = k_head(K, a, st, lh, b) + (have ? key : key_begin) * a.kst;
#pragma unroll
  for (int e = 0; e < D; ++e) kr[e] = kp[e];
  const float* rs = rowstat + ((int64_t)lh * st.B + b) * a.Mpad;
  float col = 0.f;
  for (int r0 = 0; r0 < a.M; r0 += 16) {
    __syncthreads();
    for (int i = tid; i < 16 * D; i += 256) {
      const int rr = r0 + i / D;
      qs[i / D][i % D] =
          rr < a.M ? ((const float*)q_row_ptr(Q, 4, a, l, g, b, rr))[i % D] : 0.f;
    }
    if (tid < 16) ms[tid] = r0 + tid < a.M ? rs[r0 + tid] : INFINITY;
    __syncthreads();
    const int rend = min(16, a.M - r0);
    for (int rr = 0; rr < rend; ++rr) {
      const int w = (r0 + rr) % a.W;
      const int64_t lim = a.causal ? (N - a.W + w) : (N - 1);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) dot = fmaf(qs[rr][e], kr[e], dot);
      const float p = fast_exp2(dot * a.c2 - ms[rr]);
      col += (have && key <= lim) ? p : 0.f;
    }
  }
  double hs = 0.0, ha = 0.0;
  if (have) {
    s_out[(int64_t)lh * a.T + st.cu[b] + key] = col;
    hs = (double)col;
    if (col > 0.f) ha = (double)col * (double)(__builtin_amdgcn_logf(col) * kLn2);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    hs += __shfl_xor(hs, off);
    ha += __shfl_xor(ha, off);
  }
  if (lane == 0) hred[wave] = make_double2(hs, ha);
  __syncthreads();
  if (tid == 0) {
    double S = 0.0, A = 0.0;
    for (int w = 0; w < 4; ++w) {
      S += hred[w].x;
      A += hred[w].y;
    }
    part2[(int64_t)lh * a.nchunk + chunk_g] = make_double2(S, A);
  }
}

// --------------------------------------------------------------------------
// Fold chunk partials: one thread per (layer-head, sequence, row).
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void score_combine(SeqTable st, ScoreArgs a,
                                                     const float2* __restrict__ part1,
                                                     float* __restrict__ rowstat) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  const int lh = blockIdx.z;
  if (r >= a.Mpad) return;
  float m = kMinit, s = 0.f;
  const int c0 = st.tile_off[b], c1 = st.tile_off[b + 1];
  const float2* pp = part1 + ((int64_t)lh * a.nchunk) * a.Mpad + r;
  for (int c = c0; c < c1; c += 8) {
    float2 p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      p[u] = c + u < c1 ? pp[(int64_t)(c + u) * a.Mpad] : make_float2(kMinit, 0.f);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (p[u].y > 0.f) merge_ml(m, s, p[u].x, p[u].y);
  }
  rowstat[((int64_t)lh * st.B + b) * a.Mpad + r] =
      (r < a.M && s > 0.f) ? m + __builtin_amdgcn_logf(s) : INFINITY;
}

// Per (layer, sequence, KV head): sum the chunk statistics in a fixed order.
__global__ __launch_bounds__(64) void stats_final(SeqTable st, int L, int Hkv, int nchunk,
                                                  const double2* __restrict__ part2,
                                                  double* __restrict__ stats) {
  const int u = blockIdx.x * 64 + threadIdx.x;  // (l * B + b) * Hkv + g
  if (u >= L * st.B * Hkv) return;
  const int g = u % Hkv, b = (u / Hkv) % st.B, l = u / (Hkv * st.B);
  const int lh = l * Hkv + g;
  double S = 0.0, A = 0.0;
  for (int c = st.tile_off[b]; c < st.tile_off[b + 1]; ++c) {
    const double2 p = part2[(int64_t)lh * nchunk + c];
    S += p.x;
    A += p.y;
  }
  stats[(int64_t)u * 2 + 0] = S;
  stats[(int64_t)u * 2 + 1] = A;
}

template <int D>
hipError_t run_f32(const void* q, const void* k, const SeqTable& st, const ScoreArgs& a,
                   float2* part1, float* rowstat, float* s, double2* part2, hipStream_t stream) {
  const dim3 grid(a.nchunk, a.L * a.Hkv);
  hipLaunchKernelGGL((score_stats_f32<D>), grid, dim3(256), 0, stream, (const float*)q,
                     (const float*)k, st, a, part1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(score_combine, dim3((a.Mpad + 255) / 256, st.B, a.L * a.Hkv), dim3(256), 0,
                     stream, st, a, (const float2*)part1, rowstat);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((score_probs_f32<D>), grid, dim3(256), 0, stream, (const float*)q,
                     (const float*)k, st, a, (const float*)rowstat, s, part2);
  return hipGetLastError();
}

template <int D, int NRG, int NKG>
hipError_t run_mfma(const void* q, const void* k, const SeqTable& st, const ScoreArgs& a,
                    char* ws, const ScoreGeom& geo, float* s, double* stats,
                    hipStream_t stream) {
  int* ctl = (int*)(ws + geo.off_ctl);
  const dim3 grid(a.nchunk, a.L * a.Hkv), block(64 * NRG * NKG);
  float2* part1 = (float2*)(ws + geo.off_part1);
  double2* part2 = (double2*)(ws + geo.off_part2);
  hipLaunchKernelGGL((score_pass_mfma<D, NRG, NKG, 1>), grid, block, 0, stream, (const __bf16*)q,
                     (const __bf16*)k, st, a, ctl, part1, part2, s, stats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((score_pass_mfma<D, NRG, NKG, 2>), grid, block, 0, stream, (const __bf16*)q,
                     (const __bf16*)k, st, a, ctl, part1, part2, s, stats);
  return hipGetLastError();
}

template <int D, int NRG>
hipError_t run_shared(const void* q, const void* k, const SeqTable& st, const ScoreArgs& a,
                      char* ws, const ScoreGeom& geo, float* s, double* stats,
                      hipStream_t stream) {
  int* ctl = (int*)(ws + geo.off_ctl);
  const dim3 grid(a.nchunk, a.L * a.Hkv), block(64 * NRG);
  float2* part1 = (float2*)(ws + geo.off_part1);
  double2* part2 = (double2*)(ws + geo.off_part2);
  hipLaunchKernelGGL((score_pass_shared<D, NRG, 1>), grid, block, 0, stream, (const __bf16*)q,
                     (const __bf16*)k, st, a, ctl, part1, part2, s, stats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((score_pass_shared<D, NRG, 2>), grid, block, 0, stream, (const __bf16*)q,
                     (const __bf16*)k, st, a, ctl, part1, part2, s, stats);
  return hipGetLastError();
}

template <int D>
hipError_t dispatch_mfma(const void* q, const void* k, const SeqTable& st, const ScoreArgs& a,
                         char* ws, const ScoreGeom& geo, float* s, double* stats,
                         hipStream_t stream) {
  switch (a.Mpad / 64) {
    case 1: return run_mfma<D, 1, 4>(q, k, st, a, ws, geo, s, stats, stream);
    case 2: return run_shared<D, 2>(q, k, st, a, ws, geo, s, stats, stream);
    case 3: return run_shared<D, 3>(q, k, st, a, ws, geo, s, stats, stream);
    case 4: return run_shared<D, 4>(q, k, st, a, ws, geo, s, stats, stream);
    case 5: return run_shared<D, 5>(q, k, st, a, ws, geo, s, stats, stream);
    case 6: return run_shared<D, 6>(q, k, st, a, ws, geo, s, stats, stream);
    case 7: return run_shared<D, 7>(q, k, st, a, ws, geo, s, stats, stream);
    case 8: return run_shared<D, 8>(q, k, st, a, ws, geo, s, stats, stream);
    default: return hipErrorInvalidValue;  // G*W > 512 is rejected before launch
  }
}

}  // namespace

hipError_t launch_score(const void* q, const void* k, int dtype, const SeqTable& st, int L, int Hq,
                        int Hkv, int W, int d, const ScoreStrides& sd, float scale, int causal,
                        float* s, double* head_stats, char* ws, const ScoreGeom& geo,
                        hipStream_t stream) {
  ScoreArgs a{};
  a.L = L;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.W = W;
  a.M = geo.M;
  a.Mpad = geo.Mpad;
  a.chunk = geo.chunk;
  a.nchunk = geo.nchunk;
  a.causal = causal ? 1 : 0;
  a.T = 0;
  for (int b = 0; b < st.B; ++b) a.T += st.N[b];
  a.qsl = sd.q_l;
  a.qsh = sd.q_h;
  a.qsr = sd.q_r;
  a.ksl = sd.k_l;
  a.ksh = sd.k_h;
  a.kst = sd.k_t;
  a.c2 = (float)((double)scale * 1.4426950408889634);
  if (dtype == 1)
    return d == 128 ? dispatch_mfma<128>(q, k, st, a, ws, geo, s, head_stats, stream)
                    : dispatch_mfma<64>(q, k, st, a, ws, geo, s, head_stats, stream);
  float2* part1 = (float2*)(ws + geo.off_part1);
  float* rowstat = (float*)(ws + geo.off_rowstat);
  double2* part2 = (double2*)(ws + geo.off_part2);
  hipError_t e = d == 128 ? run_f32<128>(q, k, st, a, part1, rowstat, s, part2, stream)
                          : run_f32<64>(q, k, st, a, part1, rowstat, s, part2, stream);
  if (e != hipSuccess || !head_stats) return e;
  const int units = L * st.B * Hkv;
  hipLaunchKernelGGL(stats_final, dim3((units + 63) / 64), dim3(64), 0, stream, st, L, Hkv,
                     geo.nchunk, (const double2*)part2, head_stats);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// Fixed scratch for the allocation-free score entry point.  Each device that
// runs the library holds its own copy of `scratch` until the process ends.
// Host code never passes the array's name to a kernel (on the host it only
// stands for the symbol): the device address comes from hipGetSymbolAddress,
// once per device with that device current, and is kept here.
// --------------------------------------------------------------------------
namespace {

static __device__ __align__(256) char scratch[kScoreScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t score_scratch(hipStream_t stream, char** ptr) {
  *ptr = nullptr;
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream) {
    hipDevice_t sd = 0;
    e = hipStreamGetDevice(stream, &sd);
    if (e != hipSuccess) return e;
    dev = (int)sd;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = (char*)p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace hubkv
