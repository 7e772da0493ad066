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
// of the row.  The work is split in two sweeps over the keys so that nothing
// of size rows x keys is ever stored:
//   pass 1 (stats)   per work-group chunk of keys and per query row, the
//                    running maximum m and sum l of exp2(x - m), x the logit
//                    in log2 units; written as partials;
//   combine          per row, the partials fold into M = m + log2(l);
//   pass 2 (probs)   the logits are recomputed and p = exp2(x - M) is summed
//                    down each key column; per-chunk {sum s, sum s ln s} of
//                    the finished scores are written for the head weight.
// bf16 inputs use MFMA (v_mfma_f32_16x16x32_bf16): each wave keeps 64 query
// rows of Q in registers as A fragments and streams 16-key tiles of K as B
// fragments straight from global memory.  fp32 inputs use a plain VALU path.
#include "internal.hpp"

namespace hubkv {

namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr float kMinit = -1.0e30f;   // finite "no key yet" reference
constexpr float kRescale = 8.0f;     // lazy rescale margin (log2 units)

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2) {
  const float mn = fmaxf(m, m2);
  l = l * fast_exp2(m - mn) + l2 * fast_exp2(m2 - mn);
  m = mn;
}

struct ScoreArgs {
  int L, Hq, Hkv, G, W, M, Mpad, chunk, nchunk, causal;
  int64_t T;
  float c2;  // scale * log2(e)
};

}  // namespace

// --------------------------------------------------------------------------
// Geometry
// --------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

ScoreGeom score_geometry(const SeqTable& st, int L, int Hq, int Hkv, int W, int d, int dtype) {
  (void)d;
  ScoreGeom g{};
  g.M = (Hq / Hkv) * W;
  g.Mpad = ((g.M + 63) / 64) * 64;
  g.chunk = dtype == 1 ? kScoreChunkMfma : kScoreChunkF32;
  g.nchunk = 0;
  for (int b = 0; b < st.B; ++b) g.nchunk += (int)((st.N[b] + g.chunk - 1) / g.chunk);
  const size_t LH = (size_t)L * Hkv;
  g.off_part1 = 0;
  g.off_rowstat = align256(LH * g.nchunk * g.Mpad * sizeof(float2));
  g.off_part2 = g.off_rowstat + align256(LH * st.B * g.Mpad * sizeof(float));
  g.bytes = g.off_part2 + align256(LH * g.nchunk * 2 * sizeof(double));
  return g;
}

namespace {

__device__ __forceinline__ const void* q_row_ptr(const void* Q, int esize, const ScoreArgs& a,
                                                 int l, int g, int B, int b, int r, int D) {
  const int hl = r / a.W, w = r - hl * a.W;
  const int h = g * a.G + hl;
  const int64_t row = ((int64_t)l * a.Hq + h) * ((int64_t)B * a.W) + (int64_t)b * a.W + w;
  return (const char*)Q + row * D * esize;
}

// --------------------------------------------------------------------------
// bf16 MFMA path
// --------------------------------------------------------------------------
// Work-group = NRG x NKG waves.  Wave (rg, kg) owns query rows
// [64 rg, 64 rg + 64) and key tiles kg, kg + NKG, ... of the chunk.
template <int D, int NRG, int NKG>
struct MfmaCfg {
  static constexpr int KS = D / 32;  // k-steps of 32 per MFMA
  static constexpr int WAVES = NRG * NKG;
  static constexpr int THREADS = 64 * WAVES;
};

template <int D, int NRG>
__device__ __forceinline__ void load_q_frags(bf16x8 (&qa)[4][D / 32], const __bf16* Q,
                                             const ScoreArgs& a, const SeqTable& st, int l, int g,
                                             int b, int rg, int lane) {
  const int col8 = (lane >> 4) * 8;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int r = rg * 64 + t * 16 + (lane & 15);
    if (r < a.M) {
      const __bf16* qr = (const __bf16*)q_row_ptr(Q, 2, a, l, g, st.B, b, r, D);
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) qa[t][kk] = *(const bf16x8*)(qr + kk * 32 + col8);
    } else {
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        bf16x8 z;
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.0f;
        qa[t][kk] = z;
      }
    }
  }
}

// Last visible key (inclusive) of each of the lane's 16 output rows, clamped
// to the chunk.
__device__ __forceinline__ void row_limits(int (&lim)[4][4], const ScoreArgs& a, int64_t N,
                                           int rg, int lane, int64_t chunk_last) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = rg * 64 + t * 16 + (lane >> 4) * 4 + j;
      int64_t lm;
      if (r >= a.M) {
        lm = chunk_last;  // padding row: zero Q, ignored stats, +inf normaliser
      } else {
        const int w = r % a.W;
        lm = a.causal ? (N - a.W + w) : (N - 1);
        if (lm > chunk_last) lm = chunk_last;
      }
      lim[t][j] = (int)lm;
    }
}

template <int D>
__device__ __forceinline__ void load_k_frags(bf16x8 (&kb)[D / 32], const __bf16* Kh, int64_t key,
                                             int64_t key_end, int lane) {
  const int col8 = (lane >> 4) * 8;
  if (key < key_end) {
    const __bf16* kr = Kh + key * D;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) kb[kk] = *(const bf16x8*)(kr + kk * 32 + col8);
  } else {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      bf16x8 z;
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.0f;
      kb[kk] = z;
    }
  }
}

template <int D>
__device__ __forceinline__ void mfma_tile(f32x4 (&acc)[4], const bf16x8 (&qa)[4][D / 32],
                                          const bf16x8 (&kb)[D / 32]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[t][kk], kb[kk], c, 0, 0, 0);
    acc[t] = c;
  }
}

template <int D, int NRG, int NKG>
__global__ __launch_bounds__(64 * NRG * NKG) void score_stats_mfma(const __bf16* __restrict__ Q,
                                                                    const __bf16* __restrict__ K,
                                                                    SeqTable st, ScoreArgs a,
                                                                    float2* __restrict__ part1) {
  __shared__ float2 red[NKG][64 * NRG];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rg = wave % NRG, kg = wave / NRG;
  const int lh = blockIdx.y, l = lh / a.Hkv, g = lh % a.Hkv;
  const int chunk_g = blockIdx.x;
  const int b = seq_of_tile(st, chunk_g);
  const int64_t N = st.N[b];
  const int64_t key_begin = (int64_t)(chunk_g - st.tile_off[b]) * a.chunk;
  const int64_t key_end = key_begin + a.chunk < N ? key_begin + a.chunk : N;
  const __bf16* Kh = K + ((int64_t)lh * a.T + st.cu[b]) * D;

  bf16x8 qa[4][D / 32];
  load_q_frags<D, NRG>(qa, Q, a, st, l, g, b, rg, lane);
  int lim[4][4];
  row_limits(lim, a, N, rg, lane, key_end - 1);
  int minlim = lim[0][0];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) minlim = min(minlim, lim[t][j]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) minlim = min(minlim, __shfl_xor(minlim, off));

  float m[4][4], s[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m[t][j] = kMinit;
      s[t][j] = 0.f;
    }

  for (int64_t key0 = key_begin + kg * 16; key0 < key_end; key0 += 16 * NKG) {
    bf16x8 kb[D / 32];
    const int64_t key = key0 + (lane & 15);
    load_k_frags<D>(kb, Kh, key, key_end, lane);
    f32x4 acc[4];
    mfma_tile<D>(acc, qa, kb);
    const bool full = (key0 + 15) <= minlim;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (full || key <= lim[t][j]) {
          const float x = acc[t][j] * a.c2;
          float dl = x - m[t][j];
          if (dl > kRescale) {  // new reference well above the old one
            s[t][j] *= fast_exp2(m[t][j] - x);
            m[t][j] = x;
            dl = 0.f;
          }
          s[t][j] += fast_exp2(dl);
        }
      }
  }
  // fold the 16 key columns of each row (lanes differing in bits 0..3)
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const float m2 = __shfl_xor(m[t][j], off);
        const float s2 = __shfl_xor(s[t][j], off);
        merge_ml(m[t][j], s[t][j], m2, s2);
      }
  if ((lane & 15) == 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rl = rg * 64 + t * 16 + (lane >> 4) * 4 + j;
        red[kg][rl] = make_float2(m[t][j], s[t][j]);
      }
  }
  __syncthreads();
  for (int rl = threadIdx.x; rl < 64 * NRG; rl += 64 * NRG * NKG) {
    float mm = red[0][rl].x, ss = red[0][rl].y;
#pragma unroll
    for (int q = 1; q < NKG; ++q) merge_ml(mm, ss, red[q][rl].x, red[q][rl].y);
    if (rl < a.Mpad)
      part1[((int64_t)lh * a.nchunk + chunk_g) * a.Mpad + rl] = make_float2(mm, ss);
  }
}

template <int D, int NRG, int NKG>
__global__ __launch_bounds__(64 * NRG * NKG) void score_probs_mfma(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, SeqTable st, ScoreArgs a,
    const float* __restrict__ rowstat, float* __restrict__ s_out, double2* __restrict__ part2) {
  constexpr int CK = kScoreChunkMfma;
  __shared__ float cs[NRG][CK];
  __shared__ double2 hred[64 * NRG * NKG / 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rg = wave % NRG, kg = wave / NRG;
  const int lh = blockIdx.y, l = lh / a.Hkv, g = lh % a.Hkv;
  const int chunk_g = blockIdx.x;
  const int b = seq_of_tile(st, chunk_g);
  const int64_t N = st.N[b];
  const int64_t key_begin = (int64_t)(chunk_g - st.tile_off[b]) * a.chunk;
  const int64_t key_end = key_begin + a.chunk < N ? key_begin + a.chunk : N;
  const __bf16* Kh = K + ((int64_t)lh * a.T + st.cu[b]) * D;

  bf16x8 qa[4][D / 32];
  load_q_frags<D, NRG>(qa, Q, a, st, l, g, b, rg, lane);
  int lim[4][4];
  row_limits(lim, a, N, rg, lane, key_end - 1);
  int minlim = lim[0][0];
  float Mr[4][4];
  const float* rs = rowstat + ((int64_t)lh * st.B + b) * a.Mpad;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      minlim = min(minlim, lim[t][j]);
      Mr[t][j] = rs[rg * 64 + t * 16 + (lane >> 4) * 4 + j];
    }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) minlim = min(minlim, __shfl_xor(minlim, off));

  for (int64_t key0 = key_begin + kg * 16; key0 < key_end; key0 += 16 * NKG) {
    bf16x8 kb[D / 32];
    const int64_t key = key0 + (lane & 15);
    load_k_frags<D>(kb, Kh, key, key_end, lane);
    f32x4 acc[4];
    mfma_tile<D>(acc, qa, kb);
    const bool full = (key0 + 15) <= minlim;
    float c = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p = fast_exp2(acc[t][j] * a.c2 - Mr[t][j]);
        c += (full || key <= lim[t][j]) ? p : 0.f;
      }
    c += __shfl_xor(c, 16);
    c += __shfl_xor(c, 32);
    if (lane < 16) cs[rg][key0 - key_begin + lane] = c;
  }
  __syncthreads();
  // finish the column sums, write s, and accumulate the head statistics
  double hs = 0.0, ha = 0.0;
  float* so = s_out + (int64_t)lh * a.T + st.cu[b];
  for (int i = threadIdx.x; i < key_end - key_begin; i += 64 * NRG * NKG) {
    float v = cs[0][i];
#pragma unroll
    for (int q = 1; q < NRG; ++q) v += cs[q][i];
    so[key_begin + i] = v;
    hs += (double)v;
    if (v > 0.f) ha += (double)v * (double)(__builtin_amdgcn_logf(v) * kLn2);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    hs += __shfl_xor(hs, off);
    ha += __shfl_xor(ha, off);
  }
  if (lane == 0) hred[wave] = make_double2(hs, ha);
  __syncthreads();
  if (threadIdx.x == 0) {
    double S = 0.0, A = 0.0;
    for (int w = 0; w < NRG * NKG; ++w) {
      S += hred[w].x;
      A += hred[w].y;
    }
    part2[(int64_t)lh * a.nchunk + chunk_g] = make_double2(S, A);
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
  const float* kp = K + ((int64_t)lh * a.T + st.cu[b] + (have ? key : key_begin)) * D;
#pragma unroll
  for (int e = 0; e < D; ++e) kr[e] = kp[e];
  for (int r0 = 0; r0 < a.M; r0 += 16) {
    __syncthreads();
    for (int i = tid; i < 16 * D; i += 256) {
      const int rr = r0 + i / D;
      qs[i / D][i % D] =
          rr < a.M ? ((const float*)q_row_ptr(Q, 4, a, l, g, st.B, b, rr, D))[i % D] : 0.f;
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
                                                       ScoreArgs a, const float* __restrict__ rowstat,
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
  const float* kp = K + ((int64_t)lh * a.T + st.cu[b] + (have ? key : key_begin)) * D;
#pragma unroll
  for (int e = 0; e < D; ++e) kr[e] = kp[e];
  const float* rs = rowstat + ((int64_t)lh * st.B + b) * a.Mpad;
  float col = 0.f;
  for (int r0 = 0; r0 < a.M; r0 += 16) {
    __syncthreads();
    for (int i = tid; i < 16 * D; i += 256) {
      const int rr = r0 + i / D;
      qs[i / D][i % D] =
          rr < a.M ? ((const float*)q_row_ptr(Q, 4, a, l, g, st.B, b, rr, D))[i % D] : 0.f;
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
    for (int u = 0; u < 8; ++u) p[u] = c + u < c1 ? pp[(int64_t)(c + u) * a.Mpad] : make_float2(kMinit, 0.f);
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

template <int D, int NRG, int NKG>
hipError_t run_mfma(const void* q, const void* k, const SeqTable& st, const ScoreArgs& a,
                    float2* part1, float* rowstat, float* s, double2* part2, hipStream_t stream) {
  constexpr int TH = 64 * NRG * NKG;
  const dim3 grid(a.nchunk, a.L * a.Hkv);
  hipLaunchKernelGGL((score_stats_mfma<D, NRG, NKG>), grid, dim3(TH), 0, stream,
                     (const __bf16*)q, (const __bf16*)k, st, a, part1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(score_combine, dim3((a.Mpad + 255) / 256, st.B, a.L * a.Hkv), dim3(256), 0,
                     stream, st, a, (const float2*)part1, rowstat);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((score_probs_mfma<D, NRG, NKG>), grid, dim3(TH), 0, stream,
                     (const __bf16*)q, (const __bf16*)k, st, a, (const float*)rowstat, s, part2);
  return hipGetLastError();
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

template <int D>
hipError_t dispatch_mfma(const void* q, const void* k, const SeqTable& st, const ScoreArgs& a,
                         float2* part1, float* rowstat, float* s, double2* part2,
                         hipStream_t stream) {
  const int nrg = a.Mpad / 64;
  switch (nrg) {
    case 1: return run_mfma<D, 1, 4>(q, k, st, a, part1, rowstat, s, part2, stream);
    case 2: return run_mfma<D, 2, 2>(q, k, st, a, part1, rowstat, s, part2, stream);
    case 3: return run_mfma<D, 3, 1>(q, k, st, a, part1, rowstat, s, part2, stream);
    case 4: return run_mfma<D, 4, 1>(q, k, st, a, part1, rowstat, s, part2, stream);
    case 5: return run_mfma<D, 5, 1>(q, k, st, a, part1, rowstat, s, part2, stream);
    case 6: return run_mfma<D, 6, 1>(q, k, st, a, part1, rowstat, s, part2, stream);
    case 7: return run_mfma<D, 7, 1>(q, k, st, a, part1, rowstat, s, part2, stream);
    case 8: return run_mfma<D, 8, 1>(q, k, st, a, part1, rowstat, s, part2, stream);
    default: return hipErrorInvalidValue;  // G*W > 512 is rejected before launch
  }
}

}  // namespace

hipError_t launch_score(const void* q, const void* k, int dtype, const SeqTable& st, int L, int Hq,
                        int Hkv, int W, int d, float scale, int causal, float* s,
                        double* head_stats, char* ws, const ScoreGeom& geo, hipStream_t stream) {
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
  a.c2 = (float)((double)scale * 1.4426950408889634);
  float2* part1 = (float2*)(ws + geo.off_part1);
  float* rowstat = (float*)(ws + geo.off_rowstat);
  double2* part2 = (double2*)(ws + geo.off_part2);
  hipError_t e;
  if (dtype == 1) {
    e = d == 128 ? dispatch_mfma<128>(q, k, st, a, part1, rowstat, s, part2, stream)
                 : dispatch_mfma<64>(q, k, st, a, part1, rowstat, s, part2, stream);
  } else {
    e = d == 128 ? run_f32<128>(q, k, st, a, part1, rowstat, s, part2, stream)
                 : run_f32<64>(q, k, st, a, part1, rowstat, s, part2, stream);
  }
  if (e != hipSuccess || !head_stats) return e;
  const int units = L * st.B * Hkv;
  hipLaunchKernelGGL(stats_final, dim3((units + 63) / 64), dim3(64), 0, stream, st, L, Hkv,
                     geo.nchunk, (const double2*)part2, head_stats);
  return hipGetLastError();
}

}  // namespace hubkv
