// refine_select.hip -- HubKV refinement and protected per-head Top-K.
//
// Refinement (HubKV walkthrough, "Method", four steps per head):
//   1 hub_i   <=> s_i equals the max of s over [i - pool/2, i + pool/2] of its
//               own sequence (width-5 max-pooling on the page)
//   2 q_i      = s_i on hubs, gamma * s_i elsewhere (the SMD discount)
//   3 beta_h   = clip(sel_h / mean_heads sel, lo, hi), sel_h the normalised
//               negentropy of the head's scores (a mild selectivity weight)
//   4 z_i      = s_i + r^2 (beta_h q_i - s_i) (the ratio gate)
// Selection (HubKV walkthrough: refined scores feed plain Top-K; H2O breakdown
// page, heavy + recent and per-head sections; KV-cache survey page, sections
// 4.1-4.2: sinks and the recent window are always kept): per (layer, KV head,
// sequence) keep the protected positions and the largest remaining z, ties to
// the lower position, written ascending.
//
// Selection is an exact radix select on order-preserving 32-bit keys of z
// (three histogram passes of 11, 11 and 10 bits in LDS), followed by one
// ordered emission pass in which each wave walks a contiguous segment and
// uses ballots for the in-order ranks of ties and of kept positions.  The
// result is deterministic and independent of thread timing.
#include "internal.hpp"

namespace hubkv {

static size_t align256r(size_t x) { return (x + 255) & ~(size_t)255; }

RefineGeom refine_geometry(const SeqTable& st, int L, int Hkv) {
  RefineGeom g{};
  g.nchunk = 0;
  for (int b = 0; b < st.B; ++b) g.nchunk += (int)((st.N[b] + kRefineTile - 1) / kRefineTile);
  const size_t LH = (size_t)L * Hkv;
  g.off_part = 0;
  g.off_stats = align256r(LH * g.nchunk * 2 * sizeof(double));
  g.off_beta = g.off_stats + align256r((size_t)L * st.B * Hkv * 2 * sizeof(double));
  g.bytes = g.off_beta + align256r((size_t)L * st.B * Hkv * sizeof(float));
  return g;
}

namespace {

constexpr float kLn2f = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Head statistics {sum s, sum s ln s} from a score array (used when the caller
// gives neither statistics nor beta).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void head_stats_partial(const float* __restrict__ s,
                                                          SeqTable st, int64_t T,
                                                          int nchunk, double2* __restrict__ part) {
  __shared__ double2 red[4];
  const int lh = blockIdx.y, c = blockIdx.x;
  const int b = seq_of_tile(st, c);
  const int64_t N = st.N[b];
  const int64_t i0 = (int64_t)(c - st.tile_off[b]) * kRefineTile;
  const float* sb = s + (int64_t)lh * T + st.cu[b];
  double S = 0.0, A = 0.0;
  for (int i = threadIdx.x; i < kRefineTile; i += 256) {
    if (i0 + i < N) {
      const float v = sb[i0 + i];
      S += (double)v;
      if (v > 0.f) A += (double)v * (double)(__builtin_amdgcn_logf(v) * kLn2f);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    S += __shfl_xor(S, off);
    A += __shfl_xor(A, off);
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_double2(S, A);
  __syncthreads();
  if (threadIdx.x == 0) {
    double S2 = 0.0, A2 = 0.0;
    for (int w = 0; w < 4; ++w) {
      S2 += red[w].x;
      A2 += red[w].y;
    }
    part[(int64_t)lh * nchunk + c] = make_double2(S2, A2);
  }
}

__global__ __launch_bounds__(64) void head_stats_final(SeqTable st, int L, int Hkv, int nchunk,
                                                       const double2* __restrict__ part,
                                                       double* __restrict__ stats) {
  const int u = blockIdx.x * 64 + threadIdx.x;  // (l * B + b) * Hkv + g
  if (u >= L * st.B * Hkv) return;
  const int g = u % Hkv, b = (u / Hkv) % st.B, l = u / (Hkv * st.B);
  const int lh = l * Hkv + g;
  double S = 0.0, A = 0.0;
  for (int c = st.tile_off[b]; c < st.tile_off[b + 1]; ++c) {
    const double2 p = part[(int64_t)lh * nchunk + c];
    S += p.x;
    A += p.y;
  }
  stats[(int64_t)u * 2 + 0] = S;
  stats[(int64_t)u * 2 + 1] = A;
}

// Head weight of every (layer, sequence, KV head): one work-group per
// (layer, sequence), one thread per KV head, the mean over heads by shuffles.
constexpr int kMaxHkvBeta = 1024;

__global__ __launch_bounds__(kMaxHkvBeta) void beta_kernel(SeqTable st, int Hkv,
                                                           const double* __restrict__ stats,
                                                           float lo, float hi,
                                                           float* __restrict__ beta) {
  __shared__ double part[kMaxHkvBeta / 64];
  const int lb = blockIdx.x;  // l * B + b
  const int b = lb % st.B;
  const int g = threadIdx.x;
  const double lnN = log((double)st.N[b]);
  double v = 0.0;
  if (g < Hkv) {
    const double S = stats[((int64_t)lb * Hkv + g) * 2], A = stats[((int64_t)lb * Hkv + g) * 2 + 1];
    if (st.N[b] > 1 && S > 0.0) v = 1.0 - (log(S) - A / S) / lnN;
  }
  double sum = v;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = sum;
  __syncthreads();
  if (g >= Hkv) return;
  double mean = 0.0;
  for (int w = 0; w < (int)((blockDim.x + 63) / 64); ++w) mean += part[w];
  mean /= (double)Hkv;
  double bt = 1.0;
  if (mean > 0.0 && isfinite(mean)) {
    bt = v / mean;
    if (bt < (double)lo) bt = (double)lo;
    if (bt > (double)hi) bt = (double)hi;
  }
  beta[(int64_t)lb * Hkv + g] = (float)bt;
}

// ---------------------------------------------------------------------------
// Max-pool hubs + SMD discount + ratio gate; one 1024-token tile of one
// sequence per work-group, staged with its halo in LDS.
// ---------------------------------------------------------------------------
constexpr int kMaxHalf = 31;

// SMD discount and ratio gate as this exact fp32 op sequence (no contraction):
// q = hub ? s : fl(gamma s); z = fma(r2, fl(fl(beta q) - s), s).
__device__ __forceinline__ float smd_gate(float si, bool hub, float gamma, float bt, float r2) {
#pragma clang fp contract(off)
  const float qi = hub ? si : gamma * si;
  const float t = bt * qi;
  const float d = t - si;
  return __builtin_fmaf(r2, d, si);
}

__global__ __launch_bounds__(256) void refine_kernel(const float* __restrict__ s, SeqTable st,
                                                     int64_t T, int Hkv, int half, float gamma,
                                                     float r2, const float* __restrict__ beta,
                                                     float* __restrict__ z,
                                                     float* __restrict__ beta_out) {
  __shared__ float tile[kRefineTile + 2 * kMaxHalf];
  const int lh = blockIdx.y, c = blockIdx.x;
  const int l = lh / Hkv, g = lh % Hkv;
  const int b = seq_of_tile(st, c);
  const int64_t N = st.N[b];
  const int64_t i0 = (int64_t)(c - st.tile_off[b]) * kRefineTile;
  const float* sb = s + (int64_t)lh * T + st.cu[b];
  float* zb = z + (int64_t)lh * T + st.cu[b];
  const int u = (l * st.B + b) * Hkv + g;
  const float bt = beta[u];
  if (beta_out && i0 == 0 && threadIdx.x == 0) beta_out[u] = bt;
  // tile[j] holds s[i0 - half + j]
  for (int j = threadIdx.x; j < kRefineTile + 2 * half; j += 256) {
    const int64_t i = i0 - half + j;
    tile[j] = (i >= 0 && i < N) ? sb[i] : 0.f;
  }
  __syncthreads();
  for (int j = threadIdx.x; j < kRefineTile; j += 256) {
    const int64_t i = i0 + j;
    if (i >= N) break;
    const int64_t lo = i - half < 0 ? 0 : i - half;
    const int64_t hi = i + half > N - 1 ? N - 1 : i + half;
    float mx = tile[lo - i0 + half];
    for (int64_t k = lo + 1; k <= hi; ++k) {
      const float v = tile[k - i0 + half];
      mx = v > mx ? v : mx;
    }
    const float si = tile[j + half];
    zb[i] = smd_gate(si, si == mx, gamma, bt, r2);
  }
}

// ---------------------------------------------------------------------------
// Protected Top-K by radix select.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (v != v) return 0u;             // NaN ranks below everything
  if (u == 0x80000000u) u = 0u;      // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long lanes_below(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Exclusive scan over the kSelWaves wave totals held in shared memory.
__device__ __forceinline__ void wave_totals_scan(uint32_t* v) {
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (int w = 0; w < kSelWaves; ++w) {
      const uint32_t x = v[w];
      v[w] = run;
      run += x;
    }
  }
}

// Keys of candidate positions [a, c) of one (layer, head, sequence): staged in
// LDS when they fit, else read from global memory (z stays in L2).
constexpr int kSelLdsKeys = 36864;  // 144 KiB

template <bool kLds>
struct KeySource {
  const float* zb;
  const uint32_t* lds;
  int64_t a;
  __device__ __forceinline__ uint32_t operator()(int64_t i) const {
    if constexpr (kLds) return lds[i - a];
    else return order_key(zb[i]);
  }
};

template <bool kLds>
__device__ void select_body(const float* __restrict__ zb, int32_t* __restrict__ out, int64_t N,
                            int64_t kept, int n_sink, int n_recent, uint32_t* keys,
                            uint32_t* hist, uint32_t* wt_def, uint32_t* wt_tie, uint32_t* wt_keep,
                            uint32_t* sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // protected: [0, a) and [c, N)
  const int64_t a = n_sink < N ? n_sink : N;
  int64_t c = N - n_recent > 0 ? N - n_recent : 0;
  if (c < a) c = a;
  const int64_t ncand = c - a;
  const int64_t want = kept - (a + (N - c));
  const int mode = (want <= 0) ? 0 : (want >= ncand ? 1 : 2);
  if (kLds && mode == 2) {
    // stage the candidates' order keys, four loads in flight per thread
    for (int64_t i0 = tid; i0 < ncand; i0 += 4 * kSelThreads) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t i = i0 + u * kSelThreads;
        v[u] = i < ncand ? zb[a + i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t i = i0 + u * kSelThreads;
        if (i < ncand) keys[i] = order_key(v[u]);
      }
    }
    __syncthreads();
  }
  const KeySource<kLds> key_at{zb, keys, a};

  uint32_t thr = 0, rem = 0;
  if (mode == 2) {
    uint32_t prefix = 0, pmask = 0;
    uint32_t need = (uint32_t)want;
    const int shifts[3] = {21, 10, 0};
    const int bits[3] = {11, 11, 10};
    for (int pass = 0; pass < 3; ++pass) {
      const int nb = 1 << bits[pass];
      const int shf = shifts[pass];
      for (int i = tid; i < nb; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      for (int64_t i0 = a + tid; i0 < c; i0 += 4 * kSelThreads) {
        uint32_t k4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t i = i0 + u * kSelThreads;
          k4[u] = i < c ? key_at(i) : 0u;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t i = i0 + u * kSelThreads;
          if (i < c && (k4[u] & pmask) == prefix) atomicAdd(&hist[(k4[u] >> shf) & (nb - 1)], 1u);
        }
      }
      __syncthreads();
      // counts above each digit: thread t owns digits [per*t, per*t+per) from the top
      const int per = nb / kSelThreads;  // 2 or 1
      uint32_t mine = 0;
      for (int e = 0; e < per; ++e) mine += hist[nb - 1 - (tid * per + e)];
      uint32_t incl = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      if (lane == 63) wt_def[wave] = incl;
      __syncthreads();
      wave_totals_scan(wt_def);
      __syncthreads();
      uint32_t above = wt_def[wave] + incl - mine;
      for (int e = 0; e < per; ++e) {
        const int dgt = nb - 1 - (tid * per + e);
        const uint32_t cnt = hist[dgt];
        if (above < need && above + cnt >= need) {
          sh[0] = (uint32_t)dgt;
          sh[1] = above;
        }
        above += cnt;
      }
      __syncthreads();
      prefix |= sh[0] << shf;
      pmask |= (uint32_t)(nb - 1) << shf;
      need -= sh[1];
      __syncthreads();
    }
    thr = prefix;
    rem = need;  // ties at the threshold still to take, in position order
  }

  // ordered emission: wave w walks [w * seg, (w + 1) * seg) in 64-position steps
  const int64_t seg = ((N + kSelWaves - 1) / kSelWaves + 63) / 64 * 64;
  const int64_t s0 = wave * seg;
  const int64_t s1 = s0 + seg < N ? s0 + seg : N;
  auto classify = [&](int64_t i, bool& def, bool& tie) {
    def = false;
    tie = false;
    if (i < s1) {
      if (i < a || i >= c || mode == 1) {
        def = true;
      } else if (mode == 2) {
        const uint32_t k = key_at(i);
        def = k > thr;
        tie = k == thr;
      }
    }
  };
  uint32_t n_def = 0, n_tie = 0;
  for (int64_t base = s0; base < s1; base += 64) {
    bool def, tie;
    classify(base + lane, def, tie);
    n_def += (uint32_t)__popcll(__ballot(def));
    n_tie += (uint32_t)__popcll(__ballot(tie));
  }
  if (lane == 0) {
    wt_def[wave] = n_def;
    wt_tie[wave] = n_tie;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t tie_run = 0, out_run = 0;
    for (int w = 0; w < kSelWaves; ++w) {
      const uint32_t ties = wt_tie[w];
      const uint32_t take = tie_run >= rem ? 0u : (rem - tie_run < ties ? rem - tie_run : ties);
      const uint32_t keep = wt_def[w] + take;
      wt_tie[w] = tie_run;
      wt_keep[w] = out_run;
      tie_run += ties;
      out_run += keep;
    }
  }
  __syncthreads();
  uint32_t tie_before = wt_tie[wave], out_pos = wt_keep[wave];
  for (int64_t base = s0; base < s1; base += 64) {
    const int64_t i = base + lane;
    bool def, tie;
    classify(i, def, tie);
    const unsigned long long tb = __ballot(tie);
    const uint32_t rank = tie_before + (uint32_t)__popcll(tb & lanes_below(lane));
    const bool keep = def || (tie && rank < rem);
    const unsigned long long kb = __ballot(keep);
    const uint32_t o = out_pos + (uint32_t)__popcll(kb & lanes_below(lane));
    if (keep && o < (uint32_t)kept) out[o] = (int32_t)i;  // never past this sequence's slice
    tie_before += (uint32_t)__popcll(tb);
    out_pos += (uint32_t)__popcll(kb);
  }
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ z,
                                                             SeqTable st, int64_t T, int64_t Ktot,
                                                             int n_sink, int n_recent,
                                                             int32_t* __restrict__ idx) {
  __shared__ uint32_t keys[kSelLdsKeys];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wt_def[kSelWaves], wt_tie[kSelWaves], wt_keep[kSelWaves];
  __shared__ uint32_t sh[2];
  const int lh = blockIdx.y, b = blockIdx.x;
  const int64_t N = st.N[b];
  const float* zb = z + (int64_t)lh * T + st.cu[b];
  int32_t* out = idx + (int64_t)lh * Ktot + st.ko[b];
  const int64_t a = n_sink < N ? n_sink : N;
  int64_t c = N - n_recent > 0 ? N - n_recent : 0;
  if (c < a) c = a;
  if (c - a <= kSelLdsKeys)
    select_body<true>(zb, out, N, st.kept[b], n_sink, n_recent, keys, hist, wt_def, wt_tie,
                      wt_keep, sh);
  else
    select_body<false>(zb, out, N, st.kept[b], n_sink, n_recent, keys, hist, wt_def, wt_tie,
                       wt_keep, sh);
}

}  // namespace

hipError_t launch_head_stats(const float* s, const SeqTable& st, int L, int Hkv, double* part,
                             double* stats, hipStream_t stream) {
  int64_t T = 0;
  for (int b = 0; b < st.B; ++b) T += st.N[b];
  const int nchunk = st.tile_off[st.B];
  hipLaunchKernelGGL(head_stats_partial, dim3(nchunk, L * Hkv), dim3(256), 0, stream, s, st, T,
                     nchunk, (double2*)part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int units = L * st.B * Hkv;
  hipLaunchKernelGGL(head_stats_final, dim3((units + 63) / 64), dim3(64), 0, stream, st, L, Hkv,
                     nchunk, (const double2*)part, stats);
  return hipGetLastError();
}

hipError_t launch_refine(const float* s, const SeqTable& st, int L, int Hkv,
                         const double* head_stats, const float* beta_in, int pool, float gamma,
                         float beta_lo, float beta_hi, float r2, float* z, float* beta_out,
                         float* beta_ws, hipStream_t stream) {
  int64_t T = 0;
  for (int b = 0; b < st.B; ++b) T += st.N[b];
  const float* beta = beta_in;
  hipError_t e;
  if (!beta) {
    const int threads = ((Hkv + 63) / 64) * 64;
    hipLaunchKernelGGL(beta_kernel, dim3(L * st.B), dim3(threads), 0, stream, st, Hkv, head_stats,
                       beta_lo, beta_hi, beta_ws);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    beta = beta_ws;
  }
  const int nchunk = st.tile_off[st.B];
  hipLaunchKernelGGL(refine_kernel, dim3(nchunk, L * Hkv), dim3(256), 0, stream, s, st, T, Hkv,
                     pool / 2, gamma, r2, beta, z, beta_out);
  return hipGetLastError();
}

hipError_t launch_select(const float* z, const SeqTable& st, int L, int Hkv, int n_sink,
                         int n_recent, int32_t* idx, hipStream_t stream) {
  int64_t T = 0, K = 0;
  for (int b = 0; b < st.B; ++b) {
    T += st.N[b];
    K += st.kept[b];
  }
  hipLaunchKernelGGL(select_kernel, dim3(st.B, L * Hkv), dim3(kSelThreads), 0, stream, z, st, T, K,
                     n_sink, n_recent, idx);
  return hipGetLastError();
}

}  // namespace hubkv
