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
// (histogram passes in LDS, the first one over the keys' own range), followed
// by one ordered emission pass that ranks kept positions with ballots.  The
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
  g.bytes = g.off_stats + align256r((size_t)L * st.B * Hkv * 2 * sizeof(double));
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

// Head weight of KV head g of (layer, sequence) lb, computed by wave 0 of a
// work-group: sel = 1 - (ln S - A / S) / ln N per head from {S, A} =
// {sum s, sum s ln s}, beta = clip(sel_g / mean_heads sel, lo, hi), 1 when the
// mean is not positive.  Every lane ends with beta.
__device__ float head_beta(const SeqTable& st, int lb, int b, int g, int Hkv,
                           const double* __restrict__ stats, float lo, float hi) {
  const int lane = threadIdx.x & 63;
  const double lnN = log((double)st.N[b]);
  double sum = 0.0, mine = 0.0;
  for (int h = lane; h < Hkv; h += 64) {
    const double S = stats[((int64_t)lb * Hkv + h) * 2], A = stats[((int64_t)lb * Hkv + h) * 2 + 1];
    double v = 0.0;
    if (st.N[b] > 1 && S > 0.0) v = 1.0 - (log(S) - A / S) / lnN;
    sum += v;
    if (h == g) mine = v;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    sum += __shfl_xor(sum, off);
    mine += __shfl_xor(mine, off);  // one lane holds it, the others add 0
  }
  const double mean = sum / (double)Hkv;
  double bt = 1.0;
  if (mean > 0.0 && isfinite(mean)) {
    bt = mine / mean;
    if (bt < (double)lo) bt = (double)lo;
    if (bt > (double)hi) bt = (double)hi;
  }
  return (float)bt;
}

// ---------------------------------------------------------------------------
// Max-pool hubs + SMD discount + ratio gate; one 1024-token tile of one
// sequence per work-group, staged with its halo in LDS.
// ---------------------------------------------------------------------------
constexpr int kMaxHalf = 31;
constexpr int kRefineThreads = 256;

// SMD discount and ratio gate as this exact fp32 op sequence (no contraction):
// q = hub ? s : fl(gamma s); z = fma(r2, fl(fl(beta q) - s), s).
__device__ __forceinline__ float smd_gate(float si, bool hub, float gamma, float bt, float r2) {
#pragma clang fp contract(off)
  const float qi = hub ? si : gamma * si;
  const float t = bt * qi;
  const float d = t - si;
  return __builtin_fmaf(r2, d, si);
}

__global__ __launch_bounds__(kRefineThreads) void refine_kernel(
    const float* __restrict__ s, SeqTable st, int64_t T, int Hkv, int half, float gamma, float r2,
    const float* __restrict__ beta_in, const double* __restrict__ stats, float lo, float hi,
    float* __restrict__ z, float* __restrict__ beta_out) {
  __shared__ float tile[kRefineTile + 2 * kMaxHalf];
  __shared__ float sh_beta;
  const int lh = blockIdx.y, c = blockIdx.x;
  const int l = lh / Hkv, g = lh % Hkv;
  const int b = seq_of_tile(st, c);
  const int N = (int)st.N[b];
  const int i0 = (c - st.tile_off[b]) * kRefineTile;
  const float* sb = s + (int64_t)lh * T + st.cu[b];
  float* zb = z + (int64_t)lh * T + st.cu[b];
  const int lb = l * st.B + b;
  const int u = lb * Hkv + g;
  // tile[j] holds s[i0 - half + j] (0 outside the sequence, never read)
  for (int j = threadIdx.x; j < kRefineTile + 2 * half; j += kRefineThreads) {
    const int i = i0 - half + j;
    tile[j] = (i >= 0 && i < N) ? sb[i] : 0.f;
  }
  if (threadIdx.x < 64) {
    const float bt = beta_in ? beta_in[u] : head_beta(st, lb, b, g, Hkv, stats, lo, hi);
    if (threadIdx.x == 0) {
      sh_beta = bt;
      if (beta_out && i0 == 0) beta_out[u] = bt;
    }
  }
  __syncthreads();
  const float bt = sh_beta;
  // window max scanned from its lowest in-sequence position upwards with a
  // strict compare, so that a NaN first entry stays the max as in a plain scan
  for (int j = threadIdx.x; j < kRefineTile; j += kRefineThreads) {
    const int i = i0 + j;
    if (i >= N) break;
    const float si = tile[j + half];
    float mx;
    if (half == 2 && i >= 2 && i + 2 < N) {
      mx = tile[j];
      mx = tile[j + 1] > mx ? tile[j + 1] : mx;
      mx = si > mx ? si : mx;
      mx = tile[j + 3] > mx ? tile[j + 3] : mx;
      mx = tile[j + 4] > mx ? tile[j + 4] : mx;
    } else {
      const int wlo = i - half < 0 ? 0 : i - half;
      const int whi = i + half > N - 1 ? N - 1 : i + half;
      mx = tile[wlo - i0 + half];
      for (int k = wlo + 1; k <= whi; ++k) {
        const float v = tile[k - i0 + half];
        mx = v > mx ? v : mx;
      }
    }
    zb[i] = smd_gate(si, si == mx, gamma, bt, r2);
  }
}

// ---------------------------------------------------------------------------
// Protected Top-K by radix select, one work-group per (layer, KV head,
// sequence).
//
// Layout: the sequence is cut into rounds of kSelRound positions; inside a
// round wave w owns kSelKpt sub-blocks of 64 consecutive positions and lane l
// holds position (w * kSelKpt + j) * 64 + l of sub-block j, so every load is a
// fully coalesced 256-byte row and position order inside a sub-block is lane
// order (ballots give in-order ranks).  A sequence of one round keeps its
// keys in registers through every pass; longer ones reload each round from L2.
//
// Keys: order-preserving 32-bit images of z (NaN lowest, -0 == +0), at most
// 0xff800000 (+inf).  Protected positions get kProt, above every real key, and
// positions past the end get kPad; neither is ever a candidate.  Once the
// candidates' range [kmin, kmax] is known, candidate keys are rebased to
// v = key - kmin in place.  Pass 1 bins v >> sh with the smallest shift that
// fits the range into 2047 bins (about 2047 occupied bins, few LDS-atomic
// collisions), protected and padding keys counted in bin 2047; further passes
// resolve the remaining low bits 11 at a time inside the chosen bin.  The
// result is (thr, rem): every key above thr is kept, plus the first rem keys
// equal to thr in position order.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelKpt = 32;
constexpr int kSelRound = kSelThreads * kSelKpt;
constexpr uint32_t kProt = 0xffffffffu;
constexpr uint32_t kPad = 0xfffffffeu;

__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  u = u == 0x80000000u ? 0u : u;                            // -0 == +0
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return v != v ? 0u : k;                                   // NaN ranks below everything
}

__device__ __forceinline__ unsigned long long lanes_below(int lane) {
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = __shfl_xor(v, off);
    v = o < v ? o : v;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = __shfl_xor(v, off);
    v = o > v ? o : v;
  }
  return v;
}

struct SelView {
  const float* zb;
  int N, a, c, wave, lane;
  __device__ __forceinline__ int base(int r) const {
    return r * kSelRound + wave * (64 * kSelKpt) + lane;
  }
  // keys of round r; a position past N reads a clamped address and gets kPad
  __device__ __forceinline__ void load(int r, uint32_t (&key)[kSelKpt]) const {
    const int p0 = base(r);
    float v[kSelKpt];
#pragma unroll
    for (int j = 0; j < kSelKpt; ++j) {
      const int p = p0 + 64 * j;
      v[j] = zb[p < N ? p : N - 1];
    }
#pragma unroll
    for (int j = 0; j < kSelKpt; ++j) {
      const int p = p0 + 64 * j;
      const uint32_t k = order_key(v[j]);
      const uint32_t kp = (p < a || p >= c) ? kProt : k;
      key[j] = p >= N ? kPad : kp;
    }
  }
  // rebase candidate keys to key - kmin (special keys unchanged)
  __device__ __forceinline__ void rebase(uint32_t (&key)[kSelKpt], uint32_t kmn) const {
#pragma unroll
    for (int j = 0; j < kSelKpt; ++j) key[j] = key[j] < kPad ? key[j] - kmn : key[j];
  }
};

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ z,
                                                             SeqTable st, int64_t T, int64_t Ktot,
                                                             int n_sink, int n_recent,
                                                             int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wa[kSelWaves], wb[kSelWaves];
  __shared__ uint32_t bc[2];
  const int lh = blockIdx.y, b = blockIdx.x;
  const int N = (int)st.N[b];
  const int kept = (int)st.kept[b];
  if (N <= 0 || kept <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int a = n_sink < N ? n_sink : N;
  int c = N - n_recent > 0 ? N - n_recent : 0;
  if (c < a) c = a;
  const uint32_t nprot = (uint32_t)(a + (N - c));
  const SelView sv{z + (int64_t)lh * T + st.cu[b], N, a, c, wave, lane};
  int32_t* out = idx + (int64_t)lh * Ktot + st.ko[b];
  const int nr = (N + kSelRound - 1) / kSelRound;
  const uint32_t npad = (uint32_t)(nr * kSelRound - N);

  uint32_t key[kSelKpt];
  sv.load(0, key);

  // keep rule: key > thr (kPad excluded), or key == thr among the first rem
  // such keys in position order; keys are rebased when a select ran
  uint32_t thr, rem, kmn = 0u;
  bool rebased = false;
  if ((uint32_t)kept >= (uint32_t)N) {
    thr = 0u;
    rem = (uint32_t)N;
  } else if ((uint32_t)kept <= nprot) {
    thr = kProt;
    rem = (uint32_t)kept;
  } else {
    // range of the candidate keys
    uint32_t mn = kPad, mx = 0u;
    for (int r = 0; r < nr; ++r) {
      if (nr > 1) sv.load(r, key);
#pragma unroll
      for (int j = 0; j < kSelKpt; ++j) {
        const uint32_t k = key[j];
        mn = k < mn ? k : mn;                    // specials are >= kPad
        mx = (k < kPad && k > mx) ? k : mx;
      }
    }
    mn = wave_min_u32(mn);
    mx = wave_max_u32(mx);
    if (lane == 0) {
      wa[wave] = mn;
      wb[wave] = mx;
    }
    __syncthreads();
    mn = kPad;
    mx = 0u;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
      mn = wa[w] < mn ? wa[w] : mn;
      mx = wb[w] > mx ? wb[w] : mx;
    }
    kmn = mn;
    rebased = true;
    const uint32_t range = mx - mn;  // <= 0xff800000, so sh <= 21
    int sh = 0;
    while ((range >> sh) > 2046u) ++sh;
    if (nr == 1) sv.rebase(key, kmn);

    // counted from the top: protected keys and padding sit in bin 2047
    uint32_t need = (uint32_t)kept + npad;
    uint32_t pfx = 0u;
    int pfx_sh = sh;
    bool first = true;
    for (;;) {
      const int nbits = first ? 11 : (pfx_sh < 11 ? pfx_sh : 11);
      const int sel_sh = first ? sh : pfx_sh - nbits;
      const uint32_t mask = (1u << nbits) - 1u;
      __syncthreads();  // earlier readers of hist / wa / bc are done
      hist[2 * tid] = 0u;
      hist[2 * tid + 1] = (first && tid == kSelThreads - 1) ? nprot + npad : 0u;  // bin 2047
      __syncthreads();
      for (int r = 0; r < nr; ++r) {
        if (nr > 1) {
          sv.load(r, key);
          sv.rebase(key, kmn);
        }
        if (first) {
#pragma unroll
          for (int j = 0; j < kSelKpt; ++j) {
            const uint32_t d = key[j] >> sh;  // protected and padding keys give >= 2047
            if (d < 2047u) atomicAdd(&hist[d], 1u);
          }
        } else {
#pragma unroll
          for (int j = 0; j < kSelKpt; ++j) {
            const uint32_t v = key[j];
            if ((v >> pfx_sh) == pfx) atomicAdd(&hist[(v >> sel_sh) & mask], 1u);
          }
        }
      }
      __syncthreads();
      // thread t owns bins 2047 - 2t (upper) and 2046 - 2t, counted from the top
      const int d0 = 2047 - 2 * tid;
      const uint32_t h0 = hist[d0], h1 = hist[d0 - 1];
      const uint32_t mine = h0 + h1;
      uint32_t incl = mine;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      if (lane == 63) wa[wave] = incl;
      __syncthreads();
      uint32_t above = incl - mine;
      for (int w = 0; w < wave; ++w) above += wa[w];
      if (above < need && above + h0 >= need) {
        bc[0] = (uint32_t)d0;
        bc[1] = above;
      } else if (above + h0 < need && above + mine >= need) {
        bc[0] = (uint32_t)(d0 - 1);
        bc[1] = above + h0;
      }
      __syncthreads();
      const uint32_t dsel = bc[0];
      need -= bc[1];
      pfx = first ? dsel : ((pfx << nbits) | dsel);
      pfx_sh = sel_sh;
      first = false;
      if (pfx_sh == 0) break;
    }
    thr = pfx;  // rebased
    rem = need;
  }
  // ordered emission, round by round
  uint32_t Dr = 0u, Tr = 0u;  // kept-by-rank and tied keys before this round
  const unsigned long long below = lanes_below(lane);
  for (int r = 0; r < nr; ++r) {
    if (nr > 1) {
      sv.load(r, key);
      if (rebased) sv.rebase(key, kmn);
    }
    uint32_t nd = 0u, nt = 0u;  // per lane, then per wave
#pragma unroll
    for (int j = 0; j < kSelKpt; ++j) {
      nd += (key[j] > thr && key[j] != kPad) ? 1u : 0u;
      nt += key[j] == thr ? 1u : 0u;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      nd += __shfl_xor(nd, off);
      nt += __shfl_xor(nt, off);
    }
    __syncthreads();  // earlier readers of wa / wb are done
    if (lane == 0) {
      wa[wave] = nd;
      wb[wave] = nt;
    }
    __syncthreads();
    // lanes 0..15 take one wave's counts each: totals and this wave's prefix
    const uint32_t x = lane < kSelWaves ? wa[lane] : 0u, y = lane < kSelWaves ? wb[lane] : 0u;
    uint32_t xb = lane < wave ? x : 0u, yb = lane < wave ? y : 0u, dtot = x, ttot = y;
#pragma unroll
    for (int off = kSelWaves / 2; off >= 1; off >>= 1) {
      xb += __shfl_xor(xb, off);
      yb += __shfl_xor(yb, off);
      dtot += __shfl_xor(dtot, off);
      ttot += __shfl_xor(ttot, off);
    }
    uint32_t D = Dr + __builtin_amdgcn_readfirstlane(xb), Tt = Tr + __builtin_amdgcn_readfirstlane(yb);
    dtot = __builtin_amdgcn_readfirstlane(dtot);
    ttot = __builtin_amdgcn_readfirstlane(ttot);
    const int p0 = sv.base(r);
    uint32_t thw = thr;
    asm volatile("" : "+v"(thw));  // keeps the counting compares from being reused here
#pragma unroll
    for (int j = 0; j < kSelKpt; ++j) {
      const bool def = key[j] > thw && key[j] != kPad;
      const bool tie = key[j] == thw;
      const unsigned long long bd = __ballot(def), bt = __ballot(tie);
      const uint32_t dr = (uint32_t)__popcll(bd & below), tr = (uint32_t)__popcll(bt & below);
      const uint32_t tk = Tt + tr;  // tied keys before this one
      uint32_t o = 0xffffffffu;
      if (def) o = D + dr + (tk < rem ? tk : rem);
      else if (tie && tk < rem) o = D + dr + tk;
      if (o < (uint32_t)kept) out[o] = p0 + 64 * j;  // never past this sequence's slice
      D += (uint32_t)__popcll(bd);
      Tt += (uint32_t)__popcll(bt);
    }
    Dr += dtot;
    Tr += ttot;
  }
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
                         hipStream_t stream) {
  int64_t T = 0;
  for (int b = 0; b < st.B; ++b) T += st.N[b];
  const int nchunk = st.tile_off[st.B];
  hipLaunchKernelGGL(refine_kernel, dim3(nchunk, L * Hkv), dim3(kRefineThreads), 0, stream, s, st,
                     T, Hkv, pool / 2, gamma, r2, beta_in, head_stats, beta_lo, beta_hi, z,
                     beta_out);
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
