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
// Selection is exact and integer throughout, on order-preserving 32-bit keys
// of z, with one ordered emission pass that ranks kept positions with
// ballots.  Two implementations give the same result bit for bit:
//   - many work-groups per head (msel_bin + msel_pick, below): 4096-position
//     slices binned around a sampled estimate of the threshold, every slice
//     resolving the threshold itself from all slices' bin data;
//   - one work-group per head (select_kernel): radix histogram passes in
//     LDS, the first over the keys' own range, for calls whose units fill the
//     chip alone and for sequences beyond the slices' reach.
// The result is deterministic and independent of thread timing.
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

// Refined score of position i (tile-local index j) of a sequence of N
// positions whose tile starts at i0: tile[j + half] holds s_i and the halo
// sits on both sides.  The window maximum is scanned from its lowest
// in-sequence position upwards with a strict compare, so that a NaN first
// entry stays the maximum as in a plain scan.
__device__ __forceinline__ float refined(const float* tile, int j, int i, int i0, int N, int half,
                                         float gamma, float bt, float r2) {
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
  return smd_gate(si, si == mx, gamma, bt, r2);
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
  // tile[j] holds s[i0 - half + j] (0 outside the sequence, never read);
  // every load is issued before the first LDS store
  constexpr int kPer = kRefineTile / kRefineThreads;
  const int tid = threadIdx.x;
  float v[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int i = i0 + e * kRefineThreads + tid;
    v[e] = i < N ? sb[i] : 0.f;
  }
  float hv = 0.f;
  if (tid < 2 * half) {  // halo: half positions on each side of the tile
    const int i = tid < half ? i0 - half + tid : i0 + kRefineTile - half + tid;
    hv = (i >= 0 && i < N) ? sb[i] : 0.f;
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) tile[half + e * kRefineThreads + tid] = v[e];
  if (tid < 2 * half) tile[tid < half ? tid : kRefineTile + tid] = hv;
  if (threadIdx.x < 64) {
    const float bt = beta_in ? beta_in[u] : head_beta(st, lb, b, g, Hkv, stats, lo, hi);
    if (threadIdx.x == 0) {
      sh_beta = bt;
      if (beta_out && i0 == 0) beta_out[u] = bt;
    }
  }
  __syncthreads();
  const float bt = sh_beta;
  for (int j = threadIdx.x; j < kRefineTile; j += kRefineThreads) {
    const int i = i0 + j;
    if (i >= N) break;
    zb[i] = refined(tile, j, i, i0, N, half, gamma, bt, r2);
  }
}

// ---------------------------------------------------------------------------
// Protected Top-K by radix select, one work-group per (layer, KV head,
// sequence).
//
// Layout: the sequence is cut into rounds of kSelRound positions; inside a
// round wave w owns kSelKpt rows of 64 consecutive positions and lane l holds
// position (w * kSelKpt + j) * 64 + l of row j, so every load is a fully
// coalesced 256-byte row and position order inside a row is lane order
// (ballots and mbcnt give in-order ranks).  A sequence of one round keeps its
// keys in registers through every pass; longer ones reload each round from L2.
//
// Keys: when no candidate is negative, -0 or NaN (scores are sums of
// probabilities) the raw fp32 bits already order the values and are used as
// they are; otherwise each value is mapped to an order-preserving key (NaN
// lowest, -0 == +0).  Protected positions get kProt and positions past the
// end kPad, above every real key; only the waves whose rows touch the
// protected windows or the end pay for that.  Candidate keys are rebased to
// key - kmin; pass 1 bins them with the smallest shift that fits their range
// into 2047 bins (few LDS-atomic collisions), protected and padding keys
// counted in bin 2047; later passes resolve the remaining low bits 11 at a
// time inside the chosen bin.  The result is (thr, rem): every key above thr
// is kept, plus the first rem keys equal to thr in position order.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelKpt = 32;
constexpr int kSelRound = kSelThreads * kSelKpt;
constexpr uint32_t kProt = 0xffffffffu;
constexpr uint32_t kPad = 0xfffffffeu;

__device__ __forceinline__ uint32_t order_key_bits(uint32_t u) {
  const float v = __uint_as_float(u);
  u = u == 0x80000000u ? 0u : u;                            // -0 == +0
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return v != v ? 0u : k;                                   // NaN ranks below everything
}

__device__ __forceinline__ uint32_t rank_below(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
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

typedef const __attribute__((address_space(1))) uint32_t* gbits;  // global memory

struct SelView {
  gbits zb;  // bits of z
  int N, a, c, wave, lane;
  __device__ __forceinline__ int seg0(int r) const {
    return r * kSelRound + wave * (64 * kSelKpt);
  }
  // rows of this wave in round r touch a protected window or the end
  __device__ __forceinline__ bool edge(int r) const {
    const int s0 = seg0(r);
    return s0 < a || s0 + 64 * kSelKpt > c;
  }
  // raw bits of round r; on edge waves positions past N read a clamped address
  __device__ __forceinline__ void load_raw(int r, uint32_t (&key)[kSelKpt]) const {
    const int p0 = seg0(r) + lane;
    if (edge(r)) {
#pragma unroll
      for (int j = 0; j < kSelKpt; ++j) {
        const int p = p0 + 64 * j;
        key[j] = zb[p < N ? p : N - 1];
      }
    } else {
      const gbits zr = zb + p0;
#pragma unroll
      for (int j = 0; j < kSelKpt; ++j) key[j] = zr[64 * j];
    }
  }
  __device__ __forceinline__ void specials(int r, uint32_t (&key)[kSelKpt]) const {
    const int p0 = seg0(r) + lane;
#pragma unroll
    for (int j = 0; j < kSelKpt; ++j) {
      const int p = p0 + 64 * j;
      key[j] = p >= N ? kPad : ((p < a || p >= c) ? kProt : key[j]);
    }
  }
  // keys of round r, rebased by kmn
  __device__ __forceinline__ void load(int r, uint32_t (&key)[kSelKpt], bool conv,
                                       uint32_t kmn) const {
    load_raw(r, key);
    if (conv) {
#pragma unroll
      for (int j = 0; j < kSelKpt; ++j) key[j] = order_key_bits(key[j]);
    }
    if (edge(r)) {
      specials(r, key);
#pragma unroll
      for (int j = 0; j < kSelKpt; ++j) key[j] = key[j] < kPad ? key[j] - kmn : key[j];
    } else {
#pragma unroll
      for (int j = 0; j < kSelKpt; ++j) key[j] -= kmn;
    }
  }
};

// Block-wide min and max of per-lane values and OR of a per-lane flag.
__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, uint32_t& fl,
                                             uint32_t* wa, uint32_t* wb, uint32_t* wc, int wave,
                                             int lane) {
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  fl = wave_max_u32(fl);
  __syncthreads();  // earlier readers of wa / wb / wc are done
  if (lane == 0) {
    wa[wave] = mn;
    wb[wave] = mx;
    wc[wave] = fl;
  }
  __syncthreads();
  const uint32_t x = lane < kSelWaves ? wa[lane] : 0xffffffffu;
  const uint32_t y = lane < kSelWaves ? wb[lane] : 0u;
  const uint32_t f = lane < kSelWaves ? wc[lane] : 0u;
  mn = __builtin_amdgcn_readfirstlane(wave_min_u32(x));
  mx = __builtin_amdgcn_readfirstlane(wave_max_u32(y));
  fl = __builtin_amdgcn_readfirstlane(wave_max_u32(f));
}

constexpr int kCandCap = 8192;   // keys of the threshold bin held in LDS
constexpr int kFastRounds = 16;  // sequences up to 16 rounds take the fast path

struct SelSmem {
  uint32_t hist[4096];
  uint32_t ckey[kCandCap];
  int32_t cpos[kCandCap];
  uint32_t rw_def[kFastRounds * kSelWaves];  // per (round, wave): keys above thr, then prefix
  uint32_t rw_tie[kFastRounds * kSelWaves];  // per (round, wave): keys equal to thr, then prefix
  uint32_t wa[kSelWaves], wb[kSelWaves], wc[kSelWaves];
  uint32_t bc[2];
  uint32_t ncand;
};

// Bin of hist[0 .. 1024 * kPer) holding the need-th largest count from the
// top, and the count strictly above it; thread t owns bins
// 1024 * kPer - 1 - kPer * t downwards.  Block-uniform results.
template <int kPer>
__device__ __forceinline__ void find_bin(const uint32_t* hist, uint32_t need, SelSmem& sm, int tid,
                                         int lane, int wave, uint32_t& d, uint32_t& above_d) {
  const int top = 1024 * kPer - 1 - kPer * tid;
  uint32_t h[kPer], mine = 0u;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    h[e] = hist[top - e];
    mine += h[e];
  }
  uint32_t incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) sm.wa[wave] = incl;
  __syncthreads();
  uint32_t above = incl - mine;
  for (int w = 0; w < wave; ++w) above += sm.wa[w];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    if (above < need && above + h[e] >= need) {
      sm.bc[0] = (uint32_t)(top - e);
      sm.bc[1] = above;
    }
    above += h[e];
  }
  __syncthreads();
  d = sm.bc[0];
  above_d = sm.bc[1];
}

// Ordered writes of one round: keys above thr, then the first rem keys equal
// to thr, ranked from D and Tt (keys above / equal to thr before this wave's
// rows).  Keys in registers, specials applied.
template <int R>
__device__ __forceinline__ void emit_round(const uint32_t (&key)[R], bool edge, uint32_t thr,
                                           uint32_t rem, uint32_t D, uint32_t Tt, int p0, int kept,
                                           int32_t* __restrict__ out) {
  uint32_t thw = thr;
  asm volatile("" : "+v"(thw));  // keeps earlier compares against thr from being reused
  // usual case: no key of the wave's rows equals thr, so the tie count Tt
  // stays put and each row needs one ballot
  bool anyeq = false;
#pragma unroll
  for (int j = 0; j < R; ++j) anyeq |= key[j] == thw;
  if (!__any(anyeq)) {
    uint32_t base = D + (Tt < rem ? Tt : rem);
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const uint32_t k = key[j];
      const bool def = edge ? (k > thw && k != kPad) : (k > thw);
      const unsigned long long bd = __ballot(def);
      const uint32_t o = base + rank_below(bd);
      if (def && o < (uint32_t)kept) out[o] = p0 + 64 * j;
      base += (uint32_t)__popcll(bd);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const uint32_t k = key[j];
    const bool def = edge ? (k > thw && k != kPad) : (k > thw);
    const unsigned long long bd = __ballot(def);
    const unsigned long long bt = __ballot(k == thw);
    if (bt == 0ull) {
      // no key of this row equals thr: kept ranks are those of the keys above it
      const uint32_t o = D + rank_below(bd) + (Tt < rem ? Tt : rem);
      if (def && o < (uint32_t)kept) out[o] = p0 + 64 * j;
    } else {
      const uint32_t tk = Tt + rank_below(bt);  // tied keys before this one
      uint32_t o = 0xffffffffu;
      if (def) o = D + rank_below(bd) + (tk < rem ? tk : rem);
      else if (k == thw && tk < rem) o = D + rank_below(bd) + tk;
      if (o < (uint32_t)kept) out[o] = p0 + 64 * j;  // never past this sequence's slice
    }
    D += (uint32_t)__popcll(bd);
    Tt += (uint32_t)__popcll(bt);
  }
}

// Fast path for sequences whose candidates are all +0, positive or +inf (the
// raw bits order them).  Sweep 0 finds the candidates' bit range; sweep 1
// bins the rebased bits with the smallest shift that fits that range into
// 4095 bins (bin 4095 holds protected and padding keys); sweep 2 counts the
// keys above the threshold bin per (round, wave) and copies the bin's keys to
// LDS, where the remaining low bits are resolved; sweep 3 writes.  Returns
// false, having written nothing, when a candidate needs an order key, the bin
// is larger than kCandCap or the sequence is longer than kFastRounds rounds.
__device__ __forceinline__ bool select_fast(const SelView& sv, SelSmem& sm, int nr, uint32_t nprot,
                                            uint32_t npad, int kept, int32_t* __restrict__ out,
                                            int tid, int lane, int wave) {
  if (nr > kFastRounds) return false;
  uint32_t key[kSelKpt];
  // sweep 0: range of the candidates' raw bits; bits above +inf's
  // (0x7f800000) belong to a NaN or a negative value
  uint32_t mn = 0xffffffffu, mx = 0u;
  for (int r = 0; r < nr; ++r) {
    sv.load_raw(r, key);
    if (sv.edge(r)) sv.specials(r, key);
#pragma unroll
    for (int j = 0; j < kSelKpt; ++j) {
      mn = key[j] < mn ? key[j] : mn;   // specials are above every candidate
      const uint32_t k2 = key[j] + 2u;  // specials wrap to 0 and 1
      mx = k2 > mx ? k2 : mx;
    }
  }
  uint32_t unused = 0u;
  block_minmax(mn, mx, unused, sm.wa, sm.wb, sm.wc, wave, lane);
  mx -= 2u;
  if (mx > 0x7f800000u) return false;
  const uint32_t kmn = mn, range = mx - mn;
  int sh = 0;
  while ((range >> sh) > 4094u) ++sh;

  // sweep 1: histogram of the rebased bits
  for (int i = tid; i < 4096; i += kSelThreads) sm.hist[i] = i == 4095 ? nprot + npad : 0u;
  __syncthreads();
  for (int r = 0; r < nr; ++r) {
    const bool edge = sv.edge(r);
    if (nr > 1) {
      sv.load_raw(r, key);
      if (edge) sv.specials(r, key);
    }
    if (edge) {
#pragma unroll
      for (int j = 0; j < kSelKpt; ++j) {
        if (key[j] < kPad) {
          key[j] -= kmn;
          atomicAdd(&sm.hist[key[j] >> sh], 1u);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < kSelKpt; ++j) {
        key[j] -= kmn;
        atomicAdd(&sm.hist[key[j] >> sh], 1u);
      }
    }
  }
  __syncthreads();
  // counted from the top: protected keys and padding sit in bin 4095
  uint32_t need = (uint32_t)kept + npad, d1, above;
  find_bin<4>(sm.hist, need, sm, tid, lane, wave, d1, above);
  need -= above;
  const uint32_t c1 = sm.hist[d1];
  if (c1 > (uint32_t)kCandCap) return false;

  // sweep 2: keys above bin d1 per (round, wave); keys of bin d1 to LDS
  if (tid == 0) sm.ncand = 0u;
  __syncthreads();
  for (int r = 0; r < nr; ++r) {
    const bool edge = sv.edge(r);
    if (nr > 1) {
      sv.load_raw(r, key);
      if (edge) {
        sv.specials(r, key);
#pragma unroll
        for (int j = 0; j < kSelKpt; ++j) key[j] = key[j] < kPad ? key[j] - kmn : key[j];
      } else {
#pragma unroll
        for (int j = 0; j < kSelKpt; ++j) key[j] -= kmn;
      }
    }
    const int p0 = sv.seg0(r) + lane;
    uint32_t nhi = 0u;
#pragma unroll
    for (int j = 0; j < kSelKpt; ++j) {
      const uint32_t k = key[j];
      const uint32_t bin = k < kPad ? k >> sh : 4095u;
      nhi += (uint32_t)__popcll(__ballot(bin > d1 && k != kPad));
      if (bin == d1) {
        const uint32_t slot = atomicAdd(&sm.ncand, 1u);
        sm.ckey[slot] = k;
        sm.cpos[slot] = p0 + 64 * j;
      }
    }
    if (lane == 0) sm.rw_def[r * kSelWaves + wave] = nhi;
  }
  __syncthreads();
  // the bin's low sh bits, at most 11 per pass, on the LDS copy
  uint32_t pfx = d1;
  int pfx_sh = sh;
  while (pfx_sh > 0) {
    const int nbits = pfx_sh < 11 ? pfx_sh : 11;
    const int sel_sh = pfx_sh - nbits;
    const uint32_t mask = (1u << nbits) - 1u;
    for (int i = tid; i < 2048; i += kSelThreads) sm.hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < (int)c1; i += kSelThreads) {
      const uint32_t v = sm.ckey[i];
      if ((v >> pfx_sh) == pfx) atomicAdd(&sm.hist[(v >> sel_sh) & mask], 1u);
    }
    __syncthreads();
    uint32_t dsel;
    find_bin<2>(sm.hist, need, sm, tid, lane, wave, dsel, above);
    need -= above;
    pfx = (pfx << nbits) | dsel;
    pfx_sh = sel_sh;
  }
  const uint32_t thr = pfx;  // rebased
  const uint32_t rem = need;

  // add the bin's keys above / equal to thr to the per-(round, wave) counts
  for (int i = tid; i < nr * kSelWaves; i += kSelThreads) sm.rw_tie[i] = 0u;
  __syncthreads();
  for (int i = tid; i < (int)c1; i += kSelThreads) {
    const uint32_t k = sm.ckey[i];
    const int p = sm.cpos[i];
    const int rw = (p / kSelRound) * kSelWaves + (p % kSelRound) / (64 * kSelKpt);
    if (k > thr) atomicAdd(&sm.rw_def[rw], 1u);
    else if (k == thr) atomicAdd(&sm.rw_tie[rw], 1u);
  }
  __syncthreads();
  // exclusive prefix over (round, wave) in position order, by wave 0
  if (wave == 0) {
    uint32_t Dp = 0u, Tp = 0u;
    for (int base = 0; base < nr * kSelWaves; base += 64) {
      const int i = base + lane;
      const uint32_t x = i < nr * kSelWaves ? sm.rw_def[i] : 0u;
      const uint32_t y = i < nr * kSelWaves ? sm.rw_tie[i] : 0u;
      uint32_t xi = x, yi = y;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t xs = __shfl_up(xi, off), ys = __shfl_up(yi, off);
        if (lane >= off) {
          xi += xs;
          yi += ys;
        }
      }
      if (i < nr * kSelWaves) {
        sm.rw_def[i] = Dp + xi - x;
        sm.rw_tie[i] = Tp + yi - y;
      }
      Dp += __shfl(xi, 63);
      Tp += __shfl(yi, 63);
    }
  }
  __syncthreads();

  // sweep 3: ordered writes
  for (int r = 0; r < nr; ++r) {
    const bool edge = sv.edge(r);
    if (nr > 1) {
      sv.load_raw(r, key);
      if (edge) {
        sv.specials(r, key);
#pragma unroll
        for (int j = 0; j < kSelKpt; ++j) key[j] = key[j] < kPad ? key[j] - kmn : key[j];
      } else {
#pragma unroll
        for (int j = 0; j < kSelKpt; ++j) key[j] -= kmn;
      }
    }
    const uint32_t D = sm.rw_def[r * kSelWaves + wave], Tt = sm.rw_tie[r * kSelWaves + wave];
    emit_round(key, edge, thr, rem, D, Tt, sv.seg0(r) + lane, kept, out);
  }
  return true;
}

// General path: order keys when needed, a first pass binned over the
// candidates' own key range, further radix passes over every key.
__device__ __noinline__ void select_generic(const SelView& sv, SelSmem& sm, int nr, uint32_t nprot,
                               uint32_t npad, int kept, int32_t* __restrict__ out, int tid,
                               int lane, int wave) {
  const int N = sv.N, a = sv.a, c = sv.c;

  // pass 0: candidate range in raw-bit space, and whether raw bits order them
  // (their largest raw bits above +inf's mean a NaN or a negative value)
  uint32_t key[kSelKpt];
  uint32_t mn = 0xffffffffu, mx = 0u, bad = 0u;
  for (int r = 0; r < nr; ++r) {
    sv.load_raw(r, key);
    if (sv.edge(r)) {
      const int p0 = sv.seg0(r) + lane;
#pragma unroll
      for (int j = 0; j < kSelKpt; ++j) {
        const int p = p0 + 64 * j;
        const bool cand = p < N && p >= a && p < c;
        bad = (cand && key[j] > bad) ? key[j] : bad;
        key[j] = p >= N ? kPad : (cand ? key[j] : kProt);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kSelKpt; ++j) bad = key[j] > bad ? key[j] : bad;
    }
#pragma unroll
    for (int j = 0; j < kSelKpt; ++j) {
      mn = key[j] < mn ? key[j] : mn;        // specials are above every candidate
      const uint32_t k2 = key[j] + 2u;       // specials wrap to 0 and 1
      mx = k2 > mx ? k2 : mx;
    }
  }
  block_minmax(mn, mx, bad, sm.wa, sm.wb, sm.wc, wave, lane);
  const bool conv = bad > 0x7f800000u;  // a NaN or a negative value among the candidates
  if (conv) {  // order-preserving keys instead of raw bits (not yet rebased)
    mn = 0xffffffffu;
    mx = 0u;
    uint32_t dummy = 0u;
    for (int r = 0; r < nr; ++r) {
      sv.load(r, key, true, 0u);
#pragma unroll
      for (int j = 0; j < kSelKpt; ++j) {
        mn = key[j] < mn ? key[j] : mn;
        const uint32_t k2 = key[j] + 2u;
        mx = k2 > mx ? k2 : mx;
      }
    }
    block_minmax(mn, mx, dummy, sm.wa, sm.wb, sm.wc, wave, lane);
  }
  const uint32_t kmn = mn;
  const uint32_t range = (mx - 2u) - mn;  // <= 0xff800000, so sh <= 21
  if (nr == 1) {  // rebase the keys held in registers
    if (sv.edge(0)) {
#pragma unroll
      for (int j = 0; j < kSelKpt; ++j) key[j] = key[j] < kPad ? key[j] - kmn : key[j];
    } else {
#pragma unroll
      for (int j = 0; j < kSelKpt; ++j) key[j] -= kmn;
    }
  }
  int sh = 0;
  while ((range >> sh) > 2046u) ++sh;

  // radix passes; counted from the top, protected keys and padding in bin 2047
  uint32_t need = (uint32_t)kept + npad;
  uint32_t pfx = 0u;
  int pfx_sh = sh;
  bool first = true;
  for (;;) {
    const int nbits = first ? 11 : (pfx_sh < 11 ? pfx_sh : 11);
    const int sel_sh = first ? sh : pfx_sh - nbits;
    const uint32_t mask = (1u << nbits) - 1u;
    __syncthreads();  // earlier readers of hist / wa / bc are done
    sm.hist[2 * tid] = 0u;
    sm.hist[2 * tid + 1] = (first && tid == kSelThreads - 1) ? nprot + npad : 0u;  // bin 2047
    __syncthreads();
    for (int r = 0; r < nr; ++r) {
      if (nr > 1) sv.load(r, key, conv, kmn);
      if (first) {
        if (sv.edge(r)) {
#pragma unroll
          for (int j = 0; j < kSelKpt; ++j) {
            const uint32_t d = key[j] >> sh;  // protected and padding keys give >= 2047
            if (d < 2047u) atomicAdd(&sm.hist[d], 1u);
          }
        } else {
#pragma unroll
          for (int j = 0; j < kSelKpt; ++j) atomicAdd(&sm.hist[key[j] >> sh], 1u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kSelKpt; ++j) {
          const uint32_t v = key[j];
          if ((v >> pfx_sh) == pfx) atomicAdd(&sm.hist[(v >> sel_sh) & mask], 1u);
        }
      }
    }
    __syncthreads();
    // thread t owns bins 2047 - 2t (upper) and 2046 - 2t, counted from the top
    const int d0 = 2047 - 2 * tid;
    const uint32_t h0 = sm.hist[d0], h1 = sm.hist[d0 - 1];
    const uint32_t mine = h0 + h1;
    uint32_t incl = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    if (lane == 63) sm.wa[wave] = incl;
    __syncthreads();
    uint32_t above = incl - mine;
    for (int w = 0; w < wave; ++w) above += sm.wa[w];
    if (above < need && above + h0 >= need) {
      sm.bc[0] = (uint32_t)d0;
      sm.bc[1] = above;
    } else if (above + h0 < need && above + mine >= need) {
      sm.bc[0] = (uint32_t)(d0 - 1);
      sm.bc[1] = above + h0;
    }
    __syncthreads();
    const uint32_t dsel = sm.bc[0];
    need -= sm.bc[1];
    pfx = first ? dsel : ((pfx << nbits) | dsel);
    pfx_sh = sel_sh;
    first = false;
    if (pfx_sh == 0) break;
  }
  const uint32_t thr = pfx;  // rebased; every candidate key is below kPad
  const uint32_t rem = need;

  // ordered emission, round by round
  uint32_t Dr = 0u, Tr = 0u;  // keys above thr and keys equal to thr before this round
  for (int r = 0; r < nr; ++r) {
    if (nr > 1) sv.load(r, key, conv, kmn);
    const bool edge = sv.edge(r);
    uint32_t nd = 0u, nt = 0u;
    if (edge) {
#pragma unroll
      for (int j = 0; j < kSelKpt; ++j) {
        nd += (uint32_t)__popcll(__ballot(key[j] > thr && key[j] != kPad));
        nt += (uint32_t)__popcll(__ballot(key[j] == thr));
      }
    } else {
#pragma unroll
      for (int j = 0; j < kSelKpt; ++j) {
        nd += (uint32_t)__popcll(__ballot(key[j] > thr));
        nt += (uint32_t)__popcll(__ballot(key[j] == thr));
      }
    }
    __syncthreads();  // earlier readers of wa / wb are done
    if (lane == 0) {
      sm.wa[wave] = nd;
      sm.wb[wave] = nt;
    }
    __syncthreads();
    // lanes 0..15 take one wave's counts each: totals and this wave's prefix
    const uint32_t x = lane < kSelWaves ? sm.wa[lane] : 0u, y = lane < kSelWaves ? sm.wb[lane] : 0u;
    uint32_t xb = lane < wave ? x : 0u, yb = lane < wave ? y : 0u, dtot = x, ttot = y;
#pragma unroll
    for (int off = kSelWaves / 2; off >= 1; off >>= 1) {
      xb += __shfl_xor(xb, off);
      yb += __shfl_xor(yb, off);
      dtot += __shfl_xor(dtot, off);
      ttot += __shfl_xor(ttot, off);
    }
    emit_round(key, edge, thr, rem, Dr + __builtin_amdgcn_readfirstlane(xb),
               Tr + __builtin_amdgcn_readfirstlane(yb), sv.seg0(r) + lane, kept, out);
    Dr += __builtin_amdgcn_readfirstlane(dtot);
    Tr += __builtin_amdgcn_readfirstlane(ttot);
  }
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ z,
                                                             SeqTable st, int64_t T, int64_t Ktot,
                                                             int n_sink, int n_recent,
                                                             int32_t* __restrict__ idx) {
  __shared__ SelSmem sm;
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
  int32_t* out = idx + (int64_t)lh * Ktot + st.ko[b];

  // all positions kept, or only the protected ones: no keys needed
  if ((uint32_t)kept >= (uint32_t)N || (uint32_t)kept <= nprot) {
    const bool all = (uint32_t)kept >= (uint32_t)N;
    for (int p = tid; p < N; p += kSelThreads) {
      if (all) {
        out[p] = p;
      } else if (p < a) {
        out[p] = p;
      } else if (p >= c && a + (p - c) < kept) {
        out[a + (p - c)] = p;
      }
    }
    return;
  }
  const SelView sv{(gbits)(z + (int64_t)lh * T + st.cu[b]), N, a, c, wave, lane};
  const int nr = (N + kSelRound - 1) / kSelRound;
  const uint32_t npad = (uint32_t)(nr * kSelRound - N);
  if (!select_fast(sv, sm, nr, nprot, npad, kept, out, tid, lane, wave)) {
    __syncthreads();  // the fast path's readers of LDS are done
    select_generic(sv, sm, nr, nprot, npad, kept, out, tid, lane, wave);
  }
}

// ---------------------------------------------------------------------------
// Protected Top-K over many work-groups per (layer, KV head, sequence) unit.
//
// Every sequence is cut into slices of kMsSlice positions, one 256-thread
// work-group per (layer-head, slice), so a unit is spread over ceil(N /
// kMsSlice) compute units.  Two launches; no work-group waits for another:
//   bin   z of the slice (the refinement fused in, or read from z) and the
//         order-preserving 32-bit key of every unprotected position.  Keys go
//         to 4096 bins of 2^14 key units (1/512 of an octave for normal
//         floats) placed around an estimate of the unit's threshold, the
//         outermost bins catching everything beyond; the estimate is the
//         matching quantile of 64 sample positions spread over the unit,
//         which every slice reads and sorts alike, so all slices bin the same
//         way without talking.  The slice stores its bins' starts, 64 coarse
//         counts (64 bins each) and its keys' low bits and positions sorted by
//         bin.
//   pick  every slice of the unit finds, redundantly, the coarse bin, then
//         the bin, holding the k-th largest unprotected key (from all slices'
//         coarse counts and bin starts), gathers that bin's keys from all
//         slices' sorted lists, resolves the exact threshold key and how many
//         of its ties are kept (radix passes over the gathered keys), counts
//         the kept keys of the slices before it, and writes its own kept
//         positions (protected ones included), ranked with ballots.
// Bins, thresholds and counts are integers computed identically in every
// slice, so the result equals the one-work-group select bit for bit and does
// not depend on timing.  A bin with more keys than the LDS list holds is
// resolved by streaming its keys from memory on every pass (exact, slower).
// ---------------------------------------------------------------------------
// work-group size: 1024 threads (16 waves, 4 rows of 64 positions each) when
// the grid is small enough to leave compute units idle, 256 threads (4 waves,
// 16 rows each) when many slices keep every compute unit busy
constexpr int kMsBigGrid = 1024;  // slices per launch from which 256-thread work-groups are used
constexpr int kMsBins = 4096;
constexpr int kMsShift = 14;                    // bin width in key units
constexpr int kMsCoarse = 64;                   // coarse bins (of 64 bins each)
constexpr int kMsListCap = 4096;                // threshold-bin keys held in LDS
constexpr uint32_t kNoneKept = 0xfffffffdu;     // threshold above every unprotected key

struct MselHead {     // per (layer-head, slice); 256 bytes
  uint32_t ncand;     // unprotected positions of the slice
  int32_t kc;         // window centre, in key >> kMsShift units (the same in every slice)
  uint32_t pad[30];
  uint32_t coarse[kMsCoarse / 2];  // 16-bit coarse counts, packed pairs
};

struct MselPtrs {
  MselHead* head;     // [L*Hkv][nslice]
  uint32_t* pre;      // [L*Hkv][nslice][kMsBins / 2]: 16-bit bin starts, packed pairs
  uint32_t* sorted;   // [L*Hkv][nslice][kMsSlice]: key low bits | slice position << 14
};

__device__ __forceinline__ MselPtrs msel_ptrs(char* ws, const MselGeomDev& g) {
  return MselPtrs{(MselHead*)(ws + g.off_head), (uint32_t*)(ws + g.off_pre),
                  (uint32_t*)(ws + g.off_sorted)};
}

// Protected window [0, a) U [c, N) of a sequence of N positions.
__device__ __forceinline__ void prot_bounds(int N, int n_sink, int n_recent, int& a, int& c) {
  a = n_sink < N ? n_sink : N;
  c = N - n_recent > 0 ? N - n_recent : 0;
  if (c < a) c = a;
}

// Bin of an order key in the window centred on kc (key >> kMsShift units).
__device__ __forceinline__ int msel_bin_of(uint32_t key, int kc) {
  const int d = (int)(key >> kMsShift) - kc + kMsBins / 2;
  return d < 0 ? 0 : (d > kMsBins - 1 ? kMsBins - 1 : d);
}

// Ascending bitonic sort across the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_sort_u32(uint32_t v, int lane) {
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint32_t o = __shfl_xor(v, j);
      const bool up = (lane & k) == 0 || k == 64;
      const bool lower = (lane & j) == 0;
      v = (lower == up) ? (o < v ? o : v) : (o > v ? o : v);
    }
  }
  return v;
}

// 16-bit entry i of an array of packed pairs.
__device__ __forceinline__ uint32_t ld16(const uint32_t* base, int i) {
  const uint32_t w = base[i >> 1];
  return (i & 1) ? (w >> 16) : (w & 0xffffu);
}

template <bool REFINE, int kMsThreads>
__global__ __launch_bounds__(kMsThreads) void msel_bin(const float* __restrict__ src,
                                                       float* __restrict__ z, MselArgs a,
                                                       char* __restrict__ ws) {
  constexpr int kMsWaves = kMsThreads / 64;
  constexpr int kMsRows = kMsSlice / kMsThreads;  // rows of 64 positions per wave
  __shared__ float tile[REFINE ? kMsSlice + 2 * kMaxHalf : 1];
  __shared__ uint32_t hist[kMsBins];         // counts, then scatter cursors
  __shared__ uint32_t srt[kMsSlice];         // packed keys in bin order
  __shared__ uint32_t wsum[kMsWaves];
  __shared__ float sh_beta;
  __shared__ int sh_kc;
  const MselPtrs P = msel_ptrs(ws, a.g);
  const int lh = blockIdx.y, x = blockIdx.x;
  const int l = lh / a.Hkv, g = lh - l * a.Hkv;
  const int b = seq_of_tile(a.st, x);
  const int N = (int)a.st.N[b];
  const int s0 = (x - a.st.tile_off[b]) * kMsSlice;
  int A, Cc;
  prot_bounds(N, a.n_sink, a.n_recent, A, Cc);
  const int ncand_u = Cc - A;
  const int need = (int)a.st.kept[b] - (N - ncand_u);  // unprotected positions kept
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int p0 = s0 + wave * (64 * kMsRows) + lane;
  const float* sb = src + (int64_t)lh * a.T + a.st.cu[b];
  float v[kMsRows];
#pragma unroll
  for (int j = 0; j < kMsRows; ++j) {
    const int p = p0 + 64 * j;
    v[j] = p < N ? sb[p] : 0.f;
  }
  // wave 0: the window centre from 64 sample positions of the unit's
  // unprotected range (their scores before refinement when refining)
  uint32_t samp = 0u;
  if (wave == 0 && ncand_u > 0) {
    const int ps = A + (int)(((int64_t)(2 * lane + 1) * ncand_u) / 128);
    samp = order_key_bits(__float_as_uint(sb[ps]));
  }
  float hv = 0.f;
  const int half = REFINE ? a.half : 0;
  if (REFINE && tid < 2 * half) {
    const int i = tid < half ? s0 - half + tid : s0 + kMsSlice - half + tid;
    hv = (i >= 0 && i < N) ? sb[i] : 0.f;
  }
  for (int i = tid; i < kMsBins; i += kMsThreads) hist[i] = 0u;
  if (wave == 0) {
    samp = wave_sort_u32(samp, lane);
    int q = ncand_u > 0 ? (int)(((int64_t)(ncand_u - need) * 64) / ncand_u) : 0;
    q = q < 0 ? 0 : (q > 63 ? 63 : q);
    const uint32_t kq = __shfl(samp, q);
    if (lane == 0) sh_kc = (int)(kq >> kMsShift);
  }
  if constexpr (REFINE) {
    float* zb = z + (int64_t)lh * a.T + a.st.cu[b];
#pragma unroll
    for (int j = 0; j < kMsRows; ++j) tile[half + p0 + 64 * j - s0] = v[j];
    if (tid < 2 * half) tile[tid < half ? tid : kMsSlice + tid] = hv;
    if (tid >= 64 && tid < 128) {  // wave 1: the head weight
      const int lb = l * a.st.B + b;
      const int u = lb * a.Hkv + g;
      const float bt = a.beta_in ? a.beta_in[u]
                                 : head_beta(a.st, lb, b, g, a.Hkv, a.stats, a.beta_lo, a.beta_hi);
      if (tid == 64) {
        sh_beta = bt;
        if (a.beta_out && s0 == 0) a.beta_out[u] = bt;
      }
    }
    __syncthreads();
    const float bt = sh_beta;
#pragma unroll
    for (int j = 0; j < kMsRows; ++j) {
      const int p = p0 + 64 * j;
      if (p < N) {
        v[j] = refined(tile, p - s0, p, s0, N, half, a.gamma, bt, a.r2);
        zb[p] = v[j];
      }
    }
  } else {
    __syncthreads();
  }
  const int kc = sh_kc;
  // bins of the slice's unprotected keys
  uint32_t bin[kMsRows], low[kMsRows];
#pragma unroll
  for (int j = 0; j < kMsRows; ++j) {
    const int p = p0 + 64 * j;
    const uint32_t k = order_key_bits(__float_as_uint(v[j]));
    low[j] = k & ((1u << kMsShift) - 1u);
    bin[j] = (p >= A && p < Cc) ? (uint32_t)msel_bin_of(k, kc) : 0xffffffffu;
    if (bin[j] != 0xffffffffu) atomicAdd(&hist[bin[j]], 1u);
  }
  __syncthreads();
  // this thread's 16 bins: exclusive starts (the scatter cursors), published
  constexpr int PER = kMsBins / kMsThreads;
  uint32_t h[PER], tot = 0u;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    h[e] = hist[tid * PER + e];
    tot += h[e];
  }
  uint32_t incl = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t start = incl - tot;
  for (int w = 0; w < wave; ++w) start += wsum[w];
  const int64_t sl = (int64_t)lh * a.nslice + x;
  uint32_t* pre = P.pre + sl * (kMsBins / 2);
#pragma unroll
  for (int e = 0; e < PER; e += 2) {
    const uint32_t s_e = start, s_f = start + h[e];
    pre[(tid * PER + e) >> 1] = s_e | (s_f << 16);
    hist[tid * PER + e] = s_e;
    hist[tid * PER + e + 1] = s_f;
    start = s_f + h[e + 1];
  }
  // coarse counts: TPC threads per coarse bin of 64 bins, two bins a word
  constexpr int TPC = 64 / PER;
  uint32_t cq = tot;
#pragma unroll
  for (int off = 1; off < TPC; off <<= 1) cq += __shfl_xor(cq, off);
  const uint32_t cq_hi = __shfl_down(cq, TPC);  // the next coarse bin's count
  MselHead* hd = P.head + sl;
  if ((tid & (2 * TPC - 1)) == 0) hd->coarse[tid / (2 * TPC)] = cq | (cq_hi << 16);
  __syncthreads();
  // counting sort of the slice's keys by bin (order inside a bin is free)
#pragma unroll
  for (int j = 0; j < kMsRows; ++j) {
    if (bin[j] != 0xffffffffu) {
      const uint32_t slot = atomicAdd(&hist[bin[j]], 1u);
      srt[slot] = low[j] | ((uint32_t)(p0 + 64 * j - s0) << kMsShift);
    }
  }
  __syncthreads();
  uint32_t* so = P.sorted + sl * kMsSlice;
  const int e = s0 + kMsSlice < N ? s0 + kMsSlice : N;
  const int lo = s0 > A ? s0 : A, hi = e < Cc ? e : Cc;
  const int nc = hi > lo ? hi - lo : 0;
  for (int i = tid; i < nc; i += kMsThreads) so[i] = srt[i];
  if (tid == 0) {
    hd->ncand = (uint32_t)nc;
    hd->kc = kc;
  }
}

// Bin (from the top) of a 64-bin histogram, one bin per lane of the calling
// wave, where the count from the top first reaches `need`, and the count
// strictly above it.  Wave-uniform results.
__device__ __forceinline__ void find64(uint32_t c, uint32_t need, int lane, uint32_t& d,
                                       uint32_t& above) {
  uint32_t inc = c;  // inclusive suffix: bins >= lane
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_down(inc, off);
    if (lane + off < 64) inc += y;
  }
  const uint32_t ab = inc - c;
  const bool hit = ab < need && inc >= need;
  const unsigned long long m = __ballot(hit);
  const int src = m ? (int)__builtin_ctzll(m) : 0;
  d = (uint32_t)src;
  above = __shfl(ab, src);
}

template <int kMsThreads>
__global__ __launch_bounds__(kMsThreads) void msel_pick(const float* __restrict__ z, MselArgs a,
                                                        const char* __restrict__ ws,
                                                        int32_t* __restrict__ idx) {
  constexpr int kMsWaves = kMsThreads / 64;
  constexpr int kMsRows = kMsSlice / kMsThreads;  // rows of 64 positions per wave
  // per-slice arrays, sized by the launch for its longest sequence
  extern __shared__ uint32_t slice_lds[];
  uint32_t* lst = slice_lds;
  uint32_t* lcnt = lst + a.max_nsl;
  uint32_t* abv = lcnt + a.max_nsl;
  uint32_t* loff = abv + a.max_nsl;
  __shared__ uint32_t lkey[kMsListCap];
  __shared__ uint16_t lw[kMsListCap];
  __shared__ uint32_t h2[kMsThreads];  // partial counts, then radix digits
  __shared__ uint32_t wsum[2][kMsWaves];
  __shared__ uint32_t sres[4];
  const MselPtrs P = msel_ptrs((char*)ws, a.g);
  const int lh = blockIdx.y, x = blockIdx.x;
  const int b = seq_of_tile(a.st, x);
  const int N = (int)a.st.N[b];
  const int kept = (int)a.st.kept[b];
  const int x0 = a.st.tile_off[b];
  const int nsl = a.st.tile_off[b + 1] - x0;
  const int me = x - x0;
  const int s0 = me * kMsSlice;
  int A, Cc;
  prot_bounds(N, a.n_sink, a.n_recent, A, Cc);
  const int ncand_u = Cc - A;
  const uint32_t need = (uint32_t)(kept - (N - ncand_u));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const float* zb = z + (int64_t)lh * a.T + a.st.cu[b];
  const MselHead* heads = P.head + (int64_t)lh * a.nslice + x0;
  const uint32_t* pres = P.pre + ((int64_t)lh * a.nslice + x0) * (kMsBins / 2);
  const uint32_t* srts = P.sorted + ((int64_t)lh * a.nslice + x0) * kMsSlice;
  // this slice's scores, loaded first (used only when writing, so the loads
  // overlap the threshold search)
  const int p0 = s0 + wave * (64 * kMsRows) + lane;
  float zv[kMsRows];
#pragma unroll
  for (int j = 0; j < kMsRows; ++j) {
    const int p = p0 + 64 * j;
    zv[j] = (p >= A && p < Cc) ? zb[p] : 0.f;
  }
  // protected positions before this slice: sinks below s0 and recents below s0
  const uint32_t prot_before = (uint32_t)((s0 < A ? s0 : A) + (s0 > Cc ? s0 - Cc : 0));
  uint32_t thr = kNoneKept, rem = 0u, Dbefore = prot_before, Tbefore = 0u;
  if (need > 0u) {
    const int kc = heads[0].kc;
    // 1. coarse bin: counts of every slice added up; thread t sums coarse
    // bin t % 64 over the slices w = t / 64 (mod the wave count), no atomics
    const int bj = tid & 63, grp = tid >> 6;
    uint32_t cacc = 0u;
#pragma unroll 4
    for (int w = grp; w < nsl; w += kMsWaves) {
      const uint32_t w2 = heads[w].coarse[bj >> 1];
      cacc += (bj & 1) ? (w2 >> 16) : (w2 & 0xffffu);
    }
    h2[tid] = cacc;
    __syncthreads();
    if (wave == 0) {
      uint32_t dc, ab;
      uint32_t csum = 0u;
      for (int g2 = 0; g2 < kMsWaves; ++g2) csum += h2[64 * g2 + lane];
      find64(csum, need, lane, dc, ab);
      if (lane == 0) {
        sres[0] = dc;
        sres[1] = ab;
      }
    }
    __syncthreads();
    const uint32_t dc = sres[0];
    uint32_t need1 = need - sres[1];
    // 2. the bin inside it, from every slice's bin starts, the same way
    const int fb = (int)dc * 64 + bj;
    uint32_t facc = 0u;
#pragma unroll 4
    for (int w = grp; w < nsl; w += kMsWaves) {
      const uint32_t* pw = pres + (int64_t)w * (kMsBins / 2);
      const uint32_t s_e = ld16(pw, fb);
      const uint32_t s_n = fb + 1 < kMsBins ? ld16(pw, fb + 1) : heads[w].ncand;
      facc += s_n - s_e;
    }
    __syncthreads();  // the coarse sums are read
    h2[tid] = facc;
    __syncthreads();
    if (wave == 0) {
      uint32_t df, ab;
      uint32_t csum = 0u;
      for (int g2 = 0; g2 < kMsWaves; ++g2) csum += h2[64 * g2 + lane];
      find64(csum, need1, lane, df, ab);
      if (lane == 0) {
        sres[0] = dc * 64 + df;
        sres[1] = ab;
      }
    }
    __syncthreads();
    const uint32_t d1 = sres[0];
    need1 -= sres[1];
    // 3. every slice's run of bin d1 in its sorted keys, and its keys above it
    for (int w = tid; w < nsl; w += kMsThreads) {
      const uint32_t* pw = pres + (int64_t)w * (kMsBins / 2);
      const uint32_t nc = heads[w].ncand;
      const uint32_t st0 = ld16(pw, (int)d1);
      const uint32_t en = d1 + 1 < (uint32_t)kMsBins ? ld16(pw, (int)d1 + 1) : nc;
      lst[w] = st0;
      lcnt[w] = en - st0;
      abv[w] = nc - en;
    }
    __syncthreads();
    if (wave == 0) {  // exclusive prefix of the runs over the slices
      uint32_t run = 0u;
      for (int base = 0; base < nsl; base += 64) {
        const int w = base + lane;
        const uint32_t c = w < nsl ? lcnt[w] : 0u;
        uint32_t inc = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t y = __shfl_up(inc, off);
          if (lane >= off) inc += y;
        }
        if (w < nsl) loff[w] = run + inc - c;
        run += __shfl(inc, 63);
      }
      if (lane == 0) loff[nsl] = run;
    }
    __syncthreads();
    const uint32_t nlist = loff[nsl];
    const bool edge_bin = d1 == 0u || d1 == (uint32_t)(kMsBins - 1);  // keys beyond the window
    const bool in_lds = nlist <= (uint32_t)kMsListCap;
    // entry i of the bin's list: its key (the low kMsShift bits, or the whole
    // key in an outermost bin) and its slice
    auto entry = [&](uint32_t i, uint32_t& k, int& w) {
      if (in_lds) {
        k = lkey[i];
        w = lw[i];
        return;
      }
      int lo = 0, hi = nsl - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (loff[mid] <= i) lo = mid; else hi = mid - 1;
      }
      w = lo;
      const uint32_t e = srts[(int64_t)w * kMsSlice + lst[w] + (i - loff[w])];
      k = edge_bin ? order_key_bits(__float_as_uint(zb[w * kMsSlice + (int)(e >> kMsShift)]))
                   : (e & ((1u << kMsShift) - 1u));
    };
    if (in_lds) {
      for (uint32_t i = tid; i < nlist; i += kMsThreads) {
        int lo = 0, hi = nsl - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (loff[mid] <= i) lo = mid; else hi = mid - 1;
        }
        const uint32_t e = srts[(int64_t)lo * kMsSlice + lst[lo] + (i - loff[lo])];
        lkey[i] = edge_bin ? order_key_bits(__float_as_uint(zb[lo * kMsSlice + (int)(e >> kMsShift)]))
                           : (e & ((1u << kMsShift) - 1u));
        lw[i] = (uint16_t)lo;
      }
      __syncthreads();
    }
    // 4. exact threshold in the bin: 8-bit radix passes from the top bit
    const int kbits = edge_bin ? 32 : kMsShift;
    uint32_t pfx = 0u;
    int done = 0;
    while (done < kbits) {
      const int nb = kbits - done < 8 ? kbits - done : 8;
      const int sh = kbits - done - nb;
      h2[tid] = 0u;
      __syncthreads();
      for (uint32_t i = tid; i < nlist; i += kMsThreads) {
        uint32_t k;
        int w;
        entry(i, k, w);
        if (done == 0 || (k >> (sh + nb)) == pfx) atomicAdd(&h2[(k >> sh) & ((1u << nb) - 1u)], 1u);
      }
      __syncthreads();
      // digit from the top: thread t holds digit t
      const uint32_t c = h2[tid];
      uint32_t inc = c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_down(inc, off);
        if (lane + off < 64) inc += y;
      }
      if (lane == 0) wsum[0][wave] = inc;
      __syncthreads();
      uint32_t ab = inc - c;
      for (int w2 = wave + 1; w2 < kMsWaves; ++w2) ab += wsum[0][w2];
      if (ab < need1 && ab + c >= need1) {
        sres[2] = (uint32_t)tid;
        sres[3] = ab;
      }
      __syncthreads();
      pfx = (pfx << nb) | sres[2];
      need1 -= sres[3];
      done += nb;
      __syncthreads();
    }
    rem = need1;
    // 5. the bin's keys above / equal to the threshold in the slices before
    // this one, and the keys of those slices in bins above d1
    uint32_t dl = 0u, tl = 0u;
    for (uint32_t i = tid; i < nlist; i += kMsThreads) {
      uint32_t k;
      int w;
      entry(i, k, w);
      if (w < me) {
        dl += k > pfx ? 1u : 0u;
        tl += k == pfx ? 1u : 0u;
      }
    }
    for (int w = tid; w < me; w += kMsThreads) dl += abv[w];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      dl += __shfl_xor(dl, off);
      tl += __shfl_xor(tl, off);
    }
    if (lane == 0) {
      wsum[0][wave] = dl;
      wsum[1][wave] = tl;
    }
    __syncthreads();
    dl = 0u;
    tl = 0u;
    for (int w2 = 0; w2 < kMsWaves; ++w2) {
      dl += wsum[0][w2];
      tl += wsum[1][w2];
    }
    Dbefore += dl;
    Tbefore = tl;
    const int kc_ = kc;
    thr = edge_bin ? pfx : (((uint32_t)((int)d1 - kMsBins / 2 + kc_) << kMsShift) | pfx);
  }
  // 6. ordered writes of this slice (protected positions and padding carry
  // keys above every score)
  uint32_t key[kMsRows];
#pragma unroll
  for (int j = 0; j < kMsRows; ++j) {
    const int p = p0 + 64 * j;
    key[j] = p >= N ? kPad
                    : ((p < A || p >= Cc) ? kProt : order_key_bits(__float_as_uint(zv[j])));
  }
  uint32_t nd = 0u, nt = 0u;
#pragma unroll
  for (int j = 0; j < kMsRows; ++j) {
    nd += (uint32_t)__popcll(__ballot(key[j] > thr && key[j] != kPad));
    nt += (uint32_t)__popcll(__ballot(key[j] == thr));
  }
  if (lane == 0) {
    wsum[0][wave] = nd;
    wsum[1][wave] = nt;
  }
  __syncthreads();
  uint32_t D = Dbefore, Tt = Tbefore;
  for (int w = 0; w < wave; ++w) {
    D += wsum[0][w];
    Tt += wsum[1][w];
  }
  int32_t* out = idx + (int64_t)lh * a.Ktot + a.st.ko[b];
  emit_round<kMsRows>(key, true, thr, rem, D, Tt, s0 + wave * (64 * kMsRows) + lane, kept, out);
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

MselGeom msel_geometry(const SeqTable& st, int L, int Hkv) {
  MselGeom g{};
  const size_t LH = (size_t)L * Hkv;
  const size_t ns = (size_t)st.tile_off[st.B];
  g.d.off_head = 0;
  g.d.off_pre = align256r(LH * ns * sizeof(MselHead));
  g.d.off_sorted = g.d.off_pre + align256r(LH * ns * (kMsBins / 2) * sizeof(uint32_t));
  g.bytes = g.d.off_sorted + align256r(LH * ns * kMsSlice * sizeof(uint32_t));
  return g;
}

hipError_t launch_msel(const float* src, bool refine, float* z, const SeqTable& st, int L,
                       int Hkv, int n_sink, int n_recent, const RefineParams& rp, int32_t* idx,
                       char* ws, const MselGeom& geo, hipStream_t stream) {
  MselArgs a{};
  a.st = st;
  a.Hkv = Hkv;
  a.n_sink = n_sink;
  a.n_recent = n_recent;
  a.nslice = st.tile_off[st.B];
  a.max_nsl = 1;
  for (int b = 0; b < st.B; ++b) {
    const int n = st.tile_off[b + 1] - st.tile_off[b];
    a.max_nsl = n > a.max_nsl ? n : a.max_nsl;
  }
  a.T = 0;
  a.Ktot = 0;
  for (int b = 0; b < st.B; ++b) {
    a.T += st.N[b];
    a.Ktot += st.kept[b];
  }
  a.g = geo.d;
  a.half = rp.pool / 2;
  a.gamma = rp.gamma;
  a.r2 = rp.r2;
  a.beta_lo = rp.beta_lo;
  a.beta_hi = rp.beta_hi;
  a.beta_in = rp.beta_in;
  a.stats = rp.stats;
  a.beta_out = rp.beta_out;
  const dim3 grid(a.nslice, L * Hkv);
  const bool big = (int64_t)a.nslice * L * Hkv >= kMsBigGrid;
  const dim3 block(big ? 256 : 1024);
  if (refine && big)
    hipLaunchKernelGGL((msel_bin<true, 256>), grid, block, 0, stream, src, z, a, ws);
  else if (refine)
    hipLaunchKernelGGL((msel_bin<true, 1024>), grid, block, 0, stream, src, z, a, ws);
  else if (big)
    hipLaunchKernelGGL((msel_bin<false, 256>), grid, block, 0, stream, src, z, a, ws);
  else
    hipLaunchKernelGGL((msel_bin<false, 1024>), grid, block, 0, stream, src, z, a, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)(4 * a.max_nsl + 1) * sizeof(uint32_t);
  const float* zz = refine ? (const float*)z : src;
  if (big)
    hipLaunchKernelGGL((msel_pick<256>), grid, block, lds, stream, zz, a, (const char*)ws, idx);
  else
    hipLaunchKernelGGL((msel_pick<1024>), grid, block, lds, stream, zz, a, (const char*)ws, idx);
  return hipGetLastError();
}

}  // namespace hubkv
