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
__device__ __forceinline__ void emit_round(const uint32_t (&key)[kSelKpt], bool edge, uint32_t thr,
                                           uint32_t rem, uint32_t D, uint32_t Tt, int p0, int kept,
                                           int32_t* __restrict__ out) {
  uint32_t thw = thr;
  asm volatile("" : "+v"(thw));  // keeps earlier compares against thr from being reused
  // usual case: no key of the wave's rows equals thr, so the tie count Tt
  // stays put and each row needs one ballot
  bool anyeq = false;
#pragma unroll
  for (int j = 0; j < kSelKpt; ++j) anyeq |= key[j] == thw;
  if (!__any(anyeq)) {
    uint32_t base = D + (Tt < rem ? Tt : rem);
#pragma unroll
    for (int j = 0; j < kSelKpt; ++j) {
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
  for (int j = 0; j < kSelKpt; ++j) {
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
