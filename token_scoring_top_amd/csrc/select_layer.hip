// select_layer.hip -- layer-wide budget allocation over the KV heads of a
// layer, and the compaction of its output.
//
// NestedKV summary page, head-wise memory allocation: instead of an even
// split, the layer's budget goes to the (token, head) pairs with the highest
// scores across the layer, each head keeping a minimum of its own; KV-cache
// survey page, section 4.4 (PyramidKV): the budget itself is set per layer.
// Per (layer l, sequence b), with P the protected positions and f the floor:
//   every head keeps P and its f best candidates (z descending, position
//   ascending, NaN lowest, -0 == +0);
//   the remaining candidates of all heads compete for
//   R = budget - Hkv (|P| + f) places in (z descending, head ascending,
//   position ascending) order.
// Every head then keeps a prefix of its own order, so the result is a per-head
// Top-k_h with k_h set by one layer-wide threshold.
//
// Keys are 32-bit order keys of z (larger key = kept first).  Everything is a
// radix search in three levels (key bits 31..21, 20..10, 9..0) over chunks of
// kLselChunk positions, one work-group per (layer, head, chunk):
//   floor levels   per head, the key of its f-th best candidate (phi) and how
//                  many of the candidates equal to phi the floor takes;
//   pool levels    per (layer, sequence), over the candidates outside the
//                  floors -- every key below its head's phi, plus the ties at
//                  phi the floor leaves out -- the key tau of the R-th best
//                  and how many of the ties at tau are taken (in head order);
//   count          per head, remaining keys above / at tau; the last
//                  work-group of a (layer, sequence) turns them into k_h, the
//                  head's emission threshold (kappa, r) and its output offset;
//   emission       per chunk, kept counts, then ordered writes.
// Work-groups add their LDS histograms into a global one with agent-scope
// atomics; the last one to arrive (a counter) resolves the level, clears the
// histogram and the counter for the next launch.  No work-group ever waits for
// another.
#include "internal.hpp"

namespace hubkv {

namespace {

constexpr int kT = 256;                     // threads per work-group
constexpr int kPer = kLselChunk / kT;       // positions per thread in a chunk
constexpr int kBins = 2048;
constexpr uint32_t kNone = 0xffffffffu;     // above every order key

// Order key of an fp32 score: larger value -> larger key, -0 == +0, NaN lowest.
__device__ __forceinline__ uint32_t ordkey(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return v != v ? 0u : k;
}

__device__ __forceinline__ constexpr int lv_shift(int lv) {
  return lv == 0 ? 21 : (lv == 1 ? 10 : 0);
}
__device__ __forceinline__ constexpr int lv_bits(int lv) { return lv == 2 ? 10 : 11; }

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ uint32_t ld_ag(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_ag(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void add_ag(uint32_t* p, uint32_t v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t bump_ag(uint32_t* p) {
  return __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Per (layer, sequence, head) state, 64 bytes.
struct HeadState {
  uint32_t pfx, need;   // floor search: key prefix so far, candidates still to place
  uint32_t phi;         // floor key (kNone: no floor; 0 with remf = kNone: all candidates)
  uint32_t remf;        // candidates equal to phi inside the floor
  uint32_t cties;       // candidates equal to phi outside the floor
  uint32_t gt, eq;      // pool keys above / equal to tau
  uint32_t kappa, r;    // emission: keep keys > kappa and the first r equal to kappa
  uint32_t k;           // kept count
  uint32_t search;      // the floor search runs
  uint32_t pad;
  int64_t off;          // first output row
  int64_t pad2;
};
// Per (layer, sequence) state, 32 bytes.
struct SegState {
  uint32_t pfx, need;   // pool search
  uint32_t tau, rem;    // pool threshold and ties taken at it
  uint32_t search;
  uint32_t pad[3];
};

struct Ws {
  HeadState* hs;
  SegState* ss;
  uint32_t* hh;    // [U][kBins]
  uint32_t* hg;    // [S][kBins]
  uint32_t* ch;    // [U] arrival counters (floor levels)
  uint32_t* cg;    // [S] arrival counters (pool levels, count)
  uint2* ec;       // [L * Hkv][nchunk] emission counts per chunk
};

__device__ __forceinline__ Ws ws_of(char* base, const LselGeom& g) {
  Ws w;
  w.hs = (HeadState*)(base + g.off_hs);
  w.ss = (SegState*)(base + g.off_ss);
  w.hh = (uint32_t*)(base + g.off_hh);
  w.hg = (uint32_t*)(base + g.off_hg);
  w.ch = (uint32_t*)(base + g.off_ch);
  w.cg = (uint32_t*)(base + g.off_cg);
  w.ec = (uint2*)(base + g.off_ec);
  return w;
}

__device__ __forceinline__ int seq_of_chunk(const LselArgs& a, int x) {
  int b = 0;
  while (b + 1 < a.B && a.ch_off[b + 1] <= x) ++b;
  return b;
}

__device__ __forceinline__ int64_t prot_count(int64_t N, int ns, int nr) {
  const int64_t lo = ns < N ? ns : N;
  const int64_t hi = N - nr > 0 ? N - nr : 0;
  return hi <= lo ? N : lo + (N - hi);
}

// Where a work-group's chunk sits: layer, head, sequence, chunk, positions.
struct Chunk {
  int l, h, b, c, nch, u, s;
  int64_t N, p0, p1;
  const float* zb;
};

__device__ __forceinline__ Chunk chunk_of(const LselArgs& a, const float* z) {
  Chunk k;
  const int lh = blockIdx.y;
  k.l = lh / a.Hkv;
  k.h = lh - k.l * a.Hkv;
  const int x = blockIdx.x;
  k.b = seq_of_chunk(a, x);
  k.c = x - a.ch_off[k.b];
  k.nch = a.ch_off[k.b + 1] - a.ch_off[k.b];
  k.s = k.l * a.B + k.b;
  k.u = k.s * a.Hkv + k.h;
  k.N = a.N[k.b];
  k.p0 = (int64_t)k.c * kLselChunk;
  k.p1 = k.p0 + kLselChunk < k.N ? k.p0 + kLselChunk : k.N;
  k.zb = z + (int64_t)lh * a.T + a.cu[k.b];
  return k;
}

// The chunk's keys: thread t holds positions p0 + t + kT j; kNone marks a
// protected position or one past the chunk (kNone is above every order key
// and is never counted as a candidate).
__device__ __forceinline__ void load_keys(const LselArgs& a, const Chunk& k,
                                          uint32_t (&key)[kPer]) {
  const int64_t lo = a.n_sink, hi = k.N - a.n_recent;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t p = k.p0 + threadIdx.x + kT * j;
    const bool in = p < k.p1;
    const float v = k.zb[in ? p : k.p0];
    key[j] = (!in || p < lo || p >= hi) ? kNone : ordkey(v);
  }
}

// Bin of a kBins-entry LDS histogram (entries [0, nb)) holding the need-th
// key from the top, and the count strictly above that bin.  Block-uniform.
// Returns false when the histogram holds fewer than need keys.
__device__ bool find_top(const uint32_t* hist, int nb, uint32_t need, uint32_t* red, uint32_t* res,
                         uint32_t& bin, uint32_t& above) {
  constexpr int E = kBins / kT;  // 8 bins per thread, from the top down
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int top = nb - 1 - E * tid;
  uint32_t h[E], mine = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    h[e] = top - e >= 0 ? hist[top - e] : 0u;
    mine += h[e];
  }
  uint32_t incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) red[wave] = incl;
  if (tid == 0) res[2] = 0u;
  __syncthreads();
  uint32_t ab = incl - mine;
  for (int w = 0; w < wave; ++w) ab += red[w];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (ab < need && ab + h[e] >= need) {
      res[0] = (uint32_t)(top - e);
      res[1] = ab;
      res[2] = 1u;
    }
    ab += h[e];
  }
  __syncthreads();
  bin = res[0];
  above = res[1];
  const bool ok = res[2] != 0u;
  __syncthreads();
  return ok;
}

// Copies the first nb bins of a global histogram into LDS (kBins entries, the
// rest zero) with every load in flight at once, then clears the global bins
// for the next launch.
__device__ __forceinline__ void take_hist(uint32_t* gh, int nb, uint32_t* hist) {
  constexpr int E = kBins / kT;
  uint32_t v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = e * kT + threadIdx.x;
    v[e] = i < nb ? ld_ag(gh + i) : 0u;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = e * kT + threadIdx.x;
    hist[i] = v[e];
    if (v[e]) st_ag(gh + i, 0u);
  }
}

// Adds the LDS histogram into the global one, then counts the work-group in.
// Returns true (block-uniform) in the last work-group of `total`.
__device__ bool push_and_arrive(const uint32_t* lh, uint32_t* gh, uint32_t* cnt, uint32_t total,
                                uint32_t* flag) {
  for (int i = threadIdx.x; i < kBins; i += kT)
    if (lh[i]) add_ag(gh + i, lh[i]);
  wait_vm();
  __syncthreads();
  if (threadIdx.x == 0) *flag = bump_ag(cnt) == total - 1 ? 1u : 0u;
  __syncthreads();
  return *flag != 0u;
}

// ---- initial state, histograms and counters cleared (fill kernel, no memset)
__global__ __launch_bounds__(kT) void lsel_init(LselArgs a, LselGeom g, char* base) {
  const Ws w = ws_of(base, g);
  const int u = blockIdx.x;  // (l, b, h)
  const int s = u / a.Hkv, h = u - s * a.Hkv;
  const int b = s % a.B;
  for (int i = threadIdx.x; i < kBins; i += kT) w.hh[(int64_t)u * kBins + i] = 0u;
  if (h == 0)
    for (int i = threadIdx.x; i < kBins; i += kT) w.hg[(int64_t)s * kBins + i] = 0u;
  if (threadIdx.x == 0) {
    const int64_t N = a.N[b];
    const int64_t P = prot_count(N, a.n_sink, a.n_recent);
    const int64_t f = a.f[b];
    HeadState hs;
    hs.pfx = 0u;
    hs.need = (uint32_t)f;
    hs.search = (f > 0 && f < N - P) ? 1u : 0u;
    hs.phi = f == 0 ? kNone : 0u;
    hs.remf = (f > 0 && f == N - P) ? kNone : 0u;  // every candidate is in the floor
    hs.cties = 0u;
    hs.gt = hs.eq = 0u;
    hs.kappa = hs.r = hs.k = 0u;
    hs.pad = 0u;
    hs.off = 0;
    hs.pad2 = 0;
    w.hs[u] = hs;
    w.ch[u] = 0u;
    if (h == 0) {
      const int64_t R = (int64_t)a.budget[s] - (int64_t)a.Hkv * (P + f);
      SegState ss;
      ss.pfx = 0u;
      ss.need = (uint32_t)R;
      ss.search = R > 0 ? 1u : 0u;
      ss.tau = kNone;
      ss.rem = 0u;
      ss.pad[0] = ss.pad[1] = ss.pad[2] = 0u;
      w.ss[s] = ss;
      w.cg[s] = 0u;
    }
  }
}

// ---- floor levels: per head, the f-th best candidate
template <int LV>
__global__ __launch_bounds__(kT) void lsel_floor_level(const float* __restrict__ z, LselArgs a,
                                                       LselGeom g, char* base) {
  constexpr int SH = lv_shift(LV), NB = 1 << lv_bits(LV);
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t red[kT / 64], res[3], flag;
  const Ws w = ws_of(base, g);
  const Chunk k = chunk_of(a, z);
  HeadState* hs = w.hs + k.u;
  uint32_t key[kPer];
  load_keys(a, k, key);     // in flight while the state is read
  if (!hs->search) return;  // uniform over the head's work-groups
  const uint32_t pfx = hs->pfx;
  for (int i = threadIdx.x; i < kBins; i += kT) hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint32_t x = key[j];
    if (x != kNone && (LV == 0 || (x >> (SH + lv_bits(LV))) == pfx))
      atomicAdd(&hist[(x >> SH) & (NB - 1)], 1u);
  }
  __syncthreads();
  uint32_t* gh = w.hh + (int64_t)k.u * kBins;
  if (!push_and_arrive(hist, gh, w.ch + k.u, (uint32_t)k.nch, &flag)) return;
  // last work-group of the head: resolve the level
  take_hist(gh, NB, hist);
  __syncthreads();
  uint32_t bin, above;
  const uint32_t need = hs->need;
  const bool ok = find_top(hist, NB, need, red, res, bin, above);
  if (threadIdx.x == 0) {
    const uint32_t np = (pfx << lv_bits(LV)) | (ok ? bin : 0u);
    if (LV < 2) {
      hs->pfx = np;
      hs->need = need - above;
    } else {
      hs->phi = np;
      hs->remf = need - above;
      hs->cties = (ok ? hist[bin] : 0u) - (need - above);
      hs->search = 0u;
    }
    st_ag(w.ch + k.u, 0u);
  }
}

// ---- pool levels: per (layer, sequence), over the candidates outside the floors
template <int LV>
__global__ __launch_bounds__(kT) void lsel_pool_level(const float* __restrict__ z, LselArgs a,
                                                      LselGeom g, char* base) {
  constexpr int SH = lv_shift(LV), NB = 1 << lv_bits(LV);
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t red[kT / 64], res[3], flag;
  const Ws w = ws_of(base, g);
  const Chunk k = chunk_of(a, z);
  SegState* ss = w.ss + k.s;
  uint32_t key[kPer];
  load_keys(a, k, key);     // in flight while the state is read
  if (!ss->search) return;  // uniform over the (layer, sequence)
  const uint32_t pfx = ss->pfx;
  const uint32_t phi = w.hs[k.u].phi;
  for (int i = threadIdx.x; i < kBins; i += kT) hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint32_t x = key[j];
    if (x != kNone && x < phi && (LV == 0 || (x >> (SH + lv_bits(LV))) == pfx))
      atomicAdd(&hist[(x >> SH) & (NB - 1)], 1u);
  }
  __syncthreads();
  uint32_t* gh = w.hg + (int64_t)k.s * kBins;
  if (!push_and_arrive(hist, gh, w.cg + k.s, (uint32_t)(k.nch * a.Hkv), &flag)) return;
  // last work-group of the (layer, sequence): add the floors' left-out ties
  take_hist(gh, NB, hist);
  __syncthreads();
  for (int hh = threadIdx.x; hh < a.Hkv; hh += kT) {
    const HeadState& o = w.hs[(int64_t)k.s * a.Hkv + hh];
    if (o.cties && (LV == 0 || (o.phi >> (SH + lv_bits(LV))) == pfx))
      atomicAdd(&hist[(o.phi >> SH) & (NB - 1)], o.cties);
  }
  __syncthreads();
  uint32_t bin, above;
  const uint32_t need = ss->need;
  const bool ok = find_top(hist, NB, need, red, res, bin, above);
  if (threadIdx.x == 0) {
    const uint32_t np = (pfx << lv_bits(LV)) | (ok ? bin : 0u);
    if (LV < 2) {
      ss->pfx = np;
      ss->need = need - above;
    } else {
      ss->tau = np;
      ss->rem = need - above;
      ss->search = 0u;
    }
    st_ag(w.cg + k.s, 0u);
  }
}

// ---- pool keys above / at tau per head; the last work-group of a (layer,
// sequence) sets every head's kept count, emission threshold and offset
__global__ __launch_bounds__(kT) void lsel_count(const float* __restrict__ z, LselArgs a,
                                                 LselGeom g, char* base,
                                                 int32_t* __restrict__ head_kept) {
  __shared__ uint32_t rg[kT / 64], re[kT / 64], flag;
  const Ws w = ws_of(base, g);
  const Chunk k = chunk_of(a, z);
  const SegState* ss = w.ss + k.s;
  const uint32_t tau = ss->tau;
  HeadState* hs = w.hs + k.u;
  const uint32_t phi = hs->phi;
  uint32_t key[kPer];
  load_keys(a, k, key);
  uint32_t gt = 0u, eq = 0u;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const uint32_t x = key[j];
    if (x != kNone && x < phi) {
      gt += x > tau ? 1u : 0u;
      eq += x == tau ? 1u : 0u;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    gt += __shfl_xor(gt, off);
    eq += __shfl_xor(eq, off);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    rg[wave] = gt;
    re[wave] = eq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t G = 0u, E = 0u;
    for (int i = 0; i < kT / 64; ++i) {
      G += rg[i];
      E += re[i];
    }
    if (G) add_ag(&hs->gt, G);
    if (E) add_ag(&hs->eq, E);
    wait_vm();
    flag = bump_ag(w.cg + k.s) == (uint32_t)(k.nch * a.Hkv) - 1 ? 1u : 0u;
  }
  __syncthreads();
  if (!flag || wave != 0) return;
  // the (layer, sequence)'s last work-group, wave 0: heads in groups of 64,
  // in order, with running totals carried between groups
  const int64_t P = prot_count(k.N, a.n_sink, a.n_recent);
  const int64_t f = a.f[k.b];
  int64_t seg = 0;
  for (int v = 0; v < k.s; ++v) seg += a.budget[v];
  const int64_t seg_end = seg + a.budget[k.s];
  uint32_t left = ss->rem;   // ties at tau still to hand out
  int64_t off = seg;         // first row of the group's first head
  for (int h0 = 0; h0 < a.Hkv; h0 += 64) {
    const int hh = h0 + lane;
    const bool on = hh < a.Hkv;
    HeadState* o = w.hs + (int64_t)k.s * a.Hkv + (on ? hh : 0);
    uint32_t ph = 0u, ct = 0u, remf = 0u, g2 = 0u, e2 = 0u;
    if (on) {
      ph = o->phi;
      ct = o->cties;
      remf = o->remf;
      g2 = ld_ag(&o->gt);
      e2 = ld_ag(&o->eq);
      if (ph != kNone && ph > tau) g2 += ct;  // the floor's left-out ties sit above tau
      if (ph == tau) e2 += ct;
    }
    // ties at tau go to the lower heads first: x = clamp(left - ties of the heads before)
    uint32_t incl = e2;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    const uint32_t before = incl - e2;
    const uint32_t x = before >= left ? 0u : (e2 < left - before ? e2 : left - before);
    uint32_t kap, r;
    if (ph < tau) {
      kap = ph;
      r = remf;
    } else if (ph == tau) {
      kap = tau;
      r = remf == kNone ? kNone : remf + x;
    } else {
      kap = tau;
      r = x;
    }
    const int64_t kh0 = on ? P + f + g2 + x : 0;
    int64_t kin = kh0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t y = __shfl_up(kin, d);
      if (lane >= d) kin += y;
    }
    const int64_t my_off = off + kin - kh0;
    int64_t kh = kh0;
    if (my_off + kh > seg_end) kh = seg_end > my_off ? seg_end - my_off : 0;  // stay in the slice
    if (on) {
      o->kappa = kap;
      o->r = r;
      o->k = (uint32_t)kh;
      o->off = my_off;
      head_kept[(int64_t)k.s * a.Hkv + hh] = (int32_t)kh;
    }
    const uint32_t tot_e = __shfl(incl, 63);
    left = tot_e >= left ? 0u : left - tot_e;
    off += __shfl(kin, 63);
  }
  if (lane == 0) st_ag(w.cg + k.s, 0u);
}

// Keep rule of the emission: protected, above kappa, or one of the first r
// keys equal to kappa (in position order).
__device__ __forceinline__ void emit_flags(uint32_t x, uint32_t kap, bool& def, bool& tie) {
  def = x == kNone ? true : x > kap;  // kNone here marks a protected position
  tie = x != kNone && x == kap;
}

// Chunk keys for the emission: protected positions get kNone (kept), positions
// past the chunk get 0 with `valid` false.
__device__ __forceinline__ void load_emit(const LselArgs& a, const Chunk& k, int64_t base,
                                          uint32_t (&key)[kPer], bool (&valid)[kPer]) {
  const int64_t lo = a.n_sink, hi = k.N - a.n_recent;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int64_t p = base + 64 * j + lane;
    valid[j] = p < k.p1;
    const float v = k.zb[valid[j] ? p : k.p0];
    key[j] = (p < lo || p >= hi) ? kNone : ordkey(v);
  }
}

// ---- emission counts per chunk: kept-for-sure and tied keys
__global__ __launch_bounds__(kT) void lsel_emit_count(const float* __restrict__ z, LselArgs a,
                                                      LselGeom g, char* base) {
  __shared__ uint32_t rd[kT / 64], rt[kT / 64];
  const Ws w = ws_of(base, g);
  const Chunk k = chunk_of(a, z);
  const HeadState& hs = w.hs[k.u];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t key[kPer];
  bool valid[kPer];
  load_emit(a, k, k.p0 + 64 * kPer * wave, key, valid);
  uint32_t D = 0u, Tn = 0u;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    bool def, tie;
    emit_flags(key[j], hs.kappa, def, tie);
    D += (uint32_t)__popcll(__ballot(valid[j] && def));
    Tn += (uint32_t)__popcll(__ballot(valid[j] && tie));
  }
  if (lane == 0) {
    rd[wave] = D;
    rt[wave] = Tn;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint2 c = make_uint2(0u, 0u);
    for (int i = 0; i < kT / 64; ++i) {
      c.x += rd[i];
      c.y += rt[i];
    }
    w.ec[(int64_t)blockIdx.y * a.nchunk + blockIdx.x] = c;
  }
}

__device__ __forceinline__ uint32_t rank_below(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// ---- ordered writes: wave w of a chunk owns its positions [64 kPer w,
// 64 kPer (w + 1)) in rows of 64; ranks come from the earlier chunks' counts,
// the earlier waves' counts and ballots inside a row
__global__ __launch_bounds__(kT) void lsel_emit(const float* __restrict__ z, LselArgs a, LselGeom g,
                                                char* base, int32_t* __restrict__ idx) {
  __shared__ uint32_t rd[kT / 64], rt[kT / 64];
  const Ws w = ws_of(base, g);
  const Chunk k = chunk_of(a, z);
  const HeadState& hs = w.hs[k.u];
  const uint32_t kap = hs.kappa, r = hs.r, kh = hs.k;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // counts of the head's earlier chunks of this sequence
  uint32_t D0 = 0u, T0 = 0u;
  {
    const uint2* ec = w.ec + (int64_t)blockIdx.y * a.nchunk + a.ch_off[k.b];
    for (int c = lane; c < k.c; c += 64) {
      const uint2 v = ec[c];
      D0 += v.x;
      T0 += v.y;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      D0 += __shfl_xor(D0, off);
      T0 += __shfl_xor(T0, off);
    }
  }
  uint32_t key[kPer];
  bool valid[kPer];
  const int64_t base_p = k.p0 + 64 * kPer * wave;
  load_emit(a, k, base_p, key, valid);
  uint32_t D = 0u, Tn = 0u;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    bool def, tie;
    emit_flags(key[j], kap, def, tie);
    D += (uint32_t)__popcll(__ballot(valid[j] && def));
    Tn += (uint32_t)__popcll(__ballot(valid[j] && tie));
  }
  if (lane == 0) {
    rd[wave] = D;
    rt[wave] = Tn;
  }
  __syncthreads();
  D = D0;
  Tn = T0;
  for (int i = 0; i < wave; ++i) {
    D += rd[i];
    Tn += rt[i];
  }
  int32_t* out = idx + hs.off;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    bool def, tie;
    emit_flags(key[j], kap, def, tie);
    def = def && valid[j];
    tie = tie && valid[j];
    const unsigned long long bd = __ballot(def), bt = __ballot(tie);
    const uint32_t tk = Tn + rank_below(bt);  // tied keys before this one
    uint32_t o = 0xffffffffu;
    if (def) o = D + rank_below(bd) + (tk < r ? tk : r);
    else if (tie && tk < r) o = D + rank_below(bd) + tk;
    if (o < kh) out[o] = (int32_t)(base_p + 64 * j + lane);
    D += (uint32_t)__popcll(bd);
    Tn += (uint32_t)__popcll(bt);
  }
}

// ---- compaction of a layer-wide selection: unit (l, b, h) owns rows
// [off, off + head_kept) of the packed output, off = the (layer, sequence)'s
// first row + the head_kept of the heads before it
constexpr int kCrows = 1;      // rows per thread group and block iteration
constexpr int kCblocks = 256;  // work-groups per (layer, sequence, head), grid-stride beyond

template <int LOGP>
__global__ __launch_bounds__(kT) void compact_layer_kernel(
    const u32x4* __restrict__ k_in, const u32x4* __restrict__ v_in, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ head_kept, LselArgs a, u32x4* __restrict__ k_out,
    u32x4* __restrict__ v_out) {
  constexpr int P = 1 << LOGP;
  constexpr int RPI = kT / P;
  constexpr int RB = RPI * kCrows;
  const int u = blockIdx.y;
  const int s = u / a.Hkv, h = u - s * a.Hkv;
  const int l = s / a.B, b = s - l * a.B;
  __shared__ int64_t s_off;
  __shared__ int32_t s_n;
  if (threadIdx.x == 0) {
    // rows stay inside the (layer, sequence)'s slice whatever head_kept holds
    int64_t seg = 0;
    for (int v = 0; v < s; ++v) seg += a.budget[v];
    const int64_t seg_end = seg + a.budget[s];
    int64_t off = seg;
    for (int hh = 0; hh < h; ++hh) {
      const int32_t c = head_kept[(int64_t)s * a.Hkv + hh];
      off += c > 0 ? c : 0;
    }
    int64_t n = head_kept[u];
    if (n < 0 || off >= seg_end) n = 0;
    if (off + n > seg_end) n = seg_end - off;
    s_off = off;
    s_n = (int32_t)n;
  }
  __syncthreads();
  const int64_t off = s_off;
  const int n = s_n;
  const int64_t N = a.N[b];
  const int pc = threadIdx.x & (P - 1), rsub = threadIdx.x >> LOGP;
  const u32x4* kin = k_in + ((int64_t)(l * a.Hkv + h) * a.T + a.cu[b]) * P;
  const u32x4* vin = v_in + ((int64_t)(l * a.Hkv + h) * a.T + a.cu[b]) * P;
  for (int r0 = blockIdx.x * RB; r0 < n; r0 += gridDim.x * RB) {
    int64_t src[kCrows];
#pragma unroll
    for (int q = 0; q < kCrows; ++q) {
      const int r = r0 + q * RPI + rsub;
      src[q] = -1;
      if (r < n) {
        const int32_t p = idx[off + r];
        if (p >= 0 && p < N) src[q] = (int64_t)p * P + pc;
      }
    }
    u32x4 kv[kCrows], vv[kCrows];
#pragma unroll
    for (int q = 0; q < kCrows; ++q)
      if (src[q] >= 0) {
        kv[q] = __builtin_nontemporal_load(&kin[src[q]]);
        vv[q] = __builtin_nontemporal_load(&vin[src[q]]);
      }
#pragma unroll
    for (int q = 0; q < kCrows; ++q)
      if (src[q] >= 0) {
        const int64_t dst = (off + r0 + q * RPI + rsub) * P + pc;
        __builtin_nontemporal_store(kv[q], &k_out[dst]);
        __builtin_nontemporal_store(vv[q], &v_out[dst]);
      }
  }
}

}  // namespace

LselGeom lsel_geometry(const LselArgs& a) {
  LselGeom g;
  const int64_t U = (int64_t)a.L * a.B * a.Hkv, S = (int64_t)a.L * a.B;
  size_t o = 0;
  auto take = [&](size_t n) {
    const size_t at = o;
    o += (n + 255) & ~(size_t)255;
    return at;
  };
  g.off_hs = take(U * sizeof(HeadState));
  g.off_ss = take(S * sizeof(SegState));
  g.off_hh = take(U * kBins * 4);
  g.off_hg = take(S * kBins * 4);
  g.off_ch = take(U * 4);
  g.off_cg = take(S * 4);
  g.off_ec = take((size_t)a.L * a.Hkv * a.nchunk * sizeof(uint2));
  g.bytes = o;
  return g;
}

hipError_t launch_select_layer(const float* z, const LselArgs& a, const LselGeom& g, char* ws,
                               int32_t* idx, int32_t* head_kept, hipStream_t stream) {
  const int U = a.L * a.B * a.Hkv;
  const dim3 grid(a.nchunk, a.L * a.Hkv), block(kT);
  hipLaunchKernelGGL(lsel_init, dim3(U), block, 0, stream, a, g, ws);
  hipLaunchKernelGGL(lsel_floor_level<0>, grid, block, 0, stream, z, a, g, ws);
  hipLaunchKernelGGL(lsel_floor_level<1>, grid, block, 0, stream, z, a, g, ws);
  hipLaunchKernelGGL(lsel_floor_level<2>, grid, block, 0, stream, z, a, g, ws);
  hipLaunchKernelGGL(lsel_pool_level<0>, grid, block, 0, stream, z, a, g, ws);
  hipLaunchKernelGGL(lsel_pool_level<1>, grid, block, 0, stream, z, a, g, ws);
  hipLaunchKernelGGL(lsel_pool_level<2>, grid, block, 0, stream, z, a, g, ws);
  hipLaunchKernelGGL(lsel_count, grid, block, 0, stream, z, a, g, ws, head_kept);
  hipLaunchKernelGGL(lsel_emit_count, grid, block, 0, stream, z, a, g, ws);
  hipLaunchKernelGGL(lsel_emit, grid, block, 0, stream, z, a, g, ws, idx);
  return hipGetLastError();
}

hipError_t launch_compact_layer(const void* k_in, const void* v_in, int elem_bytes,
                                const int32_t* idx, const int32_t* head_kept, const LselArgs& a,
                                int d, void* k_out, void* v_out, hipStream_t stream) {
  const int pieces = d * elem_bytes / 16;
  const int logp = pieces == 8 ? 3 : (pieces == 16 ? 4 : 5);
  int64_t nmax = 0;
  for (int b = 0; b < a.B; ++b) nmax = a.N[b] > nmax ? a.N[b] : nmax;
  const int64_t rb = (int64_t)(kT / pieces) * kCrows;
  int64_t blocks = (nmax + rb - 1) / rb;
  if (blocks > kCblocks) blocks = kCblocks;
  const dim3 grid((unsigned)blocks, a.L * a.B * a.Hkv), block(kT);
  const u32x4* ki = (const u32x4*)k_in;
  const u32x4* vi = (const u32x4*)v_in;
  if (logp == 3)
    hipLaunchKernelGGL(compact_layer_kernel<3>, grid, block, 0, stream, ki, vi, idx, head_kept, a,
                       (u32x4*)k_out, (u32x4*)v_out);
  else if (logp == 4)
    hipLaunchKernelGGL(compact_layer_kernel<4>, grid, block, 0, stream, ki, vi, idx, head_kept, a,
                       (u32x4*)k_out, (u32x4*)v_out);
  else
    hipLaunchKernelGGL(compact_layer_kernel<5>, grid, block, 0, stream, ki, vi, idx, head_kept, a,
                       (u32x4*)k_out, (u32x4*)v_out);
  return hipGetLastError();
}

}  // namespace hubkv
