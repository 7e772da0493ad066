// h2o_step.hip -- one decode step of H2O greedy eviction on fixed cache slots.
//
// H2O breakdown page: "greedy eviction" (the current query's softmax over the
// cached tokens is added to their accumulated scores, the new token enters
// with score 0, and over budget the lowest accumulated score is evicted), the
// heavy + recent section (a recent window is protected from eviction), the
// per-head section (each head evicts independently) and the FlexGen section
// (slots are preallocated; the evicted slot is overwritten by the new token,
// and the score update rides on the attention pass).
//
// One work-group per (sequence, KV head).  Waves sweep the slots, a group of
// lanes per slot row: each lane loads 16 bytes of the row and the partial dot
// products are folded with shuffles; the logits of the group's query heads
// stay in LDS.  After block-wide softmax statistics, each thread updates the
// scores of the slots it owns (the probabilities replace the logits in LDS)
// and tracks the eviction candidate with the smallest (score, position); a
// block reduction picks the slot to overwrite.
//
// Optional attention output (KV-cache page, section 1.1, decode attention;
// H2O page, problem statement: only retained tokens enter the normaliser): a
// second sweep reads the V rows of the occupied slots once and accumulates
// sum_slot p_h(slot) v_slot per query head, each lane owning a few columns;
// the partial sums are folded across the lanes of a wave with shuffles and
// across waves in LDS, in a fixed order.  The sweep reads the cache before the
// new token's row is written into its slot.
//
// Ring layout (H2O breakdown page, FlexGen section: the recent region is a
// circular queue whose head and tail advance in O(1)): slots [0, C - R) hold
// the heavy tokens and slots [C - R, C) a ring of R = n_recent slots, where
// position p always sits in slot C - R + p mod R.  The new token t takes the
// ring slot of t - R, the token leaving the recent window.  That token moves
// to a free heavy slot if there is one; otherwise the lowest (score,
// position) among the heavy candidates and the leaving token is evicted, and
// when the victim is a heavy token the leaving token's row, score and
// position are copied into the victim's slot (one extra row copy).  The
// candidates are those of the fixed layout (positions in [n_sink,
// t - n_recent]), so both layouts retain the same tokens with the same scores
// when t advances by one per step.
#include "internal.hpp"

namespace hubkv {

namespace {

constexpr int kH2OThreads = 512;
constexpr int kH2OWaves = kH2OThreads / 64;
constexpr float kLog2eH = 1.4426950408889634f;

// a lane's piece of a row: W 32-bit words
template <int W>
struct Words {
  typedef uint32_t __attribute__((ext_vector_type(W))) type;
};
template <>
struct Words<1> {
  typedef uint32_t type;
};

// Sum over each group of N consecutive lanes (N = 8, 16 or 32; groups start
// at multiples of N), left in every lane of the group.  DPP moves on the VALU
// (quad permutes [1,0,3,2] and [2,3,0,1], then the half-row and row mirrors)
// instead of LDS-crossbar shuffles; a 32-lane group adds one shuffle.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int N>
__device__ __forceinline__ float row_sum(float d) {
  static_assert(N == 8 || N == 16 || N == 32, "groups of 8, 16 or 32 lanes");
  d += dpp_mov<0xB1>(d);   // lane ^ 1
  d += dpp_mov<0x4E>(d);   // lane ^ 2: every lane holds its quad's sum
  d += dpp_mov<0x141>(d);  // half-row mirror: the other quad of its 8 lanes
  if constexpr (N >= 16) d += dpp_mov<0x140>(d);  // row mirror: the other 8 of its 16
  if constexpr (N == 32) d += __shfl_xor(d, 16);
  return d;
}

template <typename T>
__device__ __forceinline__ float to_f(T x);
template <>
__device__ __forceinline__ float to_f<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f<__bf16>(__bf16 x) { return (float)x; }

__device__ __forceinline__ uint32_t asc_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int G_of(const H2OArgs& a) { return a.Hq / a.Hkv; }

// KG: the group size G rounded up to a power of two (register arrays and
// unrolled head loops are sized by it; heads h >= G are skipped).
template <typename T, int D, int KG>
__global__ __launch_bounds__(kH2OThreads) void h2o_step_kernel(
    const T* __restrict__ q, const T* __restrict__ k_new, const T* __restrict__ v_new,
    T* __restrict__ k_cache, T* __restrict__ v_cache, float* __restrict__ acc,
    int32_t* __restrict__ pos, H2OArgs a, int32_t* __restrict__ evicted,
    float* __restrict__ probs, float* __restrict__ out) {
  constexpr int EPL = 16 / (int)sizeof(T);  // elements per lane piece
  constexpr int LPR = D / EPL;              // lanes per slot row
  constexpr int RPW = 64 / LPR;             // rows per wave per sweep step
  constexpr int WAVES = kH2OWaves;
  // dynamic LDS: [G][C] logits in log2 units (then probabilities), [C] slot
  // positions, and with an output [WAVES][G][D] per-wave partial sums
  extern __shared__ float lg[];
  int32_t* pl = (int32_t*)(lg + G_of(a) * a.C);
  float* part = (float*)(pl + a.C);
  __shared__ float qs[KG][D];
  __shared__ u32x4 newrow[2][LPR];  // the new token's K and V rows, 16 bytes a lane
  __shared__ float red[WAVES][KG], red2[WAVES][KG];
  __shared__ float Mh[KG], iLh[KG], selfx[KG], pself[KG];
  __shared__ unsigned long long cand_key[WAVES];
  __shared__ int cand_slot[WAVES], empty_w[WAVES];
  __shared__ int dec_slot, dec_move, dec_mpos;
  __shared__ float dec_acc, dec_macc, ring_acc;

  const int u = blockIdx.x;
  const int b = u / a.Hkv, g = u % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int C = a.C;
  const int64_t t = a.t[b];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float c2 = a.scale * kLog2eH;

  // ---- logits over the occupied slots.  Every load that depends on nothing
  // computed here goes out first, before the first wait: the first K row
  // groups, this thread's accumulated scores, the slot positions, the new
  // K/V rows written at the end, and the query.
  const T* Kc = k_cache + (int64_t)u * C * D;
  const int32_t* P = pos + (int64_t)u * C;
  float* A = acc + (int64_t)u * C;
  const int piece = lane % LPR, rsub = lane / LPR;
  // row groups are software-pipelined: the next kUnroll groups' loads are in
  // flight while the current kUnroll groups are reduced
  constexpr int kUnroll = 4;
  constexpr int kStep = WAVES * RPW * kUnroll;
  u32x4 nxt[kUnroll];
  auto load_group = [&](int j0, u32x4 (&dst)[kUnroll]) {
#pragma unroll
    for (int uu = 0; uu < kUnroll; ++uu) {
      const int j = j0 + uu * WAVES * RPW + rsub;
      const int jc = j < C ? j : C - 1;  // past-the-end rows read the last slot, never stored
      // a read-once stream: non-temporal loads (a plain read stream on MI355X
      // runs at ~6.1 TB/s, a non-temporal one at ~7.0 TB/s)
      dst[uu] = __builtin_nontemporal_load((const u32x4*)(Kc + (int64_t)jc * D + piece * EPL));
    }
  };
  load_group(wave * RPW, nxt);
  // the accumulated scores this thread updates after the sweep, in registers
  // (the host limits C to 8192)
  constexpr int kAccPer = 16;
  static_assert(kAccPer * kH2OThreads >= 8192, "every slot of the largest cache has a register");
  float accv[kAccPer];
#pragma unroll
  for (int i = 0; i < kAccPer; ++i) {
    const int j = tid + i * kH2OThreads;
    accv[i] = j < C ? A[j] : 0.f;
  }
  // positions of the slots, the new token's K and V rows and the query,
  // staged in LDS with coalesced loads
  if (wave == 0 && lane < LPR) {
    const int64_t src = ((int64_t)b * a.Hkv + g) * D + lane * EPL;
    newrow[0][lane] = *(const u32x4*)(k_new + src);
    newrow[1][lane] = *(const u32x4*)(v_new + src);
  }
  for (int j = tid; j < C; j += kH2OThreads) pl[j] = P[j];
  for (int i = tid; i < G * D; i += kH2OThreads)
    qs[i / D][i % D] = to_f<T>(q[((int64_t)b * a.Hq + g * G + i / D) * D + i % D]);
  __syncthreads();  // positions and query staged
  // this lane's piece of every query head, in registers for the whole sweep
  float qv[KG][EPL];
#pragma unroll
  for (int h = 0; h < KG; ++h)
#pragma unroll
    for (int x = 0; x < EPL; ++x) qv[h][x] = h < G ? qs[h][piece * EPL + x] : 0.f;
  for (int j0 = wave * RPW; j0 < C; j0 += kStep) {
    u32x4 raw[kUnroll];
#pragma unroll
    for (int uu = 0; uu < kUnroll; ++uu) raw[uu] = nxt[uu];
    if (j0 + kStep < C) load_group(j0 + kStep, nxt);
#pragma unroll
    for (int uu = 0; uu < kUnroll; ++uu) {
      const int j = j0 + uu * WAVES * RPW + rsub;
      const T* e = (const T*)&raw[uu];
      float kv[EPL];
#pragma unroll
      for (int x = 0; x < EPL; ++x) kv[x] = to_f<T>(e[x]);
      const bool occ = j < C && pl[j] >= 0;
#pragma unroll
      for (int h = 0; h < KG; ++h) {
        if (h < G) {  // G is uniform: every lane takes the same branch
          float d = 0.f;
#pragma unroll
          for (int x = 0; x < EPL; ++x) d = fmaf(qv[h][x], kv[x], d);
          d = row_sum<LPR>(d);
          const float x2 = occ ? d * c2 : -INFINITY;
          if (piece == 0 && j < C) lg[h * C + j] = x2;
        }
      }
    }
  }
  if (tid < G) {
    float d = -INFINITY;
    if (a.include_self) {
      d = 0.f;
      const T* kn = k_new + ((int64_t)b * a.Hkv + g) * D;
      for (int x = 0; x < D; ++x) d = fmaf(qs[tid][x], to_f<T>(kn[x]), d);
      d *= c2;
    }
    selfx[tid] = d;
  }
  __syncthreads();

  // ---- each thread's share of the softmax statistics, from the logits in
  // LDS (every lane busy, one exponential per logit): its slots' maximum,
  // then their sum of exp2(x - maximum)
  float om[KG], os[KG];
#pragma unroll
  for (int h = 0; h < KG; ++h) {
    om[h] = -INFINITY;
    os[h] = 0.f;
    if (h < G) {  // G is uniform: every lane takes the same branch
      float m = -INFINITY;
      for (int j = tid; j < C; j += kH2OThreads) m = fmaxf(m, lg[h * C + j]);
      float sm = 0.f;
      if (m > -INFINITY)
        for (int j = tid; j < C; j += kH2OThreads) sm += __builtin_amdgcn_exp2f(lg[h * C + j] - m);
      om[h] = m;
      os[h] = sm;
    }
  }

  // ---- softmax statistics per query head: merge the threads' (m, s)
#pragma unroll
  for (int h = 0; h < KG; ++h) {
    if (h < G) {  // G is uniform: every lane takes the same branch
      float m = om[h], sm = os[h];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(sm, off);
        const float mn = fmaxf(m, m2);
        if (mn > -INFINITY) {
          sm = sm * __builtin_amdgcn_exp2f(m - mn) + s2 * __builtin_amdgcn_exp2f(m2 - mn);
          m = mn;
        }
      }
      if (lane == 0) {
        red[wave][h] = m;
        red2[wave][h] = sm;
      }
    }
  }
  __syncthreads();
  if (tid < G) {
    float m = selfx[tid];
    for (int w = 0; w < WAVES; ++w) m = fmaxf(m, red[w][tid]);
    float sm = (m > -INFINITY && selfx[tid] > -INFINITY) ? __builtin_amdgcn_exp2f(selfx[tid] - m)
                                                          : 0.f;
    if (m > -INFINITY)
      for (int w = 0; w < WAVES; ++w)
        if (red[w][tid] > -INFINITY) sm += red2[w][tid] * __builtin_amdgcn_exp2f(red[w][tid] - m);
    Mh[tid] = m;
    iLh[tid] = sm > 0.f ? 1.f / sm : 0.f;
  }
  __syncthreads();

  // ---- value sweep geometry: a lane owns EPLV columns of a V row, sized so
  // the KG x EPLV running sums stay within 32 registers
  constexpr int EPLV = sizeof(T) == 2 ? (KG <= 4 ? 8 : 32 / KG) : (KG <= 8 ? 4 : 2);
  constexpr int WV = EPLV * (int)sizeof(T) / 4;  // 32-bit words per lane piece
  constexpr int LPRV = D / EPLV;                 // lanes per V row
  constexpr int RPWV = 64 / LPRV;                // V rows per wave per step
  constexpr int kStepV = WAVES * RPWV * kUnroll;
  typedef typename Words<WV>::type VW;
  const T* Vc = v_cache + (int64_t)u * C * D;
  const int pv = lane % LPRV, rv = lane / LPRV;
  auto load_v = [&](int j0, VW (&dst)[kUnroll]) {
#pragma unroll
    for (int uu = 0; uu < kUnroll; ++uu) {
      const int j = j0 + uu * WAVES * RPWV + rv;
      const int jc = j < C ? j : C - 1;
      dst[uu] = __builtin_nontemporal_load((const VW*)(Vc + (int64_t)jc * D + pv * EPLV));
    }
  };
  VW vnx[kUnroll];
  // the first V rows are in flight during the score update
  if (out) load_v(wave * RPWV, vnx);

  // ---- score update, eviction candidate, first empty slot (a heavy slot in
  // the ring layout)
  const int64_t lo = a.n_sink, hi = t - a.n_recent;
  const int nheavy = a.ring ? C - a.n_recent : C;
  const int rslot = a.ring ? nheavy + (int)(t % a.n_recent) : -1;  // the new token's ring slot
  unsigned long long best = ~0ull;
  int best_slot = -1, first_empty = 0x7fffffff;
#pragma unroll
  for (int i = 0; i < kAccPer; ++i) {
    const int j = tid + i * kH2OThreads;
    if (j >= C) break;
    const int32_t pj = pl[j];
    float add = 0.f;
    for (int h = 0; h < G; ++h) {
      const float p = pj >= 0 ? __builtin_amdgcn_exp2f(lg[h * C + j] - Mh[h]) * iLh[h] : 0.f;
      add += p;
      lg[h * C + j] = p;
      if (probs) probs[((int64_t)b * a.Hq + g * G + h) * (C + 1) + j] = p;
    }
    if (pj < 0) {
      if (j < nheavy) first_empty = min(first_empty, j);
    } else {
      const float na = accv[i] + add;
      A[j] = na;
      if (j == rslot) ring_acc = na;
      if (pj >= lo && pj <= hi) {
        const unsigned long long key = ((unsigned long long)asc_key(na) << 32) | (uint32_t)pj;
        if (key < best) {
          best = key;
          best_slot = j;
        }
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned long long ok = __shfl_xor(best, off);
    const int os = __shfl_xor(best_slot, off);
    if (ok < best) {
      best = ok;
      best_slot = os;
    }
    first_empty = min(first_empty, __shfl_xor(first_empty, off));
  }
  if (lane == 0) {
    cand_key[wave] = best;
    cand_slot[wave] = best_slot;
    empty_w[wave] = first_empty;
  }
  __syncthreads();
  if (tid == 0) {
    float self_acc = 0.f;
    for (int h = 0; h < G; ++h) {
      const float p = (Mh[h] > -INFINITY && selfx[h] > -INFINITY)
                          ? __builtin_amdgcn_exp2f(selfx[h] - Mh[h]) * iLh[h] : 0.f;
      self_acc += p;
      pself[h] = p;
      if (probs) probs[((int64_t)b * a.Hq + g * G + h) * (C + 1) + C] = p;
    }
    unsigned long long bk = ~0ull;
    int bs = -1, fe = 0x7fffffff;
    for (int w = 0; w < WAVES; ++w) {
      if (cand_key[w] < bk) {
        bk = cand_key[w];
        bs = cand_slot[w];
      }
      fe = min(fe, empty_w[w]);
    }
    int slot = -1, ev = -1, mv = -1;
    if (a.ring) {
      // the new token takes its ring slot; the token leaving it moves to a
      // free heavy slot, or the lowest candidate (it included) is evicted
      const int32_t pold = pl[rslot];
      if (pold < 0) {
        slot = rslot;
      } else if (fe < nheavy) {
        slot = rslot;
        mv = fe;
      } else if (bs >= 0) {
        slot = rslot;
        ev = (int)(bk & 0xffffffffu);
        if (bs != rslot) mv = bs;
      }
      dec_mpos = pold;
      dec_macc = ring_acc;
    } else if (fe < C) {
      slot = fe;
    } else {
      // the new token competes when it is outside both protected windows
      if (t >= lo && t <= hi) {
        const unsigned long long nk = ((unsigned long long)asc_key(self_acc) << 32) | (uint32_t)t;
        if (nk < bk) {
          bk = nk;
          bs = -2;
        }
      }
      if (bs == -2) {
        ev = (int)t;
      } else if (bs >= 0) {
        slot = bs;
        ev = (int)(bk & 0xffffffffu);
      }
    }
    dec_slot = slot;
    dec_move = mv;
    dec_acc = self_acc;  // 0 unless the new token attends to itself
    if (evicted) evicted[u] = ev;
  }
  __syncthreads();

  // ---- attention output: sum over occupied slots of p_h(slot) * v_slot
  if (out) {
    float o[KG][EPLV];
#pragma unroll
    for (int h = 0; h < KG; ++h)
#pragma unroll
      for (int x = 0; x < EPLV; ++x) o[h][x] = 0.f;
    for (int j0 = wave * RPWV; j0 < C; j0 += kStepV) {
      VW raw[kUnroll];
#pragma unroll
      for (int uu = 0; uu < kUnroll; ++uu) raw[uu] = vnx[uu];
      if (j0 + kStepV < C) load_v(j0 + kStepV, vnx);
#pragma unroll
      for (int uu = 0; uu < kUnroll; ++uu) {
        const int j = j0 + uu * WAVES * RPWV + rv;
        // empty slots hold no token, and their rows may hold anything
        if (j < C && pl[j] >= 0) {
          const T* e = (const T*)&raw[uu];
          float vv[EPLV];
#pragma unroll
          for (int x = 0; x < EPLV; ++x) vv[x] = to_f<T>(e[x]);
#pragma unroll
          for (int h = 0; h < KG; ++h) {
            if (h < G) {  // G is uniform: every lane takes the same branch
              const float p = lg[h * C + j];
#pragma unroll
              for (int x = 0; x < EPLV; ++x) o[h][x] = fmaf(p, vv[x], o[h][x]);
            }
          }
        }
      }
    }
    // fold the rows of a wave, then park the wave's sums in LDS
#pragma unroll
    for (int h = 0; h < KG; ++h) {
      if (h < G) {  // G is uniform: every lane takes the same branch
#pragma unroll
        for (int x = 0; x < EPLV; ++x) {
          float v = o[h][x];
#pragma unroll
          for (int off = LPRV; off < 64; off <<= 1) v += __shfl_xor(v, off);
          if (rv == 0) part[(wave * G + h) * D + pv * EPLV + x] = v;
        }
      }
    }
    __syncthreads();  // every wave's V reads are done before the slot rewrite below
    const T* vn = v_new + ((int64_t)b * a.Hkv + g) * D;
    for (int i = tid; i < G * D; i += kH2OThreads) {
      const int h = i / D, e = i % D;
      float v = 0.f;
      for (int w = 0; w < WAVES; ++w) v += part[(w * G + h) * D + e];
      v = fmaf(pself[h], to_f<T>(vn[e]), v);
      out[((int64_t)b * a.Hq + g * G + h) * D + e] = v;
    }
  }

  const int slot = dec_slot, mv = dec_move;
  // a slot's owner thread rewrites its score and position (it wrote the
  // updated score above, so program order keeps the final value)
  if (mv >= 0 && (mv % kH2OThreads) == tid) {
    A[mv] = dec_macc;
    pos[(int64_t)u * C + mv] = dec_mpos;
  }
  if (slot >= 0) {
    if ((slot % kH2OThreads) == tid) {
      A[slot] = dec_acc;
      pos[(int64_t)u * C + slot] = (int32_t)t;
    }
    if (wave == 0 && lane < LPR) {
      const int64_t dst = ((int64_t)u * C + slot) * D + lane * EPL;
      if (mv >= 0) {
        // the leaving token's row goes to its heavy slot before the new row
        // overwrites it (same lane, same addresses: program order holds)
        const int64_t mdst = ((int64_t)u * C + mv) * D + lane * EPL;
        const u32x4 kr = *(const u32x4*)(k_cache + dst);
        const u32x4 vr = *(const u32x4*)(v_cache + dst);
        *(u32x4*)(k_cache + mdst) = kr;
        *(u32x4*)(v_cache + mdst) = vr;
      }
      *(u32x4*)(k_cache + dst) = newrow[0][lane];
      *(u32x4*)(v_cache + dst) = newrow[1][lane];
    }
  }
}

}  // namespace

size_t h2o_lds_bytes(int G, int C, int d, bool with_out) {
  return (size_t)G * C * sizeof(float) + (size_t)C * sizeof(int32_t) +
         (with_out ? (size_t)kH2OWaves * G * d * sizeof(float) : 0);
}

namespace {

template <typename T, int D>
void launch_h2o_t(const void* q, const void* k_new, const void* v_new, void* k_cache,
                  void* v_cache, float* acc, int32_t* pos, const H2OArgs& a, int32_t* evicted,
                  float* probs, float* out, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const size_t lds = h2o_lds_bytes(G, a.C, D, out != nullptr);
  const dim3 grid(a.B * a.Hkv), block(kH2OThreads);
#define H2O_LAUNCH(KG)                                                                          \
  hipLaunchKernelGGL((h2o_step_kernel<T, D, KG>), grid, block, lds, stream, (const T*)q,        \
                     (const T*)k_new, (const T*)v_new, (T*)k_cache, (T*)v_cache, acc, pos, a,   \
                     evicted, probs, out)
  if (G == 1) H2O_LAUNCH(1);
  else if (G == 2) H2O_LAUNCH(2);
  else if (G <= 4) H2O_LAUNCH(4);
  else if (G <= 8) H2O_LAUNCH(8);
  else H2O_LAUNCH(16);
#undef H2O_LAUNCH
}

}  // namespace

hipError_t launch_h2o_step(const void* q, const void* k_new, const void* v_new, int dtype,
                           void* k_cache, void* v_cache, float* acc, int32_t* pos,
                           const H2OArgs& a, int32_t* evicted, float* probs, float* out,
                           hipStream_t stream) {
  if (dtype == 1) {
    if (a.d == 128)
      launch_h2o_t<__bf16, 128>(q, k_new, v_new, k_cache, v_cache, acc, pos, a, evicted, probs,
                                out, stream);
    else
      launch_h2o_t<__bf16, 64>(q, k_new, v_new, k_cache, v_cache, acc, pos, a, evicted, probs,
                               out, stream);
  } else {
    if (a.d == 128)
      launch_h2o_t<float, 128>(q, k_new, v_new, k_cache, v_cache, acc, pos, a, evicted, probs,
                               out, stream);
    else
      launch_h2o_t<float, 64>(q, k_new, v_new, k_cache, v_cache, acc, pos, a, evicted, probs,
                              out, stream);
  }
  return hipGetLastError();
}

}  // namespace hubkv
