// nestedkv.hip -- NestedKV key-only score: anomalies of each key against
// three running memories of the key stream, blended per head and routed by
// their disagreement.
//
// NestedKV summary page, continuum memory state: for every token i the key
// stream keeps a stable memory (the mean of all normalised keys), an episodic
// memory (the mean over i's block, blocks of about N / 32 keys) and a current
// memory (a moving mean over a 64-key window); each gives a cosine anomaly
// a_x(i) = -cos(k^_i, mu_x).  Outer teacher: per head, each scale's
// discriminative power (top minus bottom) goes through a softmax with a fixed
// log-prior to blend the anomalies; when the three anomalies disagree (their
// standard deviation is above a threshold) the score is the largest of them.
// Readings: k^ = k / |k| (0 for a zero key); blocks of ceil(N / nblocks) keys
// from the start; the current window is the 64 keys ending at i; power =
// max - min of the anomaly over the head; the log-prior and the threshold are
// arguments.
//
// Per (layer, KV head, sequence), in four launches:
//   1  tile sums of k^ over tiles of at most kNkvTile keys that never straddle
//      a block (16-byte pieces, a row over LPR lanes, several rows per wave
//      instruction);
//   2  block sums and their norms (tiles added in a fixed order);
//   3  anomalies over tiles of kNkvAnTile keys: the sequence sum from the
//      block sums, in order; walkers (the lanes of one row slot) each carry
//      the window sum S along a contiguous run of rows (S += k^_new - k^_old,
//      the old row reloaded from cache and renormalised with its stored
//      inverse norm), so the stable, episodic and current cosines are dot
//      products folded over a row's lanes; per-tile extremes of each anomaly;
//   4  per-head weights from the tiles' extremes, routing, the score.
// Cosines are scale-free, so sums stand in for means.
#include "internal.hpp"

namespace hubkv {

namespace {

constexpr int kT = 256;
constexpr int kWaves = kT / 64;
constexpr int kWin = 64;   // current-memory window

template <typename T>
__device__ __forceinline__ float to_f(T x);
template <>
__device__ __forceinline__ float to_f<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f<__bf16>(__bf16 x) { return (float)x; }

struct Tile {
  int lh, b, m, j;
  int64_t N, t0, t1;   // rows [t0, t1) of the sequence
  int64_t row_base;    // first packed row of (lh, b)
  int tile_g;          // tile index within (lh)
};

__device__ __forceinline__ Tile tile_of(const NkvArgs& a) {
  Tile t;
  t.lh = blockIdx.y;
  t.tile_g = blockIdx.x;
  int b = 0;
  while (b + 1 < a.B && a.tile_off[b + 1] <= t.tile_g) ++b;
  t.b = b;
  const int x = t.tile_g - a.tile_off[b];
  t.m = x / a.tpb[b];
  t.j = x - t.m * a.tpb[b];
  t.N = a.N[b];
  const int64_t blk0 = (int64_t)t.m * a.bs[b];
  const int64_t blk1 = blk0 + a.bs[b] < t.N ? blk0 + a.bs[b] : t.N;
  t.t0 = blk0 + (int64_t)t.j * kNkvTile;
  t.t1 = t.t0 + kNkvTile < blk1 ? t.t0 + kNkvTile : blk1;
  if (t.t0 > t.t1) t.t0 = t.t1;  // an empty tile of a short last block
  t.row_base = (int64_t)t.lh * a.T + a.cu[b];
  return t;
}

// A lane's 16-byte piece of a row: P elements; a row is LPR consecutive lanes,
// so one wave instruction loads RPW whole rows.
template <typename T, int D>
struct Piece {
  static constexpr int P = 16 / (int)sizeof(T);
  static constexpr int LPR = D / P;
  static constexpr int RPW = 64 / LPR;
  __device__ static u32x4 raw(const T* __restrict__ K, int64_t row, int c) {
    return *(const u32x4*)(K + row * D + c * P);
  }
  __device__ static void unpack(const u32x4& r, float (&x)[P]) {
    const T* e = (const T*)&r;
#pragma unroll
    for (int i = 0; i < P; ++i) x[i] = to_f<T>(e[i]);
  }
  __device__ static void load(const T* __restrict__ K, int64_t row, int c, float (&x)[P]) {
    unpack(raw(K, row, c), x);
  }
  // sum over the LPR lanes of one row (every lane of the row gets it)
  __device__ static float row_sum(float v) {
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) v += __shfl_xor(v, off);
    return v;
  }
};

// ---- 1: tile sums of the normalised keys.  Each wave loads RPW rows per
// instruction, kUnroll instructions in flight; the norm of a row is folded
// over its LPR lanes.
template <typename T, int D>
__global__ __launch_bounds__(kT) void nkv_tile_sum(const T* __restrict__ K, NkvArgs a,
                                                   NkvGeom g, char* ws) {
  using PC = Piece<T, D>;
  constexpr int P = PC::P, LPR = PC::LPR, RPW = PC::RPW;
  constexpr int kUnroll = 4;
  constexpr int STEP = kWaves * RPW;  // rows per unrolled step of the work-group
  __shared__ float red[kWaves][D];
  const Tile t = tile_of(a);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane % LPR, slot = lane / LPR;
  float acc[P];
#pragma unroll
  for (int i = 0; i < P; ++i) acc[i] = 0.f;
  for (int64_t r0 = t.t0 + wave * RPW + slot; r0 < t.t1; r0 += (int64_t)STEP * kUnroll) {
    float x[kUnroll][P];
    bool in[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t r = r0 + (int64_t)u * STEP;
      in[u] = r < t.t1;
      PC::load(K, t.row_base + (in[u] ? r : t.t0), c, x[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float nn = 0.f;
#pragma unroll
      for (int i = 0; i < P; ++i) nn = fmaf(x[u][i], x[u][i], nn);
      nn = PC::row_sum(nn);
      const float inv = (in[u] && nn > 0.f) ? 1.f / sqrtf(nn) : 0.f;
#pragma unroll
      for (int i = 0; i < P; ++i) acc[i] = fmaf(x[u][i], inv, acc[i]);
    }
  }
  // rows of the wave's slots, then the waves, in a fixed order
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int i = 0; i < P; ++i) acc[i] += __shfl_xor(acc[i], off);
  if (slot == 0)
#pragma unroll
    for (int i = 0; i < P; ++i) red[wave][c * P + i] = acc[i];
  __syncthreads();
  float* out = (float*)(ws + g.off_part) + ((int64_t)t.lh * a.ntile + t.tile_g) * D;
  for (int e = threadIdx.x; e < D; e += kT) {
    float v = 0.f;
    for (int w = 0; w < kWaves; ++w) v += red[w][e];
    out[e] = v;
  }
}

// Block-wide sum of one value per thread (fixed order).
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
  for (int w = 0; w < kWaves; ++w) s += red[w];
  return s;
}

// ---- 2: block sums and their norms (one work-group per (layer, head, block);
// thread e owns dimension e; tiles added in order)
__global__ __launch_bounds__(kT) void nkv_block_sum(NkvArgs a, NkvGeom g, char* ws) {
  __shared__ float red[kWaves];
  const int lh = blockIdx.y, bi = blockIdx.x;
  int b = 0;
  while (b + 1 < a.B && a.blk_off[b + 1] <= bi) ++b;
  const int m = bi - a.blk_off[b];
  const int e = threadIdx.x;
  const bool on = e < a.d;
  const float* part = (const float*)(ws + g.off_part) + (int64_t)lh * a.ntile * a.d;
  float s = 0.f;
  const int tb = a.tile_off[b] + m * a.tpb[b];
  for (int j = 0; j < a.tpb[b]; ++j)
    if (on) s += part[(int64_t)(tb + j) * a.d + e];
  if (on) ((float*)(ws + g.off_bsum))[((int64_t)lh * a.nblk_total + bi) * a.d + e] = s;
  const float n2 = block_sum(on ? s * s : 0.f, red);
  if (threadIdx.x == 0) ((float*)(ws + g.off_bnorm))[(int64_t)lh * a.nblk_total + bi] = sqrtf(n2);
}

// ---- 3: anomalies over tiles of up to kNkvAnTile rows (they may cross
// blocks).  A walker -- the LPR lanes of one row slot of a wave -- owns a
// contiguous run of the tile's rows and steps through it one row at a time,
// all walkers of the work-group in lockstep, after 64 warm-up steps over the
// rows before its run.  The window sum S is carried in the walker's lanes
// (S += k^_new - k^_old, the row 64 back reloaded from cache); lane
// (step mod 64) of register ring[w] keeps walker w's inverse norm of that
// step's row, read and written with a uniform lane index.
template <typename T, int D>
__global__ __launch_bounds__(kT) void nkv_anomaly(const T* __restrict__ K, NkvArgs a, NkvGeom g,
                                                  char* ws, float* __restrict__ an) {
  using PC = Piece<T, D>;
  constexpr int P = PC::P, LPR = PC::LPR, RPW = PC::RPW;
  constexpr int NWALK = kWaves * RPW;
  __shared__ float mm_s[kWaves][6];
  const int lh = blockIdx.y, x = blockIdx.x;
  int b = 0;
  while (b + 1 < a.B && a.at_off[b + 1] <= x) ++b;
  const int64_t N = a.N[b];
  const int64_t t0 = (int64_t)(x - a.at_off[b]) * kNkvAnTile;
  const int64_t t1 = t0 + kNkvAnTile < N ? t0 + kNkvAnTile : N;
  const int64_t row_base = (int64_t)lh * a.T + a.cu[b];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane % LPR, slot = lane / LPR;
  const int walker = wave * RPW + slot;
  const float* bsum = (const float*)(ws + g.off_bsum) + ((int64_t)lh * a.nblk_total + a.blk_off[b]) * D;
  const float* bnrm = (const float*)(ws + g.off_bnorm) + (int64_t)lh * a.nblk_total + a.blk_off[b];
  // the sequence sum, from the block sums in order, and its norm
  float ms[P];
#pragma unroll
  for (int i = 0; i < P; ++i) ms[i] = 0.f;
  // (unrolled so the block sums' loads are in flight together; added in order)
#pragma unroll 8
  for (int m = 0; m < a.nblk[b]; ++m)
#pragma unroll
    for (int i = 0; i < P; ++i) ms[i] += bsum[(int64_t)m * D + c * P + i];
  float msn = 0.f;
#pragma unroll
  for (int i = 0; i < P; ++i) msn = fmaf(ms[i], ms[i], msn);
  msn = PC::row_sum(msn);
  const float ims = msn > 0.f ? 1.f / sqrtf(msn) : 0.f;
  // this walker's run
  const int64_t len = t1 - t0;
  const int64_t R = (len + NWALK - 1) / NWALK;
  const int64_t st = t0 + R * walker < t1 ? t0 + R * walker : t1;
  const int64_t run = st + R < t1 ? R : t1 - st;
  const int bsz = a.bs[b];
  int cm = (int)(st / bsz);  // block of the current row, its sum and inverse norm
  float me[P], ime;
  auto load_block = [&](int m) {
    const int mc = m < a.nblk[b] ? m : a.nblk[b] - 1;
#pragma unroll
    for (int i = 0; i < P; ++i) me[i] = bsum[(int64_t)mc * D + c * P + i];
    const float n = bnrm[mc];
    ime = n > 0.f ? 1.f / n : 0.f;
  };
  load_block(cm);
  float S[P];
#pragma unroll
  for (int i = 0; i < P; ++i) S[i] = 0.f;
  float ring[RPW];
#pragma unroll
  for (int w = 0; w < RPW; ++w) ring[w] = 0.f;
  float mx[3] = {-INFINITY, -INFINITY, -INFINITY}, mn[3] = {INFINITY, INFINITY, INFINITY};
  float* anb = an + row_base * 3;
  // Steps in groups of kPf.  The next group's rows are in flight while a
  // group is processed in phases, so the reductions of its steps overlap:
  // the rows' norms, the ring and the window sums (the only step-to-step
  // dependency, a few adds), then the four dot products of every step.
  constexpr int kPf = 4;
  const int64_t Rmax = R;
  u32x4 nq[kPf], oq[kPf];
  auto issue = [&](int64_t jg) {
#pragma unroll
    for (int u = 0; u < kPf; ++u) {
      const int64_t j = jg + u, q = st + j;
      const bool live = j < run && q >= 0;
      const bool drop = j >= 0 && j < run && q - kWin >= 0;
      nq[u] = PC::raw(K, row_base + (live ? q : 0), c);
      oq[u] = PC::raw(K, row_base + (drop ? q - kWin : 0), c);
    }
  };
  issue(-kWin);
  for (int64_t jg = -kWin; jg < Rmax; jg += kPf) {
    u32x4 cn[kPf], co[kPf];
#pragma unroll
    for (int u = 0; u < kPf; ++u) {
      cn[u] = nq[u];
      co[u] = oq[u];
    }
    if (jg + kPf < Rmax) issue(jg + kPf);
    // norms of the group's new rows
    float inv[kPf];
#pragma unroll
    for (int u = 0; u < kPf; ++u) {
      float xn[P];
      PC::unpack(cn[u], xn);
      float nn = 0.f;
#pragma unroll
      for (int i = 0; i < P; ++i) nn = fmaf(xn[i], xn[i], nn);
      inv[u] = nn;
    }
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1)
#pragma unroll
      for (int u = 0; u < kPf; ++u) inv[u] += __shfl_xor(inv[u], off);
    // ring, window sums and the lane partials of each step's dot products
    // (with the inverse norm of the step's own block: a later step of the
    // group may move to the next block)
    float pd[kPf][4], pie[kPf];
#pragma unroll
    for (int u = 0; u < kPf; ++u) {
      const int64_t j = jg + u, q = st + j;
      const bool live = j < Rmax && j < run && q >= 0;
      const bool drop = j >= 0 && j < run && q - kWin >= 0;
      const float iv = (live && inv[u] > 0.f) ? 1.f / sqrtf(inv[u]) : 0.f;
      inv[u] = iv;
      const int L = (int)(j & (kWin - 1));
      float iold = 0.f;
#pragma unroll
      for (int w = 0; w < RPW; ++w) {
        const float o = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ring[w]), L));
        if (slot == w) iold = o;
        const float nv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(iv), w * LPR));
        if (j < Rmax) ring[w] = lane == L ? nv : ring[w];
      }
      float xn[P], xo[P];
      PC::unpack(cn[u], xn);
      PC::unpack(co[u], xo);
      float dc = 0.f, ss = 0.f, ds = 0.f, de = 0.f;
      if (j >= 0 && live && q >= (int64_t)(cm + 1) * bsz) load_block(++cm);
#pragma unroll
      for (int i = 0; i < P; ++i) {
        const float kh = xn[i] * iv;
        S[i] = S[i] + kh - (drop ? xo[i] * iold : 0.f);
        dc = fmaf(kh, S[i], dc);
        ss = fmaf(S[i], S[i], ss);
        ds = fmaf(kh, ms[i], ds);
        de = fmaf(kh, me[i], de);
      }
      pd[u][0] = dc;
      pd[u][1] = ss;
      pd[u][2] = ds;
      pd[u][3] = de;
      pie[u] = ime;
    }
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1)
#pragma unroll
      for (int u = 0; u < kPf; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) pd[u][v] += __shfl_xor(pd[u][v], off);
#pragma unroll
    for (int u = 0; u < kPf; ++u) {
      const int64_t j = jg + u, q = st + j;
      if (j < 0 || j >= run) continue;  // warm-up steps and past the run
      const float sn = pd[u][1] > 0.f ? sqrtf(pd[u][1]) : 0.f;
      const float as = -(pd[u][2] * ims);
      const float ae = -(pd[u][3] * pie[u]);
      const float ac = sn > 0.f ? -(pd[u][0] / sn) : -0.f;
      mx[0] = fmaxf(mx[0], as);
      mx[1] = fmaxf(mx[1], ae);
      mx[2] = fmaxf(mx[2], ac);
      mn[0] = fminf(mn[0], as);
      mn[1] = fminf(mn[1], ae);
      mn[2] = fminf(mn[2], ac);
      if (c < 3) anb[q * 3 + c] = c == 0 ? as : (c == 1 ? ae : ac);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      mx[k] = fmaxf(mx[k], __shfl_xor(mx[k], off));
      mn[k] = fminf(mn[k], __shfl_xor(mn[k], off));
    }
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      mm_s[wave][2 * k] = mx[k];
      mm_s[wave][2 * k + 1] = mn[k];
    }
  }
  __syncthreads();
  if (threadIdx.x < 6) {
    const int k = threadIdx.x;
    float v = mm_s[0][k];
    for (int w = 1; w < kWaves; ++w) v = (k & 1) ? fminf(v, mm_s[w][k]) : fmaxf(v, mm_s[w][k]);
    ((float*)(ws + g.off_mm))[((int64_t)lh * a.nat + x) * 6 + k] = v;
  }
}

// ---- 4: per-head weights and routing, over the anomaly tiles
__global__ __launch_bounds__(kT) void nkv_route(NkvArgs a, NkvGeom g, char* ws,
                                                const float* __restrict__ an,
                                                float* __restrict__ s,
                                                float* __restrict__ weights) {
  __shared__ float w_s[3], ext[kWaves][6];
  const int lh = blockIdx.y, x = blockIdx.x;
  int b = 0;
  while (b + 1 < a.B && a.at_off[b + 1] <= x) ++b;
  const int64_t N = a.N[b];
  const int64_t t0 = (int64_t)(x - a.at_off[b]) * kNkvAnTile;
  const int64_t t1 = t0 + kNkvAnTile < N ? t0 + kNkvAnTile : N;
  const int64_t row_base = (int64_t)lh * a.T + a.cu[b];
  {
    // extremes of each anomaly over the sequence's tiles (max / min: exact in any order)
    const float* mm = (const float*)(ws + g.off_mm) + (int64_t)lh * a.nat * 6;
    float hi[3] = {-INFINITY, -INFINITY, -INFINITY}, lo[3] = {INFINITY, INFINITY, INFINITY};
    for (int y = a.at_off[b] + (int)threadIdx.x; y < a.at_off[b + 1]; y += kT)
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        hi[k] = fmaxf(hi[k], mm[(int64_t)y * 6 + 2 * k]);
        lo[k] = fminf(lo[k], mm[(int64_t)y * 6 + 2 * k + 1]);
      }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        hi[k] = fmaxf(hi[k], __shfl_xor(hi[k], off));
        lo[k] = fminf(lo[k], __shfl_xor(lo[k], off));
      }
    if ((threadIdx.x & 63) == 0)
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        ext[threadIdx.x >> 6][2 * k] = hi[k];
        ext[threadIdx.x >> 6][2 * k + 1] = lo[k];
      }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float hi[3], lo[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      hi[k] = ext[0][2 * k];
      lo[k] = ext[0][2 * k + 1];
      for (int w = 1; w < kWaves; ++w) {
        hi[k] = fmaxf(hi[k], ext[w][2 * k]);
        lo[k] = fminf(lo[k], ext[w][2 * k + 1]);
      }
    }
    double D[3], dm = -INFINITY;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      D[k] = (double)hi[k] - (double)lo[k] + (double)a.prior[k];
      dm = D[k] > dm ? D[k] : dm;
    }
    double den = 0.0;
#pragma unroll
    for (int k = 0; k < 3; ++k) den += exp(D[k] - dm);
#pragma unroll
    for (int k = 0; k < 3; ++k) w_s[k] = (float)(exp(D[k] - dm) / den);
    if (weights && x == a.at_off[b]) {
      const int l = lh / a.Hkv, h = lh - l * a.Hkv;
#pragma unroll
      for (int k = 0; k < 3; ++k) weights[(((int64_t)l * a.B + b) * a.Hkv + h) * 3 + k] = w_s[k];
    }
  }
  __syncthreads();
  const float w0 = w_s[0], w1 = w_s[1], w2 = w_s[2];
  for (int64_t q = t0 + threadIdx.x; q < t1; q += kT) {
    const float* ai = an + (row_base + q) * 3;
    const float x0 = ai[0], x1 = ai[1], x2 = ai[2];
    const float mean = (x0 + x1 + x2) * (1.f / 3.f);
    const float v = ((x0 - mean) * (x0 - mean) + (x1 - mean) * (x1 - mean) +
                     (x2 - mean) * (x2 - mean)) * (1.f / 3.f);
    const float sg = sqrtf(v);
    s[row_base + q] = sg > a.theta ? fmaxf(fmaxf(x0, x1), x2)
                                   : fmaf(w0, x0, fmaf(w1, x1, w2 * x2));
  }
}

template <typename T, int D>
hipError_t launch_t(const void* k, const NkvArgs& a, const NkvGeom& g, char* ws, float* an,
                    float* s, float* weights, hipStream_t stream) {
  const dim3 grid(a.ntile, a.L * a.Hkv), agrid(a.nat, a.L * a.Hkv), block(kT);
  hipLaunchKernelGGL((nkv_tile_sum<T, D>), grid, block, 0, stream, (const T*)k, a, g, ws);
  hipLaunchKernelGGL(nkv_block_sum, dim3(a.nblk_total, a.L * a.Hkv), block, 0, stream, a, g, ws);
  hipLaunchKernelGGL((nkv_anomaly<T, D>), agrid, block, 0, stream, (const T*)k, a, g, ws, an);
  hipLaunchKernelGGL(nkv_route, agrid, block, 0, stream, a, g, ws, (const float*)an, s, weights);
  return hipGetLastError();
}

}  // namespace

NkvGeom nkv_geometry(const NkvArgs& a) {
  NkvGeom g;
  const int64_t LH = (int64_t)a.L * a.Hkv;
  size_t o = 0;
  auto take = [&](size_t n) {
    const size_t at = o;
    o += (n + 255) & ~(size_t)255;
    return at;
  };
  g.off_part = take((size_t)LH * a.ntile * a.d * 4);
  g.off_bsum = take((size_t)LH * a.nblk_total * a.d * 4);
  g.off_bnorm = take((size_t)LH * a.nblk_total * 4);
  g.off_mm = take((size_t)LH * a.nat * 6 * 4);
  g.off_an = take((size_t)LH * a.T * 3 * 4);
  g.bytes = o;
  return g;
}

hipError_t launch_nestedkv(const void* k, int dtype, const NkvArgs& a, const NkvGeom& g, char* ws,
                           float* anomalies, float* s, float* weights, hipStream_t stream) {
  float* an = anomalies ? anomalies : (float*)(ws + g.off_an);
  if (dtype == 1) {
    if (a.d == 128) return launch_t<__bf16, 128>(k, a, g, ws, an, s, weights, stream);
    return launch_t<__bf16, 64>(k, a, g, ws, an, s, weights, stream);
  }
  if (a.d == 128) return launch_t<float, 128>(k, a, g, ws, an, s, weights, stream);
  return launch_t<float, 64>(k, a, g, ws, an, s, weights, stream);
}

}  // namespace hubkv
