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
// Per (layer, KV head, sequence), in four launches over tiles of at most
// kNkvTile keys that never straddle a block:
//   1  tile sums of k^ (lanes across the head dimension, rows batched so the
//      norm reductions overlap);
//   2  block sums and their norms (tiles added in a fixed order);
//   3  anomalies: the sequence sum from the block sums, in order; every
//      wave walks a contiguous run of rows carrying the window sum S
//      (S += k^_new - k^_old, the old row reloaded from cache and
//      renormalised with its stored inverse norm), so the stable, episodic
//      and current cosines are dot products with per-lane partials folded by
//      butterfly shuffles; per-tile maxima and minima of each anomaly;
//   4  per-head weights from the tiles' extremes, routing, the score.
// Cosines are scale-free, so sums stand in for means.
#include "internal.hpp"

namespace hubkv {

namespace {

constexpr int kT = 256;
constexpr int kWaves = kT / 64;
constexpr int kWin = 64;   // current-memory window
constexpr int kBatch = 8;  // rows per batch of butterfly reductions

template <typename T>
__device__ __forceinline__ float to_f(T x);
template <>
__device__ __forceinline__ float to_f<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f<__bf16>(__bf16 x) { return (float)x; }

// Butterfly sum over the 64 lanes of N independent values (every lane ends
// with the totals).
template <int N>
__device__ __forceinline__ void wave_sum(float (&v)[N]) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] += __shfl_xor(v[j], off);
}

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

// Lane l owns head-dimension elements [E l, E l + E) of every row.
template <typename T, int D>
struct RowIO {
  static constexpr int E = D / 64;
  __device__ static void load(const T* __restrict__ K, int64_t row, int lane, float (&x)[E]) {
    const T* p = K + row * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = to_f<T>(p[e]);
  }
};

// ---- 1: tile sums of the normalised keys
template <typename T, int D>
__global__ __launch_bounds__(kT) void nkv_tile_sum(const T* __restrict__ K, NkvArgs a,
                                                   NkvGeom g, char* ws) {
  constexpr int E = D / 64;
  __shared__ float red[kWaves][D];
  const Tile t = tile_of(a);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  // wave w takes rows t0 + w, t0 + w + 4, ... in batches of kBatch
  for (int64_t r0 = t.t0 + wave; r0 < t.t1; r0 += (int64_t)kWaves * kBatch) {
    float x[kBatch][E], nn[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t r = r0 + (int64_t)i * kWaves;
      const int64_t rc = r < t.t1 ? r : t.t0;
      RowIO<T, D>::load(K, t.row_base + rc, lane, x[i]);
      nn[i] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) nn[i] = fmaf(x[i][e], x[i][e], nn[i]);
      if (r >= t.t1) nn[i] = 0.f;
    }
    wave_sum<kBatch>(nn);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t r = r0 + (int64_t)i * kWaves;
      const float inv = (r < t.t1 && nn[i] > 0.f) ? 1.f / sqrtf(nn[i]) : 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(x[i][e], inv, acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[wave][lane * E + e] = acc[e];
  __syncthreads();
  float* out = (float*)(ws + g.off_part) + ((int64_t)t.lh * a.ntile + t.tile_g) * D;
  for (int e = threadIdx.x; e < D; e += kT) {
    float s = 0.f;
    for (int w = 0; w < kWaves; ++w) s += red[w][e];
    out[e] = s;
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

// ---- 3: anomalies.  Wave w walks rows [r0, r1), a contiguous quarter of the
// tile, after a warm-up over the (at most 63) rows before r0 that fill its
// window.  Lane (q mod 64) keeps the inverse norm of row q for the last 64
// rows, so the row leaving the window is reloaded (from cache) and
// renormalised without a reduction.
template <typename T, int D>
__global__ __launch_bounds__(kT) void nkv_anomaly(const T* __restrict__ K, NkvArgs a, NkvGeom g,
                                                  char* ws, float* __restrict__ an) {
  constexpr int E = D / 64;
  __shared__ float mm_s[kWaves][6];
  const Tile t = tile_of(a);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the sequence sum: block sums of the sequence in order
  const float* bs_seq = (const float*)(ws + g.off_bsum) +
                        ((int64_t)t.lh * a.nblk_total + a.blk_off[t.b]) * D;
  float ms[E], me[E];
#pragma unroll
  for (int e = 0; e < E; ++e) ms[e] = 0.f;
  for (int m = 0; m < a.nblk[t.b]; ++m)
#pragma unroll
    for (int e = 0; e < E; ++e) ms[e] += bs_seq[(int64_t)m * D + lane * E + e];
  float msn[1] = {0.f};
#pragma unroll
  for (int e = 0; e < E; ++e) msn[0] = fmaf(ms[e], ms[e], msn[0]);
  wave_sum<1>(msn);
  const int bi = a.blk_off[t.b] + t.m;
  const float* eb = (const float*)(ws + g.off_bsum) + ((int64_t)t.lh * a.nblk_total + bi) * D;
  const float ebn = ((const float*)(ws + g.off_bnorm))[(int64_t)t.lh * a.nblk_total + bi];
#pragma unroll
  for (int e = 0; e < E; ++e) me[e] = eb[lane * E + e];
  const float musn = sqrtf(msn[0]);
  const float ims = musn > 0.f ? 1.f / musn : 0.f, ime = ebn > 0.f ? 1.f / ebn : 0.f;
  const int64_t len = t.t1 - t.t0;
  const int64_t q4 = (len + kWaves - 1) / kWaves;
  const int64_t r0 = t.t0 + q4 * wave < t.t1 ? t.t0 + q4 * wave : t.t1;
  const int64_t r1 = r0 + q4 < t.t1 ? r0 + q4 : t.t1;
  const int64_t w0 = r0 - (kWin - 1) > 0 ? r0 - (kWin - 1) : 0;  // first row of the warm-up
  float S[E];
#pragma unroll
  for (int e = 0; e < E; ++e) S[e] = 0.f;
  float ring = 0.f;  // lane (q mod 64): inverse norm of row q
  float mx[3] = {-INFINITY, -INFINITY, -INFINITY}, mn[3] = {INFINITY, INFINITY, INFINITY};
  float* anb = an + t.row_base * 3;
  for (int64_t q0 = w0; r0 < r1 && q0 < r1; q0 += kBatch) {
    float xn[kBatch][E], xo[kBatch][E], nn[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t q = q0 + i;
      const bool in = q < r1;
      RowIO<T, D>::load(K, t.row_base + (in ? q : w0), lane, xn[i]);
      const int64_t qo = q - kWin;
      RowIO<T, D>::load(K, t.row_base + (in && qo >= w0 ? qo : w0), lane, xo[i]);
      nn[i] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) nn[i] = fmaf(xn[i][e], xn[i][e], nn[i]);
    }
    wave_sum<kBatch>(nn);
    float part[4 * kBatch];  // per row: k^.S, S.S, k^.mu_s, k^.mu_e (lane partials)
    float inv[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t q = q0 + i;
      const bool in = q < r1;
      inv[i] = (in && nn[i] > 0.f) ? 1.f / sqrtf(nn[i]) : 0.f;
      const int slot = (int)(q & (kWin - 1));
      const float iold = __shfl(ring, slot);       // row q - 64's, when it was seen
      const bool drop = in && q - kWin >= w0;
      if (lane == slot && in) ring = inv[i];
      float kh[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        kh[e] = xn[i][e] * inv[i];
        S[e] = S[e] + kh[e] - (drop ? xo[i][e] * iold : 0.f);
      }
      float dc = 0.f, ss = 0.f, ds = 0.f, de = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        dc = fmaf(kh[e], S[e], dc);
        ss = fmaf(S[e], S[e], ss);
        ds = fmaf(kh[e], ms[e], ds);
        de = fmaf(kh[e], me[e], de);
      }
      part[4 * i + 0] = dc;
      part[4 * i + 1] = ss;
      part[4 * i + 2] = ds;
      part[4 * i + 3] = de;
    }
    wave_sum<4 * kBatch>(part);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t q = q0 + i;
      if (q < r0 || q >= r1) continue;  // warm-up rows and past the run
      const float sn = part[4 * i + 1] > 0.f ? sqrtf(part[4 * i + 1]) : 0.f;
      const float as = -(part[4 * i + 2] * ims);
      const float ae = -(part[4 * i + 3] * ime);
      const float ac = sn > 0.f ? -(part[4 * i + 0] / sn) : -0.f;
      mx[0] = fmaxf(mx[0], as);
      mx[1] = fmaxf(mx[1], ae);
      mx[2] = fmaxf(mx[2], ac);
      mn[0] = fminf(mn[0], as);
      mn[1] = fminf(mn[1], ae);
      mn[2] = fminf(mn[2], ac);
      if (lane < 3) anb[q * 3 + lane] = lane == 0 ? as : (lane == 1 ? ae : ac);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      mm_s[wave][2 * x] = mx[x];
      mm_s[wave][2 * x + 1] = mn[x];
    }
  }
  __syncthreads();
  if (threadIdx.x < 6) {
    const int x = threadIdx.x;
    float v = mm_s[0][x];
    for (int w = 1; w < kWaves; ++w) v = (x & 1) ? fminf(v, mm_s[w][x]) : fmaxf(v, mm_s[w][x]);
    ((float*)(ws + g.off_mm))[((int64_t)t.lh * a.ntile + t.tile_g) * 6 + x] = v;
  }
}

// ---- 4: per-head weights and routing
__global__ __launch_bounds__(kT) void nkv_route(NkvArgs a, NkvGeom g, char* ws,
                                                const float* __restrict__ an,
                                                float* __restrict__ s,
                                                float* __restrict__ weights) {
  __shared__ float w_s[3], ext[kWaves][6];
  const Tile t = tile_of(a);
  {
    // extremes of each anomaly over the sequence's tiles (max / min: exact in any order)
    const float* mm = (const float*)(ws + g.off_mm) + (int64_t)t.lh * a.ntile * 6;
    float hi[3] = {-INFINITY, -INFINITY, -INFINITY}, lo[3] = {INFINITY, INFINITY, INFINITY};
    const int tb = a.tile_off[t.b], te = a.tile_off[t.b + 1];
    for (int x = tb + (int)threadIdx.x; x < te; x += kT)
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        hi[k] = fmaxf(hi[k], mm[(int64_t)x * 6 + 2 * k]);
        lo[k] = fminf(lo[k], mm[(int64_t)x * 6 + 2 * k + 1]);
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
    if (weights && t.m == 0 && t.j == 0) {
      const int l = t.lh / a.Hkv, h = t.lh - l * a.Hkv;
#pragma unroll
      for (int k = 0; k < 3; ++k) weights[(((int64_t)l * a.B + t.b) * a.Hkv + h) * 3 + k] = w_s[k];
    }
  }
  __syncthreads();
  const float w0 = w_s[0], w1 = w_s[1], w2 = w_s[2];
  for (int64_t q = t.t0 + threadIdx.x; q < t.t1; q += kT) {
    const float* ai = an + (t.row_base + q) * 3;
    const float x0 = ai[0], x1 = ai[1], x2 = ai[2];
    const float mean = (x0 + x1 + x2) * (1.f / 3.f);
    const float v = ((x0 - mean) * (x0 - mean) + (x1 - mean) * (x1 - mean) +
                     (x2 - mean) * (x2 - mean)) * (1.f / 3.f);
    const float sg = sqrtf(v);
    s[t.row_base + q] = sg > a.theta ? fmaxf(fmaxf(x0, x1), x2)
                                     : fmaf(w0, x0, fmaf(w1, x1, w2 * x2));
  }
}

template <typename T, int D>
hipError_t launch_t(const void* k, const NkvArgs& a, const NkvGeom& g, char* ws, float* an,
                    float* s, float* weights, hipStream_t stream) {
  const dim3 grid(a.ntile, a.L * a.Hkv), block(kT);
  hipLaunchKernelGGL((nkv_tile_sum<T, D>), grid, block, 0, stream, (const T*)k, a, g, ws);
  hipLaunchKernelGGL(nkv_block_sum, dim3(a.nblk_total, a.L * a.Hkv), block, 0, stream, a, g, ws);
  hipLaunchKernelGGL((nkv_anomaly<T, D>), grid, block, 0, stream, (const T*)k, a, g, ws, an);
  hipLaunchKernelGGL(nkv_route, grid, block, 0, stream, a, g, ws, (const float*)an, s, weights);
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
  g.off_mm = take((size_t)LH * a.ntile * 6 * 4);
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
