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
//   3  anomalies over tiles of kNkvAnTile keys, one key row per lane: the
//      sequence sum from the block sums, in order; the current-window sum of
//      each row is a cross-lane prefix (DPP scans) of the normalised keys of
//      its 64-row segment plus the suffix of the previous segment, so the
//      stable, episodic and current cosines are lane-local dot products;
//      per-tile extremes of each anomaly;
//   4  per-head weights from the tiles' extremes, routing, the score.
// Cosines are scale-free, so sums stand in for means.
#include "internal.hpp"

namespace hubkv {

namespace {

constexpr int kT = 256;
constexpr int kWaves = kT / 64;


template <typename T>
__device__ __forceinline__ float to_f(T x);
template <>
__device__ __forceinline__ float to_f<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f<__bf16>(__bf16 x) { return (float)x; }

// Inclusive prefix sum across the 64 lanes of a wave with DPP moves (no LDS):
// shifts by 1, 2, 4 and 8 inside each 16-lane row, then row broadcasts of lane
// 15 into rows 1 and 3 and of lane 31 into rows 2 and 3.  Lanes whose source
// falls outside their row add 0.
__device__ __forceinline__ float dpp_add(float v, int y) { return v + __int_as_float(y); }
__device__ __forceinline__ float wave_prefix(float v) {
  v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, false));
  v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, false));
  v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));
  v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false));
  v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xa, 0xf, false));
  v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xc, 0xf, false));
  return v;
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

// ---- 1: tile sums of the normalised keys, and every row's inverse norm.
// Each wave loads RPW rows per instruction, kUnroll instructions in flight;
// the norm of a row is folded over its LPR lanes.
template <typename T, int D>
__global__ __launch_bounds__(kT) void nkv_tile_sum(const T* __restrict__ K, NkvArgs a,
                                                   NkvGeom g, char* ws) {
  float* invn = (float*)(ws + g.off_inv);  // every row's inverse norm, for the anomaly pass
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
      if (in[u] && c == 0) invn[t.row_base + r0 + (int64_t)u * STEP] = inv;
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

// ---- 3: anomalies over tiles of kNkvAnTile rows, rows on lanes.  Wave w
// owns NSEG segments of 64 rows; in segment s lane l owns row r = 64 s + l of
// the wave's run.  The window of the 64 rows ending at r is the segment's
// rows up to r plus the previous segment's rows after position l, so for each
// 16-element group of the head dimension
//   S = (inclusive prefix of k^ across the lanes)
//     + (exclusive suffix across the lanes of the previous segment's k^),
// the previous segment's line reloaded from cache and renormalised with its
// stored inverse norm (pass 1 wrote every row's); the scans are DPP moves and
// the suffix is the previous segment's total minus its prefix.  The dot
// products k^.S, S.S, k^.mu_s and k^.mu_e are then lane-local.  A row's
// episodic memory is its block's; a segment's blocks are walked with uniform
// loads (at most two when blocks hold 64 rows or more).  The wave's
// (segment, group) items run in order with kPf items' lines in flight.
template <typename T, int D>
__global__ __launch_bounds__(kT) void nkv_anomaly(const T* __restrict__ K, NkvArgs a, NkvGeom g,
                                                  char* ws, float* __restrict__ an) {
  constexpr int EPW = 16 / (int)sizeof(T);     // elements per 16-byte word
  constexpr int G = 16;                        // elements per scan group
  constexpr int WPG = G / EPW;                 // 16-byte words per group
  constexpr int NG = D / G;
  constexpr int NSEG = kNkvAnTile / (kWaves * 64);
  constexpr int kPf = 3;
  __shared__ float mus[D];
  __shared__ float red[kWaves];
  __shared__ float mm_s[kWaves][6];
  const int lh = blockIdx.y, x = blockIdx.x;
  int b = 0;
  while (b + 1 < a.B && a.at_off[b + 1] <= x) ++b;
  const int64_t N = a.N[b];
  const int64_t t0 = (int64_t)(x - a.at_off[b]) * kNkvAnTile;
  const int64_t t1 = t0 + kNkvAnTile < N ? t0 + kNkvAnTile : N;
  const int64_t row_base = (int64_t)lh * a.T + a.cu[b];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* bsum =
      (const float*)(ws + g.off_bsum) + ((int64_t)lh * a.nblk_total + a.blk_off[b]) * D;
  const float* bnrm = (const float*)(ws + g.off_bnorm) + (int64_t)lh * a.nblk_total + a.blk_off[b];
  const float* invn = (const float*)(ws + g.off_inv) + row_base;
  // the sequence sum (block sums in order) and its norm
  {
    const int e = threadIdx.x;
    float v = 0.f;
    if (e < D) {
#pragma unroll 8
      for (int m = 0; m < a.nblk[b]; ++m) v += bsum[(int64_t)m * D + e];
      mus[e] = v;
    }
    float q = e < D ? v * v : 0.f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) q += __shfl_xor(q, off);
    if (lane == 0) red[wave] = q;
  }
  __syncthreads();
  float msn = 0.f;
  for (int w = 0; w < kWaves; ++w) msn += red[w];
  const float ims = msn > 0.f ? 1.f / sqrtf(msn) : 0.f;
  const int bsz = a.bs[b];
  const int64_t wbase = t0 + (int64_t)wave * NSEG * 64;
  float mx[3] = {-INFINITY, -INFINITY, -INFINITY}, mn[3] = {INFINITY, INFINITY, INFINITY};
  float* anb = an + row_base * 3;
  const int64_t wend = wbase + (int64_t)NSEG * 64 < t1 ? wbase + (int64_t)NSEG * 64 : t1;
  const int nseg = wend > wbase ? (int)((wend - wbase + 63) / 64) : 0;
  const int items = nseg * NG;
  u32x4 buf[kPf][2 * WPG];  // the current and the previous segment's words of an item
  auto issue = [&](int t, u32x4 (&dst)[2 * WPG]) {
    const int s2 = t / NG, gi = t - s2 * NG;
    const int64_t row = wbase + 64 * s2 + lane, prow = row - 64;
    const T* cur = K + (row_base + (row < N ? row : 0)) * D + gi * G;
    const T* prv = K + (row_base + (prow >= 0 ? prow : 0)) * D + gi * G;
#pragma unroll
    for (int k = 0; k < WPG; ++k) {
      dst[k] = ((const u32x4*)cur)[k];
      dst[WPG + k] = ((const u32x4*)prv)[k];
    }
  };
#pragma unroll
  for (int u = 0; u < kPf; ++u)
    if (u < items) issue(u, buf[u]);
  int64_t row = 0;
  bool inseq = false;
  float iv = 0.f, ivp = 0.f, d_c = 0.f, s_s = 0.f, d_s = 0.f, d_e = 0.f;
  int mfirst = 0, mlast = 0, mine = 0;
  for (int tb = 0; tb < items; tb += kPf) {
#pragma unroll
    for (int u = 0; u < kPf; ++u) {
      const int t = tb + u;
      if (t >= items) break;
      const int s2 = t / NG, gi = t - s2 * NG;
      if (gi == 0) {
        const int64_t r0 = wbase + 64 * s2;
        row = r0 + lane;
        const int64_t prow = row - 64;
        inseq = row < N;
        iv = inseq ? invn[row] : 0.f;
        ivp = prow >= 0 ? invn[prow] : 0.f;
        const int64_t rl = r0 + 63 < t1 - 1 ? r0 + 63 : t1 - 1;
        mfirst = (int)(r0 / bsz);
        mlast = (int)(rl / bsz);
        mine = (int)((inseq && row < t1 ? row : rl) / bsz);
        d_c = s_s = d_s = d_e = 0.f;
      }
      float p[G], q[G], kh[G];
#pragma unroll
      for (int k = 0; k < WPG; ++k) {
        const T* ec = (const T*)&buf[u][k];
        const T* ep = (const T*)&buf[u][WPG + k];
#pragma unroll
        for (int i = 0; i < EPW; ++i) {
          kh[k * EPW + i] = to_f<T>(ec[i]) * iv;
          q[k * EPW + i] = to_f<T>(ep[i]) * ivp;
        }
      }
      // the slot is free: the lines kPf items ahead go into it
      if (t + kPf < items) issue(t + kPf, buf[u]);
#pragma unroll
      for (int i = 0; i < G; ++i) {
        p[i] = wave_prefix(kh[i]);
        const float pq = wave_prefix(q[i]);
        q[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pq), 63)) - pq;
      }
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float S = p[j] + q[j];
        d_c = fmaf(kh[j], S, d_c);
        s_s = fmaf(S, S, s_s);
        d_s = fmaf(kh[j], mus[gi * G + j], d_s);
      }
      for (int m = mfirst; m <= mlast; ++m) {
        const float* em = bsum + (int64_t)m * D + gi * G;
        float e = 0.f;
#pragma unroll
        for (int j = 0; j < G; ++j) e = fmaf(kh[j], em[j], e);
        if (m == mine) d_e += e;
      }
      if (gi == NG - 1 && inseq && row < t1) {
        const float en = bnrm[mine];
        const float sn = s_s > 0.f ? sqrtf(s_s) : 0.f;
        const float as = -(d_s * ims);
        const float ae = en > 0.f ? -(d_e / en) : -0.f;
        const float ac = sn > 0.f ? -(d_c / sn) : -0.f;
        mx[0] = fmaxf(mx[0], as);
        mx[1] = fmaxf(mx[1], ae);
        mx[2] = fmaxf(mx[2], ac);
        mn[0] = fminf(mn[0], as);
        mn[1] = fminf(mn[1], ae);
        mn[2] = fminf(mn[2], ac);
        anb[row * 3 + 0] = as;
        anb[row * 3 + 1] = ae;
        anb[row * 3 + 2] = ac;
      }
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
  g.off_inv = take((size_t)LH * a.T * 4);
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
