// compact.hip -- gather of the kept K/V rows into a packed cache.
//
// H2O breakdown page, "two code bases": the real-drop variant physically
// removes evicted tokens' K/V, so later attention reads only the kept rows.
//   K_out[l][g][o_b + j] = K[l][g][cu_b + idx[l][g][o_b + j]]   (same for V)
// Each thread moves 16-byte pieces of rows; a 256-byte bf16 row (d = 128) is
// 16 consecutive lanes, so every wave reads and writes whole rows with fully
// used 64-byte segments.  Several pieces per thread are loaded before any is
// stored, to keep enough reads in flight.
#include "internal.hpp"

namespace hubkv {

namespace {

constexpr int kCompactThreads = 256;
constexpr int kUnroll = 4;

__device__ __forceinline__ int seq_of_row(const SeqTable& st, int64_t row) {
  int lo = 0, hi = st.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (st.ko[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(kCompactThreads) void compact_kernel(
    const u32x4* __restrict__ k_in, const u32x4* __restrict__ v_in,
    const int32_t* __restrict__ idx, SeqTable st, int64_t T, int64_t Ktot, int pieces,
    u32x4* __restrict__ k_out, u32x4* __restrict__ v_out) {
  const int lh = blockIdx.y;
  const int64_t total = Ktot * pieces;
  const int64_t stride = (int64_t)gridDim.x * kCompactThreads;
  const int32_t* ih = idx + (int64_t)lh * Ktot;
  const u32x4* kin = k_in + (int64_t)lh * T * pieces;
  const u32x4* vin = v_in + (int64_t)lh * T * pieces;
  u32x4* ko = k_out + (int64_t)lh * Ktot * pieces;
  u32x4* vo = v_out + (int64_t)lh * Ktot * pieces;
  for (int64_t f0 = (int64_t)blockIdx.x * kCompactThreads + threadIdx.x; f0 < total;
       f0 += stride * kUnroll) {
    u32x4 kv[kUnroll], vv[kUnroll];
    int64_t dst[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t f = f0 + u * stride;
      dst[u] = -1;
      if (f < total) {
        const int64_t row = f / pieces;
        const int pc = (int)(f - row * pieces);
        const int b = seq_of_row(st, row);
        const int32_t p = ih[row];
        if (p >= 0 && p < st.N[b]) {
          const int64_t src = (st.cu[b] + p) * pieces + pc;
          kv[u] = kin[src];
          vv[u] = vin[src];
          dst[u] = f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (dst[u] >= 0) {
        ko[dst[u]] = kv[u];
        vo[dst[u]] = vv[u];
      }
    }
  }
}

}  // namespace

hipError_t launch_compact(const void* k_in, const void* v_in, int elem_bytes, const int32_t* idx,
                          const SeqTable& st, int L, int Hkv, int d, void* k_out, void* v_out,
                          hipStream_t stream) {
  int64_t T = 0, K = 0;
  for (int b = 0; b < st.B; ++b) {
    T += st.N[b];
    K += st.kept[b];
  }
  if (K == 0) return hipSuccess;
  const int pieces = d * elem_bytes / 16;
  const int64_t total = K * pieces;
  int64_t blocks = (total + (int64_t)kCompactThreads * kUnroll - 1) / ((int64_t)kCompactThreads * kUnroll);
  if (blocks > 65535) blocks = 65535;
  hipLaunchKernelGGL(compact_kernel, dim3((unsigned)blocks, L * Hkv), dim3(kCompactThreads), 0,
                     stream, (const u32x4*)k_in, (const u32x4*)v_in, idx, st, T, K, pieces,
                     (u32x4*)k_out, (u32x4*)v_out);
  return hipGetLastError();
}

}  // namespace hubkv
