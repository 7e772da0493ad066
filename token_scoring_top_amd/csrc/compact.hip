// compact.hip -- gather of the kept K/V rows into a packed cache.
//
// H2O breakdown page, "two code bases": the real-drop variant physically
// removes evicted tokens' K/V, so later attention reads only the kept rows.
//   K_out[l][g][o_b + j] = K[l][g][cu_b + idx[l][g][o_b + j]]   (same for V)
// Each operand has its own layer, head and row strides, so token-major or
// padded caches are read and written in place.
// Each thread moves 16-byte pieces of rows; a 256-byte bf16 row (d = 128) is
// 16 consecutive lanes, so every wave reads and writes whole rows with fully
// used 64-byte segments.
#include "internal.hpp"

namespace hubkv {

namespace {

constexpr int kCompactThreads = 256;
constexpr int kUnroll = 1;  // rows per thread group and block iteration (1 measured fastest:
                             // more, smaller work-groups keep more rows in flight)

__device__ __forceinline__ int seq_of_row(const SeqTable& st, int64_t row) {
  int lo = 0, hi = st.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (st.ko[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Rows of 1 << LOGP 16-byte pieces: a group of 1 << LOGP consecutive lanes
// moves one row, so a wave reads and writes whole rows.  Each thread first
// loads the kept positions of its kUnroll rows, then their K and V pieces
// (2 kUnroll 16-byte loads in flight), then stores them (non-temporal: the
// packed cache is not read again here).  On the Llama-2-7B-shaped layer one
// row per thread group ran at 6.0 TB/s against 5.5 TB/s for four.
// Row strides of the four operands (16-byte units) and the KV head count.
struct CompactStrides {
  RowStrides ki, vi, ko, vo;
  int Hkv;
};

__device__ __forceinline__ int64_t head_base(const RowStrides& r, int l, int h) {
  return (int64_t)l * r.s_l + (int64_t)h * r.s_h;
}

template <int LOGP>
__global__ __launch_bounds__(kCompactThreads) void compact_kernel(
    const u32x4* __restrict__ k_in, const u32x4* __restrict__ v_in,
    const int32_t* __restrict__ idx, SeqTable st, CompactStrides cs, int64_t Ktot,
    u32x4* __restrict__ k_out, u32x4* __restrict__ v_out) {
  constexpr int P = 1 << LOGP;
  constexpr int RPI = kCompactThreads / P;  // rows per unrolled step
  constexpr int RB = RPI * kUnroll;          // rows per block iteration
  const int lh = blockIdx.y;
  const int l = lh / cs.Hkv, h = lh - l * cs.Hkv;
  const int pc = threadIdx.x & (P - 1);
  const int rsub = threadIdx.x >> LOGP;
  const int32_t* ih = idx + (int64_t)lh * Ktot;
  const u32x4* kin = k_in + head_base(cs.ki, l, h) + pc;
  const u32x4* vin = v_in + head_base(cs.vi, l, h) + pc;
  u32x4* ko = k_out + head_base(cs.ko, l, h) + pc;
  u32x4* vo = v_out + head_base(cs.vo, l, h) + pc;
  for (int64_t row0 = (int64_t)blockIdx.x * RB; row0 < Ktot; row0 += (int64_t)gridDim.x * RB) {
    int64_t src[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t row = row0 + u * RPI + rsub;
      src[u] = -1;
      if (row < Ktot) {
        const int b = st.B == 1 ? 0 : seq_of_row(st, row);
        const int32_t p = ih[row];
        if (p >= 0 && p < st.N[b]) src[u] = st.cu[b] + p;
      }
    }
    u32x4 kv[kUnroll], vv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (src[u] >= 0) {
        kv[u] = __builtin_nontemporal_load(&kin[src[u] * cs.ki.s_t]);
        vv[u] = __builtin_nontemporal_load(&vin[src[u] * cs.vi.s_t]);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (src[u] >= 0) {
        const int64_t row = row0 + u * RPI + rsub;
        __builtin_nontemporal_store(kv[u], &ko[row * cs.ko.s_t]);
        __builtin_nontemporal_store(vv[u], &vo[row * cs.vo.s_t]);
      }
    }
  }
}

}  // namespace

hipError_t launch_compact(const void* k_in, const void* v_in, int elem_bytes, const int32_t* idx,
                          const SeqTable& st, int L, int Hkv, int d, const RowStrides& ki,
                          const RowStrides& vi, const RowStrides& ko, const RowStrides& vo,
                          void* k_out, void* v_out, hipStream_t stream) {
  int64_t K = 0;
  for (int b = 0; b < st.B; ++b) K += st.kept[b];
  if (K == 0) return hipSuccess;
  const int pieces = d * elem_bytes / 16;  // 8, 16 or 32
  const int logp = pieces == 8 ? 3 : (pieces == 16 ? 4 : 5);
  const int64_t rb = (int64_t)(kCompactThreads / pieces) * kUnroll;
  int64_t blocks = (K + rb - 1) / rb;
  if (blocks > 65535) blocks = 65535;
  const dim3 grid((unsigned)blocks, L * Hkv), block(kCompactThreads);
  const CompactStrides cs{ki, vi, ko, vo, Hkv};
  const u32x4* kp = (const u32x4*)k_in;
  const u32x4* vp = (const u32x4*)v_in;
  if (logp == 3)
    hipLaunchKernelGGL(compact_kernel<3>, grid, block, 0, stream, kp, vp, idx, st, cs, K,
                       (u32x4*)k_out, (u32x4*)v_out);
  else if (logp == 4)
    hipLaunchKernelGGL(compact_kernel<4>, grid, block, 0, stream, kp, vp, idx, st, cs, K,
                       (u32x4*)k_out, (u32x4*)v_out);
  else
    hipLaunchKernelGGL(compact_kernel<5>, grid, block, 0, stream, kp, vp, idx, st, cs, K,
                       (u32x4*)k_out, (u32x4*)v_out);
  return hipGetLastError();
}

}  // namespace hubkv
