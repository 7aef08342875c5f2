// Combination of partial attention results over disjoint key sets, the
// online-softmax merge of ring-style attention (HSAP page, Section 2.2.1 and
// the copy/rescale step of Section 3.1, Table 1; BASP page, Section VII).
//
// Per (row t, head h): M = max_k LSE_k, w_k = exp(LSE_k - M),
// LSE = M + ln sum_k w_k, O = sum_k (w_k / sum w) O_k; all -inf gives 0, -inf.
//
// Bandwidth bound: every partial byte is read once and the result written
// once.  A group of head_dim/4 lanes owns one (row, head); each lane reads
// 4 consecutive elements of every partial (16 B for fp32 partials) with all
// partial loads of a row issued before the first use.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "launch.h"
#include "profiler.h"

namespace vl {

namespace {

struct PartPtrs {
  const void* o[kMaxMergeParts];
  const float* lse[kMaxMergeParts];
};

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ f32x4 load4(const void* base, int64_t idx) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(
        reinterpret_cast<const float*>(base) + idx));
  } else {
    const u32x2 u = __builtin_nontemporal_load(
        reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(base) + idx));
    f32x4 r;
    r[0] = bf16_lo(u[0]);
    r[1] = bf16_hi(u[0]);
    r[2] = bf16_lo(u[1]);
    r[3] = bf16_hi(u[1]);
    return r;
  }
}

template <typename TO>
__device__ __forceinline__ void store4(void* base, int64_t idx, const f32x4& v) {
  if constexpr (sizeof(TO) == 4) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + idx));
  } else {
    u32x2 u;
    u[0] = pack_bf16x2(v[0], v[1]);
    u[1] = pack_bf16x2(v[2], v[3]);
    __builtin_nontemporal_store(u, reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(base) + idx));
  }
}

template <typename TI, typename TO, int NP>
__global__ void __launch_bounds__(kThreads)
lse_merge_kernel(PartPtrs parts, int n_parts, int64_t n_rows, int n_heads, int head_dim,
                 void* __restrict__ o_out, float* __restrict__ lse_out) {
  const int lanes_per_row = head_dim >> 2;
  const int rows_per_block = kThreads / lanes_per_row;
  const int sub = threadIdx.x / lanes_per_row;
  const int c4 = (threadIdx.x - sub * lanes_per_row) * 4;
  const int64_t n_pairs = n_rows * n_heads;
  if (sub >= rows_per_block) return;
  for (int64_t pr = int64_t(blockIdx.x) * rows_per_block + sub; pr < n_pairs;
       pr += int64_t(gridDim.x) * rows_per_block) {
    const int64_t t = pr / n_heads;
    const int h = int(pr - t * n_heads);
    const int64_t lidx = int64_t(h) * n_rows + t;
    const int np = NP > 0 ? NP : n_parts;
    float l[NP > 0 ? NP : kMaxMergeParts];
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < (NP > 0 ? NP : kMaxMergeParts); ++k) {
      if (k < np) {
        l[k] = parts.lse[k][lidx];
        m = fmaxf(m, l[k]);
      }
    }
    const int64_t oidx = pr * head_dim + c4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float tot = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int k = 0; k < (NP > 0 ? NP : kMaxMergeParts); ++k) {
        if (k < np) {
          const float w = __expf(l[k] - m);
          tot += w;
          const f32x4 x = load4<TI>(parts.o[k], oidx);
          acc[0] += w * x[0];
          acc[1] += w * x[1];
          acc[2] += w * x[2];
          acc[3] += w * x[3];
        }
      }
      const float inv = 1.f / tot;
      acc[0] *= inv;
      acc[1] *= inv;
      acc[2] *= inv;
      acc[3] *= inv;
    }
    store4<TO>(o_out, oidx, acc);
    if (c4 == 0) lse_out[lidx] = (m == -INFINITY) ? -INFINITY : m + __logf(tot);
  }
}

template <typename TI, typename TO>
hipError_t dispatch(const PartPtrs& p, int n_parts, int64_t n_rows, int n_heads, int head_dim,
                    void* o_out, float* lse_out, hipStream_t stream) {
  const int lanes_per_row = head_dim / 4;
  const int rows_per_block = kThreads / lanes_per_row;
  const int64_t n_pairs = n_rows * n_heads;
  const int64_t want = (n_pairs + rows_per_block - 1) / rows_per_block;
  // one pass of the grid-stride loop: more rows in flight than a capped grid
  const int blocks = int(std::max<int64_t>(1, std::min<int64_t>(want, int64_t(1) << 30)));
  ProfScope prof("lse_merge", stream);
#define VL_MERGE_CASE(N)                                                                     \
  case N:                                                                                    \
    hipLaunchKernelGGL((lse_merge_kernel<TI, TO, N>), dim3(blocks), dim3(kThreads), 0, stream, p, \
                       n_parts, n_rows, n_heads, head_dim, o_out, lse_out);                  \
    break;
  switch (n_parts) {
    VL_MERGE_CASE(1)
    VL_MERGE_CASE(2)
    VL_MERGE_CASE(4)
    VL_MERGE_CASE(8)
    VL_MERGE_CASE(16)
    default:
      hipLaunchKernelGGL((lse_merge_kernel<TI, TO, 0>), dim3(blocks), dim3(kThreads), 0, stream, p,
                         n_parts, n_rows, n_heads, head_dim, o_out, lse_out);
  }
#undef VL_MERGE_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(int32_t n_parts, const void* const* o_parts,
                            const float* const* lse_parts, int32_t in_dtype, int64_t n_rows,
                            int32_t n_heads, int32_t head_dim, void* o_out, float* lse_out,
                            int32_t out_dtype, hipStream_t stream) {
  if (n_rows == 0 || n_heads == 0) return hipSuccess;
  PartPtrs p{};
  for (int k = 0; k < n_parts; ++k) {
    p.o[k] = o_parts[k];
    p.lse[k] = lse_parts[k];
  }
  // in/out dtype 0 = bf16, 1 = fp32
  if (in_dtype == 1 && out_dtype == 1)
    return dispatch<float, float>(p, n_parts, n_rows, n_heads, head_dim, o_out, lse_out, stream);
  if (in_dtype == 1 && out_dtype == 0)
    return dispatch<float, uint16_t>(p, n_parts, n_rows, n_heads, head_dim, o_out, lse_out, stream);
  if (in_dtype == 0 && out_dtype == 1)
    return dispatch<uint16_t, float>(p, n_parts, n_rows, n_heads, head_dim, o_out, lse_out, stream);
  return dispatch<uint16_t, uint16_t>(p, n_parts, n_rows, n_heads, head_dim, o_out, lse_out, stream);
}

}  // namespace vl
