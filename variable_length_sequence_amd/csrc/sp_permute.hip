// Ulysses sequence<->head layout change of one GPU's shard (HSAP page,
// Section 2.2.2; BASP page, Section II-C).  seq2head packs x [n, H, d] into
// y [P, n, h, d] (h = H / P) so that chunk p is one contiguous message for
// rank p; head2seq is the inverse.  Pure data movement, bandwidth bound.
//
// Both directions copy n * P runs of h * d elements.  The kernel walks the
// [n, H, d] side linearly (fully coalesced) and scatters/gathers whole runs on
// the [P, n, h, d] side, so every wave touches at most a few runs of
// contiguous bytes.  Units are 16, 8, 4 or 2 bytes, the widest that divides a
// run and the pointer alignment.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "fastdiv.h"
#include "launch.h"
#include "profiler.h"

namespace vl {

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t unit16;
typedef __attribute__((ext_vector_type(2))) uint32_t unit8;

constexpr int kThreads = 256;
constexpr int kIlp = 4;  // units in flight per thread

template <typename U, int DIR>
__global__ void __launch_bounds__(kThreads)
sp_permute_kernel(const U* __restrict__ src, U* __restrict__ dst, uint32_t n_units,
                  FastDiv upc, FastDiv deg, uint32_t t0, uint32_t n_tok) {
  // flat index i over the [n, H, d] side of this launch's token range
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t base = blockIdx.x * kThreads * kIlp + threadIdx.x; base < n_units;
       base += stride * kIlp) {
    U val[kIlp];
    uint64_t other[kIlp];
#pragma unroll
    for (int r = 0; r < kIlp; ++r) {
      const uint32_t i = base + r * kThreads;
      if (i < n_units) {
        const uint32_t run = upc.div(i);           // (t, p) in token-major order
        const uint32_t off = i - run * upc.d;
        const uint32_t t = deg.div(run);
        const uint32_t p = run - t * deg.d;
        other[r] = (uint64_t(p) * n_tok + (t0 + t)) * upc.d + off;
        if (DIR == 0)
          val[r] = __builtin_nontemporal_load(src + i);
        else
          val[r] = __builtin_nontemporal_load(src + other[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < kIlp; ++r) {
      const uint32_t i = base + r * kThreads;
      if (i < n_units) {
        if (DIR == 0)
          __builtin_nontemporal_store(val[r], dst + other[r]);
        else
          __builtin_nontemporal_store(val[r], dst + i);
      }
    }
  }
}

template <typename U>
hipError_t run(const void* src, void* dst, int64_t n_tok, int32_t deg, int64_t run_bytes, int dir,
               hipStream_t stream) {
  const int64_t upc = run_bytes / int64_t(sizeof(U));
  const int64_t units_per_tok = upc * deg;
  // each launch covers a token range whose unit count fits 31 bits
  const int64_t max_units = int64_t(1) << 30;
  int64_t tok_per_launch = std::max<int64_t>(1, max_units / units_per_tok);
  const FastDiv fu{uint32_t(upc)}, fd{uint32_t(deg)};
  int dev = 0;
  (void)hipGetDevice(&dev);
  int n_cu = 256;
  (void)hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  for (int64_t t0 = 0; t0 < n_tok; t0 += tok_per_launch) {
    const int64_t nt = std::min(tok_per_launch, n_tok - t0);
    const uint32_t n_units = uint32_t(nt * units_per_tok);
    const int64_t want = (int64_t(n_units) + kThreads * kIlp - 1) / (kThreads * kIlp);
    const int blocks = int(std::max<int64_t>(1, std::min<int64_t>(want, int64_t(n_cu) * 16)));
    // the [n, H, d] side is offset to this token range; the other side is indexed globally
    ProfScope prof(dir == 0 ? "sp_seq2head" : "sp_head2seq", stream);
    if (dir == 0) {
      const U* s = reinterpret_cast<const U*>(src) + t0 * units_per_tok;
      hipLaunchKernelGGL((sp_permute_kernel<U, 0>), dim3(blocks), dim3(kThreads), 0, stream, s,
                         reinterpret_cast<U*>(dst), n_units, fu, fd, uint32_t(t0), uint32_t(n_tok));
    } else {
      U* d = reinterpret_cast<U*>(dst) + t0 * units_per_tok;
      hipLaunchKernelGGL((sp_permute_kernel<U, 1>), dim3(blocks), dim3(kThreads), 0, stream,
                         reinterpret_cast<const U*>(src), d, n_units, fu, fd, uint32_t(t0),
                         uint32_t(n_tok));
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_sp_permute(const void* src, void* dst, int64_t n_tokens, int32_t n_heads,
                             int32_t head_dim, int32_t sp_degree, int32_t elem_bytes, int dir,
                             hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  const int64_t run_bytes = int64_t(n_heads / sp_degree) * head_dim * elem_bytes;
  const uintptr_t align = reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst);
  auto fits = [&](int64_t u) { return run_bytes % u == 0 && (align % uintptr_t(u)) == 0; };
  if (fits(16)) return run<unit16>(src, dst, n_tokens, sp_degree, run_bytes, dir, stream);
  if (fits(8)) return run<unit8>(src, dst, n_tokens, sp_degree, run_bytes, dir, stream);
  if (fits(4)) return run<uint32_t>(src, dst, n_tokens, sp_degree, run_bytes, dir, stream);
  return run<uint16_t>(src, dst, n_tokens, sp_degree, run_bytes, dir, stream);
}

}  // namespace vl
