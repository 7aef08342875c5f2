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

#include "common.h"
#include "fastdiv.h"
#include "launch.h"
#include "profiler.h"

namespace vl {

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t unit16;
typedef __attribute__((ext_vector_type(2))) uint32_t unit8;

constexpr int kThreads = 256;
constexpr int kIlp = 1;  // units per thread per grid-stride step

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
  for (int64_t t0 = 0; t0 < n_tok; t0 += tok_per_launch) {
    const int64_t nt = std::min(tok_per_launch, n_tok - t0);
    const uint32_t n_units = uint32_t(nt * units_per_tok);
    // one unit per thread: many small workgroups keep more copies in flight
    // than a capped grid-stride loop (measured 78 % against 68 % of HBM peak)
    const int64_t want = (int64_t(n_units) + kThreads * kIlp - 1) / (kThreads * kIlp);
    const int blocks = int(std::max<int64_t>(1, want));
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

namespace {

// ---------------------------------------------------------------------------
// Q, K and V of one Ulysses exchange in a single launch, with the kv-head
// split of grouped-query attention: rank p holds query heads
// [p Hq/P, (p+1) Hq/P) after the exchange, and so needs the kv heads those
// read (query head h reads kv head h Hkv / Hq).  With Hkv >= P that is
// Hkv/P heads of its own; with Hkv < P it is one head that P/Hkv ranks share,
// sent to each of them, and the gradients coming back for it are summed in
// increasing rank order in fp32.
//
// One run is the hs heads (hs = H/P, or 1 under replication) of one token for
// one rank.  A segment (Q, K or V) is described by the run length in units,
// the runs per token of its [n, H, d] side (rpt = H/hs) and rep, the ranks
// that hold each run.  Both directions walk the [n, H, d] side linearly (fully
// coalesced); run c of token t belongs to ranks c rep .. c rep + rep - 1, so
// the pack stores it rep times and the unpack loads and sums rep copies.
// ---------------------------------------------------------------------------

struct QkvSeg {
  const uint32_t* src;
  uint32_t* dst;
  uint32_t n_units;   // units of the [n, H, d] side in this launch's token range
  FastDiv upr;        // units per run
  FastDiv rpt_div;    // runs per token on the [n, H, d] side
  uint32_t rpt, rep;  // runs per token; ranks holding one run
  uint32_t blk0, blk1;
};

struct QkvArgs {
  QkvSeg seg[3];
  uint32_t t0, n_tok;
};

template <typename U>
struct UnitWords;
template <> struct UnitWords<unit16> { static constexpr int n = 4; };
template <> struct UnitWords<unit8> { static constexpr int n = 2; };
template <> struct UnitWords<uint32_t> { static constexpr int n = 1; };

template <typename U>
__device__ __forceinline__ uint32_t word(const U& u, int w) {
  if constexpr (UnitWords<U>::n == 1) return u;
  else return u[w];
}
template <typename U>
__device__ __forceinline__ void set_word(U& u, int w, uint32_t x) {
  if constexpr (UnitWords<U>::n == 1) u = x;
  else u[w] = x;
}

// acc (2 floats per word: bf16 lanes, or 1 float per word: fp32) += unit
template <typename U, bool BF16>
__device__ __forceinline__ void acc_add(float (&acc)[2 * UnitWords<U>::n], const U& u, bool first) {
#pragma unroll
  for (int w = 0; w < UnitWords<U>::n; ++w) {
    const uint32_t x = word(u, w);
    if constexpr (BF16) {
      acc[2 * w] = first ? bf16_lo(x) : acc[2 * w] + bf16_lo(x);
      acc[2 * w + 1] = first ? bf16_hi(x) : acc[2 * w + 1] + bf16_hi(x);
    } else {
      acc[w] = first ? __uint_as_float(x) : acc[w] + __uint_as_float(x);
    }
  }
}

template <typename U, bool BF16>
__device__ __forceinline__ U acc_pack(const float (&acc)[2 * UnitWords<U>::n]) {
  U u;
#pragma unroll
  for (int w = 0; w < UnitWords<U>::n; ++w) {
    if constexpr (BF16) set_word(u, w, pack_bf16x2(acc[2 * w], acc[2 * w + 1]));
    else set_word(u, w, __float_as_uint(acc[w]));
  }
  return u;
}

template <typename U, int DIR, bool BF16>
__global__ void __launch_bounds__(kThreads)
sp_qkv_kernel(QkvArgs a) {
  const uint32_t b = blockIdx.x;
  const int si = b < a.seg[0].blk1 ? 0 : (b < a.seg[1].blk1 ? 1 : 2);
  const QkvSeg& sg = a.seg[si];
  const U* __restrict__ src = reinterpret_cast<const U*>(sg.src);
  U* __restrict__ dst = reinterpret_cast<U*>(sg.dst);
  const uint32_t upr = sg.upr.d, rep = sg.rep;
  // unit i of the [n, H, d] side of this launch's token range is unit x0 + i
  // of the tensor; its run c of token t lives on ranks c rep .. c rep + rep - 1
  const uint64_t x0 = uint64_t(a.t0) * sg.rpt * upr;
  const uint64_t rank_stride = uint64_t(a.n_tok) * upr;
  const uint32_t stride = (sg.blk1 - sg.blk0) * kThreads * kIlp;
  for (uint32_t base = (b - sg.blk0) * kThreads * kIlp + threadIdx.x; base < sg.n_units;
       base += stride) {
    uint64_t y0[kIlp];
    U val[kIlp];
#pragma unroll
    for (int r = 0; r < kIlp; ++r) {
      const uint32_t i = base + r * kThreads;
      if (i < sg.n_units) {
        const uint32_t run = sg.upr.div(i);
        const uint32_t off = i - run * upr;
        const uint32_t tt = sg.rpt_div.div(run);
        const uint32_t c = run - tt * sg.rpt;
        y0[r] = (uint64_t(c) * rep * a.n_tok + a.t0 + tt) * upr + off;
        val[r] = __builtin_nontemporal_load(src + (DIR == 0 ? x0 + i : y0[r]));
      }
    }
    if constexpr (DIR == 0) {
      // pack: the run goes to each rank that reads it
      for (uint32_t k = 0; k < rep; ++k) {
#pragma unroll
        for (int r = 0; r < kIlp; ++r)
          if (base + r * kThreads < sg.n_units)
            __builtin_nontemporal_store(val[r], dst + y0[r] + k * rank_stride);
      }
    } else {
      if (rep > 1) {
        // unpack: sum over the ranks that held the run, in increasing rank order
        float acc[kIlp][2 * UnitWords<U>::n];
#pragma unroll
        for (int r = 0; r < kIlp; ++r) acc_add<U, BF16>(acc[r], val[r], true);
        for (uint32_t k = 1; k < rep; ++k) {
#pragma unroll
          for (int r = 0; r < kIlp; ++r)
            if (base + r * kThreads < sg.n_units)
              val[r] = __builtin_nontemporal_load(src + y0[r] + k * rank_stride);
#pragma unroll
          for (int r = 0; r < kIlp; ++r) acc_add<U, BF16>(acc[r], val[r], false);
        }
#pragma unroll
        for (int r = 0; r < kIlp; ++r) val[r] = acc_pack<U, BF16>(acc[r]);
      }
#pragma unroll
      for (int r = 0; r < kIlp; ++r) {
        const uint32_t i = base + r * kThreads;
        if (i < sg.n_units) __builtin_nontemporal_store(val[r], dst + x0 + i);
      }
    }
  }
}

template <typename U>
hipError_t run_qkv(const QkvTensors& t, int64_t n_tok, int32_t hq, int32_t hkv, int32_t d,
                   int32_t deg, int32_t elem_bytes, bool bf16, int dir, hipStream_t stream) {
  const int64_t head_units = int64_t(d) * elem_bytes / int64_t(sizeof(U));
  struct Geo { int64_t upr, rpt, rep; };
  auto geo = [&](int32_t H) {
    const int64_t hs = H >= deg ? H / deg : 1;
    return Geo{hs * head_units, H / hs, H >= deg ? 1 : deg / H};
  };
  const Geo g[3] = {geo(hq), geo(hkv), geo(hkv)};
  // units per token of the [n, H, d] side that both directions walk
  int64_t per_tok[3];
  for (int s = 0; s < 3; ++s) per_tok[s] = g[s].rpt * g[s].upr;
  const int64_t widest = std::max(per_tok[0], per_tok[1]);
  const int64_t tok_per_launch = std::max<int64_t>(1, (int64_t(1) << 30) / widest);
  const void* srcs[3] = {t.src[0], t.src[1], t.src[2]};
  void* dsts[3] = {t.dst[0], t.dst[1], t.dst[2]};
  for (int64_t t0 = 0; t0 < n_tok; t0 += tok_per_launch) {
    const int64_t nt = std::min(tok_per_launch, n_tok - t0);
    QkvArgs a;
    a.t0 = uint32_t(t0);
    a.n_tok = uint32_t(n_tok);
    int64_t total = 0, units[3];
    for (int s = 0; s < 3; ++s) total += (units[s] = nt * per_tok[s]);
    // blocks in proportion to each segment's units, one unit per thread
    const int64_t want = (total + kThreads * kIlp - 1) / (kThreads * kIlp);
    const int64_t blocks = std::max<int64_t>(3, want);
    uint32_t b0 = 0;
    for (int s = 0; s < 3; ++s) {
      QkvSeg& sg = a.seg[s];
      sg.src = reinterpret_cast<const uint32_t*>(srcs[s]);
      sg.dst = reinterpret_cast<uint32_t*>(dsts[s]);
      sg.n_units = uint32_t(units[s]);
      sg.upr = FastDiv(uint32_t(g[s].upr));
      sg.rpt_div = FastDiv(uint32_t(g[s].rpt));
      sg.rpt = uint32_t(g[s].rpt);
      sg.rep = uint32_t(g[s].rep);
      const int64_t nb = std::max<int64_t>(1, (blocks * units[s] + total - 1) / total);
      sg.blk0 = b0;
      sg.blk1 = b0 + uint32_t(nb);
      b0 = sg.blk1;
    }
    ProfScope prof(dir == 0 ? "sp_qkv_seq2head" : "sp_qkv_head2seq", stream);
    if (dir == 0)
      hipLaunchKernelGGL((sp_qkv_kernel<U, 0, false>), dim3(b0), dim3(kThreads), 0, stream, a);
    else if (bf16)
      hipLaunchKernelGGL((sp_qkv_kernel<U, 1, true>), dim3(b0), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL((sp_qkv_kernel<U, 1, false>), dim3(b0), dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_sp_qkv(const QkvTensors& t, int64_t n_tokens, int32_t n_heads_q,
                         int32_t n_heads_kv, int32_t head_dim, int32_t sp_degree, int32_t dtype,
                         int dir, hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  const int32_t eb = dtype == 0 ? 2 : 4;
  const bool bf16 = dtype == 0;
  uintptr_t align = 0;
  for (int s = 0; s < 3; ++s)
    align |= reinterpret_cast<uintptr_t>(t.src[s]) | reinterpret_cast<uintptr_t>(t.dst[s]);
  const int64_t head_bytes = int64_t(head_dim) * eb;
  auto fits = [&](int64_t u) { return head_bytes % u == 0 && (align % uintptr_t(u)) == 0; };
  if (fits(16))
    return run_qkv<unit16>(t, n_tokens, n_heads_q, n_heads_kv, head_dim, sp_degree, eb, bf16, dir,
                           stream);
  if (fits(8))
    return run_qkv<unit8>(t, n_tokens, n_heads_q, n_heads_kv, head_dim, sp_degree, eb, bf16, dir,
                          stream);
  return run_qkv<uint32_t>(t, n_tokens, n_heads_q, n_heads_kv, head_dim, sp_degree, eb, bf16, dir,
                           stream);
}

}  // namespace vl
