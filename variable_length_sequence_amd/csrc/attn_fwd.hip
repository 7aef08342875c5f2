// Forward attention over packed variable-length documents on gfx950.
//
// Computes O = softmax(scale Q K^T) V and LSE per query, each query seeing
// only the keys of its own document (HSAP page, Section 2.1, cu_len; NSP page,
// Section 2.2) and, if causal, only keys at or before its position.  The
// softmax is evaluated online over key tiles, so the score matrix is never
// stored (BASP page, Section II-A on tiling and online softmax; HSAP page,
// Section 2.2.1).
//
// Mapping (one workgroup = one work item x one q head; 4 waves):
//   * a work item is a 128-row query tile of one document plus the number of
//     64-row key tiles it needs (tiles past the causal diagonal are never
//     listed); the kernel runs them as 32-key tiles, skipping a last half
//     that no query of the item sees;  wave w owns query rows 32w .. 32w+31;
//   * three workgroups share a compute unit (48 KB of LDS and at most 168
//     VGPRs each), so each SIMD interleaves three waves: a third wave hides
//     more of each wave's softmax and load latency than pairing matrix and
//     vector work inside one wave did with 64-key tiles at two waves;
//   * scores are computed transposed, S^T = K Q^T, on 32x32x16 bf16 MFMAs, so
//     each lane owns one query (its column) and row statistics need only one
//     exchange with the other half-wave;
//   * the key rows of the MFMA A operand are permuted (bits 2 and 3 of the row
//     swapped) so that the fp32 S^T values a lane holds are, after rounding
//     P to bf16, exactly the B operand of O^T += V^T P^T with no shuffles;
//   * K and V tiles are staged in LDS row-major with XOR-swizzled 16-byte
//     chunks; the V^T operand is read with the gfx950 transpose read
//     (ds_read_b64_tr_b16), so no transposed copy is stored; tiles are
//     double-buffered and filled by direct global->LDS loads issued one tile
//     ahead (one barrier per tile, no staging registers); the tile loop is
//     unrolled by two so both buffers have fixed addresses;
//   * the Q tile also arrives by direct loads (whole rows, into the second
//     key buffer and a third one beside it) and each wave reads its Q
//     fragments from LDS; the epilogue stages each wave's 32 x D block of O in LDS and writes
//     whole rows of 16-byte chunks (both replace scattered 16- and 8-byte
//     accesses of 32 rows per instruction);
//   * work items are ordered longest first and the workgroup id is remapped
//     so all q heads of one item run on the same XCD (shared K/V in its L2).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "launch.h"
#include "profiler.h"

namespace vl {

namespace {

constexpr int BQ = kFwdBQ;  // 128
constexpr int BK = kFwdBK / 2;   // 32 keys per tile (the work lists count 64-key tiles)
constexpr int kThreads = 256;

template <int D>
struct FwdSmem {
  // [buffer][K, V]: double-buffered K and V tiles (buffers 0 and 1),
  // row-major with swizzled chunks; key row r is kept at LDS row
  // swap_bits23(r) (the row order the MFMA operands want).  Buffers 1 and 2
  // (64 rows each) take the Q tile before the loop; buffer 2 and the buffer
  // the last key tile did not use stage the epilogue.
  uint16_t kv[3][2][BK * D];
};

// OUT: kOutBf16 / kOutF32 write O and LSE; kOutAcc folds them into fp32
// running (O, LSE) accumulators (see the epilogue).
template <int D, int OUT>
__global__ void __launch_bounds__(kThreads, 3)
attn_fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                const uint16_t* __restrict__ v, const DevItem* __restrict__ items,
                int hq, int hkv, float scale, int causal,
                void* __restrict__ out,
                float* __restrict__ lse, int64_t total_q) {
  constexpr int NKS = D / 16;  // k-steps over the head dim
  constexpr int NCB = D / 32;  // 32-wide blocks of the head dim
  __shared__ FwdSmem<D> sm;

  // workgroup -> (item, head): XCD b % 8 runs its own item list, longest
  // first, and all heads of one item stay on that XCD (shared K/V in its L2)
  const int b = blockIdx.x;
  const int xcd = b & (kXcds - 1);
  const int r = b / kXcds;
  const DevItem it = items[(r / hq) * kXcds + xcd];
  const int h = __builtin_amdgcn_readfirstlane(r % hq);
  if (it.n_slices == 0) return;   // empty slot
  const int g = __builtin_amdgcn_readfirstlane(h / (hq / hkv));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int lq = it.lq, lk = it.lk;
  const int q0 = it.tile * BQ;
  const int qrow = q0 + w * 32 + l32;        // doc-relative query row of this lane
  const int off = lk - lq;                   // causal diagonal offset
  const int64_t q_tok = int64_t(hq) * D;
  const int64_t kv_tok = int64_t(hkv) * D;
  const float c = scale * kLog2e;

  // The Q tile arrives by direct loads into LDS buffers 1 (rows 0-63; free
  // until the prefetch of key tile 1) and 2 (rows 64-127); rows past the
  // document repeat its last row.
  load_rows128_lds<D>(q + (int64_t(it.q_start) + q0) * q_tok + int64_t(h) * D, uint32_t(q_tok * 2),
                      lq - q0, lds_addr(sm.kv[1][0]), lds_addr(sm.kv[2][0]), w, lane);

  bf16x8 qf[NKS];
  f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[cb][i] = 0.f;
  float m_run = -INFINITY;  // reference max of raw scores of this lane's query
  float l_run = 0.f;        // running sum (this half-wave's keys)

  const uint16_t* kbase = k + int64_t(it.k_start) * kv_tok + int64_t(g) * D;
  const uint16_t* vbase = v + int64_t(it.k_start) * kv_tok + int64_t(g) * D;
  const PairLoader<D, BK, kThreads / 64> loader(w, lane, uint32_t(kv_tok * 2));
  // the next key tile to load, advanced by one tile per tile
  const int64_t kv_step = int64_t(BK) * kv_tok;
  const uint16_t* knext = kbase + kv_step;
  const uint16_t* vnext = vbase + kv_step;

  // first and last query rows of this wave (for skipping / masking)
  const int wq_first = q0 + w * 32;
  const int wq_last = min(q0 + w * 32 + 31, lq - 1);
  // 32-key tiles this item needs: up to the last key its last query sees
  const int last_q = min(q0 + BQ, lq) - 1;
  const int kend = causal ? min(lk, last_q + off + 1) : lk;
  const int n_kv = kend > 0 ? min(2 * it.count, (kend + BK - 1) / BK) : 0;

  // one key tile; the buffer index is a compile-time constant so every LDS
  // address is a loop-invariant register plus an immediate offset
  auto tile = [&](int kt, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int kv0 = kt * BK;
    // tile kt has landed in every wave's part of buffer `buf`, and every wave
    // is done with the other buffer (read during tile kt - 1)
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    __syncthreads();
    if (kt + 1 < n_kv) {
      loader.load_from(knext, vnext, lk - kv0 - BK, uint32_t(kv_tok * 2), lds_addr(sm.kv[buf ^ 1][0]),
                       lds_addr(sm.kv[buf ^ 1][1]), w, lane);
      knext += kv_step;
      vnext += kv_step;
    }
    const uint16_t* ks = sm.kv[buf][0];
    const uint16_t* vs = sm.kv[buf][1];

    // wave-uniform: skip tiles no query of this wave can see
    const bool wave_live = (wq_first < lq) && (!causal || kv0 <= wq_last + off);
    if (!wave_live) return;
    const bool need_mask = (kv0 + BK > lk) || (causal && kv0 + BK - 1 > wq_first + off);
    // key kv0 + 8 half + e (e = 16 (i / 8) + i % 8) of S^T is visible iff
    // e <= lim - kv0 - 8 half
    const int lim = causal ? min(lk - 1, qrow + off) : lk - 1;
    auto mask = [&](f32x16& x) {
      const int thr = lim - kv0 - 8 * half;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (16 * (i >> 3) + (i & 7) > thr) x[i] = -INFINITY;
    };

    // A tile: S^T = K Q^T (8 MFMAs at d = 128), the softmax, O^T += V^T P^T
    // (8 MFMAs).  K fragments of the score chain are read two ahead and the
    // V^T fragments of the output chain two ahead, the first two before the
    // softmax; the other waves of the SIMD fill the gaps.
    auto kfrag = [&](int f) {
      return as_bf16x8(*reinterpret_cast<const u32x4*>(&ks[SwzTile<D>::chunk(l32, 2 * f + half)]));
    };
    // V^T operand of step j (keys 16 j .. 16 j + 15): dims 32 cb + l32
    auto vfrag = [&](int cb, int j) { return tr_frag<D>(vs, lane, 16 * j, 32 * cb); };

    // softmax of the tile: P (bf16, two 16-key steps), the reference max and
    // the tile's row sum; returns whether the reference max moved
    float m_use = m_run, psum = 0.f;
    auto softmax = [&](const f32x16& x, bf16x8* p) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, x[i]);
      mx = halves_max(mx);
      // m_run is the reference max of the exponent.  It moves (and O and l
      // are rescaled) only when the running max exceeds it by more than 2^8
      // in probability, so p <= 256 and most tiles skip the rescale.
      const float m_new = fmaxf(m_run, mx);
      const bool grow = (m_new - m_run) * c > 8.f;   // false while both are -inf
      m_use = grow ? m_new : m_run;
      const float mc = (m_use == -INFINITY) ? 0.f : m_use * c;
      psum = 0.f;
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        u32x4 u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(x[8 * hs + 2 * e], c, -mc));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(x[8 * hs + 2 * e + 1], c, -mc));
          psum += p0 + p1;
          u[e] = pack_bf16x2(p0, p1);
        }
        p[hs] = as_bf16x8(u);
      }
      return grow;
    };
    // A lane that has seen no visible key yet holds O = 0 and l = 0, so its
    // first reference max needs no rescale (the first tile of every item).
    auto commit = [&](bool grow) {
      const bool scale_acc = grow && m_run != -INFINITY;
      if (__ballot(scale_acc)) {
        const float alpha = scale_acc ? __builtin_amdgcn_exp2f((m_run - m_use) * c) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[cb][i] *= alpha;
      }
      m_run = m_use;
      l_run += psum;
    };

    constexpr int kPf = 2;   // K fragments in flight
    constexpr int kVa = 2;   // V^T fragments in flight
    bf16x8 kr[kPf];
    // The score chain is fenced step by step: with only instruction kinds
    // pinned, the scheduler filled its read slots with later reads and sank
    // each K read to just before its MFMA.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < kPf; ++f) kr[f] = kfrag(f);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 st;
#pragma unroll
    for (int f = 0; f < NKS; ++f) {
      const bf16x8 a = kr[f % kPf];
      st = mfma32(a, qf[f], f == 0 ? f32x16{} : st);
      if (f + kPf < NKS) kr[f % kPf] = kfrag(f + kPf);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (need_mask) mask(st);
    // O^T += V^T P^T: MFMA i takes V^T fragment (cb, j) = (i % NCB, i / NCB)
    bf16x8 vr[kVa];
#pragma unroll
    for (int i = 0; i < kVa; ++i) vr[i] = vfrag(i % NCB, i / NCB);
    bf16x8 pt[2];
    commit(softmax(st, pt));
#pragma unroll
    for (int i = 0; i < 2 * NCB; ++i) {
      acc[i % NCB] = mfma32(vr[i % kVa], pt[i / NCB], acc[i % NCB]);
      if (i + kVa < 2 * NCB) vr[i % kVa] = vfrag((i + kVa) % NCB, (i + kVa) / NCB);
    }
  };

  if (n_kv > 0)
    loader.load(kbase, vbase, kv_tok, 0, lk, lds_addr(sm.kv[0][0]), lds_addr(sm.kv[0][1]), w, lane);
  // Q fragments (B operand of S^T = K Q^T): query l32, dims 16s + 8 half .. +8
  __builtin_amdgcn_s_waitcnt(kWaitAll);
  __syncthreads();
  {
    const int row = w * 32 + l32;
    const uint16_t* qs = row < 64 ? sm.kv[1][0] : sm.kv[2][0];
#pragma unroll
    for (int s = 0; s < NKS; ++s)
      qf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(&qs[SwzTile<D>::chunk(row & 63, 2 * s + half)]));
  }
  int kt = 0;
  for (; kt + 1 < n_kv; kt += 2) {
    tile(kt, IC<0>{});
    tile(kt + 1, IC<1>{});
  }
  if (kt < n_kv) tile(kt, IC<0>{});

  // epilogue: O = acc / l, LSE = m scale + ln l
  const float l_tot = halves_sum(l_run);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if constexpr (OUT == kOutBf16) {
    // each wave stages its 32 x D block of O in LDS and writes whole rows of
    // 16-byte chunks (chunk c of row r sits at chunk c ^ (r % (D / 8))).  The
    // staging goes to buffer 2 (waves 2, 3) and to the K/V buffer the last
    // key tile did not use (waves 0, 1): every wave is done with both since
    // that tile's barrier and no load went into them, so no wave waits for
    // the others here, except in an item without key tiles, whose Q
    // fragments other waves may still be reading from buffer 2.
    const int fb = n_kv & 1;
    if (n_kv == 0) __syncthreads();
    uint32_t* stg = reinterpret_cast<uint32_t*>(w < 2 ? &sm.kv[fb][0][0] : &sm.kv[2][0][0]) +
                    (w & 1) * (32 * D / 2);
    constexpr int RCH = D / 8;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int cc = 4 * cb + gq;
        const u32x2 o2{pack_bf16x2(acc[cb][4 * gq] * inv, acc[cb][4 * gq + 1] * inv),
                       pack_bf16x2(acc[cb][4 * gq + 2] * inv, acc[cb][4 * gq + 3] * inv)};
        *reinterpret_cast<u32x2*>(&stg[l32 * (D / 2) + ((cc ^ (l32 & (RCH - 1))) << 2) + 2 * half]) = o2;
      }
    constexpr int RPI = 64 / RCH;
    const int64_t orow0 = (int64_t(it.q_start) + q0 + w * 32) * q_tok + int64_t(h) * D;
    uint16_t* outp = reinterpret_cast<uint16_t*>(out);
#pragma unroll
    for (int t = 0; t < 32 / RPI; ++t) {
      const int r = t * RPI + lane / RCH, cc = lane % RCH;
      const u32x4 x = *reinterpret_cast<const u32x4*>(&stg[r * (D / 2) + ((cc ^ (r & (RCH - 1))) << 2)]);
      if (q0 + w * 32 + r < lq)
        *reinterpret_cast<u32x4*>(outp + orow0 + int64_t(r) * q_tok + 8 * cc) = x;
    }
    if (qrow < lq && half == 0) {
      const int64_t lrow = int64_t(h) * total_q + it.q_start + qrow;
      lse[lrow] = (l_tot > 0.f) ? (m_run * scale + __logf(l_tot)) : -INFINITY;
    }
  } else if (qrow < lq) {
    const int64_t orow = (int64_t(it.q_start) + qrow) * q_tok + int64_t(h) * D;
    const int64_t lrow = int64_t(h) * total_q + it.q_start + qrow;
    const float lv = (l_tot > 0.f) ? (m_run * scale + __logf(l_tot)) : -INFINITY;
    if constexpr (OUT == kOutAcc) {
      // Fold this key chunk's (O, LSE) into the running pair (the online
      // combination of ring attention: HSAP page, Section 2.2.1, with its
      // rescale step done here instead of in a separate pass, Section 3.1):
      // M = max(LSE_a, LSE), w = exp(. - M), O_a = (w_a O_a + w O) / (w_a + w),
      // LSE_a = M + ln(w_a + w).  Two -inf LSEs leave the pair unchanged.
      float* oa = reinterpret_cast<float*>(out);
      const float la = lse[lrow];
      const float mm = fmaxf(la, lv);
      float ca = 1.f, cn = 0.f, ln = la;
      if (mm != -INFINITY) {
        const float wa = __expf(la - mm), wn = __expf(lv - mm);
        const float rden = 1.f / (wa + wn);
        ca = wa * rden;
        cn = wn * rden * inv;
        ln = mm + __logf(wa + wn);
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int cc = cb * 32 + 8 * gq + 4 * half;
          f32x4 o4 = *reinterpret_cast<const f32x4*>(oa + orow + cc);
#pragma unroll
          for (int j = 0; j < 4; ++j) o4[j] = fmaf(ca, o4[j], cn * acc[cb][4 * gq + j]);
          *reinterpret_cast<f32x4*>(oa + orow + cc) = o4;
        }
      // the one load of LSE_a above (both half-waves) precedes this store
      if (half == 0) lse[lrow] = ln;
    } else {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int cc = cb * 32 + 8 * gq + 4 * half;
          if constexpr (OUT == kOutF32) {
            f32x4 o4;
#pragma unroll
            for (int j = 0; j < 4; ++j) o4[j] = acc[cb][4 * gq + j] * inv;
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + orow + cc) = o4;
          } else {
            u32x2 o2;
            o2[0] = pack_bf16x2(acc[cb][4 * gq] * inv, acc[cb][4 * gq + 1] * inv);
            o2[1] = pack_bf16x2(acc[cb][4 * gq + 2] * inv, acc[cb][4 * gq + 3] * inv);
            *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + orow + cc) = o2;
          }
        }
      if (half == 0) lse[lrow] = lv;
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd(const AttnShape& s, const void* q, const void* k, const void* v,
                           const ItemMap& map, int32_t out_kind, void* out, float* lse,
                           hipStream_t stream) {
  if (map.rows == 0) return hipSuccess;
  const dim3 grid(unsigned(map.rows) * unsigned(kXcds) * unsigned(s.hq));
  const auto* qq = reinterpret_cast<const uint16_t*>(q);
  const auto* kk = reinterpret_cast<const uint16_t*>(k);
  const auto* vv = reinterpret_cast<const uint16_t*>(v);
  ProfScope prof("attn_fwd", stream);
#define VL_FWD(DD, OUTK)                                                                       \
  hipLaunchKernelGGL((attn_fwd_kernel<DD, OUTK>), grid, dim3(kThreads), 0, stream, qq, kk, vv,  \
                     map.items, s.hq, s.hkv, s.scale, s.causal, out, lse, s.total_q)
  if (s.d == 128) {
    if (out_kind == kOutAcc) VL_FWD(128, kOutAcc);
    else if (out_kind == kOutF32) VL_FWD(128, kOutF32);
    else VL_FWD(128, kOutBf16);
  } else {
    if (out_kind == kOutAcc) VL_FWD(64, kOutAcc);
    else if (out_kind == kOutF32) VL_FWD(64, kOutF32);
    else VL_FWD(64, kOutBf16);
  }
#undef VL_FWD
  return hipGetLastError();
}

}  // namespace vl
