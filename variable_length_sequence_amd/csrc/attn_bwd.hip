// Backward attention over packed variable-length documents on gfx950.
//
// The exact gradient of the forward (the pages do not write it out; P is
// recomputed from the saved LSE, the attention recompute the NSP page
// discusses in Sections 2.3 and 4.2.2):
//   D_i = dO_i . O_i,  P_ij = exp(S_ij - LSE_i),  dP_ij = dO_i . V_j,
//   dS_ij = P_ij (dP_ij - D_i),
//   dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij Q_i,  dQ_i = scale sum_j dS_ij K_j.
//
// Three kernels, no atomics on dQ:
//   1. bwd_pre: D = rowsum(dO * O) in fp32, [Hq, T].
//   2. dkdv: one workgroup per (128-key tile of a document, kv head[, slice of
//      its q heads]); each wave owns 32 keys and keeps their K, V operands and
//      fp32 dK, dV accumulators in registers while 32-row query tiles of every
//      q head of the group stream through LDS (row-major and transposed).
//      Scores are computed as S = Q K^T so a lane owns one key; the query rows
//      of the A operand are permuted so P and dS come out of the MFMA already
//      in the A-operand layout of dV += P^T dO and dK += dS^T Q.
//   3. dq: the forward's mapping (a lane owns one query): S^T = K Q^T and
//      dP^T = V dO^T per 64-key tile, then dQ^T += K^T dS^T.
// The extra two contractions of (3) replace a zeroed fp32 dQ accumulator, its
// atomics and a conversion pass, and keep dQ deterministic.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "launch.h"
#include "profiler.h"

namespace vl {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- D = rowsum(dO O)
template <int D>
__global__ void __launch_bounds__(kThreads)
bwd_pre_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
               float* __restrict__ delta, int64_t total_q, int hq) {
  constexpr int LPR = D / 8;                 // lanes per (row, head)
  constexpr int RPB = kThreads / LPR;        // rows per block
  const int sub = threadIdx.x / LPR;
  const int c8 = threadIdx.x % LPR;
  const int64_t n_pairs = total_q * hq;
  for (int64_t pr = int64_t(blockIdx.x) * RPB + sub; pr < n_pairs;
       pr += int64_t(gridDim.x) * RPB) {
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(o + pr * D + c8 * 8));
    const u32x4 b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dout + pr * D + c8 * 8));
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = fmaf(bf16_lo(a[j]), bf16_lo(b[j]), acc);
      acc = fmaf(bf16_hi(a[j]), bf16_hi(b[j]), acc);
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if (c8 == 0) {
      const int64_t t = pr / hq;
      const int h = int(pr - t * hq);
      delta[int64_t(h) * total_q + t] = acc;
    }
  }
}

__global__ void __launch_bounds__(kThreads)
fill_zero_kernel(f32x4* __restrict__ p, int64_t n4) {
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n4;
       i += int64_t(gridDim.x) * kThreads)
    p[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// fp32 [T, H, D] accumulator -> bf16
__global__ void __launch_bounds__(kThreads)
f32_to_bf16_kernel(const f32x4* __restrict__ src, u32x2* __restrict__ dst, int64_t n4) {
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n4;
       i += int64_t(gridDim.x) * kThreads) {
    const f32x4 x = src[i];
    dst[i] = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
  }
}

// A chain of N dependent-accumulator MFMAs whose LDS operand fragment f is
// read PF fragments ahead of its use; the schedule is pinned to (MFMA, LDS
// read) pairs so the read latency hides behind the matrix pipe.
template <int N, int PF, int SYNC, typename Load, typename Mac>
__device__ __forceinline__ void mfma_chain(Load load, Mac mac) {
  bf16x8 r[PF];
#pragma unroll
  for (int f = 0; f < PF; ++f) r[f] = load(f);
#pragma unroll
  for (int f = 0; f < N; ++f) {
    const bf16x8 a = r[f % PF];
    if (f + PF < N) r[f % PF] = load(f + PF);
    mac(f, a);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, PF, SYNC);
#pragma unroll
  for (int f = 0; f < N - PF; ++f) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, SYNC);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, SYNC);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, PF, SYNC);
}

// ---------------------------------------------------------------- dK, dV
constexpr int KB_Q = kBwdBQ;   // 32 query rows per step
constexpr int KB_K = kBwdBK;   // 128 keys per workgroup
constexpr int kKvThreads = 512;

template <int D>
struct KvSmem {
  // double-buffered Q and dO tiles, row-major with swizzled chunks; query row
  // r is kept at LDS row swap_bits23(r).  The transposed operands (dO for
  // dV += P^T dO, Q for dK += dS^T Q) are read from the same tiles with the
  // transpose read.
  uint16_t q[2][KB_Q * D];
  uint16_t dout[2][KB_Q * D];
  alignas(16) float lse2[2][KB_Q];
  alignas(16) float delta[2][KB_Q];
};

// Direct global->LDS loads of a tile of `ROWS` rows of two [T, H, D] tensors
// (same rows of both), spread over the NW waves of a workgroup.  The lane
// that lands on LDS row p, chunk pc fetches source row swap_bits23(p), chunk
// pc ^ swz(p); rows at or past `n_valid` are clamped to the last valid row
// (those rows are masked out wherever they are used).
template <int D, int ROWS, int NW>
__device__ __forceinline__ void issue_pair(uint16_t* dst_a, uint16_t* dst_b,
                                           const uint16_t* __restrict__ src_a,
                                           const uint16_t* __restrict__ src_b,
                                           int64_t tok_stride, int row0, int n_valid, int wave,
                                           int lane) {
  constexpr int NCH = D / 8;
  constexpr int RPL = 64 / NCH;                // rows per wave load (1 KB)
  constexpr int BLKS = ROWS / RPL;             // 1 KB blocks per tensor
#pragma unroll
  for (int blk = wave; blk < BLKS; blk += NW) {
    const int p = blk * RPL + lane / NCH;
    const int pc = lane % NCH;
    const int row = min(row0 + swap_bits23(p), n_valid - 1);
    const int64_t o = int64_t(row) * tok_stride + ((pc ^ SwzTile<D>::swz(p)) << 3);
    load_lds16(src_a + o, dst_a + blk * 512);
    load_lds16(src_b + o, dst_b + blk * 512);
  }
}

// 8 waves: waves 0-3 accumulate dV, waves 4-7 dK, for the same four 32-key
// blocks (wave w and w + 4 share block w & 3 and, being w apart by 4, the same
// SIMD).  Both roles recompute S = Q K^T; the dV role then needs only
// P^T dO, the dK role dP = dO V^T and dS^T Q.  Splitting the roles halves the
// accumulators a wave holds, so two waves fit per SIMD and one wave's
// exponentials overlap the other's MFMAs.
template <int D>
__global__ void __launch_bounds__(kKvThreads)
attn_bwd_dkdv_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                     const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                     const float* __restrict__ lse, const float* __restrict__ delta,
                     const DevItem* __restrict__ items, int n_items, int hq, int hkv,
                     int head_split, float scale, int causal, int64_t total_q,
                     uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                     float* __restrict__ dkv_acc, int64_t total_k) {
  constexpr int NKS = D / 16;
  constexpr int NCB = D / 32;
  __shared__ KvSmem<D> sm;

  const int b = blockIdx.x;
  const int xcd = b & 7;
  const int r = b >> 3;
  const int per_item = hkv * head_split;
  const int item_idx = (r / per_item) * 8 + xcd;
  const int g = (r % per_item) / head_split;
  const int split = r % head_split;
  if (item_idx >= n_items) return;
  const DevItem it = items[item_idx];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int role = wave >> 2;                  // 0: dV, 1: dK
  const int w = wave & 3;                      // key block
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int lq = it.lq, lk = it.lk;
  const int off = lk - lq;
  const int j0 = it.tile * KB_K;               // first key of the tile (doc-relative)
  const int key = j0 + w * 32 + l32;           // this lane's key
  const int64_t q_tok = int64_t(hq) * D;
  const int64_t kv_tok = int64_t(hkv) * D;
  const float c = scale * kLog2e;
  const int grp = hq / hkv;
  const int hpg = grp / head_split;            // q heads handled here
  const int h_begin = g * grp + split * hpg;

  // K (both roles) and V (dK role) as B operands: key l32, dims 16s + 8 half ..
  bf16x8 kf[NKS], vf[NKS];
  {
    const int64_t row = int64_t(it.k_start) + key;
    const uint16_t* kp = k + row * kv_tok + int64_t(g) * D + 8 * half;
    const uint16_t* vp = v + row * kv_tok + int64_t(g) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      u32x4 a = u32x4{0, 0, 0, 0}, bb = u32x4{0, 0, 0, 0};
      if (key < lk) {
        a = *reinterpret_cast<const u32x4*>(kp + 16 * s);
        if (role) bb = *reinterpret_cast<const u32x4*>(vp + 16 * s);
      }
      kf[s] = as_bf16x8(a);
      vf[s] = as_bf16x8(bb);
    }
  }

  f32x16 acc[NCB];                             // dV (role 0) or dK (role 1)
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[cb][i] = 0.f;

  const int wk_first = j0 + w * 32;
  const int n_steps = hpg * it.count;

  // Q/dO tiles arrive by direct global->LDS loads one step ahead; the per-row
  // LSE and D values go through registers (threads 0..31 and 64..95)
  auto issue = [&](int step, int buf) {
    const int h = h_begin + step / it.count;
    const int i0 = (it.first + step % it.count) * KB_Q;
    const int64_t hoff = int64_t(it.q_start) * q_tok + int64_t(h) * D;
    issue_pair<D, KB_Q, 8>(sm.q[buf], sm.dout[buf], q + hoff, dout + hoff, q_tok, i0, lq, wave,
                           lane);
  };
  auto fetch_rows = [&](int step) {
    const int h = h_begin + step / it.count;
    const int i0 = (it.first + step % it.count) * KB_Q;
    float x = 0.f;
    if (tid < KB_Q) {
      const int i = i0 + tid;
      x = (i < lq) ? lse[int64_t(h) * total_q + it.q_start + i] : INFINITY;
      x = (x == -INFINITY) ? INFINITY : x * kLog2e;
    } else if (tid >= 64 && tid < 64 + KB_Q) {
      const int i = i0 + tid - 64;
      x = (i < lq) ? delta[int64_t(h) * total_q + it.q_start + i] * scale : 0.f;
    }
    return x;
  };
  auto store_rows = [&](float x, int buf) {
    if (tid < KB_Q) sm.lse2[buf][tid] = x;
    else if (tid >= 64 && tid < 64 + KB_Q) sm.delta[buf][tid - 64] = x;
  };

  if (n_steps > 0) {
    issue(0, 0);
    store_rows(fetch_rows(0), 0);
  }
  for (int step = 0; step < n_steps; ++step) {
    const int i0 = (it.first + step % it.count) * KB_Q;
    const int buf = step & 1;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    float nxt = 0.f;
    if (step + 1 < n_steps) {
      issue(step + 1, buf ^ 1);
      nxt = fetch_rows(step + 1);
    }
    const uint16_t* qs = sm.q[buf];
    const uint16_t* ds = sm.dout[buf];

    // per-query LSE (and scaled D for the dK role) of this lane's 16 queries
    // 16s + 8 half + t, read before the MFMAs so their latency is hidden
    f32x4 lr[4], dr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lr[j] = *reinterpret_cast<const f32x4*>(&sm.lse2[buf][16 * (j >> 1) + 8 * half + 4 * (j & 1)]);
      dr[j] = *reinterpret_cast<const f32x4*>(&sm.delta[buf][16 * (j >> 1) + 8 * half + 4 * (j & 1)]);
    }

    // S = Q K^T (rows: queries 16s + 8 half + t; cols: this wave's keys).
    // Waves whose keys this query tile cannot see still run the step, fully
    // masked: every wave meets at the next barrier anyway.
    f32x16 sacc;
    {
      mfma_chain<NKS, 4, 0>(
          [&](int f) {
            return as_bf16x8(*reinterpret_cast<const u32x4*>(&qs[SwzTile<D>::chunk(l32, 2 * f + half)]));
          },
          [&](int f, const bf16x8& a) { sacc = mfma32(a, kf[f], f == 0 ? f32x16{} : sacc); });
    }

    // P; element i holds query qb + e, e = 16 (i / 8) + i % 8.  It is visible
    // iff e < lq - qb (a real row), key < lk, and (causal) e >= key - off - qb.
    float p[16];
    {
      const int qb = i0 + 8 * half;
      const int e_min = causal ? key - off - qb : INT32_MIN;
      const int e_cap = (key < lk) ? lq - qb : INT32_MIN;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = 16 * (i >> 3) + (i & 7);
        const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[i], c, -lr[i >> 2][i & 3]));
        p[i] = (e < e_cap && e >= e_min) ? pv : 0.f;
      }
    }

    // A operand of the accumulation: P (dV role) or dS = P (dP - D) scale (dK role)
    bf16x8 af[2];
    if (role == 0) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 u;
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] = pack_bf16x2(p[8 * s + 2 * j], p[8 * s + 2 * j + 1]);
        af[s] = as_bf16x8(u);
      }
    } else {
      f32x16 pacc;
      mfma_chain<NKS, 4, 1>(
          [&](int f) {
            return as_bf16x8(*reinterpret_cast<const u32x4*>(&ds[SwzTile<D>::chunk(l32, 2 * f + half)]));
          },
          [&](int f, const bf16x8& a) { pacc = mfma32(a, vf[f], f == 0 ? f32x16{} : pacc); });
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        u32x4 u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 8 * s + 2 * j;
          u[j] = pack_bf16x2(p[i] * fmaf(pacc[i], scale, -dr[i >> 2][i & 3]),
                             p[i + 1] * fmaf(pacc[i + 1], scale, -dr[(i + 1) >> 2][(i + 1) & 3]));
        }
        af[s] = as_bf16x8(u);
      }
    }

    // dV += P^T dO or dK += dS^T Q  (B operands read transposed)
    {
      const uint16_t* bt = role == 0 ? ds : qs;
      mfma_chain<2 * NCB, 4, 2>(
          [&](int f) { return tr_frag<D>(bt, lane, 16 * (f & 1), 32 * (f >> 1)); },
          [&](int f, const bf16x8& bfr) { acc[f >> 1] = mfma32(af[f & 1], bfr, acc[f >> 1]); });
    }
    if (step + 1 < n_steps) store_rows(nxt, buf ^ 1);
  }

  // epilogue: lane holds column c = 32 cb + l32 of keys 32 w + 8 (v/4) + 4 half + v%4
  uint16_t* outp = role == 0 ? dv : dk;
  float* accp = dkv_acc + (role == 0 ? total_k * kv_tok : 0);
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = j0 + w * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
      if (kk < lk) {
        const int64_t idx = (int64_t(it.k_start) + kk) * kv_tok + int64_t(g) * D + cb * 32 + l32;
        if (head_split == 1)
          outp[idx] = __builtin_bit_cast(uint16_t, (__bf16)acc[cb][i]);
        else
          atomicAdd(accp + idx, acc[cb][i]);
      }
    }
  }
  (void)wk_first;
}

// ---------------------------------------------------------------- dQ
constexpr int QB_Q = kFwdBQ;  // 128 queries per workgroup (4 waves x 32)
constexpr int QB_K = kFwdBK;  // 64 keys per step

template <int D>
struct QSmem {
  // double-buffered K and V tiles, row-major with swizzled chunks; key row r
  // at LDS row swap_bits23(r).  K^T for dQ^T += K^T dS^T is read with the
  // transpose read.
  uint16_t k[2][QB_K * D];
  uint16_t v[2][QB_K * D];
};

template <int D>
__global__ void __launch_bounds__(kThreads, 2)
attn_bwd_dq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                   const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                   const float* __restrict__ lse, const float* __restrict__ delta,
                   const DevItem* __restrict__ items, int n_items, int hq, int hkv, float scale,
                   int causal, int64_t total_q, uint16_t* __restrict__ dq) {
  constexpr int NKS = D / 16;
  constexpr int NCB = D / 32;
  __shared__ QSmem<D> sm;

  const int b = blockIdx.x;
  const int xcd = b & 7;
  const int r = b >> 3;
  const int item_idx = (r / hq) * 8 + xcd;
  const int h = r % hq;
  if (item_idx >= n_items) return;
  const DevItem it = items[item_idx];
  const int g = h / (hq / hkv);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int lq = it.lq, lk = it.lk;
  const int off = lk - lq;
  const int q0 = it.tile * QB_Q;
  const int qrow = q0 + w * 32 + l32;
  const int64_t q_tok = int64_t(hq) * D;
  const int64_t kv_tok = int64_t(hkv) * D;
  const float c = scale * kLog2e;

  bf16x8 qf[NKS], df[NKS];
  {
    const int64_t row = int64_t(it.q_start) + qrow;
    const uint16_t* qp = q + row * q_tok + int64_t(h) * D + 8 * half;
    const uint16_t* dp = dout + row * q_tok + int64_t(h) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      u32x4 a = u32x4{0, 0, 0, 0}, bb = u32x4{0, 0, 0, 0};
      if (qrow < lq) {
        a = *reinterpret_cast<const u32x4*>(qp + 16 * s);
        bb = *reinterpret_cast<const u32x4*>(dp + 16 * s);
      }
      qf[s] = as_bf16x8(a);
      df[s] = as_bf16x8(bb);
    }
  }
  float lse2 = INFINITY, dl = 0.f;
  if (qrow < lq) {
    const float l = lse[int64_t(h) * total_q + it.q_start + qrow];
    lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
    dl = delta[int64_t(h) * total_q + it.q_start + qrow];
  }

  f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[cb][i] = 0.f;

  const uint16_t* kbase = k + int64_t(it.k_start) * kv_tok + int64_t(g) * D;
  const uint16_t* vbase = v + int64_t(it.k_start) * kv_tok + int64_t(g) * D;
  const int wq_first = q0 + w * 32;
  const int wq_last = min(q0 + w * 32 + 31, lq - 1);

  const int n_kv = it.count;
  if (n_kv > 0) issue_pair<D, QB_K, 4>(sm.k[0], sm.v[0], kbase, vbase, kv_tok, 0, lk, w, lane);
  for (int kt = 0; kt < n_kv; ++kt) {
    const int kv0 = kt * QB_K;
    const int buf = kt & 1;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kt + 1 < n_kv)
      issue_pair<D, QB_K, 4>(sm.k[buf ^ 1], sm.v[buf ^ 1], kbase, vbase, kv_tok, kv0 + QB_K, lk, w,
                             lane);
    const uint16_t* ks = sm.k[buf];
    const uint16_t* vs = sm.v[buf];

    const bool live = (wq_first < lq) && (!causal || kv0 <= wq_last + off);
    if (!live) continue;
    const bool need_mask = (kv0 + QB_K > lk) || (causal && kv0 + QB_K - 1 > wq_first + off);

    // per 32-key half kb: S^T and dP^T (16 MFMAs), then dS^T packed to bf16;
    // one half at a time keeps only one pair of accumulators live
    const int lim = causal ? min(lk - 1, qrow + off) : lk - 1;
    bf16x8 dsf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 sa, da;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sa[i] = 0.f;
        da[i] = 0.f;
      }
      const int prow = kb * 32 + l32;
#pragma unroll
      for (int st = 0; st < NKS; ++st) {
        const int o = SwzTile<D>::chunk(prow, 2 * st + half);
        sa = mfma32(as_bf16x8(*reinterpret_cast<const u32x4*>(&ks[o])), qf[st], sa);
        da = mfma32(as_bf16x8(*reinterpret_cast<const u32x4*>(&vs[o])), df[st], da);
      }
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        u32x4 u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float dsv[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int i = 8 * hs + 2 * j + e;
            float pv_ = __builtin_amdgcn_exp2f(fmaf(sa[i], c, -lse2));
            if (need_mask) {
              const int kk = kv0 + kb * 32 + 16 * hs + 8 * half + 2 * j + e;
              if (kk > lim) pv_ = 0.f;
            }
            dsv[e] = pv_ * (da[i] - dl) * scale;
          }
          u[j] = pack_bf16x2(dsv[0], dsv[1]);
        }
        dsf[kb][hs] = as_bf16x8(u);
      }
    }

    // dQ^T += K^T dS^T
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hs = 0; hs < 2; ++hs)
          acc[cb] = mfma32(tr_frag<D>(ks, lane, 32 * kb + 16 * hs, 32 * cb), dsf[kb][hs], acc[cb]);
  }

  if (qrow < lq) {
    const int64_t orow = (int64_t(it.q_start) + qrow) * q_tok + int64_t(h) * D;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int cc = cb * 32 + 8 * gq + 4 * half;
        u32x2 o2;
        o2[0] = pack_bf16x2(acc[cb][4 * gq], acc[cb][4 * gq + 1]);
        o2[1] = pack_bf16x2(acc[cb][4 * gq + 2], acc[cb][4 * gq + 3]);
        *reinterpret_cast<u32x2*>(dq + orow + cc) = o2;
      }
  }
}

int device_cus() {
  int dev = 0, n = 256;
  (void)hipGetDevice(&dev);
  (void)hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  return n;
}

template <int D>
hipError_t run_bwd(const AttnShape& s, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                   const uint16_t* o, const uint16_t* dout, const float* lse,
                   const DevItem* fwd_list, int32_t n_fwd, const DevItem* bwd_list, int32_t n_bwd,
                   int32_t head_split, uint16_t* dq, uint16_t* dk, uint16_t* dv, float* delta,
                   float* dkv_acc, hipStream_t stream) {
  const int n_cu = device_cus();
  {
    constexpr int RPB = kThreads / (D / 8);
    const int64_t want = (s.total_q * s.hq + RPB - 1) / RPB;
    const int blocks = int(std::max<int64_t>(1, std::min<int64_t>(want, int64_t(n_cu) * 16)));
    ProfScope prof("bwd_pre", stream);
    if (s.total_q > 0)
      hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3(blocks), dim3(kThreads), 0, stream, o, dout,
                         delta, s.total_q, s.hq);
  }
  const int64_t kv_elems = s.total_k * s.hkv * D;
  if (head_split > 1 && kv_elems > 0) {
    const int64_t n4 = 2 * kv_elems / 4;
    const int blocks = int(std::min<int64_t>((n4 + kThreads - 1) / kThreads, int64_t(n_cu) * 16));
    ProfScope prof("bwd_dkv_zero", stream);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                       reinterpret_cast<f32x4*>(dkv_acc), n4);
  }
  if (n_bwd > 0) {
    const int groups = (n_bwd + 7) / 8;
    const dim3 grid(unsigned(groups) * 8u * unsigned(s.hkv * head_split));
    ProfScope prof("bwd_dkdv", stream);
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D>), grid, dim3(kKvThreads), 0, stream, q, k, v, dout,
                       lse, delta, bwd_list, n_bwd, s.hq, s.hkv, head_split, s.scale, s.causal,
                       s.total_q, dk, dv, dkv_acc, s.total_k);
  }
  if (head_split > 1 && kv_elems > 0) {
    const int64_t n4 = kv_elems / 4;
    const int blocks = int(std::min<int64_t>((n4 + kThreads - 1) / kThreads, int64_t(n_cu) * 16));
    ProfScope prof("bwd_dkv_convert", stream);
    hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                       reinterpret_cast<const f32x4*>(dkv_acc), reinterpret_cast<u32x2*>(dk), n4);
    hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(blocks), dim3(kThreads), 0, stream,
                       reinterpret_cast<const f32x4*>(dkv_acc + kv_elems),
                       reinterpret_cast<u32x2*>(dv), n4);
  }
  if (n_fwd > 0) {
    const int groups = (n_fwd + 7) / 8;
    const dim3 grid(unsigned(groups) * 8u * unsigned(s.hq));
    ProfScope prof("bwd_dq", stream);
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D>), grid, dim3(kThreads), 0, stream, q, k, v, dout, lse,
                       delta, fwd_list, n_fwd, s.hq, s.hkv, s.scale, s.causal, s.total_q, dq);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const AttnShape& s, const void* q, const void* k, const void* v,
                           const void* o, const void* dout, const float* lse,
                           const DevItem* fwd_list, int32_t n_fwd, const DevItem* bwd_list,
                           int32_t n_bwd, int32_t head_split, void* dq, void* dk, void* dv,
                           float* delta, float* dkv_acc, hipStream_t stream) {
  auto* Q = reinterpret_cast<const uint16_t*>(q);
  auto* K = reinterpret_cast<const uint16_t*>(k);
  auto* V = reinterpret_cast<const uint16_t*>(v);
  auto* O = reinterpret_cast<const uint16_t*>(o);
  auto* DO = reinterpret_cast<const uint16_t*>(dout);
  auto* DQ = reinterpret_cast<uint16_t*>(dq);
  auto* DK = reinterpret_cast<uint16_t*>(dk);
  auto* DV = reinterpret_cast<uint16_t*>(dv);
  if (s.d == 128)
    return run_bwd<128>(s, Q, K, V, O, DO, lse, fwd_list, n_fwd, bwd_list, n_bwd, head_split, DQ,
                        DK, DV, delta, dkv_acc, stream);
  return run_bwd<64>(s, Q, K, V, O, DO, lse, fwd_list, n_fwd, bwd_list, n_bwd, head_split, DQ, DK,
                     DV, delta, dkv_acc, stream);
}

}  // namespace vl
