// Backward attention over packed variable-length documents on gfx950.
//
// The exact gradient of the forward (the pages do not write it out; P is
// recomputed from the saved LSE, the attention recompute the NSP page
// discusses in Sections 2.3 and 4.2.2):
//   D_i = dO_i . O_i,  P_ij = exp(S_ij - LSE_i),  dP_ij = dO_i . V_j,
//   dS_ij = P_ij (dP_ij - D_i),
//   dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij Q_i,  dQ_i = scale sum_j dS_ij K_j.
//
// Two kernels (three when a key tile's q heads are split), no atomics:
//   1. dq: the forward's mapping (a lane owns one query): S^T = K Q^T and
//      dP^T = V dO^T per 64-key tile, then dQ^T += K^T dS^T; the Q, dO and O
//      tiles arrive in LDS by direct loads and dQ leaves through LDS, all in
//      whole rows.  D = rowsum(dO * O) of its rows is computed in the
//      prologue (the O tile rides beside the first K/V tile) and also stored,
//      fp32 [Hq, T], for (2): no separate pass over O and dO.
//   2. dkdv: one workgroup per (128-key tile of a document, kv head[, slice of
//      its q heads]); each wave owns 32 keys and keeps their K, V operands and
//      fp32 dK, dV accumulators in registers while 32-row query tiles of every
//      q head of the group stream through LDS (row-major and transposed).
//      Scores are computed as S = Q K^T so a lane owns one key; the query rows
//      of the A operand are permuted so P and dS come out of the MFMA already
//      in the A-operand layout of dV += P^T dO and dK += dS^T Q.
//   A key tile whose q-head group would outlast the average per-CU share of
//   the pass is cut into 2-4 slices of its q heads, one workgroup each; each
//   slice stores its fp32 dK/dV partial and a third kernel adds the partials
//   of those tiles in slice order (plain stores run at several times the rate
//   of fp32 atomic adds, and the sum is deterministic).  The other tiles
//   write bf16 dK/dV directly.
// The extra two contractions of (1) replace a zeroed fp32 dQ accumulator, its
// atomics and a conversion pass, and keep dQ deterministic.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "launch.h"
#include "profiler.h"

namespace vl {

namespace {

constexpr int kThreads = 256;

// dK and dV of the kv tiles whose q-head group the dK/dV list cut into
// slices: the sum of the slices' fp32 partials ([slice][dK, dV][T, H, D]),
// added in slice order (deterministic), -> bf16.  `cut` lists the first
// slice of every cut tile; `chunks` workgroups per tile, enough for about one
// 16-byte group of each tensor per thread, so every load of a tile is in
// flight at once (the pass is short and latency-bound).
template <int D>
__global__ void __launch_bounds__(kThreads)
dkv_convert_kernel(const DevItem* __restrict__ cut, const f32x4* __restrict__ src,
                   u32x2* __restrict__ dk, u32x2* __restrict__ dv, int64_t total_k, int hkv,
                   int chunks) {
  const DevItem it = cut[blockIdx.x / chunks];
  const int chunk = blockIdx.x % chunks;
  if (it.n_slices <= 1) return;
  const int j0 = it.tile * kBwdBK;
  const int nk = min(kBwdBK, it.lk - j0);
  if (nk <= 0) return;
  const int64_t row4 = int64_t(hkv) * (D / 4);            // float4 per key row
  const int64_t base = (int64_t(it.k_start) + j0) * row4;  // the tile's first key
  const int64_t n4 = int64_t(nk) * row4;                   // per tensor
  const int64_t plane = total_k * row4;
  const int64_t end = 2 * n4 * (chunk + 1) / chunks;
  for (int64_t i = 2 * n4 * chunk / chunks + threadIdx.x; i < end; i += kThreads) {
    const int t = i >= n4;                                 // 0: dK, 1: dV
    const int64_t j = base + (i - t * n4);
    f32x4 x = src[int64_t(t) * plane + j];
    for (int sp = 1; sp < it.n_slices; ++sp) {
      const f32x4 y = src[(int64_t(sp) * 2 + t) * plane + j];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] += y[e];
    }
    (t ? dv : dk)[j] = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
  }
}

// A chain of N dependent-accumulator MFMAs whose LDS operand fragment f is
// read PF fragments ahead of its use, with every step fenced so the reads
// keep that distance.  Pinning only the kinds of instructions
// (sched_group_barrier) let the scheduler fill a chain's read slots with
// other reads of the region and sink the chain's own reads to just before
// their MFMA: the fenced form is 1-2 % faster in dQ and 1-3.5 % in dK/dV
// (there the second chain's transpose reads had taken the first chain's read
// slots, leaving three of its MFMAs each waiting for a fresh read).
template <int N, int PF, typename Load, typename Mac>
__device__ __forceinline__ void mfma_chain_fenced(Load load, Mac mac) {
  bf16x8 r[PF];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int f = 0; f < PF; ++f) r[f] = load(f);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int f = 0; f < N; ++f) {
    const bf16x8 a = r[f % PF];
    mac(f, a);
    if (f + PF < N) r[f % PF] = load(f + PF);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------- dK, dV
constexpr int KB_Q = kBwdBQ;   // 32 query rows per step
constexpr int KB_K = kBwdBK;   // 128 keys per workgroup
constexpr int kKvThreads = 512;

constexpr int kKvBufs = 3;      // steps in flight: t - 1 (dK role), t (dV role), t + 1 (loading)

template <int D>
struct KvSmemLoop {
  // Q and dO tiles, row-major with swizzled chunks; query row r is kept at
  // LDS row swap_bits23(r).  The transposed operands (dO for dV += P^T dO, Q
  // for dK += dS^T Q) are read from the same tiles with the transpose read.
  uint16_t q[kKvBufs][KB_Q * D];
  uint16_t dout[kKvBufs][KB_Q * D];
  alignas(16) float lse2[kKvBufs][KB_Q];   // LSE log2(e)
  alignas(16) float delta[kKvBufs][KB_Q];  // D scale
  // P of recent steps, bf16, in the A-operand layout of each dV wave:
  // [step buffer][key block][operand half][lane][8]
  alignas(16) uint16_t p[kKvBufs][4][2][64 * 8];
};

// After the step loop the same LDS holds each wave's 32 x D block of dK or dV
// (fp32 for a split partial, else bf16), row-major with 16-byte chunks
// XOR-swizzled by row, so the block leaves in full rows of 16-byte stores.
template <int D>
union KvSmem {
  KvSmemLoop<D> loop;
  alignas(16) uint32_t stage[8][32 * D];   // [wave][32 rows x D fp32 (or 2 D bf16)]
};

// 8 waves per workgroup, 128 keys of one document and one kv head; waves
// w and w + 4 (same SIMD) share key block w & 3.  Iteration t:
//  * waves 0-3 (dV role) take step t: S = Q K^T (a lane owns a key),
//    P = exp(S - LSE) masked, P -> LDS (bf16), dV += P^T dO;
//  * waves 4-7 (dK role) take step t - 1: dP = dO V^T, P from LDS,
//    dS = P (dP - D) scale, dK += dS^T Q.
// Both roles run the same two MFMA chains on role-dependent LDS tiles (only
// the elementwise middle differs); the two waves of a SIMD work on different
// steps and overlap freely.
template <int D>
__global__ void __launch_bounds__(kKvThreads)
attn_bwd_dkdv_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                     const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                     const float* __restrict__ lse, const float* __restrict__ delta,
                     const DevItem* __restrict__ items,
                     int hq, int hkv, float scale, int causal, int64_t total_q,
                     uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                     float* __restrict__ dkv_acc, int64_t total_k) {
  constexpr int NKS = D / 16;
  constexpr int NCB = D / 32;
  __shared__ KvSmem<D> sm;

  // workgroup -> (entry, kv head) on XCD b % 8's entry list; the entry is
  // its item's q-head slice `split` of n_slices
  const int b = blockIdx.x;
  const int xcd = b & (kXcds - 1);
  const int r = b / kXcds;
  const DevItem it = items[(r / hkv) * kXcds + xcd];
  const int g = __builtin_amdgcn_readfirstlane(r % hkv);
  if (it.n_slices == 0) return;   // empty slot
  const int split = __builtin_amdgcn_readfirstlane(it.slice);
  const int head_split = __builtin_amdgcn_readfirstlane(it.n_slices);

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
  const int kw0 = j0 + w * 32;                 // first key of this wave
  const int key = kw0 + l32;                   // this lane's key
  const int64_t q_tok = int64_t(hq) * D;
  const int64_t kv_tok = int64_t(hkv) * D;
  const int grp = __builtin_amdgcn_readfirstlane(hq / hkv);
  const int hpg = __builtin_amdgcn_readfirstlane(grp / head_split);   // q heads handled here
  const int h_begin = g * grp + split * hpg;
  // the first chain's result x becomes fma(x, alpha, -row)
  const float alpha = role == 0 ? scale * kLog2e : scale;

  // B operand of S = Q K^T (dV role: K) or dP = dO V^T (dK role: V):
  // key l32, dims 16s + 8 half .. +8
  bf16x8 bf[NKS];
  {
    const int64_t row = int64_t(it.k_start) + key;
    const uint16_t* bp = (role == 0 ? k : v) + row * kv_tok + int64_t(g) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      u32x4 a = u32x4{0, 0, 0, 0};
      if (key < lk) a = *reinterpret_cast<const u32x4*>(bp + 16 * s);
      bf[s] = as_bf16x8(a);
    }
  }

  // loop-invariant element offsets of this lane's LDS reads within a tile:
  // A fragments of the first chain (row l32, chunk 2f + half) and the two
  // halves of the transposed B fragments of the second chain (rows
  // 4 (g4 / 2) + j4 and + 8, columns 32 cb + 16 (g4 & 1) + 4 m4)
  uint32_t a_off[NKS];
#pragma unroll
  for (int f = 0; f < NKS; ++f) a_off[f] = uint32_t(SwzTile<D>::chunk(l32, 2 * f + half));
  uint32_t t_off[NCB][2];
  {
    const int g4 = lane >> 4, j4 = (lane >> 2) & 3, m4 = lane & 3;
    const int row = 4 * (g4 >> 1) + j4;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int col = 32 * cb + 16 * (g4 & 1) + 4 * m4;
      t_off[cb][0] = uint32_t(SwzTile<D>::elem(row, col));
      t_off[cb][1] = uint32_t(SwzTile<D>::elem(row + 8, col));
    }
  }

  f32x16 acc[NCB];                             // dV (role 0) or dK (role 1)
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[cb][i] = 0.f;

  // Steps run over (32-row query tile, q head) pairs, heads innermost and
  // tiles from the end of the document back to the first one this key tile
  // sees: the workgroups of the other key tiles of the document (and kv
  // head) then stream the same query rows at the same time, which they share
  // in the L2 instead of each fetching them from memory.
  const int n_steps = hpg * it.count;
  const int i_last = (it.first + it.count - 1) * KB_Q;
  auto advance = [&](int& i0, int& h) {
    if (++h == h_begin + hpg) {
      h = h_begin;
      i0 -= KB_Q;
    }
  };
  const uint16_t* qdoc = q + int64_t(it.q_start) * q_tok;
  const uint16_t* ddoc = dout + int64_t(it.q_start) * q_tok;
  const PairLoader<D, KB_Q, kKvThreads / 64> loader(wave, lane, uint32_t(q_tok * 2));

  // Q/dO tiles arrive by direct global->LDS loads one step ahead; the 32 LSE
  // (wave 0) and D (wave 1) values of a step go through registers and are
  // scaled when stored, so their load latency hides behind the step's
  // compute.  Rows past the document repeat its last row (P is masked there).
  auto issue = [&](int i0, int h, uint32_t dq_, uint32_t dd_) {
    const int64_t ho = int64_t(h) * D;
    loader.load(qdoc + ho, ddoc + ho, q_tok, i0, lq, dq_, dd_, wave, lane);
  };
  auto fetch_rows = [&](int i0, int h) {
    float x = 0.f;
    if (wave < 2) {
      const int i = min(i0 + l32, lq - 1);
      x = (wave == 0 ? lse : delta)[int64_t(h) * total_q + it.q_start + i];
    }
    return x;
  };
  auto store_rows = [&](float x, int buf) {
    if (wave < 2 && lane < KB_Q) {
      if (wave == 0) sm.loop.lse2[buf][lane] = x * kLog2e;
      else sm.loop.delta[buf][lane] = x * scale;
    }
  };

  int nxt_i0 = i_last, nxt_h = h_begin;        // step t + 1
  int cur_i0 = i_last;                         // step t (dV role)
  if (n_steps > 0) {
    issue(nxt_i0, nxt_h, lds_addr(sm.loop.q[0]), lds_addr(sm.loop.dout[0]));
    store_rows(fetch_rows(nxt_i0, nxt_h), 0);
    advance(nxt_i0, nxt_h);
  }
  // One loop iteration t.  The loop is unrolled by three and compiled once
  // per role, so the step buffer (t % 3) and the role are compile-time
  // constants and every LDS address is a loop-invariant register plus an
  // immediate offset (a runtime buffer index and role select cost about a
  // fifth of the vector instructions of a step).
  auto iteration = [&](int t, auto cc, auto rc) {
    constexpr int cur = decltype(cc)::value;
    constexpr int role = decltype(rc)::value;   // this wave's role
    constexpr int nxt = (cur + 1) % kKvBufs;
    constexpr int prv = (cur + kKvBufs - 1) % kKvBufs;
    // step t has landed; nobody reads buffer nxt any more (step t - 2)
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    __syncthreads();
    float rows = 0.f;
    if (t + 1 < n_steps) {
      issue(nxt_i0, nxt_h, lds_addr(sm.loop.q[0]) + uint32_t(nxt) * (KB_Q * D * 2),
            lds_addr(sm.loop.dout[0]) + uint32_t(nxt) * (KB_Q * D * 2));
      rows = fetch_rows(nxt_i0, nxt_h);
    }
    const int st = t - role;                   // this wave's step
    if (st >= 0 && st < n_steps) {
      const int sb = role == 0 ? cur : prv;    // its buffer
      const uint16_t* tile1 = role == 0 ? sm.loop.q[sb] : sm.loop.dout[sb];
      const uint16_t* tile2 = role == 0 ? sm.loop.dout[sb] : sm.loop.q[sb];
      const float* rowv = role == 0 ? sm.loop.lse2[sb] : sm.loop.delta[sb];
      // this lane's 16 queries 16s + 8 half + u: LSE log2(e) or D scale
      f32x4 rr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        rr[j] = *reinterpret_cast<const f32x4*>(&rowv[16 * (j >> 1) + 8 * half + 4 * (j & 1)]);
      // dK role: P of step t - 1 from the dV wave
      u32x4 pr[2];
      if (role == 1) {
        const uint16_t* pp = &sm.loop.p[prv][w][0][lane * 8];
        pr[0] = *reinterpret_cast<const u32x4*>(pp);
        pr[1] = *reinterpret_cast<const u32x4*>(pp + 64 * 8);
      }
      // S = Q K^T or dP = dO V^T (rows: queries 16s + 8 half + u; cols: keys)
      f32x16 x;
      mfma_chain_fenced<NKS, 4>(
          [&](int f) { return as_bf16x8(*reinterpret_cast<const u32x4*>(tile1 + a_off[f])); },
          [&](int f, const bf16x8& a) { x = mfma32(a, bf[f], f == 0 ? f32x16{} : x); });
      // B fragments of the second chain (transposed reads), issued now so
      // their latency hides behind the elementwise middle
      bf16x8 tb[2 * NCB];
#pragma unroll
      for (int f = 0; f < 2 * NCB; ++f) {
        const uint16_t* tp = tile2 + 16 * D * (f & 1);
        const s16x4 lo = ds_read_tr16(tp + t_off[f >> 1][0]);
        const s16x4 hi = ds_read_tr16(tp + t_off[f >> 1][1]);
        tb[f] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      __builtin_amdgcn_sched_barrier(0);
      // element i holds query i0 + 8 half + e, e = 16 (i / 8) + i % 8
      u32x4 au[2];
      if (role == 0) {
        uint16_t* pp = &sm.loop.p[cur][w][0][lane * 8];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i = 8 * s2 + 2 * j;
            au[s2][j] = pack_bf16x2(
                __builtin_amdgcn_exp2f(fmaf(x[i], alpha, -rr[i >> 2][i & 3])),
                __builtin_amdgcn_exp2f(fmaf(x[i + 1], alpha, -rr[(i + 1) >> 2][(i + 1) & 3])));
          }
        // Masking is needed only where the step crosses the causal diagonal or
        // an end of the document (wave-uniform test).  Element e is visible
        // iff e < lq - qb (a real row), key < lk, and (causal) e >= key - off - qb.
        const int i0 = cur_i0;
        const bool need_mask = (i0 + KB_Q > lq) || (kw0 + 32 > lk) ||
                               (causal && kw0 + 31 > i0 + off);
        if (need_mask) {
          const int qb = i0 + 8 * half;
          const int e_min = causal ? key - off - qb : INT32_MIN;
          const int e_cap = (key < lk) ? lq - qb : INT32_MIN;
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int e = 16 * s2 + 2 * j;
              const uint32_t lo = (e < e_cap && e >= e_min) ? 0xffffu : 0u;
              const uint32_t hi = (e + 1 < e_cap && e + 1 >= e_min) ? 0xffff0000u : 0u;
              au[s2][j] &= lo | hi;
            }
        }
        // hand P to the dK wave of this key block (read one iteration later)
        *reinterpret_cast<u32x4*>(pp) = au[0];
        *reinterpret_cast<u32x4*>(pp + 64 * 8) = au[1];
      } else {
        // dS = P (dP - D) scale
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const u32x4 pw = pr[s2];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i = 8 * s2 + 2 * j;
            au[s2][j] = pack_bf16x2(
                bf16_lo(pw[j]) * fmaf(x[i], alpha, -rr[i >> 2][i & 3]),
                bf16_hi(pw[j]) * fmaf(x[i + 1], alpha, -rr[(i + 1) >> 2][(i + 1) & 3]));
          }
        }
      }
      // dV^T += dO^T P or dK^T += Q^T dS: the transposed products, so a lane
      // holds 4 consecutive head dims of its key (the operands are the same
      // registers: a B fragment read as an A fragment is its transpose)
#pragma unroll
      for (int f = 0; f < 2 * NCB; ++f)
        acc[f >> 1] = mfma32(tb[f], as_bf16x8(au[f & 1]), acc[f >> 1]);
    }
    if (t + 1 < n_steps) store_rows(rows, nxt);
    cur_i0 = nxt_i0;
    advance(nxt_i0, nxt_h);
  };
  auto run = [&](auto rc) {
    int t = 0;
    for (; t + 2 <= n_steps; t += 3) {
      iteration(t, IC<0>{}, rc);
      iteration(t + 1, IC<1>{}, rc);
      iteration(t + 2, IC<2>{}, rc);
    }
    if (t <= n_steps) iteration(t, IC<0>{}, rc);
    if (t + 1 <= n_steps) iteration(t + 1, IC<1>{}, rc);
  };
  if (role == 0) run(IC<0>{});
  else run(IC<1>{});

  // epilogue: lane holds key kw0 + l32, head dims 32 cb + 8 j + 4 half + 0..3
  // in acc[cb][4 j .. 4 j + 3].  Each wave stages its 32 x D block in LDS
  // (the step buffers are free once every wave is past the loop) and writes
  // it out as whole rows of 16-byte chunks.
  __syncthreads();
  uint32_t* stg = sm.stage[wave];
  const int64_t row0 = (int64_t(it.k_start) + kw0) * kv_tok + int64_t(g) * D;   // key kw0
  if (head_split == 1) {
    // bf16: a row is D / 8 chunks; chunk c of row r sits at chunk
    // c ^ (r % (D / 8))
    constexpr int RCH = D / 8;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 4 * cb + j;
        const u32x2 v2{pack_bf16x2(acc[cb][4 * j], acc[cb][4 * j + 1]),
                       pack_bf16x2(acc[cb][4 * j + 2], acc[cb][4 * j + 3])};
        *reinterpret_cast<u32x2*>(&stg[l32 * (D / 2) + ((c ^ (l32 & (RCH - 1))) << 2) + 2 * half]) = v2;
      }
    uint16_t* outp = role == 0 ? dv : dk;
    constexpr int RPI = 64 / RCH;              // rows per read
#pragma unroll
    for (int t = 0; t < 32 / RPI; ++t) {
      const int r = t * RPI + lane / RCH, c = lane % RCH;
      const u32x4 x = *reinterpret_cast<const u32x4*>(&stg[r * (D / 2) + ((c ^ (r & (RCH - 1))) << 2)]);
      if (kw0 + r < lk)
        *reinterpret_cast<u32x4*>(outp + row0 + int64_t(r) * kv_tok + 8 * c) = x;
    }
  } else {
    // fp32 partial: a row is D / 4 chunks; chunk c of row r sits at chunk
    // c ^ (r % (D / 4))
    constexpr int RCH = D / 4;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 8 * cb + 2 * j + half;
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = acc[cb][4 * j + e];
        *reinterpret_cast<f32x4*>(&stg[l32 * D + ((c ^ (l32 & (RCH - 1))) << 2)]) = v4;
      }
    float* accp = dkv_acc + (int64_t(split) * 2 + (role == 0 ? 1 : 0)) * total_k * kv_tok;
    constexpr int RPI = 64 / RCH;
#pragma unroll
    for (int t = 0; t < 32 / RPI; ++t) {
      const int r = t * RPI + lane / RCH, c = lane % RCH;
      const f32x4 x = *reinterpret_cast<const f32x4*>(&stg[r * D + ((c ^ (r & (RCH - 1))) << 2)]);
      if (kw0 + r < lk)
        *reinterpret_cast<f32x4*>(accp + row0 + int64_t(r) * kv_tok + 4 * c) = x;
    }
  }
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
                   const uint16_t* __restrict__ o, const float* __restrict__ lse,
                   float* __restrict__ delta, const DevItem* __restrict__ items, int hq,
                   int hkv, float scale, int causal, int64_t total_q, uint16_t* __restrict__ dq) {
  constexpr int NKS = D / 16;
  constexpr int NCB = D / 32;
  __shared__ QSmem<D> sm;

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
  const int off = lk - lq;
  const int q0 = it.tile * QB_Q;
  const int qrow = q0 + w * 32 + l32;
  const int64_t q_tok = int64_t(hq) * D;
  const int64_t kv_tok = int64_t(hkv) * D;
  const float c = scale * kLog2e;

  // The Q and dO tiles arrive by direct loads in whole rows (Q into buffer 1,
  // dO into buffer 0; rows past the document repeat its last row, whose P is
  // zero) and are read back as fragments below; the first K/V tile follows
  // once buffer 0 is free again.
  load_rows128_lds<D>(q + (int64_t(it.q_start) + q0) * q_tok + int64_t(h) * D,
                      uint32_t(q_tok * 2), lq - q0, lds_addr(sm.k[1]), lds_addr(sm.v[1]), w, lane);
  load_rows128_lds<D>(dout + (int64_t(it.q_start) + q0) * q_tok + int64_t(h) * D,
                      uint32_t(q_tok * 2), lq - q0, lds_addr(sm.k[0]), lds_addr(sm.v[0]), w, lane);
  bf16x8 qf[NKS], df[NKS];
  float lse2 = INFINITY;
  if (qrow < lq) {
    const float l = lse[int64_t(h) * total_q + it.q_start + qrow];
    lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
  }
  float dls;   // D scale, computed once the O tile has landed

  f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[cb][i] = 0.f;

  const uint16_t* kbase = k + int64_t(it.k_start) * kv_tok + int64_t(g) * D;
  const uint16_t* vbase = v + int64_t(it.k_start) * kv_tok + int64_t(g) * D;
  const PairLoader<D, QB_K, kThreads / 64> loader(w, lane, uint32_t(kv_tok * 2));
  // the next key tile to load, advanced by one tile per tile
  const int64_t kv_step = int64_t(QB_K) * kv_tok;
  const uint16_t* knext = kbase + kv_step;
  const uint16_t* vnext = vbase + kv_step;
  const int wq_first = q0 + w * 32;
  const int wq_last = min(q0 + w * 32 + 31, lq - 1);
  const int lim = causal ? min(lk - 1, qrow + off) : lk - 1;

  // one key tile (buffer index fixed at compile time, as in the forward)
  auto tile = [&](int kt, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int kv0 = kt * QB_K;
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    __syncthreads();
    if (kt + 1 < it.count) {
      loader.load_from(knext, vnext, lk - kv0 - QB_K, uint32_t(kv_tok * 2),
                       lds_addr(sm.k[buf ^ 1]), lds_addr(sm.v[buf ^ 1]), w, lane);
      knext += kv_step;
      vnext += kv_step;
    }
    const uint16_t* ks = sm.k[buf];
    const uint16_t* vs = sm.v[buf];

    const bool live = (wq_first < lq) && (!causal || kv0 <= wq_last + off);
    if (!live) return;
    const bool need_mask = (kv0 + QB_K > lk) || (causal && kv0 + QB_K - 1 > wq_first + off);

    // per 32-key half kb: S^T and dP^T (16 MFMAs), then dS^T packed to bf16;
    // one half at a time keeps only one pair of accumulators live
    bf16x8 dsf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 sa, da;
      const int prow = kb * 32 + l32;
      // S^T and dP^T chains interleaved; fragment f = (st, K or V), read
      // four fragments ahead
      mfma_chain_fenced<2 * NKS, 4>(
          [&](int f) {
            const uint16_t* t = (f & 1) ? vs : ks;
            return as_bf16x8(*reinterpret_cast<const u32x4*>(&t[SwzTile<D>::chunk(prow, 2 * (f >> 1) + half)]));
          },
          [&](int f, const bf16x8& a) {
            const int st = f >> 1;
            if (f & 1) da = mfma32(a, df[st], st == 0 ? f32x16{} : da);
            else sa = mfma32(a, qf[st], st == 0 ? f32x16{} : sa);
          });
      // on tiles crossing the diagonal or the document's end: key kv0 + 32 kb
      // + 8 half + e (e = 16 (i / 8) + i % 8) is visible iff e <= thr; a
      // hidden score becomes -inf, so its P is exactly zero
      if (need_mask) {
        const int thr = lim - kv0 - 32 * kb - 8 * half;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (16 * (i >> 3) + (i & 7) > thr) sa[i] = -INFINITY;
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
            dsv[e] = __builtin_amdgcn_exp2f(fmaf(sa[i], c, -lse2)) * fmaf(da[i], scale, -dls);
          }
          u[j] = pack_bf16x2(dsv[0], dsv[1]);
        }
        dsf[kb][hs] = as_bf16x8(u);
      }
      // dS of this half is complete before the next half's chains start (the
      // mask branch would otherwise let the compiler sink it below them and
      // keep both halves' accumulators live)
      asm volatile("" ::"v"(as_u32x4(dsf[kb][0])), "v"(as_u32x4(dsf[kb][1])));
    }

    // dQ^T += K^T dS^T; fragment f = (cb, kb, hs), read transposed, two ahead
    mfma_chain_fenced<4 * NCB, 2>(
        [&](int f) { return tr_frag<D>(ks, lane, 16 * (f & 3), 32 * (f >> 2)); },
        [&](int f, const bf16x8& a) { acc[f >> 2] = mfma32(a, dsf[(f >> 1) & 1][f & 1], acc[f >> 2]); });
  };

  const int n_kv = it.count;
  // Q and dO fragments (B operands of S^T = K Q^T and dP^T = V dO^T): query
  // l32, dims 16s + 8 half .. +8
  __builtin_amdgcn_s_waitcnt(kWaitAll);
  __syncthreads();
  {
    const int row = w * 32 + l32;
    const uint16_t* qs = row < 64 ? sm.k[1] : sm.v[1];
    const uint16_t* ds = row < 64 ? sm.k[0] : sm.v[0];
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      qf[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(&qs[SwzTile<D>::chunk(row & 63, 2 * s + half)]));
      df[s] = as_bf16x8(*reinterpret_cast<const u32x4*>(&ds[SwzTile<D>::chunk(row & 63, 2 * s + half)]));
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitAll);
  __syncthreads();
  if (n_kv > 0)
    loader.load(kbase, vbase, kv_tok, 0, lk, lds_addr(sm.k[0]), lds_addr(sm.v[0]), w, lane);
  // the O tile lands in buffer 1 beside the first K/V tile
  load_rows128_lds<D>(o + (int64_t(it.q_start) + q0) * q_tok + int64_t(h) * D,
                      uint32_t(q_tok * 2), lq - q0, lds_addr(sm.k[1]), lds_addr(sm.v[1]), w, lane);
  __builtin_amdgcn_s_waitcnt(kWaitAll);
  __syncthreads();
  // D = dO . O of this lane's query row: each lane sums its 16-byte chunks
  // (2s + half) one by one, the chunks pairwise in a fixed tree, then the two
  // halves of the row; the row's D is stored for the dK/dV kernel
  float dl;
  {
    const int row = w * 32 + l32;
    const uint16_t* os = row < 64 ? sm.k[1] : sm.v[1];
    float part[NKS];
#pragma unroll
    for (int s2 = 0; s2 < NKS; ++s2) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(&os[SwzTile<D>::chunk(row & 63, 2 * s2 + half)]);
      const u32x4 b = as_u32x4(df[s2]);
      float x = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x = fmaf(bf16_lo(a[j]), bf16_lo(b[j]), x);
        x = fmaf(bf16_hi(a[j]), bf16_hi(b[j]), x);
      }
      part[s2] = x;
    }
#pragma unroll
    for (int m = NKS / 2; m >= 1; m >>= 1)
#pragma unroll
      for (int s2 = 0; s2 < m; ++s2) part[s2] += part[s2 + m];
    dl = halves_sum(part[0]);
    if (half == 0 && qrow < lq) delta[int64_t(h) * total_q + it.q_start + qrow] = dl;
  }
  dls = dl * scale;
  int kt = 0;
  for (; kt + 1 < n_kv; kt += 2) {
    tile(kt, IC<0>{});
    tile(kt + 1, IC<1>{});
  }
  if (kt < n_kv) tile(kt, IC<0>{});

  // each wave stages its 32 x D block of dQ in LDS and writes whole rows of
  // 16-byte chunks (chunk c of row r sits at chunk c ^ (r % (D / 8))), in the
  // K/V buffer the last key tile did not use (free since that tile's barrier;
  // no load went into it), so no wave waits for the others here
  const int fb = n_kv & 1;
  uint32_t* stg = reinterpret_cast<uint32_t*>(w < 2 ? &sm.k[fb][0] : &sm.v[fb][0]) +
                  (w & 1) * (32 * D / 2);
  constexpr int RCH = D / 8;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int cc = 4 * cb + gq;
      const u32x2 o2{pack_bf16x2(acc[cb][4 * gq], acc[cb][4 * gq + 1]),
                     pack_bf16x2(acc[cb][4 * gq + 2], acc[cb][4 * gq + 3])};
      *reinterpret_cast<u32x2*>(&stg[l32 * (D / 2) + ((cc ^ (l32 & (RCH - 1))) << 2) + 2 * half]) = o2;
    }
  constexpr int RPI = 64 / RCH;
  const int64_t orow0 = (int64_t(it.q_start) + q0 + w * 32) * q_tok + int64_t(h) * D;
#pragma unroll
  for (int t = 0; t < 32 / RPI; ++t) {
    const int r = t * RPI + lane / RCH, cc = lane % RCH;
    const u32x4 x = *reinterpret_cast<const u32x4*>(&stg[r * (D / 2) + ((cc ^ (r & (RCH - 1))) << 2)]);
    if (q0 + w * 32 + r < lq)
      *reinterpret_cast<u32x4*>(dq + orow0 + int64_t(r) * q_tok + 8 * cc) = x;
  }
}

template <int D>
hipError_t run_bwd(const AttnShape& s, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                   const uint16_t* o, const uint16_t* dout, const float* lse,
                   const ItemMap& fwd_map, const ItemMap& bwd_map, int32_t head_split,
                   uint16_t* dq, uint16_t* dk, uint16_t* dv, float* delta, float* dkv_acc,
                   hipStream_t stream) {
  const int64_t kv_elems = s.total_k * s.hkv * D;
  if (fwd_map.rows > 0) {
    const dim3 grid(unsigned(fwd_map.rows) * unsigned(kXcds) * unsigned(s.hq));
    ProfScope prof("bwd_dq", stream);
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D>), grid, dim3(kThreads), 0, stream, q, k, v, dout, o,
                       lse, delta, fwd_map.items, s.hq, s.hkv, s.scale, s.causal,
                       s.total_q, dq);
  }
  if (bwd_map.rows > 0) {
    const dim3 grid(unsigned(bwd_map.rows) * unsigned(kXcds) * unsigned(s.hkv));
    ProfScope prof("bwd_dkdv", stream);
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D>), grid, dim3(kKvThreads), 0, stream, q, k, v, dout,
                       lse, delta, bwd_map.items, s.hq, s.hkv, s.scale,
                       s.causal, s.total_q, dk, dv, dkv_acc, s.total_k);
  }
  if (head_split > 1 && bwd_map.n_cut > 0 && kv_elems > 0) {
    // 2 kBwdBK hkv D / 4 groups of a tile over kThreads-thread workgroups
    const int chunks = std::max(1, int(2 * kBwdBK * s.hkv * (D / 4) / kThreads));
    const dim3 grid(unsigned(bwd_map.n_cut) * unsigned(chunks));
    ProfScope prof("bwd_dkv_convert", stream);
    hipLaunchKernelGGL((dkv_convert_kernel<D>), grid, dim3(kThreads), 0, stream,
                       bwd_map.items + size_t(bwd_map.rows) * kXcds,
                       reinterpret_cast<const f32x4*>(dkv_acc), reinterpret_cast<u32x2*>(dk),
                       reinterpret_cast<u32x2*>(dv), s.total_k, s.hkv, chunks);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const AttnShape& s, const void* q, const void* k, const void* v,
                           const void* o, const void* dout, const float* lse,
                           const ItemMap& fwd_map, const ItemMap& bwd_map, int32_t head_split,
                           void* dq, void* dk, void* dv, float* delta, float* dkv_acc,
                           hipStream_t stream) {
  auto* Q = reinterpret_cast<const uint16_t*>(q);
  auto* K = reinterpret_cast<const uint16_t*>(k);
  auto* V = reinterpret_cast<const uint16_t*>(v);
  auto* O = reinterpret_cast<const uint16_t*>(o);
  auto* DO = reinterpret_cast<const uint16_t*>(dout);
  auto* DQ = reinterpret_cast<uint16_t*>(dq);
  auto* DK = reinterpret_cast<uint16_t*>(dk);
  auto* DV = reinterpret_cast<uint16_t*>(dv);
  if (s.d == 128)
    return run_bwd<128>(s, Q, K, V, O, DO, lse, fwd_map, bwd_map, head_split, DQ, DK, DV, delta,
                        dkv_acc, stream);
  return run_bwd<64>(s, Q, K, V, O, DO, lse, fwd_map, bwd_map, head_split, DQ, DK, DV, delta,
                     dkv_acc, stream);
}

}  // namespace vl
