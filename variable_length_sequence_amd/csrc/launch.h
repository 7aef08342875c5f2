// Internal host launchers of the HIP kernels (not part of the C ABI).
// Arguments are assumed validated by the caller (api.cpp); each returns the
// hipError_t of its launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scheduler.h"

namespace vl {

// Ulysses pack/unpack: dir 0 = seq2head (x -> y), dir 1 = head2seq (y -> x).
hipError_t launch_sp_permute(const void* src, void* dst, int64_t n_tokens, int32_t n_heads,
                             int32_t head_dim, int32_t sp_degree, int32_t elem_bytes, int dir,
                             hipStream_t stream);

// Q, K and V (or dQ, dK, dV) of one Ulysses exchange in one launch, with the
// kv heads of grouped-query attention split over the ranks (replicated when
// n_heads_kv < sp_degree; their gradients summed on the way back).
// dir 0: src = x-side tensors [n, H, d], dst = [P, n, hs, d];
// dir 1: src = [P, n, hs, d], dst = [n, H, d].  dtype VL_BF16 (0) / VL_F32 (1).
struct QkvTensors {
  const void* src[3];
  void* dst[3];
};
hipError_t launch_sp_qkv(const QkvTensors& t, int64_t n_tokens, int32_t n_heads_q,
                         int32_t n_heads_kv, int32_t head_dim, int32_t sp_degree, int32_t dtype,
                         int dir, hipStream_t stream);

// Matrix-core throughput probe (independent MFMA chains, no memory traffic);
// n_wg workgroups of 4 waves, each writing one float to sink.
hipError_t launch_mfma_probe(int32_t iters, int32_t n_wg, float* sink, hipStream_t stream);
int64_t mfma_probe_flops(int32_t iters, int32_t n_wg);

constexpr int kMaxMergeParts = 64;

hipError_t launch_lse_merge(int32_t n_parts, const void* const* o_parts,
                            const float* const* lse_parts, int32_t in_dtype, int64_t n_rows,
                            int32_t n_heads, int32_t head_dim, void* o_out, float* lse_out,
                            int32_t out_dtype, hipStream_t stream);

// Tile sizes of the attention kernels (rows of a query tile / key tile).
constexpr int kFwdBQ = 128;   // forward and dQ kernels: 4 waves x 32 queries
constexpr int kFwdBK = 64;    // key tiles of their work list (the forward runs halves)
constexpr int kBwdBQ = 32;    // dK/dV kernel: query rows per step
constexpr int kBwdBK = 128;   // dK/dV kernel: 4 waves x 32 keys

// The work items of one pass, laid out by their assignment to the 8 XCDs:
// workgroup b runs on XCD b % 8 (dispatch order), and the j-th item of XCD x
// is items[j * 8 + x] (n_slices == 0: none), so a workgroup finds its item
// with one load.  Every item is run by consecutive workgroups of its XCD, one
// per q head (forward, dQ) or per kv head (a dK/dV entry, one q-head slice).
constexpr int kXcds = 8;

struct ItemMap {
  const DevItem* items;  // [rows * kXcds]
  int32_t rows;          // items of the longest XCD list
  int32_t n_cut;         // dK/dV list: cut key tiles, at items[rows * kXcds ..]
};

struct AttnShape {
  int64_t total_q, total_k;
  int32_t hq, hkv, d;
  float scale;
  int32_t causal;
};

// out_kind: kOutBf16 / kOutF32 write O (bf16 / fp32) and LSE; kOutAcc folds
// O and LSE into running fp32 accumulators held in out and lse.
constexpr int kOutBf16 = 0, kOutF32 = 1, kOutAcc = 2;
hipError_t launch_attn_fwd(const AttnShape& s, const void* q, const void* k, const void* v,
                           const ItemMap& map, int32_t out_kind, void* out, float* lse,
                           hipStream_t stream);

// Backward: dQ over the query-tile list, which also stores D_i = dO_i . O_i
// in delta ([hq, total_q] fp32), then dK/dV over the kv-tile list.  Entries
// of the dK/dV list cut into n_slices > 1 slices of their q heads (at most
// head_split) store fp32 partials in dkv_acc, [head_split][dK, dV][total_k,
// hkv, d], which a conversion kernel adds for those kv tiles.
constexpr int kMaxHeadSplit = 4;
hipError_t launch_attn_bwd(const AttnShape& s, const void* q, const void* k, const void* v,
                           const void* o, const void* dout, const float* lse,
                           const ItemMap& fwd_map, const ItemMap& bwd_map,
                           int32_t head_split, void* dq, void* dk, void* dv,
                           float* delta, float* dkv_acc, hipStream_t stream);

// The device scratch of varlen_attn_bwd_noalloc (defined in noalloc.hip):
// its size, and the address of the current device's copy (looked up once per
// device).
constexpr size_t kNoallocScratchBytes = size_t(128) << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace vl
