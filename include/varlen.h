/*
 * varlen.h - C ABI of libvarlen, causal attention over packed variable-length
 * sequences on AMD Instinct MI355X (gfx950), with the per-GPU pieces of the
 * Ulysses and ring sequence-parallel schemes.
 *
 * Conventions shared by every entry point
 *   - Tensors are caller-owned, contiguous device buffers (any allocator);
 *     the library never frees them.  Layouts are row-major and named
 *     outermost first: [T, H, d] means d fastest, then head, then token.
 *   - cu_seqlens arrays are HOST int32 arrays of n_docs + 1 entries: entry 0
 *     is 0, entries never decrease and the last one equals the total token
 *     count (packing leaves no padding between documents).
 *   - Every call validates its arguments first.  On failure nothing is
 *     enqueued, a negative VL_E* code is returned and varlen_last_error()
 *     describes it.  No C++ exception leaves the library.
 *   - Device work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and the call returns without waiting.  By default every call
 *     schedules its cu_seqlens pattern and enqueues the upload of its work
 *     lists on `stream` (see varlen_set_plan_cache).  With the plan cache
 *     switched on, the first call with a new pattern uploads its work list
 *     synchronously and caches it (see varlen_cache_clear); later calls with
 *     that pattern only launch kernels (no allocation, copy or memset), so
 *     they can be captured into a HIP graph.
 *   - bf16 values are IEEE binary32 truncated to the top 16 bits; results are
 *     rounded to nearest-even.  Scores, softmax and accumulation are fp32.
 */
#ifndef VARLEN_H
#define VARLEN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define VL_API __attribute__((visibility("default")))
#else
#define VL_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
enum { VL_BF16 = 0, VL_F32 = 1 };

/* status codes */
enum {
  VL_OK = 0,
  VL_EINVAL = -1,       /* null pointer, bad enum or non-positive size      */
  VL_ESHAPE = -2,       /* head counts / dims / degrees that do not fit      */
  VL_ESEQLENS = -3,     /* cu_seqlens not a valid cumulative-length array    */
  VL_EUNSUPPORTED = -4, /* valid but not implemented (e.g. head_dim 96)      */
  VL_EHIP = -5,         /* a HIP runtime call or kernel launch failed        */
  VL_EWORKSPACE = -6    /* workspace missing or smaller than required        */
};

/*
 * varlen_attn_fwd - softmax attention of every query over the keys of its own
 * document, optionally causal.
 *
 * Computes, for each document b, query row i < Lq(b) and q head h with kv head
 * g = h / (Hq / Hkv):  S_ij = scale * q_i . k_j,  LSE_i = ln sum_j exp(S_ij),
 * O_i = sum_j exp(S_ij - LSE_i) v_j over the visible keys j of the same
 * document (scaled dot-product attention: BASP page, Section II-A; HSAP page,
 * Section 2.2.1; documents kept apart by cumulative lengths: HSAP page,
 * Section 2.1, and the segmented mask of packing, NSP page, Section 2.2).
 * With causal != 0 key j is visible iff j <= i + (Lk - Lq) (diagonal aligned
 * to the bottom-right).  A query with no visible key gets O = 0, LSE = -inf.
 *
 *   q            bf16 [total_q, n_heads_q, head_dim]
 *   k, v         bf16 [total_k, n_heads_kv, head_dim]
 *   cu_seqlens_q, cu_seqlens_k  host int32 [n_docs + 1]
 *   head_dim     64 or 128; n_heads_q a multiple of n_heads_kv
 *   softmax_scale  <= 0 selects 1/sqrt(head_dim)
 *   out_dtype    VL_BF16 or VL_F32 (fp32 partials for a later attn_lse_merge)
 *   out          [total_q, n_heads_q, head_dim] of out_dtype
 *   lse          fp32 [n_heads_q, total_q], natural log
 * Errors: VL_EINVAL, VL_ESHAPE, VL_ESEQLENS, VL_EUNSUPPORTED, VL_EHIP.
 */
VL_API int varlen_attn_fwd(const void* q, const void* k, const void* v,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                    int32_t n_docs, int64_t total_q, int64_t total_k,
                    int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                    float softmax_scale, int32_t causal, int32_t out_dtype,
                    void* out, float* lse, void* stream);

/*
 * varlen_attn_fwd_acc - the forward over one key chunk folded into running
 * fp32 (O, LSE) accumulators: the online combination of ring attention
 * (HSAP page, Section 2.2.1) with its copy/rescale step (Section 3.1,
 * Table 1), which the page leaves as separate operations, done in the
 * forward kernel's epilogue.  Per query row and head, with (O, LSE) of this
 * call's keys:  M = max(LSE_acc, LSE),  w_acc = exp(LSE_acc - M),
 * w = exp(LSE - M),  O_acc <- (w_acc O_acc + w O) / (w_acc + w),
 * LSE_acc <- M + ln(w_acc + w); rows where both are -inf keep O_acc.
 * Calling it once per key chunk, from o_acc = 0 and lse_acc = -inf, gives
 * the result of attn_lse_merge over the chunks' partials (up to fp32
 * rounding) without storing them.
 *
 *   q, k, v, cu_*, sizes, scale, causal   as varlen_attn_fwd
 *   o_acc        fp32 [total_q, n_heads_q, head_dim], read and written
 *   lse_acc      fp32 [n_heads_q, total_q], read and written
 * Errors: as varlen_attn_fwd.
 */
VL_API int varlen_attn_fwd_acc(const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        int32_t n_docs, int64_t total_q, int64_t total_k,
                        int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                        float softmax_scale, int32_t causal, float* o_acc, float* lse_acc,
                        void* stream);

/*
 * varlen_attn_bwd_workspace_size - an upper bound on the device workspace
 * varlen_attn_bwd needs for any batch of these sizes: the fp32 per-row terms
 * D [n_heads_q, total_q] plus the fp32 dK/dV partials of the largest q-head
 * split the backward may choose (4 when the group size allows it).  0 for
 * invalid sizes.
 */
VL_API size_t varlen_attn_bwd_workspace_size(int64_t total_q, int64_t total_k,
                                      int32_t n_heads_q, int32_t n_heads_kv,
                                      int32_t head_dim);

/*
 * varlen_attn_bwd_workspace_size_cu - the device workspace varlen_attn_bwd
 * needs for this batch on the current device: D plus one fp32 dK/dV partial
 * per slice of the most finely cut key tile of its q-head split (none when
 * no tile is cut; which tiles are cut depends on the batch's key-tile counts
 * and the device's compute-unit count, see varlen_schedule_export_dkdv).
 * Host only.  Arguments as varlen_attn_bwd; 0 for invalid arguments.
 */
VL_API size_t varlen_attn_bwd_workspace_size_cu(const int32_t* cu_seqlens_q,
                                         const int32_t* cu_seqlens_k, int32_t n_docs,
                                         int64_t total_q, int64_t total_k,
                                         int32_t n_heads_q, int32_t n_heads_kv,
                                         int32_t head_dim, int32_t causal);

/*
 * varlen_attn_bwd - exact gradients of the forward above for an upstream dO.
 *
 * The pages do not write the backward; it is the analytic gradient of the
 * forward, with P recomputed from the saved LSE (the activation recompute the
 * NSP page discusses in Sections 2.3 and 4.2.2):
 *   D_i = dO_i . O_i,  P_ij = exp(S_ij - LSE_i),  dP_ij = dO_i . v_j,
 *   dS_ij = P_ij (dP_ij - D_i),  dq_i = scale sum_j dS_ij k_j,
 *   dk_j = scale sum_{h,i} dS_ij q_i,  dv_j = sum_{h,i} P_ij dO_i,
 * the kv sums running over the q heads that share kv head g.
 *
 *   q, k, v, cu_*, sizes, scale, causal   exactly as passed to the forward
 *   out          bf16 [total_q, n_heads_q, head_dim], the forward's O
 *   dout         bf16 [total_q, n_heads_q, head_dim]
 *   lse          fp32 [n_heads_q, total_q], the forward's LSE
 *   dq           bf16 [total_q, n_heads_q, head_dim]
 *   dk, dv       bf16 [total_k, n_heads_kv, head_dim]
 *   workspace    device memory of at least varlen_attn_bwd_workspace_size_cu()
 *                bytes for this batch (varlen_attn_bwd_workspace_size() bounds
 *                it for any batch), 256-byte aligned; contents on entry are
 *                ignored
 * No atomics: results are bitwise deterministic for given inputs (the dK/dV
 * sums over a kv group's q heads run in a fixed order, the partials of a cut
 * key tile are added in slice order).  D is computed by the dQ pass and kept
 * in the workspace for the dK/dV pass.
 * Errors: as the forward, plus VL_EWORKSPACE.
 */
VL_API int varlen_attn_bwd(const void* q, const void* k, const void* v,
                    const void* out, const void* dout, const float* lse,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                    int32_t n_docs, int64_t total_q, int64_t total_k,
                    int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                    float softmax_scale, int32_t causal,
                    void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * varlen_attn_bwd_noalloc - varlen_attn_bwd for callers that cannot allocate
 * device memory (tight serving or training loops, harnesses that forbid
 * allocation): the same arguments minus the workspace, the same kernels,
 * split and results.  D, the dK/dV partials and the two work lists go into a
 * 128 MiB device scratch array inside the library (one per device, held
 * until the process ends; its address is looked up once per device, with the
 * device current, on the first call there).  It allocates nothing: the work
 * lists are built on the host and copied from pageable host memory with
 * hipMemcpyAsync on `stream`, so a call on a capturing stream fails with
 * VL_EUNSUPPORTED (a captured copy would read host memory the call has
 * released).
 *
 * Limit: D [n_heads_q, total_q] fp32, plus the fp32 dK/dV partials of the
 * q-head split when the batch is split (varlen_attn_bwd_workspace_size_cu
 * gives both), plus the work lists, must fit the 128 MiB; a larger call
 * returns VL_EWORKSPACE before any work is enqueued.
 * Every call on one device shares that device's scratch, which keeps the last
 * call's contents: calls that overlap on one device (other streams, other
 * host threads) race and must be ordered by the caller.
 * Errors: as varlen_attn_bwd; VL_EWORKSPACE when the scratch is too small;
 * VL_EUNSUPPORTED on a capturing stream.
 */
VL_API int varlen_attn_bwd_noalloc(const void* q, const void* k, const void* v,
                            const void* out, const void* dout, const float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            int32_t n_docs, int64_t total_q, int64_t total_k,
                            int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                            float softmax_scale, int32_t causal,
                            void* dq, void* dk, void* dv, void* stream);

/*
 * attn_lse_merge - combine partial attention results computed over disjoint
 * key sets (the online combination of ring-style attention: HSAP page,
 * Section 2.2.1; its copy/rescale step, Section 3.1 Table 1; BASP page,
 * Section VII).  Per (row t, head h): M = max_k LSE_k, w_k = exp(LSE_k - M),
 * LSE = M + ln sum_k w_k, O = sum_k w_k O_k / sum_k w_k; all LSE_k = -inf
 * gives O = 0, LSE = -inf.
 *
 *   n_parts      1 .. 64
 *   o_parts      HOST array of n_parts device pointers, each
 *                [n_rows, n_heads, head_dim] of in_dtype (VL_BF16 / VL_F32)
 *   lse_parts    HOST array of n_parts device pointers, each fp32 [n_heads, n_rows]
 *   o_out        [n_rows, n_heads, head_dim] of out_dtype; may alias no input
 *   lse_out      fp32 [n_heads, n_rows]
 *   head_dim     a power of two from 4 to 256
 * Errors: VL_EINVAL, VL_ESHAPE, VL_EUNSUPPORTED, VL_EHIP.
 */
VL_API int attn_lse_merge(int32_t n_parts, const void* const* o_parts,
                   const float* const* lse_parts, int32_t in_dtype,
                   int64_t n_rows, int32_t n_heads, int32_t head_dim,
                   void* o_out, float* lse_out, int32_t out_dtype, void* stream);

/*
 * sp_seq2head - the local pack of the Ulysses layout change (HSAP page,
 * Section 2.2.2, IntraSP: an n x H x d shard becomes N x H/P x d after the
 * all-to-all; BASP page, Section II-C; NSP page, Section 2.1).
 *   y[p, t, j, :] = x[t, p*h + j, :],  h = n_heads / sp_degree,
 * so chunk p of y ([n_tokens, h, head_dim], contiguous) is what goes to rank p.
 *
 *   x            [n_tokens, n_heads, head_dim], elements of elem_bytes (2 or 4)
 *   y            [sp_degree, n_tokens, n_heads / sp_degree, head_dim]
 *   sp_degree    >= 1 and dividing n_heads
 * x and y must not overlap.  Bit-exact copy.
 * Errors: VL_EINVAL, VL_ESHAPE, VL_EHIP.
 */
VL_API int sp_seq2head(const void* x, void* y, int64_t n_tokens, int32_t n_heads,
                int32_t head_dim, int32_t sp_degree, int32_t elem_bytes, void* stream);

/*
 * sp_head2seq - the inverse unpack after the output all-to-all:
 *   x[t, p*h + j, :] = y[p, t, j, :].
 * Arguments as sp_seq2head, with y the source and x the destination.
 */
VL_API int sp_head2seq(const void* y, void* x, int64_t n_tokens, int32_t n_heads,
                int32_t head_dim, int32_t sp_degree, int32_t elem_bytes, void* stream);

/*
 * sp_qkv_seq2head - the send-side packs of Q, K and V for one Ulysses
 * exchange in a single launch, with the kv heads of grouped-query attention
 * split over the ranks (HSAP page, Section 2.2.2; BASP page, Section II-C and
 * Figure 2: Q, K and V are all moved from the sequence split to the head
 * split; NSP page, Section 2.1).  After the exchange rank p holds query heads
 * [p Hq/P, (p+1) Hq/P); query head h reads kv head h * Hkv / Hq, so rank p
 * needs hk kv heads:
 *   Hkv >= P:  hk = Hkv/P, kv heads [p hk, (p+1) hk)
 *   Hkv <  P:  hk = 1, kv head p / (P/Hkv), sent to each of the P/Hkv ranks
 *              that read it (replicated)
 *   yq[p, t, j, :] = q[t, p*Hq/P + j, :]
 *   yk[p, t, j, :] = k[t, g0(p) + j, :]   (likewise yv), g0 as above
 *
 *   q            [n_tokens, n_heads_q, head_dim]
 *   k, v         [n_tokens, n_heads_kv, head_dim]
 *   yq           [sp_degree, n_tokens, n_heads_q / sp_degree, head_dim]
 *   yk, yv       [sp_degree, n_tokens, hk, head_dim]
 *   dtype        VL_BF16 or VL_F32 (element size only: the pack is a copy)
 *   sp_degree and n_heads_kv divide n_heads_q; one of sp_degree, n_heads_kv
 *   divides the other; head_dim * element size a multiple of 4 bytes; every
 *   pointer 4-byte aligned.  No output may overlap an input or another
 *   output.  Bit-exact copy.
 * Errors: VL_EINVAL, VL_ESHAPE, VL_EUNSUPPORTED, VL_EHIP.
 */
VL_API int sp_qkv_seq2head(const void* q, const void* k, const void* v, void* yq, void* yk,
                    void* yv, int64_t n_tokens, int32_t n_heads_q, int32_t n_heads_kv,
                    int32_t head_dim, int32_t sp_degree, int32_t dtype, void* stream);

/*
 * sp_qkv_head2seq - the receive-side unpacks of dQ, dK and dV after the
 * gradient exchange, in a single launch: the adjoint of sp_qkv_seq2head.
 *   dq[t, p*Hq/P + j, :] = yq[p, t, j, :]
 *   Hkv >= P:  dk[t, p hk + j, :] = yk[p, t, j, :]        (likewise dv)
 *   Hkv <  P:  dk[t, g, :] = sum over the r = P/Hkv ranks p = g r .. g r + r - 1
 *              of yk[p, t, 0, :], added in that order in fp32 and rounded once
 *              to the output dtype (bf16: nearest, ties to even)
 * Arguments and constraints as sp_qkv_seq2head, with the [P, n, h, d]
 * tensors as sources and dq [n, Hq, d], dk/dv [n, Hkv, d] as destinations.
 * Deterministic; bit-exact copy when Hkv >= P.
 */
VL_API int sp_qkv_head2seq(const void* yq, const void* yk, const void* yv, void* dq, void* dk,
                    void* dv, int64_t n_tokens, int32_t n_heads_q, int32_t n_heads_kv,
                    int32_t head_dim, int32_t sp_degree, int32_t dtype, void* stream);

/*
 * basp_shard - host-only: batch-aware sequence partitioning (BASP page,
 * Section IV-A/B, Algorithms 1 and 2, Figure 4).  world ranks, a micro-batch
 * of `batch` sequences of seq_len tokens each.  Ranks form groups of
 * K = world / batch consecutive ranks (group g = ranks g K .. g K + K - 1);
 * group g takes sequence g and its rank at local position l = rank mod K
 * holds tokens [l seq_len / K, (l+1) seq_len / K), so each group runs its own
 * K-way exchange (sp_degree = K).  batch > world falls back to data
 * parallelism: K = 1 and rank r holds sequences [r b, (r+1) b), b =
 * batch / world, whole.
 *
 *   outputs      group, group_size (K), sequences [seq_begin, seq_end),
 *                tokens [tok_begin, tok_end) of each of them
 * Errors: VL_EINVAL (null output), VL_ESHAPE (rank out of range, world not a
 * multiple of batch (or batch of world when batch > world), seq_len not a
 * multiple of K).
 */
VL_API int basp_shard(int32_t rank, int32_t world, int32_t batch, int64_t seq_len,
               int32_t* group, int32_t* group_size, int32_t* seq_begin, int32_t* seq_end,
               int64_t* tok_begin, int64_t* tok_end);

/*
 * varlen_schedule_export - host-only: the work list the kernels run for these
 * cu_seqlens (no GPU needed).  Documents are cut into query tiles of *bq rows
 * and key tiles of *bk rows, never crossing a document; tile pairs holding no
 * visible pair are skipped (the "N" blocks of the HSAP page, Figure 3).
 *
 *   pass 0 (forward):  items[4*i..] = (doc, q_tile, first kv tile, kv tiles)
 *                      (the forward kernel runs each listed kv tile as two of
 *                      *bk / 2 keys and skips a last half that no query of
 *                      the item sees; the dQ kernel runs the same list whole)
 *   pass 1 (backward): items[4*i..] = (doc, kv_tile, first q tile, q tiles)
 *   ordered by decreasing tile count, then doc, then tile.
 *   items        host int32 [4 * cap], or NULL to query *n_items only
 *   useful_pairs visible (query, key) pairs per head
 *   issued_pairs pairs covered by the issued tiles per head (tile area)
 *   bq, bk       the tile sizes used for this head_dim and pass
 * Errors: VL_EINVAL, VL_ESEQLENS, VL_EUNSUPPORTED, VL_EWORKSPACE (cap too small).
 */
VL_API int varlen_schedule_export(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                           int32_t n_docs, int32_t causal, int32_t pass, int32_t head_dim,
                           int32_t* items, int64_t cap, int64_t* n_items,
                           int64_t* useful_pairs, int64_t* issued_pairs,
                           int32_t* bq, int32_t* bk);

/*
 * varlen_schedule_export_dkdv - host-only: the dK/dV work list as the kernel
 * runs it, with its q-head split.  A kv tile whose group of Hq / Hkv q heads
 * (each `count` query steps) would outlast the average per-CU share of the
 * pass, Hq times the summed counts over n_cu, is cut into 2 or 4 slices of
 * those heads (at most min(4, Hq / Hkv), a power of two dividing it), the
 * fewest that bring a slice within that share; the other tiles stay whole.
 *
 *   entries      host int32 [6 * cap], or NULL to query *n_entries only:
 *                (doc, kv_tile, first q tile, q tiles, slice, n_slices),
 *                longest first by q tiles x Hq / (Hkv n_slices)
 *   n_cu         compute units the pass spreads over (the library uses the
 *                device's count)
 * The largest n_slices is the number of fp32 dK/dV partials the backward
 * workspace holds.  Errors: VL_EINVAL, VL_ESEQLENS, VL_ESHAPE (head counts),
 * VL_EWORKSPACE (cap too small).
 */
VL_API int varlen_schedule_export_dkdv(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int32_t n_docs, int32_t causal, int32_t n_heads_q,
                                int32_t n_heads_kv, int32_t n_cu, int32_t* entries, int64_t cap,
                                int64_t* n_entries);

/*
 * varlen_ring_block - host-only: one (query chunk, key chunk) block of ring
 * attention over a packed causal batch.  The packed token axis is cut into
 * contiguous chunks, one per ring rank, and every block of the chunk grid has
 * one of the attention patterns of the HSAP page, Figure 3 (Section 3.2):
 * A1 the diagonal block (causal within each document), A2 every pair
 * visible, A3 the top rows see every key, A4 every row sees the right-hand
 * keys, A5 the top rows see the right-hand keys, N nothing visible.
 *
 *   cu_seqlens   host int32 [n_docs + 1] of the whole packed batch
 *   q_begin, q_end, k_begin, k_end   token ranges of the query and key
 *                chunks: equal (the diagonal block) or disjoint
 *   cu_q_out, cu_k_out  host int32 [n_docs + 1]: per document, its tokens
 *                inside the query chunk and inside the key chunk
 *   causal_out   the causal flag of the block's attention call
 *   cls_out      0 N, 1 A1, 2 A2, 3 A3, 4 A4, 5 A5
 * varlen_attn_fwd(q[q_begin:q_end], k[k_begin:k_end], v[k_begin:k_end],
 * cu_q_out, cu_k_out, causal = *causal_out) then computes the block's partial
 * (O, LSE) (skip class N), and attn_lse_merge over the key chunks gives the
 * rows of the query chunk; varlen_attn_bwd of the block with the merged O and
 * LSE gives its share of dq, dk and dv (the shares sum to the gradients).
 * Errors: VL_EINVAL (null pointer, ranges out of order or overlapping
 * unequally), VL_ESEQLENS.
 */
VL_API int varlen_ring_block(const int32_t* cu_seqlens, int32_t n_docs,
                             int64_t q_begin, int64_t q_end, int64_t k_begin, int64_t k_end,
                             int32_t* cu_q_out, int32_t* cu_k_out,
                             int32_t* causal_out, int32_t* cls_out);

/*
 * vl_cost_model - the per-GPU cost model the NSP planner scores plans with
 * (NSP page, Section 4.1.2).  For a sample of length L routed to an SP tree
 * node of degree s, each of the node's GPUs pays, per pass (fwd / bwd):
 *   compute   flops_per_pair * L (L + 1) / 2 / s FLOPs at the per-GPU
 *             throughput measured for documents of length L (piecewise
 *             linear between curve points, clamped outside);
 *   exchange  for s > 1, per phase (prologue, epilogue),
 *             ((s - 1) / s) * (L / s) * bytes_per_token[phase] / a2a_gbs, plus
 *             a latency alpha (s - 1) once per non-empty node and phase (the
 *             alpha-beta all-to-all model of the BASP page, Section IV);
 *   dense     (L / s) * dense_*_flops_per_token / dense_tflops.
 *
 *   n_points, curve_len[n_points] (strictly increasing, > 0),
 *   fwd_tflops / bwd_tflops[n_points] (> 0): host arrays, read during the call
 *   bytes_per_token: fwd prologue, fwd epilogue, bwd prologue, bwd epilogue
 */
typedef struct vl_cost_model {
  int32_t n_points;
  const double* curve_len;
  const double* fwd_tflops;
  const double* bwd_tflops;
  double fwd_flops_per_pair;
  double bwd_flops_per_pair;
  double bytes_per_token[4];
  double a2a_gbs;
  double a2a_alpha_us;
  double dense_fwd_flops_per_token;
  double dense_bwd_flops_per_token;
  double dense_tflops;
} vl_cost_model;

/*
 * nsp_route - host-only: route a batch of samples onto the SP tree (NSP page,
 * Section 4.1.1 Definition 1 and Figure 4; Section 4.1.3 Algorithm 1).
 * The tree over sp_max = 2^K GPUs has nodes (depth d, index i), an SP group
 * of degree 2^(K-d) on ranks [i 2^(K-d), (i+1) 2^(K-d)); n_gpus / sp_max
 * trees sit side by side.  Samples are taken longest first (ties by index);
 * the first `prefix` are searched with a beam of `beam` states (every
 * enabled node tried, states whose token peak max_p T_p exceeds
 * token_budget dropped, the `beam` with the smallest max_p C_p kept, ties in
 * generation order); each surviving state is completed by placing the rest,
 * longest first, on the least-loaded node of the deepest enabled level that
 * keeps the budget (else the one with the smallest token load); the completed
 * state with the smallest max_p C_p is returned.  T_p = sum of L_j / |R| over
 * the nodes on p's chain; C_p = forward + backward stage time of GPU p.
 *
 *   lengths       [n_samples] host, >= 0
 *   level_mask    bit d enables depth d (-1: all)
 *   monotone      non-zero: a longer sample never takes a smaller SP degree
 *                 than a shorter one
 *   node_depth, node_index   [n_samples] outputs: the node of each sample
 *   gpu_fwd, gpu_bwd, gpu_tokens   [n_gpus] outputs (each may be NULL)
 *   within_budget            output: 1 if max_p T_p <= token_budget (may be NULL)
 * Work is O(prefix * beam * nodes * n_gpus).  If no prefix extension keeps
 * the budget, the `beam` with the smallest token peak are kept and the plan
 * is reported over budget.
 * Errors: VL_EINVAL (null, negative or non-finite input, bad cost model),
 * VL_ESHAPE (sp_max not a power of two dividing n_gpus, no level enabled).
 */
VL_API int nsp_route(const int64_t* lengths, int32_t n_samples, int32_t n_gpus, int32_t sp_max,
              const vl_cost_model* cost, double token_budget, int32_t prefix, int32_t beam,
              int32_t monotone, int32_t level_mask, int32_t* node_depth, int32_t* node_index,
              double* gpu_fwd, double* gpu_bwd, double* gpu_tokens, int32_t* within_budget);

/*
 * nsp_plan_cost - host-only: the per-GPU forward / backward stage times and
 * token loads of a given plan (node_depth / node_index per sample, as
 * nsp_route returns them) under the same cost model.
 * Errors: VL_EINVAL, VL_ESHAPE (a node outside the tree).
 */
VL_API int nsp_plan_cost(const int64_t* lengths, int32_t n_samples, int32_t n_gpus,
                  int32_t sp_max, const vl_cost_model* cost, const int32_t* node_depth,
                  const int32_t* node_index, double* gpu_fwd, double* gpu_bwd,
                  double* gpu_tokens);

/*
 * varlen_mfma_probe - measurement aid: a kernel of n_workgroups workgroups
 * (4 waves each) whose waves issue iters rounds of 8 independent 32x32x16
 * bf16 MFMAs from registers, with no memory traffic in the loop.  Timing it
 * (events on `stream`) gives the matrix-core rate the chip sustains under
 * full load, the reachable ceiling beside the spec peak.
 *   sink     device float[n_workgroups] (one checksum per workgroup)
 *   flops    output: the FLOPs the launch performs (may be NULL)
 * Errors: VL_EINVAL, VL_EHIP.
 */
VL_API int varlen_mfma_probe(int32_t iters, int32_t n_workgroups, float* sink, int64_t* flops,
                      void* stream);

/*
 * varlen_profile_enable / varlen_profile_read - optional per-kernel timing.
 * While enabled, every kernel the library launches is bracketed by two HIP
 * events recorded on its launch stream.  Enabling clears earlier records.
 * varlen_profile_read(idx, ...) reports the idx-th distinct kernel name seen
 * (first-launch order): its launch count and summed elapsed milliseconds; it
 * waits for those events and returns VL_EINVAL past the last name.
 *   name      buffer of name_cap bytes for the NUL-terminated kernel name
 */
VL_API int varlen_profile_enable(int32_t on);
VL_API int varlen_profile_read(int32_t idx, char* name, int32_t name_cap,
                               int64_t* launches, double* total_ms);

/* Message of the last failed call on this thread ("" if none). */
VL_API const char* varlen_last_error(void);

/* Free the cached device work lists, those pinned by captured graphs
 * included.  The caller guarantees no launched kernel and no graph that may
 * still be replayed reads them (e.g. after a device synchronize, once the
 * graphs captured with the plan cache on are destroyed). */
VL_API void varlen_cache_clear(void);

/* Plan cache switch, process-wide; returns the previous setting (1 = on).
 * Off (the default): every attention call validates its cu_seqlens, builds
 * its work lists on the host (the scheduling of the HSAP page's Fig. 3 block
 * classes with the NSP page's longest-first order, Section 4.1.3) and
 * enqueues their upload on its own stream, as a training loop that packs a
 * new batch every step needs: the lists are copied into pinned host staging
 * and by one asynchronous copy into a per-device ring of device memory,
 * whose regions are handed out again once the kernels that read them have
 * completed (an event recorded behind them).  Such a call allocates nothing
 * and does not wait, unless the host is a whole ring ahead of the device or
 * the call's lists outgrow half the ring (1 MiB at first, then grown once,
 * after the regions in flight have drained).  A call on a capturing stream
 * fails with VL_EUNSUPPORTED in this mode.
 * On: work lists are cached per cu_seqlens pattern as above, for patterns
 * that repeat and for graph capture.  Warm a pattern up before capturing: a
 * new pattern on a capturing stream fails with VL_EUNSUPPORTED.  A plan used
 * under capture is pinned (the graph holds its device address).  The cache
 * keeps up to 4096 plans; a call with a new pattern on a full cache waits for
 * the device and frees every plan that is not pinned, or fails with
 * VL_EUNSUPPORTED when all 4096 are pinned (varlen_cache_clear frees them). */
VL_API int varlen_set_plan_cache(int32_t on);

/* ABI version, currently 1. */
VL_API int varlen_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VARLEN_H */
