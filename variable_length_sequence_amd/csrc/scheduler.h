// Host-side work-list scheduler for packed variable-length attention.
//
// Documents sit back to back in the packed token axis, delimited by the
// cumulative lengths (HSAP page, Section 2.1, cu_len).  Each document is cut
// into query tiles and key tiles that never cross a document boundary, so no
// tile can mix two documents.  For causal attention a (query tile, key tile)
// pair entirely above the diagonal holds no visible pair -- the "N" block of
// the HSAP page's Figure 3 -- and is never issued.  Items are ordered longest
// first, the same rule the NSP planner applies to samples (NSP page,
// Section 4.1.3, Algorithm 1), so the longest tiles start first on the GPU.
//
// Pure C++17: no HIP, so it builds and runs on any host.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

namespace vl {

struct Doc {
  int64_t q_start, lq, k_start, lk;
};

// One unit of kernel work, as exported: for the forward pass
// (doc, q_tile, first kv tile, kv tile count); for the backward pass
// (doc, kv_tile, first q tile, q tile count).
struct Item {
  int32_t doc, tile, first, count;
};

// What a kernel reads per work item (self-contained, 32 bytes).  On the
// dK/dV list an item may be cut into n_slices entries that each take slice
// `slice` of the q heads of its kv head's group; n_slices == 0 marks an empty
// slot of the XCD layout.
struct DevItem {
  int32_t q_start, lq, k_start, lk;
  int32_t tile, first, count;
  int16_t slice, n_slices;
};

// One entry of a work list: an item, the slice of its q-head group it takes
// (of n_slices), and its weight for the assignment to XCDs.
struct Entry {
  Item item;
  int32_t slice, n_slices;
  int64_t weight;
};

// Validates one cumulative-length array: n_docs + 1 entries, cu[0] == 0,
// non-decreasing, cu[n_docs] == total.  Returns false and sets err otherwise.
bool validate_cu(const int32_t* cu, int32_t n_docs, int64_t total, std::string& err);

std::vector<Doc> doc_table(const int32_t* cu_q, const int32_t* cu_k, int32_t n_docs);

std::vector<Item> fwd_items(const std::vector<Doc>& docs, bool causal, int bq, int bk);
std::vector<Item> bwd_items(const std::vector<Doc>& docs, bool causal, int bq, int bk);

// Visible (query, key) pairs per head.
int64_t visible_pairs(const std::vector<Doc>& docs, bool causal);
// Pairs covered by issued tiles per head (full tile area).
int64_t issued_pairs(const std::vector<Item>& items, int bq, int bk);

// The forward / dQ list as entries: one per item (its q heads are separate
// workgroups anyway), weight count + 1 (its key tiles plus its start-up).
std::vector<Entry> fwd_entries(const std::vector<Item>& items);

// The q-head split of the dK/dV pass, item by item.  A dK/dV workgroup runs
// `count` query steps for every q head of its slice of a kv head's group of
// grp heads.  per_cu is the average per-CU share of the whole pass, grp hkv
// times the summed counts over n_cu.  An item whose group would outlast it is
// cut into 2 or 4 slices of its q heads (at most max_split, a power of two
// dividing grp) until a slice no longer does; the other items stay whole, so
// only the cut ones leave fp32 partials for a conversion pass to add.
double bwd_per_cu(const std::vector<Item>& items, int grp, int hkv, int n_cu);
int item_head_split(int64_t count, int grp, double per_cu, int max_split);

// The dK/dV list as entries (item_head_split per item, slices in order),
// ordered by their work count grp / n_slices, longest first, with weight
// that work plus kBwdEntryStartup (the measured start-up and epilogue of an
// entry, in query steps of one q head).
constexpr int64_t kBwdEntryStartup = 2;
std::vector<Entry> bwd_entries(const std::vector<Item>& items, int grp, int hkv, int n_cu,
                               int max_split);

std::vector<DevItem> device_items(const std::vector<Doc>& docs, const std::vector<Entry>& entries);

// Assignment of a longest-first entry list to the n_xcd XCDs of the device:
// each entry, in list order, goes to the XCD with the least weight so far,
// so every XCD keeps the longest-first order and all XCDs end within about
// one short entry of each other (round-robin dealing would give the first
// XCD the longest entry of every round).  Returns slots[j * n_xcd + x] =
// index of the j-th entry of XCD x, or -1; rows = the longest XCD list.
std::vector<int32_t> xcd_slots(const std::vector<Entry>& entries, int n_xcd, int32_t& rows);

// One (query chunk, key chunk) block of ring attention over a packed causal
// batch (HSAP page, Section 3.2, Figure 3).  Fills per-document token counts
// inside each chunk (as cumulative arrays of n_docs + 1 entries), the causal
// flag of the block's attention call and its class (RingClass).  Supported:
// equal ranges (the diagonal) and disjoint ranges.  Returns false with err
// set for anything else.
enum RingClass { kRingN = 0, kRingA1 = 1, kRingA2 = 2, kRingA3 = 3, kRingA4 = 4, kRingA5 = 5 };
bool ring_block(const int32_t* cu, int32_t n_docs, int64_t q_begin, int64_t q_end,
                int64_t k_begin, int64_t k_end, int32_t* cu_q, int32_t* cu_k, int32_t& causal,
                int32_t& cls, std::string& err);

// Batch-aware sequence partitioning (BASP page, Section IV-A/B, Algorithms 1
// and 2): world ranks and a micro-batch of `batch` sequences of seq_len
// tokens.  Groups are K = world / batch consecutive ranks; group g takes
// sequence g and its rank at local position l holds tokens
// [l seq_len / K, (l+1) seq_len / K).  batch > world falls back to data
// parallelism (K = 1, rank r holds sequences [r b, (r+1) b), b = batch/world,
// whole).  Returns false with err set when the sizes do not divide.
struct BaspShard {
  int32_t group, group_size, seq_begin, seq_end;
  int64_t tok_begin, tok_end;
};
bool basp_shard(int32_t rank, int32_t world, int32_t batch, int64_t seq_len, BaspShard& out,
                std::string& err);

}  // namespace vl
