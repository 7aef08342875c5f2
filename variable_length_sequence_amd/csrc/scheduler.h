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

// What a kernel reads per work item (self-contained, 32 bytes).
struct DevItem {
  int32_t q_start, lq, k_start, lk;
  int32_t tile, first, count, doc;
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

std::vector<DevItem> device_items(const std::vector<Doc>& docs, const std::vector<Item>& items);

// Assignment of an LPT-ordered item list to the n_xcd XCDs of the device:
// each item, in list order, goes to the XCD with the least work so far
// (weight count + 1: its tiles plus its start-up), so every XCD keeps the
// longest-first order and all XCDs end within about one short item of each
// other (round-robin dealing would give the first XCD the longest item of
// every round).  Returns slots[j * n_xcd + x] = index of the j-th item of XCD
// x, or -1; rows = the longest XCD list.
std::vector<int32_t> xcd_slots(const std::vector<Item>& items, int n_xcd, int32_t& rows);

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
