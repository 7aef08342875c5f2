// Host-side work-list scheduler; see scheduler.h.
#include "scheduler.h"

#include <algorithm>

namespace vl {

static inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static inline int64_t floor_div(int64_t a, int64_t b) {
  int64_t q = a / b;
  return (a % b != 0 && ((a < 0) != (b < 0))) ? q - 1 : q;
}

bool validate_cu(const int32_t* cu, int32_t n_docs, int64_t total, std::string& err) {
  if (!cu) { err = "cu_seqlens is null"; return false; }
  if (n_docs < 0) { err = "n_docs is negative"; return false; }
  if (cu[0] != 0) { err = "cu_seqlens[0] must be 0"; return false; }
  for (int32_t i = 0; i < n_docs; ++i) {
    if (cu[i + 1] < cu[i]) {
      err = "cu_seqlens must be non-decreasing (entry " + std::to_string(i + 1) + ")";
      return false;
    }
  }
  if (int64_t(cu[n_docs]) != total) {
    err = "cu_seqlens[n_docs] = " + std::to_string(cu[n_docs]) +
          " does not equal the total token count " + std::to_string(total);
    return false;
  }
  return true;
}

std::vector<Doc> doc_table(const int32_t* cu_q, const int32_t* cu_k, int32_t n_docs) {
  std::vector<Doc> d(static_cast<size_t>(n_docs));
  for (int32_t i = 0; i < n_docs; ++i)
    d[size_t(i)] = Doc{cu_q[i], int64_t(cu_q[i + 1]) - cu_q[i], cu_k[i], int64_t(cu_k[i + 1]) - cu_k[i]};
  return d;
}

static void lpt_sort(std::vector<Item>& items) {
  std::stable_sort(items.begin(), items.end(), [](const Item& a, const Item& b) {
    if (a.count != b.count) return a.count > b.count;
    if (a.doc != b.doc) return a.doc < b.doc;
    return a.tile < b.tile;
  });
}

std::vector<Item> fwd_items(const std::vector<Doc>& docs, bool causal, int bq, int bk) {
  std::vector<Item> out;
  for (size_t b = 0; b < docs.size(); ++b) {
    const Doc& d = docs[b];
    const int64_t n_k = ceil_div(d.lk, bk);
    const int64_t n_t = ceil_div(d.lq, bq);
    for (int64_t t = 0; t < n_t; ++t) {
      int64_t n_kv = n_k;
      if (causal) {
        // the tile's last row sees keys up to last_row + (Lk - Lq)
        const int64_t last_row = std::min(d.lq, (t + 1) * bq) - 1;
        const int64_t last_key = last_row + (d.lk - d.lq);
        n_kv = std::min(std::max(floor_div(last_key, bk) + 1, int64_t(0)), n_k);
      }
      out.push_back(Item{int32_t(b), int32_t(t), 0, int32_t(n_kv)});
    }
  }
  lpt_sort(out);
  return out;
}

std::vector<Item> bwd_items(const std::vector<Doc>& docs, bool causal, int bq, int bk) {
  std::vector<Item> out;
  for (size_t b = 0; b < docs.size(); ++b) {
    const Doc& d = docs[b];
    const int64_t n_q = ceil_div(d.lq, bq);
    const int64_t n_j = ceil_div(d.lk, bk);
    for (int64_t j = 0; j < n_j; ++j) {
      int64_t t0 = 0;
      if (causal) {
        // key j*bk is first seen by query row j*bk - (Lk - Lq)
        const int64_t first_row = std::max(int64_t(0), j * bk - (d.lk - d.lq));
        t0 = std::min(first_row / bq, n_q);
      }
      out.push_back(Item{int32_t(b), int32_t(j), int32_t(t0), int32_t(n_q - t0)});
    }
  }
  lpt_sort(out);
  return out;
}

int64_t visible_pairs(const std::vector<Doc>& docs, bool causal) {
  int64_t tot = 0;
  for (const Doc& d : docs) {
    if (!causal) { tot += d.lq * d.lk; continue; }
    // row i sees min(max(i + off + 1, 0), Lk) keys, off = Lk - Lq
    const int64_t off = d.lk - d.lq;
    // rows with i + off + 1 <= 0 see nothing; rows with i + off + 1 >= Lk see Lk
    const int64_t i_lo = std::max(int64_t(0), -off);           // first row seeing >= 1 key
    const int64_t i_hi = std::min(d.lq, d.lk - off - 1);        // rows [i_lo, i_hi) see < Lk
    if (i_hi > i_lo) {
      // sum_{i=i_lo}^{i_hi-1} (i + off + 1)
      const int64_t a = i_lo + off + 1, z = i_hi - 1 + off + 1, n = i_hi - i_lo;
      tot += (a + z) * n / 2;
    }
    const int64_t full_from = std::max(i_lo, std::max(i_hi, int64_t(0)));
    if (d.lq > full_from) tot += (d.lq - full_from) * d.lk;
  }
  return tot;
}

int64_t issued_pairs(const std::vector<Item>& items, int bq, int bk) {
  int64_t n = 0;
  for (const Item& it : items) n += it.count;
  return n * int64_t(bq) * bk;
}

std::vector<Entry> fwd_entries(const std::vector<Item>& items) {
  std::vector<Entry> out;
  out.reserve(items.size());
  for (const Item& it : items) out.push_back(Entry{it, 0, 1, int64_t(it.count) + 1});
  return out;
}

double bwd_per_cu(const std::vector<Item>& items, int grp, int hkv, int n_cu) {
  int64_t total = 0;
  for (const Item& it : items) total += it.count;
  return double(total) * grp * hkv / double(std::max(n_cu, 1));
}

int item_head_split(int64_t count, int grp, double per_cu, int max_split) {
  int split = 1;
  while (split < max_split && double(count) * grp / split > per_cu) split *= 2;
  return split;
}

std::vector<Entry> bwd_entries(const std::vector<Item>& items, int grp, int hkv, int n_cu,
                               int max_split) {
  const double per_cu = bwd_per_cu(items, grp, hkv, n_cu);
  std::vector<Entry> out;
  out.reserve(items.size());
  for (const Item& it : items) {
    const int n = item_head_split(it.count, grp, per_cu, max_split);
    const int64_t work = int64_t(it.count) * (grp / n);
    for (int s = 0; s < n; ++s) out.push_back(Entry{it, s, n, work + kBwdEntryStartup});
  }
  // longest first by the entries' own work (the items came longest first by
  // count, which is kept among equal weights)
  std::stable_sort(out.begin(), out.end(),
                   [](const Entry& a, const Entry& b) { return a.weight > b.weight; });
  return out;
}

std::vector<DevItem> device_items(const std::vector<Doc>& docs, const std::vector<Entry>& entries) {
  std::vector<DevItem> out(entries.size());
  for (size_t i = 0; i < entries.size(); ++i) {
    const Item& it = entries[i].item;
    const Doc& d = docs[size_t(it.doc)];
    out[i] = DevItem{int32_t(d.q_start), int32_t(d.lq), int32_t(d.k_start), int32_t(d.lk),
                     it.tile, it.first, it.count, int16_t(entries[i].slice),
                     int16_t(entries[i].n_slices)};
  }
  return out;
}

std::vector<int32_t> xcd_slots(const std::vector<Entry>& entries, int n_xcd, int32_t& rows) {
  std::vector<std::vector<int32_t>> lists(size_t(std::max(n_xcd, 1)));
  std::vector<int64_t> load(lists.size(), 0);
  for (size_t i = 0; i < entries.size(); ++i) {
    const size_t x = size_t(std::min_element(load.begin(), load.end()) - load.begin());
    lists[x].push_back(int32_t(i));
    load[x] += entries[i].weight;
  }
  rows = 0;
  for (const auto& l : lists) rows = std::max(rows, int32_t(l.size()));
  std::vector<int32_t> slots(size_t(rows) * lists.size(), -1);
  for (size_t x = 0; x < lists.size(); ++x)
    for (size_t j = 0; j < lists[x].size(); ++j) slots[j * lists.size() + x] = lists[x][j];
  return slots;
}

bool ring_block(const int32_t* cu, int32_t n_docs, int64_t q_begin, int64_t q_end,
                int64_t k_begin, int64_t k_end, int32_t* cu_q, int32_t* cu_k, int32_t& causal,
                int32_t& cls, std::string& err) {
  const int64_t total = cu[n_docs];
  if (q_begin < 0 || q_begin > q_end || q_end > total || k_begin < 0 || k_begin > k_end ||
      k_end > total) {
    err = "chunk ranges must satisfy 0 <= begin <= end <= total tokens";
    return false;
  }
  const bool diagonal = q_begin == k_begin && q_end == k_end;
  const bool keys_before = k_end <= q_begin;
  const bool keys_after = k_begin >= q_end;
  if (!diagonal && !keys_before && !keys_after) {
    err = "the query and key chunks must be equal or disjoint";
    return false;
  }
  // per-document overlap with each chunk; the document spanning both chunks
  // (at most one when they are disjoint) is the only one with visible pairs
  cu_q[0] = 0;
  cu_k[0] = 0;
  int32_t spanning = -1;
  for (int32_t b = 0; b < n_docs; ++b) {
    const int64_t lo = cu[b], hi = cu[b + 1];
    const int64_t lq = std::max<int64_t>(0, std::min(hi, q_end) - std::max(lo, q_begin));
    const int64_t lk = std::max<int64_t>(0, std::min(hi, k_end) - std::max(lo, k_begin));
    cu_q[b + 1] = cu_q[b] + int32_t(lq);
    cu_k[b + 1] = cu_k[b] + int32_t(lk);
    if (lq > 0 && lk > 0) spanning = b;
  }
  if (diagonal) {
    causal = 1;
    cls = kRingA1;
    return true;
  }
  causal = 0;
  if (keys_after || spanning < 0) {
    cls = kRingN;   // keys after the queries, or no document in both chunks
    return true;
  }
  // the spanning document covers the top rows of the query chunk and the
  // right-hand columns of the key chunk
  const int64_t rows = cu_q[spanning + 1] - cu_q[spanning];
  const int64_t cols = cu_k[spanning + 1] - cu_k[spanning];
  const bool all_rows = rows == q_end - q_begin, all_cols = cols == k_end - k_begin;
  cls = all_rows ? (all_cols ? kRingA2 : kRingA4) : (all_cols ? kRingA3 : kRingA5);
  return true;
}

bool basp_shard(int32_t rank, int32_t world, int32_t batch, int64_t seq_len, BaspShard& out,
                std::string& err) {
  if (world <= 0 || batch <= 0) return err = "world and batch must be positive", false;
  if (rank < 0 || rank >= world) return err = "rank out of range", false;
  if (seq_len < 0) return err = "seq_len must be >= 0", false;
  if (batch > world) {
    // more sequences than ranks: plain data parallelism, whole sequences
    if (batch % world) return err = "batch must be a multiple of world when batch > world", false;
    const int32_t per = batch / world;
    out = BaspShard{rank, 1, rank * per, (rank + 1) * per, 0, seq_len};
    return true;
  }
  if (world % batch) return err = "world must be a multiple of batch", false;
  const int32_t k = world / batch;
  if (seq_len % k) return err = "seq_len must be a multiple of the group size", false;
  const int32_t g = rank / k, l = rank % k;
  const int64_t chunk = seq_len / k;
  out = BaspShard{g, k, g, g + 1, l * chunk, (l + 1) * chunk};
  return true;
}

}  // namespace vl
