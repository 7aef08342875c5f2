// C ABI of libvarlen (declared in include/varlen.h): argument validation, the
// cached device work lists, and dispatch to the HIP kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <deque>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "varlen.h"
#include "launch.h"
#include "plan_cache.h"
#include "router.h"
#include "scheduler.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return VL_EHIP;
}

// ------------------------------------------------------------ work-list cache
struct Plan {
  vl::DevItem* dev = nullptr;   // the entries in XCD slot order (rows * kXcds)
  int32_t n = 0;
  int32_t rows = 0;             // entries of the longest XCD list
  int32_t max_count = 0;
  int64_t total_count = 0;
  int32_t max_slices = 1;       // the most slices any item is cut into
  int32_t n_cut = 0;            // cut key tiles, listed after the slots
  vl::ItemMap map() const { return vl::ItemMap{dev, rows, n_cut}; }
};

std::mutex g_mu;
constexpr size_t kMaxPlans = 4096;
vl::PlanCache<Plan> g_plans(kMaxPlans);

// The dK/dV list (pass 1) also depends on the head counts (its q-head split).
std::string plan_key(int dev, int pass, int causal, const int32_t* cu_q, const int32_t* cu_k,
                     int32_t n_docs, int32_t hq, int32_t hkv) {
  std::string key;
  const int32_t hdr[6] = {dev, pass, causal, n_docs, pass == 1 ? hq : 0, pass == 1 ? hkv : 0};
  key.append(reinterpret_cast<const char*>(hdr), sizeof(hdr));
  key.append(reinterpret_cast<const char*>(cu_q), sizeof(int32_t) * size_t(n_docs + 1));
  key.append(reinterpret_cast<const char*>(cu_k), sizeof(int32_t) * size_t(n_docs + 1));
  return key;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

void release_plan(Plan& p) {
  if (p.dev) (void)hipFree(p.dev);
  p.dev = nullptr;
}

void clear_plans_locked() { g_plans.clear(release_plan); }

int max_head_split(int32_t hq, int32_t hkv);
int device_cus();

// pass 0: forward / dQ list (query tiles); pass 1: dK/dV list (key tiles,
// cut by the q-head split).  Builds the list on the host in XCD slot order (a
// workgroup reads its entry with one load; an empty slot has n_slices = 0),
// followed on the dK/dV list by the first slice of every cut key tile (the
// conversion pass's list), and fills the plan's counts.
void build_list(int pass, int causal, const int32_t* cu_q, const int32_t* cu_k, int32_t n_docs,
                int32_t hq, int32_t hkv, std::vector<vl::DevItem>& host, Plan& p) {
  const std::vector<vl::Doc> docs = vl::doc_table(cu_q, cu_k, n_docs);
  const std::vector<vl::Item> items =
      pass == 0 ? vl::fwd_items(docs, causal != 0, vl::kFwdBQ, vl::kFwdBK)
                : vl::bwd_items(docs, causal != 0, vl::kBwdBQ, vl::kBwdBK);
  const std::vector<vl::Entry> entries =
      pass == 0 ? vl::fwd_entries(items)
                : vl::bwd_entries(items, hq / hkv, hkv, device_cus(), max_head_split(hq, hkv));
  const std::vector<vl::DevItem> di = vl::device_items(docs, entries);
  int32_t rows = 0;
  const std::vector<int32_t> slots = vl::xcd_slots(entries, vl::kXcds, rows);
  p = Plan{};
  p.n = int32_t(di.size());
  p.rows = rows;
  for (const auto& it : items) {
    p.max_count = std::max(p.max_count, it.count);
    p.total_count += it.count;
  }
  host.assign(di.empty() ? 0 : slots.size(), vl::DevItem{});
  for (size_t j = 0; j < host.size(); ++j) {
    if (slots[j] < 0) continue;
    host[j] = di[size_t(slots[j])];
    p.max_slices = std::max<int32_t>(p.max_slices, host[j].n_slices);
  }
  for (const vl::DevItem& e : di) {
    if (e.n_slices > 1 && e.slice == 0) {
      host.push_back(e);
      ++p.n_cut;
    }
  }
}

// capturing: the caller's stream is being captured (the plan gets pinned).
int get_plan(int pass, int causal, const int32_t* cu_q, const int32_t* cu_k, int32_t n_docs,
             int32_t hq, int32_t hkv, bool capturing, Plan& out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  const std::string key = plan_key(dev, pass, causal, cu_q, cu_k, n_docs, hq, hkv);
  std::lock_guard<std::mutex> lock(g_mu);
  if (const Plan* hit = g_plans.find(key, capturing)) {
    out = *hit;
    return VL_OK;
  }
  if (capturing)
    return fail(VL_EUNSUPPORTED,
                "a new cu_seqlens pattern under stream capture: run the call once before capturing");
  std::vector<vl::DevItem> host;
  Plan p;
  build_list(pass, causal, cu_q, cu_k, n_docs, hq, hkv, host, p);
  if (!host.empty()) {
    // a new pattern: when the cache is full, drain the device and release the
    // plans no captured graph holds
    if (g_plans.size() >= kMaxPlans) {
      (void)hipDeviceSynchronize();
      if (!g_plans.make_room(release_plan))
        return fail(VL_EUNSUPPORTED,
                    "the plan cache is full of plans captured graphs may use: call "
                    "varlen_cache_clear once those graphs are destroyed");
    }
    const size_t bytes = host.size() * sizeof(vl::DevItem);
    e = hipMalloc(&p.dev, bytes);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(work list)");
    e = hipMemcpy(p.dev, host.data(), bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(p.dev);
      return hip_fail(e, "hipMemcpy(work list)");
    }
  }
  g_plans.insert(key, p, false);
  out = p;
  return VL_OK;
}

// ------------------------------------------------------------ per-call work lists
// With the plan cache off, every call builds its work lists on the host and
// enqueues their upload on its own stream: the lists go into pinned host
// staging and from there, by one asynchronous copy, into a per-device ring
// of device memory.  A region is handed out again only after the event
// recorded behind the last kernel that read it has completed, so a call
// allocates nothing and waits for nothing unless the host runs a whole ring
// ahead of the device, or its lists outgrow half the ring (which then grows
// once, after its in-flight regions have drained).
struct Ring {
  struct Use {
    size_t off, size;
    hipEvent_t ev;
  };
  char* dev = nullptr;
  char* host = nullptr;   // pinned staging, same offsets as dev
  size_t cap = 0, head = 0;
  std::deque<Use> live;   // in reservation order
  std::vector<hipEvent_t> spare;
};

std::atomic<int> g_cache_on{0};   // per-call work lists unless a caller opts in
std::mutex g_ring_mu;
std::map<int, Ring> g_rings;
constexpr size_t kRingMin = size_t(1) << 20;

int ring_retire(Ring& r, std::deque<Ring::Use>::iterator it, bool wait) {
  if (wait) {
    const hipError_t e = hipEventSynchronize(it->ev);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize(work-list ring)");
  }
  r.spare.push_back(it->ev);
  r.live.erase(it);
  return VL_OK;
}

int ring_reserve(Ring& r, size_t bytes, size_t& off) {
  // regions whose readers have finished go back first, oldest first
  while (!r.live.empty() && hipEventQuery(r.live.front().ev) == hipSuccess)
    (void)ring_retire(r, r.live.begin(), false);
  if (bytes > r.cap / 2) {
    while (!r.live.empty()) {
      const int rc = ring_retire(r, r.live.begin(), true);
      if (rc) return rc;
    }
    if (r.dev) (void)hipFree(r.dev);
    if (r.host) (void)hipHostFree(r.host);
    r.dev = r.host = nullptr;
    r.cap = r.head = 0;
    size_t cap = kRingMin;
    while (cap < 4 * bytes) cap *= 2;
    hipError_t e = hipMalloc(reinterpret_cast<void**>(&r.dev), cap);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(work-list ring)");
    e = hipHostMalloc(reinterpret_cast<void**>(&r.host), cap, hipHostMallocDefault);
    if (e != hipSuccess) {
      (void)hipFree(r.dev);
      r.dev = nullptr;
      return hip_fail(e, "hipHostMalloc(work-list staging)");
    }
    r.cap = cap;
  }
  off = r.head + bytes <= r.cap ? r.head : 0;
  for (auto it = r.live.begin(); it != r.live.end();) {
    if (it->off < off + bytes && off < it->off + it->size) {
      const int rc = ring_retire(r, it, true);
      if (rc) return rc;
      it = r.live.begin();
    } else {
      ++it;
    }
  }
  r.head = off + bytes;
  return VL_OK;
}

// The work lists of one call: from the cache, or (cache off) built for this
// call and uploaded into the ring.  With the ring, the lock is held until the
// destructor has recorded the event behind the call's kernels.
class CallPlans {
 public:
  ~CallPlans() {
    if (!ring_) return;
    hipEvent_t ev = nullptr;
    if (!ring_->spare.empty()) {
      ev = ring_->spare.back();
      ring_->spare.pop_back();
    } else if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) {
      ev = nullptr;
    }
    if (ev && hipEventRecord(ev, st_) == hipSuccess) {
      ring_->live.push_back(Ring::Use{off_, size_, ev});
    } else {
      // no event: the region is free once the stream has drained
      if (ev) ring_->spare.push_back(ev);
      (void)hipStreamSynchronize(st_);
    }
  }

  int get(int causal, const int32_t* cu_q, const int32_t* cu_k, int32_t n_docs, int32_t hq,
          int32_t hkv, hipStream_t st, int n_pass, const int* passes, Plan* out) {
    if (n_pass < 1 || n_pass > 2) return fail(VL_EINVAL, "internal: one or two work lists per call");
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const bool capturing =
        hipStreamIsCapturing(st, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone;
    if (g_cache_on.load()) {
      for (int i = 0; i < n_pass; ++i) {
        const int rc = get_plan(passes[i], causal, cu_q, cu_k, n_docs, hq, hkv, capturing, out[i]);
        if (rc) return rc;
      }
      return VL_OK;
    }
    if (capturing)
      return fail(VL_EUNSUPPORTED,
                  "with the plan cache off a call uploads its work lists and cannot be captured");
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::vector<vl::DevItem> host[2];
    size_t at[2] = {0, 0}, total = 0;
    for (int i = 0; i < n_pass; ++i) {
      build_list(passes[i], causal, cu_q, cu_k, n_docs, hq, hkv, host[i], out[i]);
      at[i] = total;
      total += align256(host[i].size() * sizeof(vl::DevItem));
    }
    if (total == 0) return VL_OK;
    lock_ = std::unique_lock<std::mutex>(g_ring_mu);
    Ring& r = g_rings[dev];
    size_t off = 0;
    const int rc = ring_reserve(r, total, off);
    if (rc) return rc;
    for (int i = 0; i < n_pass; ++i) {
      if (host[i].empty()) continue;
      std::memcpy(r.host + off + at[i], host[i].data(), host[i].size() * sizeof(vl::DevItem));
      out[i].dev = reinterpret_cast<vl::DevItem*>(r.dev + off + at[i]);
    }
    e = hipMemcpyAsync(r.dev + off, r.host + off, total, hipMemcpyHostToDevice, st);
    // from here on the region is in flight: the destructor records its event
    ring_ = &r;
    off_ = off;
    size_ = total;
    st_ = st;
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(work list)");
    return VL_OK;
  }

 private:
  std::unique_lock<std::mutex> lock_;
  Ring* ring_ = nullptr;
  size_t off_ = 0, size_ = 0;
  hipStream_t st_ = nullptr;
};

// ------------------------------------------------------------ validation
int check_attn_common(const void* q, const void* k, const void* v, const int32_t* cu_q,
                      const int32_t* cu_k, int32_t n_docs, int64_t total_q, int64_t total_k,
                      int32_t hq, int32_t hkv, int32_t d) {
  if (!q || !k || !v) return fail(VL_EINVAL, "q, k and v must be non-null device pointers");
  if (!cu_q || !cu_k) return fail(VL_EINVAL, "cu_seqlens_q and cu_seqlens_k must be non-null");
  if (n_docs < 0) return fail(VL_EINVAL, "n_docs must be >= 0");
  if (total_q < 0 || total_k < 0) return fail(VL_EINVAL, "total token counts must be >= 0");
  if (total_q > INT32_MAX || total_k > INT32_MAX)
    return fail(VL_ESHAPE, "total token counts must fit int32");
  if (hq <= 0 || hkv <= 0) return fail(VL_ESHAPE, "head counts must be positive");
  if (hq % hkv != 0) return fail(VL_ESHAPE, "n_heads_q must be a multiple of n_heads_kv");
  if (d != 64 && d != 128) return fail(VL_EUNSUPPORTED, "head_dim must be 64 or 128");
  std::string err;
  if (!vl::validate_cu(cu_q, n_docs, total_q, err)) return fail(VL_ESEQLENS, "cu_seqlens_q: " + err);
  if (!vl::validate_cu(cu_k, n_docs, total_k, err)) return fail(VL_ESEQLENS, "cu_seqlens_k: " + err);
  const uintptr_t al = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                       reinterpret_cast<uintptr_t>(v);
  if (al % 16) return fail(VL_EINVAL, "q, k and v must be 16-byte aligned");
  return VL_OK;
}

float resolve_scale(float s, int d) { return s > 0.f ? s : 1.0f / std::sqrt(float(d)); }

// The largest q-head split the backward may choose: a power of two dividing
// the group size, at most vl::kMaxHeadSplit.
int max_head_split(int32_t hq, int32_t hkv) {
  const int grp = hkv > 0 ? hq / hkv : 1;
  int split = 1;
  while (split < grp && grp % (split * 2) == 0 && split * 2 <= vl::kMaxHeadSplit) split *= 2;
  return split;
}

// Compute units of the current device (cached per device).
int device_cus() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int n_cu = 0;
  if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n_cu <= 0)
    n_cu = 256;
  cache[dev] = n_cu;
  return n_cu;
}

// The most slices the dK/dV list cuts any item into (the q heads of a group
// go to 2-4 workgroups for the items that would otherwise outlast the
// average per-CU share of the pass): the number of fp32 partials the
// workspace holds.
int choose_split(const int32_t* cu_q, const int32_t* cu_k, int32_t n_docs, int causal,
                 int32_t hq, int32_t hkv, int n_cu) {
  const std::vector<vl::Doc> docs = vl::doc_table(cu_q, cu_k, n_docs);
  const std::vector<vl::Item> items = vl::bwd_items(docs, causal != 0, vl::kBwdBQ, vl::kBwdBK);
  int32_t max_count = 0;
  for (const auto& it : items) max_count = std::max(max_count, it.count);
  return vl::item_head_split(max_count, hq / hkv, vl::bwd_per_cu(items, hq / hkv, hkv, n_cu),
                             max_head_split(hq, hkv));
}

// Workspace of one backward call: D [Hq, Tq] fp32, then the fp32 dK/dV
// partials of the q-head slices when the group is split.
size_t bwd_workspace_bytes(int64_t total_q, int64_t total_k, int32_t hq, int32_t hkv, int32_t d,
                           int split) {
  return align256(size_t(total_q) * size_t(hq) * 4) +
         (split > 1 ? align256(size_t(split) * 2 * size_t(total_k) * size_t(hkv) * size_t(d) * 4)
                    : 0);
}

}  // namespace

extern "C" {

const char* varlen_last_error(void) { return g_err.c_str(); }

int varlen_version(void) { return 1; }

void varlen_cache_clear(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  clear_plans_locked();
}

int varlen_set_plan_cache(int32_t on) { return g_cache_on.exchange(on != 0 ? 1 : 0); }

int varlen_attn_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                    const int32_t* cu_seqlens_k, int32_t n_docs, int64_t total_q, int64_t total_k,
                    int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, float softmax_scale,
                    int32_t causal, int32_t out_dtype, void* out, float* lse, void* stream) {
  try {
    g_err.clear();
    int rc = check_attn_common(q, k, v, cu_seqlens_q, cu_seqlens_k, n_docs, total_q, total_k,
                               n_heads_q, n_heads_kv, head_dim);
    if (rc) return rc;
    if (out_dtype != VL_BF16 && out_dtype != VL_F32) return fail(VL_EINVAL, "out_dtype must be VL_BF16 or VL_F32");
    if (!out || !lse) return fail(VL_EINVAL, "out and lse must be non-null");
    if (reinterpret_cast<uintptr_t>(out) % 16) return fail(VL_EINVAL, "out must be 16-byte aligned");
    if (total_q == 0) return VL_OK;
    Plan p;
    CallPlans plans;
    const int pass0 = 0;
    rc = plans.get(causal != 0, cu_seqlens_q, cu_seqlens_k, n_docs, n_heads_q, n_heads_kv,
                   reinterpret_cast<hipStream_t>(stream), 1, &pass0, &p);
    if (rc) return rc;
    vl::AttnShape s{total_q, total_k, n_heads_q, n_heads_kv, head_dim,
                    resolve_scale(softmax_scale, head_dim), causal != 0};
    hipError_t e = vl::launch_attn_fwd(s, q, k, v, p.map(), out_dtype == VL_F32 ? vl::kOutF32 : vl::kOutBf16, out, lse,
                                       reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "attn_fwd launch");
    return VL_OK;
  } catch (const std::exception& ex) {
    return fail(VL_EHIP, std::string("internal error: ") + ex.what());
  } catch (...) {
    return fail(VL_EHIP, "internal error");
  }
}

int varlen_attn_fwd_acc(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_k, int32_t n_docs, int64_t total_q,
                        int64_t total_k, int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                        float softmax_scale, int32_t causal, float* o_acc, float* lse_acc,
                        void* stream) {
  try {
    g_err.clear();
    int rc = check_attn_common(q, k, v, cu_seqlens_q, cu_seqlens_k, n_docs, total_q, total_k,
                               n_heads_q, n_heads_kv, head_dim);
    if (rc) return rc;
    if (!o_acc || !lse_acc) return fail(VL_EINVAL, "o_acc and lse_acc must be non-null");
    if (reinterpret_cast<uintptr_t>(o_acc) % 16) return fail(VL_EINVAL, "o_acc must be 16-byte aligned");
    if (total_q == 0) return VL_OK;
    Plan p;
    CallPlans plans;
    const int pass0 = 0;
    rc = plans.get(causal != 0, cu_seqlens_q, cu_seqlens_k, n_docs, n_heads_q, n_heads_kv,
                   reinterpret_cast<hipStream_t>(stream), 1, &pass0, &p);
    if (rc) return rc;
    vl::AttnShape s{total_q, total_k, n_heads_q, n_heads_kv, head_dim,
                    resolve_scale(softmax_scale, head_dim), causal != 0};
    hipError_t e = vl::launch_attn_fwd(s, q, k, v, p.map(), vl::kOutAcc, o_acc, lse_acc,
                                       reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "attn_fwd launch");
    return VL_OK;
  } catch (const std::exception& ex) {
    return fail(VL_EHIP, std::string("internal error: ") + ex.what());
  } catch (...) {
    return fail(VL_EHIP, "internal error");
  }
}

size_t varlen_attn_bwd_workspace_size(int64_t total_q, int64_t total_k, int32_t n_heads_q,
                                      int32_t n_heads_kv, int32_t head_dim) {
  if (total_q < 0 || total_k < 0 || n_heads_q <= 0 || n_heads_kv <= 0 || head_dim <= 0) return 0;
  if (n_heads_q % n_heads_kv) return 0;
  return bwd_workspace_bytes(total_q, total_k, n_heads_q, n_heads_kv, head_dim,
                             max_head_split(n_heads_q, n_heads_kv));
}

size_t varlen_attn_bwd_workspace_size_cu(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                         int32_t n_docs, int64_t total_q, int64_t total_k,
                                         int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                                         int32_t causal) {
  try {
    g_err.clear();
    if (!cu_seqlens_q || !cu_seqlens_k || n_docs < 0 || total_q < 0 || total_k < 0 ||
        n_heads_q <= 0 || n_heads_kv <= 0 || head_dim <= 0 || n_heads_q % n_heads_kv)
      return 0;
    std::string err;
    if (!vl::validate_cu(cu_seqlens_q, n_docs, total_q, err) ||
        !vl::validate_cu(cu_seqlens_k, n_docs, total_k, err))
      return 0;
    const int split = choose_split(cu_seqlens_q, cu_seqlens_k, n_docs, causal, n_heads_q,
                                   n_heads_kv, device_cus());
    return bwd_workspace_bytes(total_q, total_k, n_heads_q, n_heads_kv, head_dim, split);
  } catch (...) {
    return 0;
  }
}

int varlen_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                    const float* lse, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                    int32_t n_docs, int64_t total_q, int64_t total_k, int32_t n_heads_q,
                    int32_t n_heads_kv, int32_t head_dim, float softmax_scale, int32_t causal,
                    void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                    void* stream) {
  try {
    g_err.clear();
    int rc = check_attn_common(q, k, v, cu_seqlens_q, cu_seqlens_k, n_docs, total_q, total_k,
                               n_heads_q, n_heads_kv, head_dim);
    if (rc) return rc;
    if (!out || !dout || !lse || !dq || !dk || !dv)
      return fail(VL_EINVAL, "out, dout, lse, dq, dk and dv must be non-null");
    const uintptr_t al = reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(dout) |
                         reinterpret_cast<uintptr_t>(dq) | reinterpret_cast<uintptr_t>(dk) |
                         reinterpret_cast<uintptr_t>(dv);
    if (al % 16) return fail(VL_EINVAL, "out, dout, dq, dk and dv must be 16-byte aligned");
    const int n_cu = device_cus();
    const int split = choose_split(cu_seqlens_q, cu_seqlens_k, n_docs, causal, n_heads_q,
                                   n_heads_kv, n_cu);
    const size_t need = bwd_workspace_bytes(total_q, total_k, n_heads_q, n_heads_kv, head_dim, split);
    if (!workspace || workspace_bytes < need)
      return fail(VL_EWORKSPACE, "workspace must hold at least " + std::to_string(need) + " bytes");
    if (reinterpret_cast<uintptr_t>(workspace) % 256) return fail(VL_EWORKSPACE, "workspace must be 256-byte aligned");
    if (total_q == 0 && total_k == 0) return VL_OK;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    Plan pp[2];
    CallPlans plans;
    const int passes[2] = {0, 1};
    rc = plans.get(causal != 0, cu_seqlens_q, cu_seqlens_k, n_docs, n_heads_q, n_heads_kv, st, 2,
                   passes, pp);
    if (rc) return rc;
    const Plan& pf = pp[0];
    const Plan& pb = pp[1];
    // dK/dV of kv tiles that no query tile reaches are zeros written by the kernel
    float* delta = reinterpret_cast<float*>(workspace);
    float* dkv_acc = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                              align256(size_t(total_q) * size_t(n_heads_q) * 4));
    vl::AttnShape s{total_q, total_k, n_heads_q, n_heads_kv, head_dim,
                    resolve_scale(softmax_scale, head_dim), causal != 0};
    if (pb.max_slices > split) return fail(VL_EHIP, "internal: the dK/dV list outgrew its workspace");
    hipError_t e = vl::launch_attn_bwd(s, q, k, v, out, dout, lse, pf.map(), pb.map(), split, dq,
                                       dk, dv, delta, dkv_acc, st);
    if (e != hipSuccess) return hip_fail(e, "attn_bwd launch");
    return VL_OK;
  } catch (const std::exception& ex) {
    return fail(VL_EHIP, std::string("internal error: ") + ex.what());
  } catch (...) {
    return fail(VL_EHIP, "internal error");
  }
}

int varlen_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* out,
                            const void* dout, const float* lse, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, int32_t n_docs, int64_t total_q,
                            int64_t total_k, int32_t n_heads_q, int32_t n_heads_kv,
                            int32_t head_dim, float softmax_scale, int32_t causal, void* dq,
                            void* dk, void* dv, void* stream) {
  try {
    g_err.clear();
    int rc = check_attn_common(q, k, v, cu_seqlens_q, cu_seqlens_k, n_docs, total_q, total_k,
                               n_heads_q, n_heads_kv, head_dim);
    if (rc) return rc;
    if (!out || !dout || !lse || !dq || !dk || !dv)
      return fail(VL_EINVAL, "out, dout, lse, dq, dk and dv must be non-null");
    const uintptr_t al = reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(dout) |
                         reinterpret_cast<uintptr_t>(dq) | reinterpret_cast<uintptr_t>(dk) |
                         reinterpret_cast<uintptr_t>(dv);
    if (al % 16) return fail(VL_EINVAL, "out, dout, dq, dk and dv must be 16-byte aligned");
    // the same split and work lists as varlen_attn_bwd, laid out in the
    // device scratch: D, the dK/dV partials, then the two work lists
    const int split = choose_split(cu_seqlens_q, cu_seqlens_k, n_docs, causal, n_heads_q,
                                   n_heads_kv, device_cus());
    const size_t ws = bwd_workspace_bytes(total_q, total_k, n_heads_q, n_heads_kv, head_dim, split);
    std::vector<vl::DevItem> host[2];
    Plan pl[2];
    for (int i = 0; i < 2; ++i)
      build_list(i, causal != 0, cu_seqlens_q, cu_seqlens_k, n_docs, n_heads_q, n_heads_kv,
                 host[i], pl[i]);
    const size_t off0 = ws;
    const size_t off1 = off0 + align256(host[0].size() * sizeof(vl::DevItem));
    const size_t need = off1 + align256(host[1].size() * sizeof(vl::DevItem));
    if (need > vl::kNoallocScratchBytes)
      return fail(VL_EWORKSPACE, "this call needs " + std::to_string(need) +
                                     " bytes of device scratch; varlen_attn_bwd_noalloc has " +
                                     std::to_string(vl::kNoallocScratchBytes) +
                                     " (use varlen_attn_bwd with a workspace)");
    if (total_q == 0 && total_k == 0) return VL_OK;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone)
      return fail(VL_EUNSUPPORTED,
                  "varlen_attn_bwd_noalloc copies its work lists from host memory and cannot be "
                  "captured");
    void* base = nullptr;
    hipError_t e = vl::noalloc_scratch(&base);
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    char* sc = reinterpret_cast<char*>(base);
    for (int i = 0; i < 2; ++i) {
      if (host[i].empty()) continue;
      pl[i].dev = reinterpret_cast<vl::DevItem*>(sc + (i == 0 ? off0 : off1));
      // the lists live in pageable host memory: the copy has read them when it returns
      e = hipMemcpyAsync(pl[i].dev, host[i].data(), host[i].size() * sizeof(vl::DevItem),
                         hipMemcpyHostToDevice, st);
      if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(work list)");
    }
    float* delta = reinterpret_cast<float*>(sc);
    float* dkv_acc = reinterpret_cast<float*>(sc + align256(size_t(total_q) * size_t(n_heads_q) * 4));
    vl::AttnShape s{total_q, total_k, n_heads_q, n_heads_kv, head_dim,
                    resolve_scale(softmax_scale, head_dim), causal != 0};
    if (pl[1].max_slices > split) return fail(VL_EHIP, "internal: the dK/dV list outgrew its scratch");
    e = vl::launch_attn_bwd(s, q, k, v, out, dout, lse, pl[0].map(), pl[1].map(), split, dq, dk,
                            dv, delta, dkv_acc, st);
    if (e != hipSuccess) return hip_fail(e, "attn_bwd launch");
    return VL_OK;
  } catch (const std::exception& ex) {
    return fail(VL_EHIP, std::string("internal error: ") + ex.what());
  } catch (...) {
    return fail(VL_EHIP, "internal error");
  }
}

int attn_lse_merge(int32_t n_parts, const void* const* o_parts, const float* const* lse_parts,
                   int32_t in_dtype, int64_t n_rows, int32_t n_heads, int32_t head_dim,
                   void* o_out, float* lse_out, int32_t out_dtype, void* stream) {
  try {
    g_err.clear();
    if (n_parts < 1 || n_parts > vl::kMaxMergeParts)
      return fail(VL_EINVAL, "n_parts must be in [1, 64]");
    if (!o_parts || !lse_parts || !o_out || !lse_out)
      return fail(VL_EINVAL, "pointer arguments must be non-null");
    if ((in_dtype != VL_BF16 && in_dtype != VL_F32) || (out_dtype != VL_BF16 && out_dtype != VL_F32))
      return fail(VL_EINVAL, "dtypes must be VL_BF16 or VL_F32");
    if (n_rows < 0 || n_heads <= 0) return fail(VL_ESHAPE, "n_rows must be >= 0 and n_heads > 0");
    if (head_dim < 4 || head_dim > 256 || (head_dim & (head_dim - 1)))
      return fail(VL_EUNSUPPORTED, "head_dim must be a power of two in [4, 256]");
    const uintptr_t need_in = in_dtype == VL_F32 ? 16 : 8;
    const uintptr_t need_out = out_dtype == VL_F32 ? 16 : 8;
    for (int i = 0; i < n_parts; ++i) {
      if (!o_parts[i] || !lse_parts[i]) return fail(VL_EINVAL, "partial pointers must be non-null");
      if (reinterpret_cast<uintptr_t>(o_parts[i]) % need_in)
        return fail(VL_EINVAL, "partial O buffers must be aligned to 4 elements");
      if (o_parts[i] == o_out) return fail(VL_EINVAL, "o_out must not alias a partial");
    }
    if (reinterpret_cast<uintptr_t>(o_out) % need_out) return fail(VL_EINVAL, "o_out must be aligned to 4 elements");
    hipError_t e = vl::launch_lse_merge(n_parts, o_parts, lse_parts, in_dtype, n_rows, n_heads,
                                        head_dim, o_out, lse_out, out_dtype,
                                        reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "lse_merge launch");
    return VL_OK;
  } catch (...) {
    return fail(VL_EHIP, "internal error");
  }
}

static int permute_common(const void* src, void* dst, int64_t n_tokens, int32_t n_heads,
                          int32_t head_dim, int32_t sp_degree, int32_t elem_bytes, int dir,
                          void* stream) {
  g_err.clear();
  if (n_tokens < 0 || n_heads <= 0 || head_dim <= 0) return fail(VL_ESHAPE, "sizes must be positive");
  if (n_tokens > 0 && (!src || !dst)) return fail(VL_EINVAL, "x and y must be non-null");
  if (elem_bytes != 2 && elem_bytes != 4) return fail(VL_EINVAL, "elem_bytes must be 2 or 4");
  if (sp_degree <= 0 || n_heads % sp_degree) return fail(VL_ESHAPE, "sp_degree must divide n_heads");
  if (n_tokens == 0) return VL_OK;
  const int64_t bytes = n_tokens * n_heads * int64_t(head_dim) * elem_bytes;
  const char* s = reinterpret_cast<const char*>(src);
  const char* d = reinterpret_cast<const char*>(dst);
  if (n_tokens > 0 && s < d + bytes && d < s + bytes) return fail(VL_EINVAL, "x and y must not overlap");
  if (int64_t(n_heads) * head_dim * elem_bytes >= (int64_t(1) << 30))
    return fail(VL_ESHAPE, "a token row must be below 1 GiB");
  if (n_tokens >= (int64_t(1) << 31)) return fail(VL_ESHAPE, "n_tokens must fit int32");
  hipError_t e = vl::launch_sp_permute(src, dst, n_tokens, n_heads, head_dim, sp_degree, elem_bytes,
                                       dir, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sp_permute launch");
  return VL_OK;
}

int sp_seq2head(const void* x, void* y, int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                int32_t sp_degree, int32_t elem_bytes, void* stream) {
  try {
    return permute_common(x, y, n_tokens, n_heads, head_dim, sp_degree, elem_bytes, 0, stream);
  } catch (...) {
    return fail(VL_EHIP, "internal error");
  }
}

int sp_head2seq(const void* y, void* x, int64_t n_tokens, int32_t n_heads, int32_t head_dim,
                int32_t sp_degree, int32_t elem_bytes, void* stream) {
  try {
    return permute_common(y, x, n_tokens, n_heads, head_dim, sp_degree, elem_bytes, 1, stream);
  } catch (...) {
    return fail(VL_EHIP, "internal error");
  }
}

static int qkv_common(const void* const src[3], void* const dst[3], int64_t n_tokens,
                      int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, int32_t sp_degree,
                      int32_t dtype, int dir, void* stream) {
  g_err.clear();
  if (n_tokens < 0 || n_heads_q <= 0 || n_heads_kv <= 0 || head_dim <= 0 || sp_degree <= 0)
    return fail(VL_ESHAPE, "sizes must be positive");
  if (n_heads_q % sp_degree) return fail(VL_ESHAPE, "sp_degree must divide n_heads_q");
  if (n_heads_q % n_heads_kv) return fail(VL_ESHAPE, "n_heads_kv must divide n_heads_q");
  if (n_heads_kv % sp_degree && sp_degree % n_heads_kv)
    return fail(VL_ESHAPE, "one of sp_degree, n_heads_kv must divide the other");
  if (dtype != VL_BF16 && dtype != VL_F32) return fail(VL_EINVAL, "dtype must be VL_BF16 or VL_F32");
  const int64_t eb = dtype == VL_BF16 ? 2 : 4;
  if (head_dim * eb % 4) return fail(VL_EUNSUPPORTED, "head_dim * element size must be a multiple of 4 bytes");
  if (n_tokens >= (int64_t(1) << 31)) return fail(VL_ESHAPE, "n_tokens must fit int32");
  if (int64_t(n_heads_q) * head_dim * eb >= (int64_t(1) << 30))
    return fail(VL_ESHAPE, "a token row must be below 1 GiB");
  if (n_tokens == 0) return VL_OK;
  const int64_t hk = n_heads_kv >= sp_degree ? n_heads_kv / sp_degree : 1;
  // bytes of the [n, H, d] side and of the [P, n, hs, d] side, for Q, K, V
  const int64_t xb[3] = {n_tokens * n_heads_q * head_dim * eb, n_tokens * n_heads_kv * head_dim * eb,
                         n_tokens * n_heads_kv * head_dim * eb};
  const int64_t yb[3] = {xb[0], sp_degree * n_tokens * hk * head_dim * eb,
                         sp_degree * n_tokens * hk * head_dim * eb};
  const char* lo[6];
  int64_t len[6];
  for (int i = 0; i < 3; ++i) {
    if (!src[i] || !dst[i]) return fail(VL_EINVAL, "tensors must be non-null");
    if ((reinterpret_cast<uintptr_t>(src[i]) | reinterpret_cast<uintptr_t>(dst[i])) % 4)
      return fail(VL_EINVAL, "tensors must be 4-byte aligned");
    lo[i] = reinterpret_cast<const char*>(src[i]);
    lo[3 + i] = reinterpret_cast<const char*>(dst[i]);
    len[i] = dir == 0 ? xb[i] : yb[i];
    len[3 + i] = dir == 0 ? yb[i] : xb[i];
  }
  // an output may overlap no input and no other output (inputs may alias each other)
  for (int a = 3; a < 6; ++a)
    for (int b = 0; b < 6; ++b)
      if (a != b && lo[a] < lo[b] + len[b] && lo[b] < lo[a] + len[a])
        return fail(VL_EINVAL, "an output overlaps another tensor");
  vl::QkvTensors t{{src[0], src[1], src[2]}, {dst[0], dst[1], dst[2]}};
  hipError_t e = vl::launch_sp_qkv(t, n_tokens, n_heads_q, n_heads_kv, head_dim, sp_degree, dtype,
                                   dir, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sp_qkv launch");
  return VL_OK;
}

int sp_qkv_seq2head(const void* q, const void* k, const void* v, void* yq, void* yk, void* yv,
                    int64_t n_tokens, int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                    int32_t sp_degree, int32_t dtype, void* stream) {
  try {
    const void* src[3] = {q, k, v};
    void* dst[3] = {yq, yk, yv};
    return qkv_common(src, dst, n_tokens, n_heads_q, n_heads_kv, head_dim, sp_degree, dtype, 0,
                      stream);
  } catch (...) {
    return fail(VL_EHIP, "internal error");
  }
}

int sp_qkv_head2seq(const void* yq, const void* yk, const void* yv, void* dq, void* dk, void* dv,
                    int64_t n_tokens, int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                    int32_t sp_degree, int32_t dtype, void* stream) {
  try {
    const void* src[3] = {yq, yk, yv};
    void* dst[3] = {dq, dk, dv};
    return qkv_common(src, dst, n_tokens, n_heads_q, n_heads_kv, head_dim, sp_degree, dtype, 1,
                      stream);
  } catch (...) {
    return fail(VL_EHIP, "internal error");
  }
}

int basp_shard(int32_t rank, int32_t world, int32_t batch, int64_t seq_len, int32_t* group,
               int32_t* group_size, int32_t* seq_begin, int32_t* seq_end, int64_t* tok_begin,
               int64_t* tok_end) {
  try {
    g_err.clear();
    if (!group || !group_size || !seq_begin || !seq_end || !tok_begin || !tok_end)
      return fail(VL_EINVAL, "null argument");
    vl::BaspShard sh;
    std::string err;
    if (!vl::basp_shard(rank, world, batch, seq_len, sh, err)) return fail(VL_ESHAPE, err);
    *group = sh.group;
    *group_size = sh.group_size;
    *seq_begin = sh.seq_begin;
    *seq_end = sh.seq_end;
    *tok_begin = sh.tok_begin;
    *tok_end = sh.tok_end;
    return VL_OK;
  } catch (...) {
    return fail(VL_EINVAL, "internal error");
  }
}

static bool finite_nonneg(double x) { return std::isfinite(x) && x >= 0.0; }

static int cost_params(const vl_cost_model* c, vl::CostParams& cm) {
  if (!c) return fail(VL_EINVAL, "cost model is null");
  if (c->n_points < 1 || !c->curve_len || !c->fwd_tflops || !c->bwd_tflops)
    return fail(VL_EINVAL, "cost model needs a throughput curve of >= 1 point");
  for (int32_t i = 0; i < c->n_points; ++i) {
    if (!(std::isfinite(c->curve_len[i]) && c->curve_len[i] > 0) ||
        (i > 0 && !(c->curve_len[i] > c->curve_len[i - 1])))
      return fail(VL_EINVAL, "curve lengths must be positive and strictly increasing");
    if (!(std::isfinite(c->fwd_tflops[i]) && c->fwd_tflops[i] > 0) ||
        !(std::isfinite(c->bwd_tflops[i]) && c->bwd_tflops[i] > 0))
      return fail(VL_EINVAL, "curve throughputs must be positive");
  }
  const double scalars[] = {c->fwd_flops_per_pair, c->bwd_flops_per_pair, c->bytes_per_token[0],
                            c->bytes_per_token[1], c->bytes_per_token[2], c->bytes_per_token[3],
                            c->a2a_alpha_us, c->dense_fwd_flops_per_token,
                            c->dense_bwd_flops_per_token};
  for (double x : scalars)
    if (!finite_nonneg(x)) return fail(VL_EINVAL, "cost model terms must be finite and >= 0");
  if (!(std::isfinite(c->a2a_gbs) && c->a2a_gbs > 0) ||
      !(std::isfinite(c->dense_tflops) && c->dense_tflops > 0))
    return fail(VL_EINVAL, "bandwidth and dense throughput must be positive");
  cm.curve_len.assign(c->curve_len, c->curve_len + c->n_points);
  cm.fwd_tflops.assign(c->fwd_tflops, c->fwd_tflops + c->n_points);
  cm.bwd_tflops.assign(c->bwd_tflops, c->bwd_tflops + c->n_points);
  cm.fwd_flops_per_pair = c->fwd_flops_per_pair;
  cm.bwd_flops_per_pair = c->bwd_flops_per_pair;
  for (int i = 0; i < 4; ++i) cm.bytes_per_token[i] = c->bytes_per_token[i];
  cm.a2a_gbs = c->a2a_gbs;
  cm.a2a_alpha_us = c->a2a_alpha_us;
  cm.dense_fwd_flops_per_token = c->dense_fwd_flops_per_token;
  cm.dense_bwd_flops_per_token = c->dense_bwd_flops_per_token;
  cm.dense_tflops = c->dense_tflops;
  return VL_OK;
}

static int sample_lengths(const int64_t* lengths, int32_t n, std::vector<double>& L) {
  if (n < 0) return fail(VL_EINVAL, "n_samples must be >= 0");
  if (n > 0 && !lengths) return fail(VL_EINVAL, "lengths is null");
  L.resize(size_t(n));
  for (int32_t j = 0; j < n; ++j) {
    if (lengths[j] < 0) return fail(VL_EINVAL, "lengths must be >= 0");
    L[j] = double(lengths[j]);
  }
  return VL_OK;
}

static void copy_out(const std::vector<double>& v, double* dst) {
  if (dst) std::memcpy(dst, v.data(), sizeof(double) * v.size());
}

int nsp_route(const int64_t* lengths, int32_t n_samples, int32_t n_gpus, int32_t sp_max,
              const vl_cost_model* cost, double token_budget, int32_t prefix, int32_t beam,
              int32_t monotone, int32_t level_mask, int32_t* node_depth, int32_t* node_index,
              double* gpu_fwd, double* gpu_bwd, double* gpu_tokens, int32_t* within_budget) {
  try {
    g_err.clear();
    std::vector<double> L;
    vl::CostParams cm;
    int rc = sample_lengths(lengths, n_samples, L);
    if (rc) return rc;
    if ((rc = cost_params(cost, cm))) return rc;
    if (n_samples > 0 && (!node_depth || !node_index)) return fail(VL_EINVAL, "node outputs are null");
    if (std::isnan(token_budget)) return fail(VL_EINVAL, "token_budget is NaN");
    if (prefix < 0 || beam < 1) return fail(VL_EINVAL, "prefix must be >= 0 and beam >= 1");
    std::vector<vl::TreeNode> nodes;
    vl::RouteResult r;
    std::string err;
    if (!vl::sp_tree(n_gpus, sp_max, level_mask, nodes, err)) return fail(VL_ESHAPE, err);
    if (!vl::nsp_route(L, n_gpus, sp_max, cm, token_budget, prefix, beam, monotone != 0,
                       level_mask, nodes, r, err))
      return fail(VL_EINVAL, err);
    for (int32_t j = 0; j < n_samples; ++j) {
      node_depth[j] = nodes[r.node[j]].depth;
      node_index[j] = nodes[r.node[j]].index;
    }
    copy_out(r.dfwd, gpu_fwd);
    copy_out(r.dbwd, gpu_bwd);
    copy_out(r.tok, gpu_tokens);
    if (within_budget) *within_budget = r.within_budget ? 1 : 0;
    return VL_OK;
  } catch (const std::exception& ex) {
    return fail(VL_EINVAL, std::string("internal error: ") + ex.what());
  }
}

int nsp_plan_cost(const int64_t* lengths, int32_t n_samples, int32_t n_gpus, int32_t sp_max,
                  const vl_cost_model* cost, const int32_t* node_depth, const int32_t* node_index,
                  double* gpu_fwd, double* gpu_bwd, double* gpu_tokens) {
  try {
    g_err.clear();
    std::vector<double> L;
    vl::CostParams cm;
    int rc = sample_lengths(lengths, n_samples, L);
    if (rc) return rc;
    if ((rc = cost_params(cost, cm))) return rc;
    if (n_samples > 0 && (!node_depth || !node_index)) return fail(VL_EINVAL, "plan is null");
    std::vector<vl::TreeNode> nodes;
    std::string err;
    if (!vl::sp_tree(n_gpus, sp_max, -1, nodes, err)) return fail(VL_ESHAPE, err);
    // node (d, i) sits at offset (trees (2^d - 1)) + i in the full node list
    const int32_t trees = n_gpus / sp_max;
    const int32_t K = nodes.back().depth;
    std::vector<int32_t> node_of(static_cast<size_t>(n_samples));
    for (int32_t j = 0; j < n_samples; ++j) {
      const int32_t d = node_depth[j], i = node_index[j];
      if (d < 0 || d > K || i < 0 || i >= (trees << d))
        return fail(VL_ESHAPE, "a node lies outside the tree");
      node_of[j] = trees * ((1 << d) - 1) + i;
    }
    std::vector<double> f, b, t;
    vl::nsp_plan_cost(L, nodes, node_of, n_gpus, cm, f, b, t);
    copy_out(f, gpu_fwd);
    copy_out(b, gpu_bwd);
    copy_out(t, gpu_tokens);
    return VL_OK;
  } catch (const std::exception& ex) {
    return fail(VL_EINVAL, std::string("internal error: ") + ex.what());
  }
}

int varlen_mfma_probe(int32_t iters, int32_t n_workgroups, float* sink, int64_t* flops,
                      void* stream) {
  try {
    g_err.clear();
    if (iters <= 0 || n_workgroups <= 0) return fail(VL_EINVAL, "iters and n_workgroups must be positive");
    if (!sink) return fail(VL_EINVAL, "sink must be non-null");
    if (flops) *flops = vl::mfma_probe_flops(iters, n_workgroups);
    hipError_t e = vl::launch_mfma_probe(iters, n_workgroups, sink,
                                         reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "mfma_probe launch");
    return VL_OK;
  } catch (...) {
    return fail(VL_EHIP, "internal error");
  }
}

int varlen_ring_block(const int32_t* cu_seqlens, int32_t n_docs, int64_t q_begin, int64_t q_end,
                      int64_t k_begin, int64_t k_end, int32_t* cu_q_out, int32_t* cu_k_out,
                      int32_t* causal_out, int32_t* cls_out) {
  try {
    g_err.clear();
    if (!cu_seqlens || !cu_q_out || !cu_k_out || !causal_out || !cls_out)
      return fail(VL_EINVAL, "null argument");
    if (n_docs < 0) return fail(VL_EINVAL, "n_docs must be >= 0");
    std::string err;
    if (!vl::validate_cu(cu_seqlens, n_docs, cu_seqlens[n_docs], err))
      return fail(VL_ESEQLENS, "cu_seqlens: " + err);
    if (!vl::ring_block(cu_seqlens, n_docs, q_begin, q_end, k_begin, k_end, cu_q_out, cu_k_out,
                        *causal_out, *cls_out, err))
      return fail(VL_EINVAL, err);
    return VL_OK;
  } catch (const std::exception& ex) {
    return fail(VL_EINVAL, std::string("internal error: ") + ex.what());
  }
}

int varlen_schedule_export(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                           int32_t n_docs, int32_t causal, int32_t pass, int32_t head_dim,
                           int32_t* items, int64_t cap, int64_t* n_items, int64_t* useful_pairs,
                           int64_t* issued_pairs, int32_t* bq, int32_t* bk) {
  try {
    g_err.clear();
    if (!cu_seqlens_q || !cu_seqlens_k || !n_items) return fail(VL_EINVAL, "null argument");
    if (n_docs < 0) return fail(VL_EINVAL, "n_docs must be >= 0");
    if (pass != 0 && pass != 1) return fail(VL_EINVAL, "pass must be 0 or 1");
    if (head_dim != 64 && head_dim != 128) return fail(VL_EUNSUPPORTED, "head_dim must be 64 or 128");
    std::string err;
    if (!vl::validate_cu(cu_seqlens_q, n_docs, cu_seqlens_q[n_docs], err))
      return fail(VL_ESEQLENS, "cu_seqlens_q: " + err);
    if (!vl::validate_cu(cu_seqlens_k, n_docs, cu_seqlens_k[n_docs], err))
      return fail(VL_ESEQLENS, "cu_seqlens_k: " + err);
    const int tq = pass == 0 ? vl::kFwdBQ : vl::kBwdBQ;
    const int tk = pass == 0 ? vl::kFwdBK : vl::kBwdBK;
    const auto docs = vl::doc_table(cu_seqlens_q, cu_seqlens_k, n_docs);
    const auto list = pass == 0 ? vl::fwd_items(docs, causal != 0, tq, tk)
                                : vl::bwd_items(docs, causal != 0, tq, tk);
    *n_items = int64_t(list.size());
    if (useful_pairs) *useful_pairs = vl::visible_pairs(docs, causal != 0);
    if (issued_pairs) *issued_pairs = vl::issued_pairs(list, tq, tk);
    if (bq) *bq = tq;
    if (bk) *bk = tk;
    if (items) {
      if (cap < int64_t(list.size())) return fail(VL_EWORKSPACE, "items capacity too small");
      for (size_t i = 0; i < list.size(); ++i) {
        items[4 * i + 0] = list[i].doc;
        items[4 * i + 1] = list[i].tile;
        items[4 * i + 2] = list[i].first;
        items[4 * i + 3] = list[i].count;
      }
    }
    return VL_OK;
  } catch (const std::exception& ex) {
    return fail(VL_EINVAL, std::string("internal error: ") + ex.what());
  }
}

int varlen_schedule_export_dkdv(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int32_t n_docs, int32_t causal, int32_t n_heads_q,
                                int32_t n_heads_kv, int32_t n_cu, int32_t* entries, int64_t cap,
                                int64_t* n_entries) {
  try {
    g_err.clear();
    if (!cu_seqlens_q || !cu_seqlens_k || !n_entries) return fail(VL_EINVAL, "null argument");
    if (n_docs < 0) return fail(VL_EINVAL, "n_docs must be >= 0");
    if (n_cu <= 0) return fail(VL_EINVAL, "n_cu must be positive");
    if (n_heads_q <= 0 || n_heads_kv <= 0 || n_heads_q % n_heads_kv)
      return fail(VL_ESHAPE, "n_heads_q must be a positive multiple of n_heads_kv");
    std::string err;
    if (!vl::validate_cu(cu_seqlens_q, n_docs, cu_seqlens_q[n_docs], err))
      return fail(VL_ESEQLENS, "cu_seqlens_q: " + err);
    if (!vl::validate_cu(cu_seqlens_k, n_docs, cu_seqlens_k[n_docs], err))
      return fail(VL_ESEQLENS, "cu_seqlens_k: " + err);
    const auto docs = vl::doc_table(cu_seqlens_q, cu_seqlens_k, n_docs);
    const auto items = vl::bwd_items(docs, causal != 0, vl::kBwdBQ, vl::kBwdBK);
    const auto list = vl::bwd_entries(items, n_heads_q / n_heads_kv, n_heads_kv, n_cu,
                                      max_head_split(n_heads_q, n_heads_kv));
    *n_entries = int64_t(list.size());
    if (entries) {
      if (cap < int64_t(list.size())) return fail(VL_EWORKSPACE, "entries capacity too small");
      for (size_t i = 0; i < list.size(); ++i) {
        const vl::Entry& e = list[i];
        const int32_t row[6] = {e.item.doc, e.item.tile, e.item.first, e.item.count, e.slice,
                                e.n_slices};
        for (int f = 0; f < 6; ++f) entries[6 * i + f] = row[f];
      }
    }
    return VL_OK;
  } catch (const std::exception& ex) {
    return fail(VL_EINVAL, std::string("internal error: ") + ex.what());
  }
}

}  // extern "C"
