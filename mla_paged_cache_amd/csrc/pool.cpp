// Host side of the splice / evict library: the paged pool, the lowest-free
// page allocator, directive validation, the page planner and the C ABI
// (include/leyline.h).  Device work goes through the launchers in
// kernels.hip; every call enqueues it on the caller's stream.
//
// Operations: "Leyline: KV Cache Directives for Agentic Inference" (sections
// 2.1 directive and modes, 2.2 shift and delta-rotation, 2.3 serving steps);
// "KV-streams" ("how it works": in-engine eviction with kept entries
// unchanged; "assumptions and limits": 16-token and 1-token blocks).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <memory>
#include <string>
#include <utility>
#include <vector>

#include "../../include/leyline.h"
#include "host_common.h"
#include "leyline_internal.h"
#include "rows_internal.h"
#include "alloc_internal.h"

namespace ll {

namespace {
thread_local std::string g_error;
}  // namespace

ll_status fail(ll_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  try {
    g_error = buf;
  } catch (...) {
    // no memory even for the message: the status still says what happened
  }
  return s;
}

const char* last_error() { return g_error.c_str(); }

}  // namespace ll

namespace {

using ll::fail;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Lowest-free-first page allocator over a bitmap (bit set = free).
class FreePages {
 public:
  void init(int64_t n) {
    n_ = n;
    words_.assign(static_cast<size_t>(ceil_div(n, 64)), ~0ull);
    if (n % 64) words_.back() = (1ull << (n % 64)) - 1;
    count_ = n;
    hint_ = 0;
  }
  int64_t count() const { return count_; }
  bool is_free(int64_t p) const { return (words_[p >> 6] >> (p & 63)) & 1ull; }
  void take(int64_t p) {
    words_[p >> 6] &= ~(1ull << (p & 63));
    --count_;
  }
  void give(int64_t p) {
    words_[p >> 6] |= 1ull << (p & 63);
    ++count_;
    hint_ = std::min<int64_t>(hint_, p >> 6);
  }
  // The k lowest free pages, in increasing order (not taken).
  void lowest(int64_t k, std::vector<int32_t>& out) const {
    out.clear();
    out.reserve(static_cast<size_t>(k));
    for (size_t w = static_cast<size_t>(hint_); w < words_.size() && static_cast<int64_t>(out.size()) < k; ++w) {
      uint64_t bits = words_[w];
      while (bits && static_cast<int64_t>(out.size()) < k) {
        const int b = __builtin_ctzll(bits);
        out.push_back(static_cast<int32_t>(w * 64 + b));
        bits &= bits - 1;
      }
    }
  }
  // Pages marked in `bits` return to the free set, in one pass; false if one
  // of them was free already or is not a page (the caller then treats the
  // set as broken).
  bool give_bits_checked(const uint64_t* bits) {
    const size_t n = words_.size();
    if (n && (bits[n - 1] & ~tail_mask())) return false;
    // branch-free: freed words come in any order of zero and non-zero
    uint64_t clash = 0;
    int64_t added = 0;
    for (size_t w = 0; w < n; ++w) {
      const uint64_t b = bits[w];
      clash |= b & words_[w];
      words_[w] |= b;
      added += __builtin_popcountll(b);
    }
    size_t first = 0;
    while (first < n && !bits[first]) ++first;
    count_ += added;
    hint_ = std::min<int64_t>(hint_, static_cast<int64_t>(first));
    return clash == 0;
  }
  // Pages marked in `bits` (all taken now) return to the free set.
  void give_bits(const uint64_t* bits) {
    for (size_t w = 0; w < words_.size(); ++w) {
      if (!bits[w]) continue;
      count_ += __builtin_popcountll(bits[w] & ~words_[w]);
      words_[w] |= bits[w];
      hint_ = std::min<int64_t>(hint_, static_cast<int64_t>(w));
    }
  }
  size_t num_words() const { return words_.size(); }
  // The bitmap words (bit set = free), for the device's page plan.
  void copy_words(uint64_t* out) const { std::memcpy(out, words_.data(), words_.size() * sizeof(uint64_t)); }
  void advance_hint() {
    while (hint_ < static_cast<int64_t>(words_.size()) && words_[hint_] == 0) ++hint_;
  }

 private:
  // bits of the last word that are pages
  uint64_t tail_mask() const { return n_ % 64 ? (1ull << (n_ % 64)) - 1 : ~0ull; }

  int64_t n_ = 0, count_ = 0, hint_ = 0;
  std::vector<uint64_t> words_;
};

struct SeqState {
  bool used = false;
  int64_t len = 0;
  int64_t next_pos = 0;
  std::vector<int32_t> pages;
  // pages is out of date: the device page-table row (written by an eviction
  // the device planned) holds the sequence's table; copied back on demand
  bool stale = false;
};

// The region of the staging ring one call fills on the host and sends to the
// device with one copy (pinned host memory and device memory at the same
// offsets).
struct Staging {
  char* host = nullptr;
  char* dev = nullptr;
  size_t start = 0;
  size_t cap = 0;
  size_t used = 0;
};

// A region still in use by device work, and the event that marks its end.
struct RingRegion {
  size_t start, end;
  hipEvent_t done;
};

// The staging ring starts this large and doubles when one call needs more.
constexpr size_t kRingBytes = size_t{16} << 20;
// Uploads at least this large go through the pool's copy stream, so they can
// run while earlier work still occupies the caller's stream.
constexpr size_t kCopyStreamBytes = size_t{16} << 10;

struct ProfRec {
  hipEvent_t start, stop;
  int64_t bytes;
};

// Current-device guard.
class DeviceGuard {
 public:
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&old_) != hipSuccess) old_ = -1;
    if (old_ != dev) ok_ = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (old_ >= 0 && hipGetDevice(&cur) == hipSuccess && cur != old_) (void)hipSetDevice(old_);
  }
  bool ok() const { return ok_; }

 private:
  int old_ = -1;
  bool ok_ = true;
};

}  // namespace

namespace {

// A dispatch packet counts its work-items in 32 bits.  A row kernel whose
// grid would pass that (every layer of a batch that moves more than 2^32
// 16-byte chunks in all) is issued as several dispatches in order on one
// stream, each over a range of whole page tasks and every layer; the
// page-table rewrites ride in the last one.
constexpr int64_t kMaxDispatchItems = int64_t{0xFFFFFFFF};

// Page tasks per dispatch: `units_per_task` units of each task in each of
// `planes` planes, `units_per_block` units per block of `block_threads`
// threads, `extra_blocks` more blocks in the dispatch.  At least one.
int64_t tasks_per_dispatch(int64_t limit, int64_t units_per_task, int64_t planes, int64_t block_threads,
                           int64_t units_per_block, int64_t extra_blocks) {
  const int64_t blocks = limit / block_threads - extra_blocks;
  return std::max<int64_t>(1, blocks / planes * units_per_block / units_per_task);
}

// The timing events of the part of a split launch: the first part stamps the
// start, the last the stop.
ll::Stamp part_stamp(const ll::Stamp& t, bool first, bool last) {
  return ll::Stamp{first ? t.start : nullptr, last ? t.stop : nullptr};
}

}  // namespace

struct ll_pool {
  ll_pool_desc desc{};       // GQA pools: kv_lora_rank 0, rope_dim = rotary_dim
  int page_shift = 0;
  int64_t P = 1;
  bool gqa = false;          // K and V planes with per-head RoPE bands
  int32_t num_planes = 0;    // MLA: num_layers; GQA: 2 * num_layers (K then V)
  int64_t row_bytes = 0;     // one row of one plane
  int64_t band_bytes = 0;    // RoPE bytes of one row of a rotated plane
  int32_t heads = 0, head_chunks = 0, rot_shift = 0;  // GQA row shape
  std::vector<void*> layer_ptrs;  // the planes
  void** d_layers = nullptr;
  // chunks from one plane to the next when every plane's base is the first
  // one's plus a multiple of one fixed stride (one caller allocation), else 0
  int64_t plane_stride_chunks = 0;
  std::vector<SeqState> seqs;
  FreePages free;
  // staging ring: one pinned + one device buffer; calls take consecutive
  // regions and a region is reused once its call's event has fired
  char* ring_host = nullptr;
  char* ring_dev = nullptr;
  size_t ring_cap = 0;
  size_t ring_head = 0;
  std::deque<RingRegion> ring_inflight;
  std::vector<hipEvent_t> ring_events;  // idle events for new regions
  Staging cur;                          // region of the call in progress
  hipEvent_t upload_ev = nullptr;
  // eviction scratch: device [counts | reuse | src_of_dst], pinned readback
  float* d_rowtab = nullptr;    // per-row cos/sin tables of ll_rope_rows
  size_t rowtab_cap = 0;        // floats
  char* d_scratch = nullptr;
  size_t scratch_cap = 0;
  char* h_readback = nullptr;
  size_t readback_cap = 0;
  hipEvent_t readback_ev = nullptr;
  hipStream_t copy_stream = nullptr;
  hipEvent_t last_done = nullptr;  // end of the last call's device work
  hipStream_t last_stream = nullptr;  // the stream that work ran on
  // Calls that take no staging (splices planned on the device) record no
  // event: last_done then lags, and last_work() records lazy_ev on
  // last_stream when a later step needs the end of all work issued so far.
  bool unevented = false;
  hipEvent_t lazy_ev = nullptr;
  int32_t splice_planner = LL_SPLICE_PLAN_AUTO;
  bool page_reuse = true;       // false: every new page of a rewritten sequence is fresh
  int64_t dispatch_items = kMaxDispatchItems;  // work-items one row-kernel dispatch may hold
  char* d_direct = nullptr;     // tasks, tables and rotation tables of device-planned splices
  size_t direct_cap = 0;
  bool poisoned = false;
  std::vector<double> theta;    // RoPE frequencies of the pool's band (float64)
  ll_plan_stats last{};
  int32_t prof_every = 0;       // time every n-th launch of each kernel (0: none)
  int64_t prof_tick[3] = {0, 0, 0};
  std::vector<ProfRec> prof[3];  // row-moving kernel, keep scan, per-row rotation
  std::vector<hipEvent_t> spare_events;
  std::vector<int32_t> page_slot;  // per physical page: scratch marks of ll_seq_set_pages
  std::vector<int32_t> table_rows;     // host copy of device page-table rows (stale tables)
  // An eviction at page size 1 (no page is ever fresh): the call returns at
  // once and the host learns its result -- new lengths and the bitmap of
  // freed pages -- from a small readback that the next call on the pool
  // applies (settles) first.
  struct PendingEvict {
    bool active = false;
    hipEvent_t done = nullptr;   // the readback has landed
    std::vector<int32_t> seq_ids;
    size_t off_info = 0, off_freed = 0;  // in h_readback (counts at 0)
    int64_t n_words = 0;         // words of the freed bitmap
    int64_t prof_index = -1;     // prof[0] entry whose bytes are known only then
  } pending;
};

namespace {

// No exception crosses the C ABI: an exported function that catches one (in
// practice std::bad_alloc from host bookkeeping) returns LL_ENOMEM, and its
// pool, which the interrupted call may have left half-updated, is poisoned.
ll_status host_exception(ll_pool* p) noexcept {
  if (p) p->poisoned = true;
  return fail(LL_ENOMEM, "host memory exhausted during the call%s", p ? "; the pool is poisoned" : "");
}

ll_status device_fail(ll_pool* p, hipError_t e, const char* what) {
  p->poisoned = true;
  return fail(LL_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

ll_status check_pool(const ll_pool* p) {
  if (!p) return fail(LL_EINVAL, "pool is NULL");
  if (p->poisoned) return fail(LL_EPOISONED, "pool is poisoned by an earlier device failure");
  return LL_OK;
}

// Apply the result of a device-planned eviction to the host bookkeeping, from
// its readback: counts[i] rows kept by sequence seq_ids[i]; info[0] fresh
// pages, which are the info[0] lowest free pages (the device picked them from
// the free set as the call found it, and nothing has changed the free set
// since); the bitmap of old pages no new page keeps returns to the free set.
// The new page tables are on the device: the host copies are marked stale.
ll_status apply_evict(ll_pool* p, const int32_t* seq_ids, size_t n_seqs, const int64_t* counts,
                      const int32_t* info, const uint64_t* freed, int64_t n_words, int64_t prof_index) {
  const int64_t P = p->P;
  auto bad_plan = [p](const char* what) {
    p->poisoned = true;
    return fail(LL_EDEVICE, "the device page plan returned %s", what);
  };
  if (info[1]) return bad_plan("a shortage the host did not expect");
  for (size_t i = 0; i < n_seqs; ++i)
    if (counts[i] < 0 || counts[i] > p->seqs[seq_ids[i]].len) return bad_plan("a bad length");
  const int64_t fresh = info[0];
  if (fresh < 0 || fresh > p->free.count() || (P == 1 && fresh != 0)) return bad_plan("a bad fresh-page count");
  if (n_words != static_cast<int64_t>(p->free.num_words())) return bad_plan("a bitmap of the wrong size");
  ll_plan_stats stats{};
  std::vector<int32_t> taken;
  p->free.lowest(fresh, taken);
  for (int32_t pg : taken) p->free.take(pg);
  // freed pages were the sequences' own: none of them may be free now
  const int64_t before = p->free.count();
  if (!p->free.give_bits_checked(freed)) return bad_plan("a freed page that was already free");
  p->free.advance_hint();
  stats.freed_pages = p->free.count() - before;
  stats.fresh_pages = fresh;
  stats.rows_moved = static_cast<int64_t>(*reinterpret_cast<const uint64_t*>(info + 2));
  for (size_t i = 0; i < n_seqs; ++i) {
    SeqState& s = p->seqs[seq_ids[i]];
    s.len = counts[i];
    s.stale = true;
    stats.table_entries += ceil_div(counts[i], P);
  }
  stats.alg_bytes = p->num_planes * 2 * p->row_bytes * stats.rows_moved;
  stats.planned_on_device = 1;
  // page size 1: the timed kernel reads the kept rows' pages (4 B each) and
  // the freed-page bytes (one per pool page) and writes the table entries
  // (4 B each) and the freed-page bitmap
  if (prof_index >= 0 && prof_index < static_cast<int64_t>(p->prof[0].size()))
    p->prof[0][prof_index].bytes = 8 * stats.table_entries + 72 * n_words;
  p->last = stats;
  return LL_OK;
}

// Settle a pending eviction (page size 1): wait for its readback, apply it.
ll_status settle(ll_pool* p) {
  ll_pool::PendingEvict& pe = p->pending;
  if (!pe.active) return LL_OK;
  pe.active = false;
  hipError_t e = hipEventSynchronize(pe.done);
  if (e != hipSuccess) return device_fail(p, e, "eviction readback");
  return apply_evict(p, pe.seq_ids.data(), pe.seq_ids.size(), reinterpret_cast<const int64_t*>(p->h_readback),
                     reinterpret_cast<const int32_t*>(p->h_readback + pe.off_info),
                     reinterpret_cast<const uint64_t*>(p->h_readback + pe.off_freed), pe.n_words, pe.prof_index);
}

// check_pool, then settle a pending device-planned eviction.
ll_status enter(ll_pool* p) {
  ll_status rc = check_pool(p);
  if (rc) return rc;
  return settle(p);
}

hipEvent_t take_event(ll_pool* p) {
  if (!p->spare_events.empty()) {
    hipEvent_t e = p->spare_events.back();
    p->spare_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  // timing only: the host never reads device results behind these, so they
  // skip the system-scope fence (a cache writeback and invalidate per event)
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// Drop finished regions from the front of the ring's in-flight list.  Calls on
// one pool finish in order, so when the newest region is done all are (one
// query, however many regions a run of small calls left behind).
void ring_reap(ll_pool* p) {
  if (!p->ring_inflight.empty() && hipEventQuery(p->ring_inflight.back().done) == hipSuccess) {
    for (RingRegion& r : p->ring_inflight) p->ring_events.push_back(r.done);
    p->ring_inflight.clear();
    return;
  }
  while (!p->ring_inflight.empty() && hipEventQuery(p->ring_inflight.front().done) == hipSuccess) {
    p->ring_events.push_back(p->ring_inflight.front().done);
    p->ring_inflight.pop_front();
  }
}

// Wait until every region up to and including `upto` (an index into the
// in-flight list) has finished.  Calls on one pool are ordered on the device,
// so regions finish in the order they were taken.
ll_status ring_wait(ll_pool* p, size_t upto) {
  hipError_t e = hipEventSynchronize(p->ring_inflight[upto].done);
  if (e != hipSuccess) return device_fail(p, e, "hipEventSynchronize(staging)");
  for (size_t k = 0; k <= upto; ++k) {
    p->ring_events.push_back(p->ring_inflight.front().done);
    p->ring_inflight.pop_front();
  }
  return LL_OK;
}

// Take `bytes` of the staging ring for the current call.  Waits only if the
// region still holds data of unfinished earlier calls.
ll_status stage_acquire(ll_pool* p, size_t bytes, Staging** out) {
  bytes = align_up(std::max<size_t>(bytes, 256), 256);
  ring_reap(p);
  if (bytes > p->ring_cap) {
    // rare: one call needs more than the whole ring
    if (!p->ring_inflight.empty()) {
      ll_status rc = ring_wait(p, p->ring_inflight.size() - 1);
      if (rc) return rc;
    }
    if (p->ring_host) (void)hipHostFree(p->ring_host);
    if (p->ring_dev) (void)hipFree(p->ring_dev);
    p->ring_host = nullptr;
    p->ring_dev = nullptr;
    const size_t cap = std::max(2 * p->ring_cap, align_up(2 * bytes, size_t{1} << 20));
    p->ring_cap = 0;
    if (hipHostMalloc(reinterpret_cast<void**>(&p->ring_host), cap, hipHostMallocDefault) != hipSuccess ||
        hipMalloc(reinterpret_cast<void**>(&p->ring_dev), cap) != hipSuccess)
      return fail(LL_ENOMEM, "cannot allocate %zu bytes of staging", cap);
    std::memset(p->ring_host, 0, cap);  // fault the pages in now, not call by call
    p->ring_cap = cap;
    p->ring_head = 0;
  }
  if (p->ring_head + bytes > p->ring_cap) p->ring_head = 0;
  const size_t lo = p->ring_head, hi = lo + bytes;
  size_t last = SIZE_MAX;
  for (size_t k = 0; k < p->ring_inflight.size(); ++k) {
    const RingRegion& r = p->ring_inflight[k];
    if (r.start < hi && lo < r.end) last = k;
  }
  if (last != SIZE_MAX) {
    ll_status rc = ring_wait(p, last);
    if (rc) return rc;
  }
  p->ring_head = hi;
  Staging& s = p->cur;
  s.host = p->ring_host + lo;
  s.dev = p->ring_dev + lo;
  s.start = lo;
  s.cap = bytes;
  s.used = 0;
  *out = &s;
  return LL_OK;
}

// Append `bytes` to the staging slot; returns the offset.
size_t stage_put(Staging* s, const void* src, size_t bytes) {
  const size_t off = align_up(s->used, 256);
  // stage_bytes_for() sized the region for every part of the call
  if (off + bytes > s->cap) std::abort();
  if (bytes && src) std::memcpy(s->host + off, src, bytes);
  s->used = off + bytes;
  return off;
}

size_t stage_bytes_for(std::initializer_list<size_t> parts) {
  size_t t = 0;
  for (size_t x : parts) t = align_up(t, 256) + x;
  return t + 256;
}

// An event that fires once every call issued so far on the pool has finished
// on the device (nullptr: nothing issued yet).
hipEvent_t last_work(ll_pool* p, hipError_t* err) {
  *err = hipSuccess;
  if (p->unevented) {
    *err = hipEventRecord(p->lazy_ev, p->last_stream);
    if (*err != hipSuccess) return nullptr;
    p->last_done = p->lazy_ev;
    p->unevented = false;
  }
  return p->last_done;
}

// Wait on the host until the pool's device work has finished (before buffers
// it may still use are freed or grown).
ll_status wait_idle(ll_pool* p) {
  hipError_t e;
  hipEvent_t ev = last_work(p, &e);
  if (e == hipSuccess && ev) e = hipEventSynchronize(ev);
  if (e != hipSuccess) return device_fail(p, e, "hipEventSynchronize");
  return LL_OK;
}

// Bring the host page tables of `seqs` up to date where an eviction left them
// stale: wait for the pool's device work, then copy the device page-table rows
// back -- every stale sequence's, in one copy spanning them (an eviction
// leaves a whole batch stale, and its tables are usually needed together).
ll_status fresh_tables(ll_pool* p, const int32_t* seqs, size_t n) {
  bool any = false;
  for (size_t i = 0; i < n && !any; ++i) {
    const int32_t s = seqs[i];
    any = s >= 0 && s < p->desc.max_seqs && p->seqs[s].used && p->seqs[s].stale;
  }
  if (!any) return LL_OK;
  int32_t lo = INT32_MAX, hi = -1;
  for (int32_t s = 0; s < p->desc.max_seqs; ++s)
    if (p->seqs[s].used && p->seqs[s].stale) {
      lo = std::min(lo, s);
      hi = s;
    }
  if (ll_status rc = wait_idle(p)) return rc;
  const int64_t w = p->desc.max_pages_per_seq;
  const size_t count = static_cast<size_t>(hi - lo + 1) * static_cast<size_t>(w);
  p->table_rows.resize(count);
  DeviceGuard g(p->desc.device);
  hipError_t e = hipMemcpy(p->table_rows.data(), p->desc.page_table + static_cast<int64_t>(lo) * w,
                           count * sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return device_fail(p, e, "hipMemcpy(page-table rows)");
  for (int32_t s = lo; s <= hi; ++s) {
    SeqState& st = p->seqs[s];
    if (!st.used || !st.stale) continue;
    const int32_t* row = p->table_rows.data() + static_cast<int64_t>(s - lo) * w;
    st.pages.assign(row, row + ceil_div(st.len, p->P));
    st.stale = false;
  }
  return LL_OK;
}

ll_status fresh_table(ll_pool* p, int32_t seq) { return fresh_tables(p, &seq, 1); }

// Order this call after the previous call on the pool (any stream; calls on
// one stream are ordered already).
ll_status begin_call(ll_pool* p, hipStream_t st) {
  if (p->last_stream != st && (p->last_done || p->unevented)) {
    hipError_t e;
    hipEvent_t ev = last_work(p, &e);
    if (e == hipSuccess && ev) e = hipStreamWaitEvent(st, ev, 0);
    if (e != hipSuccess) return device_fail(p, e, "hipStreamWaitEvent");
  }
  return LL_OK;
}

ll_status end_call(ll_pool* p, Staging* s, hipStream_t st) {
  hipEvent_t ev = nullptr;
  if (!p->ring_events.empty()) {
    ev = p->ring_events.back();
    p->ring_events.pop_back();
  } else {
    // These mark when the device has finished reading a staging region and
    // order calls across streams of this device; the host never reads device
    // results behind them, so they skip the system-scope fence.
    hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming | hipEventDisableSystemFence);
    if (e != hipSuccess) return device_fail(p, e, "hipEventCreate(staging)");
  }
  hipError_t e = hipEventRecord(ev, st);
  if (e != hipSuccess) {
    p->ring_events.push_back(ev);
    return device_fail(p, e, "hipEventRecord");
  }
  p->ring_inflight.push_back({s->start, s->start + s->cap, ev});
  p->last_done = ev;
  p->last_stream = st;
  p->unevented = false;
  return LL_OK;
}

// Send the staging region to the device before the work that `st` runs next.
// The region is free (the device finished its last use), so a large upload does
// not have to wait behind earlier work on `st`: it runs on the copy stream and
// `st` waits for it.
ll_status upload(ll_pool* p, Staging* s, hipStream_t st) {
  if (s->used == 0) return LL_OK;
  hipError_t e;
  // Only this call's region is in flight: nothing earlier is queued, so the
  // copy goes straight onto `st` (fewer calls, lower latency).
  const bool idle = p->ring_inflight.empty();
  if (s->used >= kCopyStreamBytes && !idle) {
    e = hipMemcpyAsync(s->dev, s->host, s->used, hipMemcpyHostToDevice, p->copy_stream);
    if (e == hipSuccess) e = hipEventRecord(p->upload_ev, p->copy_stream);
    if (e == hipSuccess) e = hipStreamWaitEvent(st, p->upload_ev, 0);
  } else {
    e = hipMemcpyAsync(s->dev, s->host, s->used, hipMemcpyHostToDevice, st);
  }
  if (e != hipSuccess) return device_fail(p, e, "hipMemcpyAsync(H2D staging)");
  return LL_OK;
}

// theta_j = base^(-2j/rope_dim), j < rope_dim / 2, in float64.
std::vector<double> rope_thetas(double base, int rope_dim) {
  std::vector<double> t(static_cast<size_t>(rope_dim / 2));
  for (int j = 0; j < rope_dim / 2; ++j) t[static_cast<size_t>(j)] = std::pow(base, -2.0 * j / rope_dim);
  return t;
}

// The float32 cos/sin of the angles delta * theta_j (float64 angle, cos and
// sin, then rounding), from a precomputed theta table.
void rope_table_from(const std::vector<double>& theta, int64_t delta, float* c, float* s) {
  for (size_t j = 0; j < theta.size(); ++j) {
    const double ang = static_cast<double>(delta) * theta[j];
    c[j] = static_cast<float>(std::cos(ang));
    s[j] = static_cast<float>(std::sin(ang));
  }
}

void rope_table(double base, int rope_dim, int64_t delta, float* c, float* s) {
  for (int j = 0; j < rope_dim / 2; ++j) {
    const double theta = std::pow(base, -2.0 * j / rope_dim);
    const double ang = static_cast<double>(delta) * theta;
    c[j] = static_cast<float>(std::cos(ang));
    s[j] = static_cast<float>(std::sin(ang));
  }
}

// Page-table rewrite of whole rows, via the packed table array in staging.
struct TablePlan {
  std::vector<ll::TableWrite> writes;
  std::vector<int32_t> packed;
  void add(int32_t seq, const std::vector<int32_t>& t) {
    ll::TableWrite w{};
    w.src_off = static_cast<int64_t>(packed.size());
    w.seq = seq;
    w.count = static_cast<int32_t>(t.size());
    packed.insert(packed.end(), t.begin(), t.end());
    writes.push_back(w);
  }
};

// Upload and launch a stand-alone page-table rewrite on `st`.
ll_status write_tables(ll_pool* p, const TablePlan& tp, hipStream_t st) {
  ll_status rc = begin_call(p, st);
  if (rc) return rc;
  Staging* s = nullptr;
  if (tp.writes.size() == 1) {
    // one row: copy it straight from pinned staging into the page table
    const ll::TableWrite& w = tp.writes[0];
    if ((rc = stage_acquire(p, stage_bytes_for({tp.packed.size() * 4}), &s))) return rc;
    const size_t o = stage_put(s, tp.packed.data(), tp.packed.size() * 4);
    if (w.count > 0) {
      hipError_t e = hipMemcpyAsync(p->desc.page_table + static_cast<int64_t>(w.seq) * p->desc.max_pages_per_seq,
                                    s->host + o, static_cast<size_t>(w.count) * 4, hipMemcpyHostToDevice, st);
      if (e != hipSuccess) return device_fail(p, e, "hipMemcpyAsync(page table row)");
    }
    return end_call(p, s, st);
  }
  rc = stage_acquire(p, stage_bytes_for({tp.writes.size() * sizeof(ll::TableWrite), tp.packed.size() * 4}), &s);
  if (rc) return rc;
  const size_t o_w = stage_put(s, tp.writes.data(), tp.writes.size() * sizeof(ll::TableWrite));
  const size_t o_t = stage_put(s, tp.packed.data(), tp.packed.size() * 4);
  if ((rc = upload(p, s, st))) return rc;
  ll::TableLaunch a{};
  a.twrites = reinterpret_cast<const ll::TableWrite*>(s->dev + o_w);
  a.tables = reinterpret_cast<const int32_t*>(s->dev + o_t);
  a.n_twrites = static_cast<int32_t>(tp.writes.size());
  a.max_pages_per_seq = p->desc.max_pages_per_seq;
  a.page_table = p->desc.page_table;
  hipError_t e = ll::launch_table_write(a, st);
  if (e != hipSuccess) return device_fail(p, e, "table_write_kernel launch");
  return end_call(p, s, st);
}

// Whether this launch of `kernel` is timed: every prof_every-th one.
bool prof_pick(ll_pool* p, int kernel) {
  if (p->prof_every <= 0) return false;
  return p->prof_tick[kernel]++ % p->prof_every == 0;
}

// A timed launch takes two events; its launcher stamps them from the dispatch
// packets, so timing adds no packets of its own to the stream.
ll_status prof_begin(ll_pool* p, ProfRec* rec, ll::Stamp* t) {
  rec->start = take_event(p);
  rec->stop = take_event(p);
  if (!rec->start || !rec->stop) return fail(LL_EDEVICE, "hipEventCreate failed");
  t->start = rec->start;
  t->stop = rec->stop;
  return LL_OK;
}

void prof_end(ll_pool* p, int kernel, const ProfRec& rec) { p->prof[kernel].push_back(rec); }

// ------------------------------------------------------------------ splice --

struct SplicePlan {
  int32_t seq = 0;
  int32_t mode = LL_AMORTIZE;
  int64_t n_old = 0, n_new = 0, delta = 0, next_pos = 0;
  std::vector<int32_t> reuse;     // per new page: old logical page, or -1 (fresh)
  std::vector<char> inplace;      // per new page: rotate k_pe in place
  int64_t fresh = 0;
};

// The page plan of one directive in closed form (no per-row loop):
// a new page reuses an old one iff all its live rows are old rows of one old
// page at unchanged offsets.
void plan_splice(const ll_pool* p, const ll_directive& d, const SeqState& s, SplicePlan* out) {
  const int64_t P = p->P;
  out->seq = d.seq_id;
  out->mode = d.mode;
  out->n_old = s.len;
  if (d.mode == LL_FORGET) {
    out->n_new = d.s_start;
    out->delta = 0;
    out->next_pos = s.next_pos - (s.len - d.s_start);
  } else {
    out->delta = d.r_len - (d.s_end - d.s_start);
    out->n_new = s.len + out->delta;
    out->next_pos = s.next_pos + out->delta;
  }
  const int64_t pages = ceil_div(out->n_new, P);
  out->reuse.assign(static_cast<size_t>(pages), -1);
  out->inplace.assign(static_cast<size_t>(pages), 0);
  out->fresh = 0;
  const int64_t s0 = d.s_start;
  const int64_t r = d.mode == LL_FORGET ? 0 : d.r_len;
  const int64_t delta = out->delta;
  for (int64_t q = 0; q < pages; ++q) {
    const int64_t a = q * P, b = std::min(a + P, out->n_new);
    const bool has_pre = a < s0;
    const bool has_stub = r > 0 && a < s0 + r && b > s0;
    const bool has_down = b > s0 + r;
    int64_t reuse = -1;
    if (has_stub) {
      reuse = -1;
    } else if (has_pre && has_down) {
      reuse = delta == 0 ? q : -1;  // span and stub both empty
    } else if (has_pre) {
      reuse = q;
    } else {
      const int64_t src0 = a - delta;  // first source row, page-aligned iff delta % P == 0
      if ((src0 & (P - 1)) == 0) reuse = src0 / P;
    }
    if (!p->page_reuse) reuse = -1;
    out->reuse[q] = static_cast<int32_t>(reuse);
    if (reuse < 0) ++out->fresh;
    else if (has_down && delta != 0 && d.mode == LL_AMORTIZE) out->inplace[q] = 1;
  }
}

// Grow the eviction scratch (device) and readback (pinned) buffers; growing
// waits for earlier device work, which may still use them.
ll_status ensure_evict_buffers(ll_pool* p, size_t scratch, size_t readback) {
  if (scratch <= p->scratch_cap && readback <= p->readback_cap) return LL_OK;
  if (ll_status rc = wait_idle(p)) return rc;
  if (scratch > p->scratch_cap) {
    if (p->d_scratch) (void)hipFree(p->d_scratch);
    p->d_scratch = nullptr;
    p->scratch_cap = 0;
    if (hipMalloc(reinterpret_cast<void**>(&p->d_scratch), scratch) != hipSuccess)
      return fail(LL_ENOMEM, "cannot allocate %zu bytes of eviction scratch", scratch);
    p->scratch_cap = scratch;
  }
  if (readback > p->readback_cap) {
    if (p->h_readback) (void)hipHostFree(p->h_readback);
    p->h_readback = nullptr;
    p->readback_cap = 0;
    if (hipHostMalloc(reinterpret_cast<void**>(&p->h_readback), readback, hipHostMallocDefault) != hipSuccess)
      return fail(LL_ENOMEM, "cannot allocate %zu bytes of pinned readback", readback);
    std::memset(p->h_readback, 0, readback);
    p->readback_cap = readback;
  }
  return LL_OK;
}

// Eviction with the page plan made on the device (kernels_alloc.hip): keep
// scan (new indices, sources, per-page reuse, the bitmap of freed old pages),
// fresh-page ranks and the verdict (fresh pages, or a shortage), a readback of
// [counts | verdict | freed bitmap], then the new tables and the row moves.
// At page size > 1 the call waits for that readback only -- tens of
// microseconds, the scan's time -- so that a shortage returns LL_ENOMEM with
// nothing changed and the row-move kernel gets an exact grid; the host's books
// are then brought up to date in the same call.  At page size 1 no page is
// fresh and nothing moves: the call does not wait, and the next call on the
// pool applies the readback.
ll_status evict_device_plan(ll_pool* p, const int32_t* seq_ids, int32_t n, const uint8_t* keep_dev,
                            const std::vector<ll::EvictSeq>& es, int64_t total_rows, int64_t total_pages,
                            hipStream_t st) {
  const int64_t P = p->P;
  const int64_t rc_chunks = p->row_bytes / 16;
  if (total_pages * P * rc_chunks >= (int64_t{1} << 32) - 1024)
    return fail(LL_EUNSUPPORTED, "one eviction may move at most 2^32 16-byte chunks per layer");
  const int64_t n_words = static_cast<int64_t>(p->free.num_words());
  const int32_t n_free_words = P == 1 ? 0 : static_cast<int32_t>(n_words);
  // device scratch: [counts n | info 16 | freed n_words] (read back in one
  // copy), then reuse tp | new_table tp | src_rows rows | src_logical rows |
  // kept tp (bytes) | rank tp | fresh_count n | fresh_base n | moved n |
  // word_base n_free_words | tasks tp
  const size_t tp = static_cast<size_t>(total_pages), rows = static_cast<size_t>(total_rows);
  const size_t nn = static_cast<size_t>(n);
  const size_t off_info = align_up(8 * nn, 16);
  const size_t off_freed = align_up(off_info + 16, 256);
  const size_t readback = off_freed + 8 * static_cast<size_t>(n_words);
  const size_t off_reuse = align_up(readback, 256);
  const size_t off_nt = align_up(off_reuse + 4 * tp, 256);
  const size_t off_src = align_up(off_nt + 4 * tp, 256);
  const size_t off_logical = align_up(off_src + 4 * rows, 256);
  const size_t off_kept = align_up(off_logical + 4 * rows, 256);
  const size_t off_rank = align_up(off_kept + tp, 256);
  const size_t off_fc = align_up(off_rank + 4 * tp, 256);
  const size_t off_fb = align_up(off_fc + 4 * nn, 256);
  const size_t off_mv = align_up(off_fb + 4 * nn, 256);
  const size_t off_wb = align_up(off_mv + 4 * nn, 256);
  const size_t off_tasks = align_up(off_wb + 4 * static_cast<size_t>(n_free_words), 256);
  const size_t off_fbytes = align_up(off_tasks + sizeof(ll::EvictTask) * tp, 256);  // page size 1
  const size_t scratch = off_fbytes + (P == 1 ? 64 * static_cast<size_t>(n_words) : 0) + 256;
  ll_status rc = begin_call(p, st);
  if (rc) return rc;
  if ((rc = ensure_evict_buffers(p, scratch, readback))) return rc;

  Staging* sg = nullptr;
  const size_t words_bytes = 8 * static_cast<size_t>(n_free_words);
  if ((rc = stage_acquire(p, stage_bytes_for({es.size() * sizeof(ll::EvictSeq), words_bytes}), &sg))) return rc;
  const size_t o_es = stage_put(sg, es.data(), es.size() * sizeof(ll::EvictSeq));
  const size_t o_w = stage_put(sg, nullptr, words_bytes);
  if (n_free_words) p->free.copy_words(reinterpret_cast<uint64_t*>(sg->host + o_w));
  if ((rc = upload(p, sg, st))) return rc;

  char* d = p->d_scratch;
  ll::ScanLaunch sc{};
  sc.keep = keep_dev;
  sc.seqs = reinterpret_cast<const ll::EvictSeq*>(sg->dev + o_es);
  sc.n_seqs = n;
  sc.page_shift = p->page_shift;
  sc.page_table = p->desc.page_table;
  sc.max_pages_per_seq = p->desc.max_pages_per_seq;
  sc.counts = reinterpret_cast<int64_t*>(d);
  sc.reuse = reinterpret_cast<int32_t*>(d + off_reuse);
  sc.src_rows = reinterpret_cast<int32_t*>(d + off_src);
  sc.src_logical = reinterpret_cast<int32_t*>(d + off_logical);
  sc.kept = reinterpret_cast<uint8_t*>(d + off_kept);
  sc.freed = reinterpret_cast<unsigned long long*>(d + off_freed);
  sc.freed_bytes = reinterpret_cast<uint8_t*>(d + off_fbytes);
  sc.page_reuse = p->page_reuse ? 1 : 0;
  const bool moves = P > 1;
  // page size > 1 ORs freed pages into the bitmap; page size 1 marks bytes
  hipError_t e = moves ? ll::launch_zero_words(sc.freed, n_words, st)
                       : ll::launch_zero_words(reinterpret_cast<unsigned long long*>(sc.freed_bytes), 8 * n_words, st);
  if (e != hipSuccess) return device_fail(p, e, "zero_words_kernel launch");
  ProfRec rec1{};
  ll::Stamp t1;
  if (prof_pick(p, 1) && (rc = prof_begin(p, &rec1, &t1))) return rc;
  e = ll::launch_keep_scan(sc, st, t1);
  if (e != hipSuccess) return device_fail(p, e, "keep_scan_kernel launch");
  if (rec1.start) {
    rec1.bytes = total_rows + 4 * total_rows;
    prof_end(p, 1, rec1);
  }

  ll::AllocLaunch al{};
  al.seqs = sc.seqs;
  al.n = n;
  al.page_shift = p->page_shift;
  al.counts = sc.counts;
  al.reuse = sc.reuse;
  al.page_table = p->desc.page_table;
  al.max_pages_per_seq = p->desc.max_pages_per_seq;
  al.n_words = n_free_words;
  al.free_words = reinterpret_cast<const uint64_t*>(sg->dev + o_w);
  al.rank = reinterpret_cast<int32_t*>(d + off_rank);
  al.fresh_count = reinterpret_cast<int32_t*>(d + off_fc);
  al.fresh_base = reinterpret_cast<int32_t*>(d + off_fb);
  al.moved_count = reinterpret_cast<int32_t*>(d + off_mv);
  al.word_base = reinterpret_cast<int32_t*>(d + off_wb);
  al.new_table = reinterpret_cast<int32_t*>(d + off_nt);
  al.tasks = reinterpret_cast<ll::EvictTask*>(d + off_tasks);
  al.src_logical = sc.src_logical;
  al.info = reinterpret_cast<int32_t*>(d + off_info);
  // kernel 0's record: at page size 1 the new tables; above it the row moves
  ProfRec rec{};
  ll::Stamp t0;
  if (prof_pick(p, 0) && (rc = prof_begin(p, &rec, &t0))) return rc;
  if (!moves) {
    // page size 1: the new tables are the kept rows' pages (src_rows)
    ll::UnitPageLaunch up{};
    up.seqs = sc.seqs;
    up.n = n;
    up.counts = sc.counts;
    up.src_rows = sc.src_rows;
    up.page_table = p->desc.page_table;
    up.max_pages_per_seq = p->desc.max_pages_per_seq;
    up.freed_bytes = sc.freed_bytes;
    up.freed = sc.freed;
    up.n_words = n_words;
    up.info = al.info;
    if ((e = ll::launch_unit_page(up, st, t0)) != hipSuccess) return device_fail(p, e, "unit_page_kernel launch");
    e = hipMemcpyAsync(p->h_readback, d, readback, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipEventRecord(p->pending.done, st);
    if (e != hipSuccess) return device_fail(p, e, "eviction readback");
    int64_t prof_index = -1;
    if (rec.start) {
      rec.bytes = 0;  // known when the call settles
      prof_end(p, 0, rec);
      prof_index = static_cast<int64_t>(p->prof[0].size()) - 1;
    }
    if ((rc = end_call(p, sg, st))) return rc;
    ll_pool::PendingEvict& pe = p->pending;
    pe.active = true;
    pe.seq_ids.assign(seq_ids, seq_ids + n);
    pe.off_info = off_info;
    pe.off_freed = off_freed;
    pe.n_words = n_words;
    pe.prof_index = prof_index;
    return LL_OK;
  }

  // page size > 1: the verdict decides, then the exact grid
  if ((e = ll::launch_alloc_scan(al, st)) != hipSuccess) return device_fail(p, e, "page allocator launch");
  e = hipMemcpyAsync(p->h_readback, d, readback, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipEventRecord(p->pending.done, st);
  if (e != hipSuccess) return device_fail(p, e, "eviction readback");
  e = hipEventSynchronize(p->pending.done);
  if (e != hipSuccess) return device_fail(p, e, "eviction readback");
  const int64_t* counts = reinterpret_cast<const int64_t*>(p->h_readback);
  const int32_t* info = reinterpret_cast<const int32_t*>(p->h_readback + off_info);
  if (info[1]) {
    // nothing has changed: the kernels so far wrote scratch only
    if (rec.start) p->spare_events.insert(p->spare_events.end(), {rec.start, rec.stop});
    if ((rc = end_call(p, sg, st))) return rc;
    int64_t need = 0;
    for (int32_t i = 0; i < n; ++i) need += ceil_div(counts[i], P);
    return fail(LL_ENOMEM, "the eviction needs more fresh pages than the %lld free (at most %lld new pages)",
                (long long)p->free.count(), (long long)need);
  }
  if (info[0] < 0 || info[0] > total_pages) return device_fail(p, hipErrorUnknown, "eviction verdict out of range");
  if ((e = ll::launch_alloc_tables(al, st)) != hipSuccess) return device_fail(p, e, "page allocator launch");
  const int64_t n_tasks = info[0];
  if (p->gqa) {
    ll::PlaneEvictLaunch a{};
    a.planes = reinterpret_cast<const ll::chunk_t* const*>(p->d_layers);
    a.num_planes = p->num_planes;
    a.page_shift = p->page_shift;
    a.row_chunks = static_cast<int32_t>(rc_chunks);
    a.tasks = al.tasks;
    a.n_tasks = n_tasks;
    a.src_rows = sc.src_rows;
    a.n_twrites = 0;
    // ranges of whole tasks over every plane (src0 indexes src_rows globally)
    const int64_t per = tasks_per_dispatch(p->dispatch_items, P * rc_chunks, a.num_planes, ll::kEvictThreads,
                                           ll::kEvictThreads, 0);
    for (int64_t k0 = 0; k0 == 0 || k0 < n_tasks; k0 += per) {  // one launch when there is no task
      const int64_t cnt = std::min(per, n_tasks - k0);
      a.tasks = al.tasks + k0;
      a.n_tasks = cnt;
      a.blocks_per_plane = ll::flat_blocks(cnt * P * rc_chunks, 1, ll::kEvictThreads);
      e = ll::launch_plane_evict(a, st, part_stamp(t0, k0 == 0, k0 + cnt == n_tasks));
      if (e != hipSuccess) return device_fail(p, e, "plane_evict_kernel launch");
    }
  } else {
    ll::EvictLaunch a{};
    a.layers = reinterpret_cast<const ll::chunk_t* const*>(p->d_layers);
    a.num_layers = p->desc.num_layers;
    a.page_shift = p->page_shift;
    a.tasks = al.tasks;
    a.n_tasks = n_tasks;
    a.src_rows = sc.src_rows;
    a.n_twrites = 0;
    const int64_t per = tasks_per_dispatch(p->dispatch_items, P * rc_chunks, a.num_layers, ll::kEvictThreads,
                                           ll::kEvictThreads, 0);
    for (int64_t k0 = 0; k0 == 0 || k0 < n_tasks; k0 += per) {  // one launch when there is no task
      const int64_t cnt = std::min(per, n_tasks - k0);
      a.tasks = al.tasks + k0;
      a.n_tasks = cnt;
      a.blocks_per_layer = ll::flat_blocks(cnt * P * rc_chunks, 1, ll::kEvictThreads);
      e = ll::launch_evict_move(a, st, part_stamp(t0, k0 == 0, k0 + cnt == n_tasks));
      if (e != hipSuccess) return device_fail(p, e, "evict_move_kernel launch");
    }
  }
  if ((rc = end_call(p, sg, st))) return rc;
  if ((rc = apply_evict(p, seq_ids, static_cast<size_t>(n), counts, info,
                        reinterpret_cast<const uint64_t*>(p->h_readback + off_freed), n_words, -1)))
    return rc;
  if (rec.start) {
    rec.bytes = p->last.alg_bytes;
    prof_end(p, 0, rec);
  }
  return LL_OK;
}

ll_status validate_directives(const ll_pool* p, const ll_directive* dirs, int32_t n) {
  std::vector<char> seen(static_cast<size_t>(p->desc.max_seqs), 0);
  for (int32_t i = 0; i < n; ++i) {
    const ll_directive& d = dirs[i];
    if (d.mode == LL_PIN || d.mode == LL_DECAY || d.mode == LL_SCRATCH)
      return fail(LL_EUNSUPPORTED, "directive %d: mode %d is reserved", i, d.mode);
    if (d.mode != LL_AMORTIZE && d.mode != LL_FORGET) return fail(LL_EINVAL, "directive %d: unknown mode %d", i, d.mode);
    if (d.seq_id < 0 || d.seq_id >= p->desc.max_seqs || !p->seqs[d.seq_id].used)
      return fail(LL_EINVAL, "directive %d: unknown sequence %d", i, d.seq_id);
    if (seen[d.seq_id]) return fail(LL_EINVAL, "directive %d: sequence %d appears twice", i, d.seq_id);
    seen[d.seq_id] = 1;
    const int64_t len = p->seqs[d.seq_id].len;
    if (d.s_start < 0 || d.s_start > d.s_end || d.s_end > len)
      return fail(LL_EINVAL, "directive %d: span [%lld, %lld) outside [0, %lld]", i, (long long)d.s_start,
                  (long long)d.s_end, (long long)len);
    if (d.mode == LL_FORGET) continue;
    if (d.r_len < 0) return fail(LL_EINVAL, "directive %d: r_len < 0", i);
    if ((d.r_len > 0) != (d.r_rows != nullptr))
      return fail(LL_EINVAL, "directive %d: r_rows must be given iff r_len > 0", i);
    if (d.r_rows && (reinterpret_cast<uintptr_t>(d.r_rows) & 15))
      return fail(LL_EINVAL, "directive %d: r_rows is not 16-byte aligned", i);
    if (d.r_layer_stride_bytes < 0 || (d.r_layer_stride_bytes & 15) ||
        (d.r_layer_stride_bytes && d.r_layer_stride_bytes < d.r_len * p->row_bytes && p->desc.num_layers > 1))
      return fail(LL_EINVAL, "directive %d: bad r_layer_stride_bytes", i);
    if (!p->gqa) {
      if (d.r_rows_v) return fail(LL_EINVAL, "directive %d: r_rows_v is for GQA / MHA pools only", i);
    } else {
      if ((d.r_len > 0) != (d.r_rows_v != nullptr))
        return fail(LL_EINVAL, "directive %d: r_rows_v must be given iff r_len > 0", i);
      if (d.r_rows_v && (reinterpret_cast<uintptr_t>(d.r_rows_v) & 15))
        return fail(LL_EINVAL, "directive %d: r_rows_v is not 16-byte aligned", i);
      if (d.r_layer_stride_bytes_v < 0 || (d.r_layer_stride_bytes_v & 15) ||
          (d.r_layer_stride_bytes_v && d.r_layer_stride_bytes_v < d.r_len * p->row_bytes && p->desc.num_layers > 1))
        return fail(LL_EINVAL, "directive %d: bad r_layer_stride_bytes_v", i);
    }
    const int64_t n_new = len + d.r_len - (d.s_end - d.s_start);
    if (ceil_div(n_new, p->P) > p->desc.max_pages_per_seq)
      return fail(LL_ERANGE, "directive %d: %lld rows exceed the page-table row", i, (long long)n_new);
  }
  return LL_OK;
}

}  // namespace

// =================================================================== C ABI ==

extern "C" {

const char* ll_last_error(void) { return ll::last_error(); }

const char* ll_status_str(ll_status s) {
  switch (s) {
    case LL_OK: return "LL_OK";
    case LL_EINVAL: return "LL_EINVAL";
    case LL_ERANGE: return "LL_ERANGE";
    case LL_ENOMEM: return "LL_ENOMEM";
    case LL_EUNSUPPORTED: return "LL_EUNSUPPORTED";
    case LL_EDEVICE: return "LL_EDEVICE";
    case LL_EPOISONED: return "LL_EPOISONED";
  }
  return "unknown";
}

ll_status ll_rope_delta_table(double base, int32_t rope_dim, int64_t delta, float* cos_out, float* sin_out) try {
  if (!cos_out || !sin_out) return fail(LL_EINVAL, "NULL output");
  if (rope_dim <= 0 || (rope_dim & 1)) return fail(LL_EINVAL, "rope_dim must be even and positive");
  if (!(base > 0.0)) return fail(LL_EINVAL, "base must be positive");
  rope_table(base, rope_dim, delta, cos_out, sin_out);
  return LL_OK;
} catch (...) {
  return host_exception(nullptr);
}

}  // extern "C"

namespace {

// Checks shared by both pool kinds.
ll_status check_common(int32_t num_layers, int32_t page_size, int32_t num_pages, int32_t max_seqs,
                       int32_t max_pages_per_seq, int32_t rope_pairing, double rope_base,
                       const int32_t* page_table, int32_t device) {
  if (num_layers < 1 || num_pages < 1 || max_seqs < 1 || max_pages_per_seq < 1)
    return fail(LL_EINVAL, "num_layers, num_pages, max_seqs and max_pages_per_seq must be >= 1");
  if (page_size < 1 || page_size > 256 || (page_size & (page_size - 1)))
    return fail(LL_EINVAL, "page_size must be a power of two in [1, 256]");
  if (rope_pairing != LL_ROPE_INTERLEAVED && rope_pairing != LL_ROPE_HALF) return fail(LL_EINVAL, "unknown rope_pairing");
  if (!(rope_base > 0.0)) return fail(LL_EINVAL, "rope_base must be positive");
  if (!page_table) return fail(LL_EINVAL, "page_table is required");
  if (static_cast<int64_t>(num_pages) * page_size >= (int64_t{1} << 31) ||
      static_cast<int64_t>(max_pages_per_seq) * page_size >= (int64_t{1} << 31))
    return fail(LL_EUNSUPPORTED, "more than 2^31 rows per layer or per sequence");
  if (device < 0) return fail(LL_EINVAL, "device must be >= 0");
  return LL_OK;
}

ll_status check_planes(void* const* base, int32_t n, const char* name) {
  if (!base) return fail(LL_EINVAL, "%s is required", name);
  for (int i = 0; i < n; ++i) {
    if (!base[i]) return fail(LL_EINVAL, "%s[%d] is NULL", name, i);
    if (reinterpret_cast<uintptr_t>(base[i]) & 15) return fail(LL_EINVAL, "%s[%d] is not 16-byte aligned", name, i);
  }
  return LL_OK;
}

// Allocation and device setup shared by both pool kinds; p->desc, the row
// shape and p->layer_ptrs (the planes) are filled in by the caller.
ll_status setup_pool(ll_pool* p, ll_pool** out) {
  const ll_pool_desc& d = p->desc;
  DeviceGuard g(d.device);
  if (!g.ok()) {
    delete p;
    return fail(LL_EDEVICE, "hipSetDevice(%d) failed", d.device);
  }
  p->num_planes = static_cast<int32_t>(p->layer_ptrs.size());
  if (p->num_planes > 1) {
    const intptr_t b0 = reinterpret_cast<intptr_t>(p->layer_ptrs[0]);
    const intptr_t st = reinterpret_cast<intptr_t>(p->layer_ptrs[1]) - b0;
    bool even = st > 0 && st % 16 == 0;
    for (int32_t l = 2; even && l < p->num_planes; ++l)
      even = reinterpret_cast<intptr_t>(p->layer_ptrs[l]) - b0 == st * l;
    p->plane_stride_chunks = even ? st / 16 : 0;
  }
  p->P = d.page_size;
  while ((1 << p->page_shift) < d.page_size) ++p->page_shift;
  p->seqs.resize(static_cast<size_t>(d.max_seqs));
  p->free.init(d.num_pages);
  p->page_slot.assign(static_cast<size_t>(d.num_pages), -1);
  p->theta = rope_thetas(d.rope_base, d.rope_dim);
  // once per device, with it current: the address of the no-allocation scratch
  hipError_t e = ll::noalloc_scratch_init(d.device);
  if (e != hipSuccess) {
    delete p;
    return fail(LL_EDEVICE, "hipGetSymbolAddress(no-allocation scratch): %s", hipGetErrorString(e));
  }
  e = hipMalloc(reinterpret_cast<void**>(&p->d_layers), sizeof(void*) * p->num_planes);
  if (e == hipSuccess)
    e = hipMemcpy(p->d_layers, p->layer_ptrs.data(), sizeof(void*) * p->num_planes, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&p->readback_ev, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&p->pending.done, hipEventDisableTiming);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&p->copy_stream, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&p->upload_ev, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&p->lazy_ev, hipEventDisableTiming | hipEventDisableSystemFence);
  if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void**>(&p->ring_host), kRingBytes, hipHostMallocDefault);
  // touch every page now: first writes to fresh pinned pages fault one page
  // at a time (tens of microseconds per call while the ring is new)
  if (e == hipSuccess) std::memset(p->ring_host, 0, kRingBytes);
  if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void**>(&p->ring_dev), kRingBytes);
  if (e == hipSuccess) p->ring_cap = kRingBytes;
  if (e != hipSuccess) {
    ll_pool_destroy(p);
    return fail(LL_EDEVICE, "pool setup: %s", hipGetErrorString(e));
  }
  *out = p;
  return LL_OK;
}

}  // namespace

extern "C" {

ll_status ll_pool_create(const ll_pool_desc* desc, ll_pool** out) try {
  if (!desc || !out) return fail(LL_EINVAL, "NULL argument");
  *out = nullptr;
  const ll_pool_desc& d = *desc;
  ll_status rc = check_common(d.num_layers, d.page_size, d.num_pages, d.max_seqs, d.max_pages_per_seq, d.rope_pairing,
                              d.rope_base, d.page_table, d.device);
  if (rc) return rc;
  if (d.kv_lora_rank != ll::kKvLoraRank || d.rope_dim != ll::kRopeDim)
    return fail(LL_EUNSUPPORTED, "row shape %d + %d is not supported (512 + 64 only)", d.kv_lora_rank, d.rope_dim);
  if ((rc = check_planes(d.layer_base, d.num_layers, "layer_base"))) return rc;
  ll_pool* p = new ll_pool();
  p->desc = d;
  p->desc.layer_base = nullptr;
  p->layer_ptrs.assign(d.layer_base, d.layer_base + d.num_layers);
  p->row_bytes = ll::kRowBytes;
  p->band_bytes = 2 * ll::kRopeDim;
  return setup_pool(p, out);
} catch (...) {
  return host_exception(nullptr);
}

ll_status ll_pool_create_gqa(const ll_gqa_pool_desc* desc, ll_pool** out) try {
  if (!desc || !out) return fail(LL_EINVAL, "NULL argument");
  *out = nullptr;
  const ll_gqa_pool_desc& d = *desc;
  ll_status rc = check_common(d.num_layers, d.page_size, d.num_pages, d.max_seqs, d.max_pages_per_seq, d.rope_pairing,
                              d.rope_base, d.page_table, d.device);
  if (rc) return rc;
  if (d.num_kv_heads < 1 || d.head_dim < 8 || d.head_dim % 8)
    return fail(LL_EUNSUPPORTED, "num_kv_heads must be >= 1 and head_dim a multiple of 8");
  if (static_cast<int64_t>(d.num_kv_heads) * d.head_dim > 32768)
    return fail(LL_EUNSUPPORTED, "num_kv_heads * head_dim above 32768");
  if (d.rotary_dim < 16 || d.rotary_dim > 2 * ll::kMaxBandPairs || (d.rotary_dim & (d.rotary_dim - 1)) ||
      d.head_dim % d.rotary_dim)
    return fail(LL_EUNSUPPORTED, "rotary_dim must be a power of two in [16, 256] that divides head_dim");
  if ((rc = check_planes(d.k_layer_base, d.num_layers, "k_layer_base"))) return rc;
  if ((rc = check_planes(d.v_layer_base, d.num_layers, "v_layer_base"))) return rc;
  ll_pool* p = new ll_pool();
  ll_pool_desc& pd = p->desc;
  pd.num_layers = d.num_layers;
  pd.page_size = d.page_size;
  pd.num_pages = d.num_pages;
  pd.max_seqs = d.max_seqs;
  pd.max_pages_per_seq = d.max_pages_per_seq;
  pd.kv_lora_rank = 0;
  pd.rope_dim = d.rotary_dim;
  pd.rope_pairing = d.rope_pairing;
  pd.rope_base = d.rope_base;
  pd.layer_base = nullptr;
  pd.page_table = d.page_table;
  pd.device = d.device;
  p->gqa = true;
  p->layer_ptrs.assign(d.k_layer_base, d.k_layer_base + d.num_layers);
  p->layer_ptrs.insert(p->layer_ptrs.end(), d.v_layer_base, d.v_layer_base + d.num_layers);
  p->heads = d.num_kv_heads;
  p->head_chunks = d.head_dim / 8;
  while ((8 << p->rot_shift) < d.rotary_dim) ++p->rot_shift;
  p->row_bytes = static_cast<int64_t>(d.num_kv_heads) * d.head_dim * 2;
  p->band_bytes = static_cast<int64_t>(d.num_kv_heads) * d.rotary_dim * 2;
  return setup_pool(p, out);
} catch (...) {
  return host_exception(nullptr);
}

void ll_pool_destroy(ll_pool* p) try {
  if (!p) return;
  DeviceGuard g(p->desc.device);
  {
    hipError_t e;
    hipEvent_t ev = last_work(p, &e);
    if (ev) (void)hipEventSynchronize(ev);
  }
  if (p->pending.active) (void)hipEventSynchronize(p->pending.done);
  for (auto& r : p->ring_inflight) (void)hipEventDestroy(r.done);
  for (auto e : p->ring_events) (void)hipEventDestroy(e);
  if (p->upload_ev) (void)hipEventDestroy(p->upload_ev);
  if (p->ring_host) (void)hipHostFree(p->ring_host);
  if (p->ring_dev) (void)hipFree(p->ring_dev);
  for (auto& v : p->prof)
    for (auto& r : v) {
      (void)hipEventDestroy(r.start);
      (void)hipEventDestroy(r.stop);
    }
  for (auto e : p->spare_events) (void)hipEventDestroy(e);
  if (p->readback_ev) (void)hipEventDestroy(p->readback_ev);
  if (p->pending.done) (void)hipEventDestroy(p->pending.done);
  if (p->copy_stream) {
    (void)hipStreamSynchronize(p->copy_stream);
    (void)hipStreamDestroy(p->copy_stream);
  }
  if (p->h_readback) (void)hipHostFree(p->h_readback);
  if (p->d_scratch) (void)hipFree(p->d_scratch);
  if (p->d_rowtab) (void)hipFree(p->d_rowtab);
  if (p->d_direct) (void)hipFree(p->d_direct);
  if (p->lazy_ev) (void)hipEventDestroy(p->lazy_ev);
  if (p->d_layers) (void)hipFree(p->d_layers);
  delete p;
} catch (...) {
  return;
}

ll_status ll_pool_free_pages(const ll_pool* p, int64_t* n_free) try {
  if (!p || !n_free) return fail(LL_EINVAL, "NULL argument");
  ll_status rc = settle(const_cast<ll_pool*>(p));
  if (rc) return rc;
  *n_free = p->free.count();
  return LL_OK;
} catch (...) {
  return host_exception(const_cast<ll_pool*>(p));
}

ll_status ll_seq_get(const ll_pool* p, int32_t seq, int64_t* len, int64_t* next_position, int32_t* pages_out,
                     int32_t cap, int32_t* n_pages_out) try {
  if (!p) return fail(LL_EINVAL, "pool is NULL");
  ll_status rc = settle(const_cast<ll_pool*>(p));
  if (rc) return rc;
  if (seq < 0 || seq >= p->desc.max_seqs || !p->seqs[seq].used) return fail(LL_EINVAL, "unknown sequence %d", seq);
  if (cap > 0 && !pages_out) return fail(LL_EINVAL, "pages_out is NULL");
  if (pages_out || n_pages_out)
    if ((rc = fresh_table(const_cast<ll_pool*>(p), seq))) return rc;
  const SeqState& s = p->seqs[seq];
  if (len) *len = s.len;
  if (next_position) *next_position = s.next_pos;
  if (n_pages_out) *n_pages_out = static_cast<int32_t>(s.pages.size());
  const int32_t k = std::min<int32_t>(cap, static_cast<int32_t>(s.pages.size()));
  if (k > 0) std::memcpy(pages_out, s.pages.data(), sizeof(int32_t) * k);
  return LL_OK;
} catch (...) {
  return host_exception(const_cast<ll_pool*>(p));
}

ll_status ll_seq_alloc(ll_pool* p, int64_t n_tokens, int32_t* seq_id_out, void* stream) try {
  ll_status rc = enter(p);
  if (rc) return rc;
  if (!seq_id_out || n_tokens < 0) return fail(LL_EINVAL, "bad argument");
  const int64_t need = ceil_div(n_tokens, p->P);
  if (need > p->desc.max_pages_per_seq) return fail(LL_ERANGE, "%lld rows exceed the page-table row", (long long)n_tokens);
  int32_t seq = -1;
  for (int32_t i = 0; i < p->desc.max_seqs; ++i)
    if (!p->seqs[i].used) {
      seq = i;
      break;
    }
  if (seq < 0) return fail(LL_ENOMEM, "no free sequence id");
  if (need > p->free.count()) return fail(LL_ENOMEM, "need %lld pages, %lld free", (long long)need, (long long)p->free.count());
  std::vector<int32_t> pages;
  p->free.lowest(need, pages);
  DeviceGuard g(p->desc.device);
  TablePlan tp;
  tp.add(seq, pages);
  rc = write_tables(p, tp, static_cast<hipStream_t>(stream));
  if (rc) return rc;
  for (int32_t pg : pages) p->free.take(pg);
  p->free.advance_hint();
  SeqState& s = p->seqs[seq];
  s.used = true;
  s.len = n_tokens;
  s.next_pos = n_tokens;
  s.pages = std::move(pages);
  *seq_id_out = seq;
  return LL_OK;
} catch (...) {
  return host_exception(p);
}

ll_status ll_seq_set_pages(ll_pool* p, int32_t seq, const int32_t* pages, int64_t n_tokens, void* stream) try {
  ll_status rc = enter(p);
  if (rc) return rc;
  if (seq < 0 || seq >= p->desc.max_seqs) return fail(LL_EINVAL, "bad sequence id %d", seq);
  if (n_tokens < 0) return fail(LL_EINVAL, "n_tokens < 0");
  const int64_t need = ceil_div(n_tokens, p->P);
  if (need > p->desc.max_pages_per_seq) return fail(LL_ERANGE, "%lld rows exceed the page-table row", (long long)n_tokens);
  if (need > 0 && !pages) return fail(LL_EINVAL, "pages is NULL");
  if ((rc = fresh_table(p, seq))) return rc;
  SeqState& s = p->seqs[seq];
  // page_slot marks (reset before returning): -2 owned, -3 listed, -4 both
  std::vector<int32_t>& mark = p->page_slot;
  if (s.used)
    for (int32_t pg : s.pages) mark[pg] = -2;
  ll_status bad = LL_OK;
  int64_t listed = 0;
  for (; listed < need; ++listed) {
    const int32_t pg = pages[listed];
    if (pg < 0 || pg >= p->desc.num_pages) {
      bad = fail(LL_EINVAL, "page %d out of range", pg);
      break;
    }
    if (mark[pg] == -3 || mark[pg] == -4) {
      bad = fail(LL_EINVAL, "page %d listed twice", pg);
      break;
    }
    if (!p->free.is_free(pg) && mark[pg] != -2) {
      bad = fail(LL_EINVAL, "page %d is not free", pg);
      break;
    }
    mark[pg] = mark[pg] == -2 ? -4 : -3;
  }
  std::vector<int32_t> released;
  if (s.used)
    for (int32_t pg : s.pages)
      if (mark[pg] == -2) released.push_back(pg);
  for (int64_t i = 0; i < listed; ++i) mark[pages[i]] = -1;
  if (s.used)
    for (int32_t pg : s.pages) mark[pg] = -1;
  if (bad) return bad;
  std::vector<int32_t> t(pages, pages + need);
  DeviceGuard g(p->desc.device);
  TablePlan tp;
  tp.add(seq, t);
  rc = write_tables(p, tp, static_cast<hipStream_t>(stream));
  if (rc) return rc;
  for (int32_t pg : released) p->free.give(pg);
  for (int32_t pg : t)
    if (p->free.is_free(pg)) p->free.take(pg);
  p->free.advance_hint();
  s.used = true;
  s.len = n_tokens;
  s.next_pos = n_tokens;
  s.pages = std::move(t);
  return LL_OK;
} catch (...) {
  return host_exception(p);
}

ll_status ll_seq_free(ll_pool* p, int32_t seq) try {
  ll_status rc = enter(p);
  if (rc) return rc;
  if (seq < 0 || seq >= p->desc.max_seqs || !p->seqs[seq].used) return fail(LL_EINVAL, "unknown sequence %d", seq);
  if ((rc = fresh_table(p, seq))) return rc;
  SeqState& s = p->seqs[seq];
  for (int32_t pg : s.pages) p->free.give(pg);
  s = SeqState();
  return LL_OK;
} catch (...) {
  return host_exception(p);
}

// The splice.  noalloc: the plan always goes to the device as kernel
// arguments and its expansion lands in the library's static device scratch
// (no device or pinned memory is allocated, no event is created, no launch
// is timed); a batch that the device cannot plan, or whose plan exceeds the
// scratch, is refused before anything changes.
static ll_status splice_impl(ll_pool* p, const ll_directive* dirs, int32_t n, void* stream, bool noalloc) {
  ll_status rc = enter(p);
  if (rc) return rc;
  if (n < 0 || (n > 0 && !dirs)) return fail(LL_EINVAL, "bad directive array");
  if (n == 0) return LL_OK;
  if ((rc = validate_directives(p, dirs, n))) return rc;
  {
    std::vector<int32_t> ids(static_cast<size_t>(n));
    for (int32_t i = 0; i < n; ++i) ids[i] = dirs[i].seq_id;
    if ((rc = fresh_tables(p, ids.data(), ids.size()))) return rc;
  }

  // --- plan (host only, no state change yet)
  const int64_t P = p->P;
  std::vector<SplicePlan> plans(static_cast<size_t>(n));
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    plan_splice(p, dirs[i], p->seqs[dirs[i].seq_id], &plans[i]);
    need += plans[i].fresh;
  }
  if (need > p->free.count())
    return fail(LL_ENOMEM, "need %lld fresh pages, %lld free", (long long)need, (long long)p->free.count());
  std::vector<int32_t> fresh;
  p->free.lowest(need, fresh);

  int64_t n_move_tasks = 0, n_rot_tasks = 0, n_entries = 0;
  for (int32_t i = 0; i < n; ++i) {
    n_move_tasks += plans[i].fresh;
    for (char x : plans[i].inplace) n_rot_tasks += x;
    n_entries += static_cast<int64_t>(plans[i].reuse.size());
  }
  const int64_t row_chunks = p->row_bytes / 16;
  // chunk indices are 32-bit, with room for the last block's overhang
  if (n_move_tasks * P * row_chunks >= (int64_t{1} << 32) - 1024 || n_rot_tasks * P * row_chunks >= (int64_t{1} << 32) - 1024)
    return fail(LL_EUNSUPPORTED, "one splice may write at most 2^32 16-byte chunks per layer");
  const size_t dir_bytes = p->gqa ? sizeof(ll::GqaDir) : sizeof(ll::SpliceDir);
  const int pairs = p->gqa ? p->desc.rope_dim / 2 : ll::kHalfPairs;

  // --- who expands the plan.  The device does (from kernel arguments, no
  // staging and no upload) when the batch is small, its fresh pages form few
  // runs of consecutive ids, and every directive's fresh pages and
  // rotate-in-place pages each form one range of q.
  bool direct = (noalloc || p->splice_planner == LL_SPLICE_PLAN_AUTO) && n <= ll::kDirectMaxDirs &&
                n * 2 * pairs <= ll::kDirectTrigFloats;
  std::vector<int32_t> run_page, run_first;
  std::vector<int32_t> q_fresh0(static_cast<size_t>(n), 0), q_rot0(static_cast<size_t>(n), 0);
  std::vector<int32_t> n_rot_of(static_cast<size_t>(n), 0);
  for (size_t k = 0; direct && k < fresh.size(); ++k) {
    if (k > 0 && fresh[k] == fresh[k - 1] + 1) continue;
    if (run_page.size() == static_cast<size_t>(ll::kDirectMaxRuns)) direct = false;
    run_page.push_back(fresh[k]);
    run_first.push_back(static_cast<int32_t>(k));
  }
  for (int32_t i = 0; direct && i < n; ++i) {
    const SplicePlan& pl = plans[i];
    const int64_t pages = static_cast<int64_t>(pl.reuse.size());
    int64_t f0 = -1, nf = 0, r0 = -1, nr = 0;
    for (int64_t q = 0; q < pages; ++q) {
      if (pl.reuse[q] < 0) {
        if (f0 < 0) f0 = q;
        direct = direct && q == f0 + nf;
        ++nf;
      } else if (pl.inplace[q]) {
        if (r0 < 0) r0 = q;
        direct = direct && q == r0 + nr;
        ++nr;
      }
    }
    q_fresh0[i] = static_cast<int32_t>(std::max<int64_t>(f0, 0));
    q_rot0[i] = static_cast<int32_t>(std::max<int64_t>(r0, 0));
    n_rot_of[i] = static_cast<int32_t>(nr);
  }
  const size_t n_tasks = static_cast<size_t>(n_move_tasks + n_rot_tasks);
  // offsets of the tasks, rotation tables, table writes and tables from the
  // base of the plan space (device-planned) or of the staging region
  size_t o_t = 0;
  size_t o_d = align_up(o_t + n_tasks * sizeof(ll::SpliceTask), 256);
  size_t o_w = align_up(o_d + n * dir_bytes, 256);
  size_t o_p = align_up(o_w + n * sizeof(ll::TableWrite), 256);
  const size_t direct_bytes = o_p + static_cast<size_t>(n_entries) * 4;
  char* scratch = nullptr;
  if (noalloc) {
    if (!direct)
      return fail(LL_EUNSUPPORTED,
                  "leyline_splice_noalloc plans on the device only: at most %d directives (%d on this pool) whose "
                  "fresh pages form at most %d runs of consecutive ids",
                  ll::kDirectMaxDirs, ll::kDirectTrigFloats / (2 * pairs), ll::kDirectMaxRuns);
    if (direct_bytes > ll::kNoAllocScratchBytes)
      return fail(LL_EUNSUPPORTED, "leyline_splice_noalloc: the plan needs %zu bytes, the scratch holds %zu",
                  direct_bytes, ll::kNoAllocScratchBytes);
    scratch = static_cast<char*>(ll::noalloc_scratch(p->desc.device));
    if (!scratch) return fail(LL_EDEVICE, "the no-allocation scratch of device %d was not found", p->desc.device);
  } else if (direct && direct_bytes > p->direct_cap) {
    // grows rarely (a larger batch than any before); waits for earlier work
    if ((rc = wait_idle(p))) return rc;
    if (p->d_direct) (void)hipFree(p->d_direct);
    p->d_direct = nullptr;
    p->direct_cap = 0;
    const size_t cap = std::max(align_up(direct_bytes, size_t{1} << 20), size_t{1} << 20);
    if (hipMalloc(reinterpret_cast<void**>(&p->d_direct), cap) != hipSuccess)
      return fail(LL_ENOMEM, "cannot allocate %zu bytes of splice plan space", cap);
    p->direct_cap = cap;
  }

  // --- device work: one launch on the host-planned path (descriptors written
  // straight into pinned staging, one upload), two on the device-planned one
  // (plan expansion, then the same row kernel)
  DeviceGuard g(p->desc.device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((rc = begin_call(p, st))) return rc;
  Staging* sg = nullptr;
  char* dev_base = noalloc ? scratch : p->d_direct;
  ll::DirectPlanArgs da{};
  ll::SpliceDir* ddirs = nullptr;
  ll::GqaDir* gdirs = nullptr;
  ll::SpliceTask* move_out = nullptr;
  ll::SpliceTask* rot_out = nullptr;
  ll::TableWrite* writes = nullptr;
  int32_t* packed = nullptr;
  if (!direct) {
    rc = stage_acquire(p, stage_bytes_for({n * dir_bytes, n_tasks * sizeof(ll::SpliceTask),
                                           n * sizeof(ll::TableWrite), static_cast<size_t>(n_entries) * 4}),
                       &sg);
    if (rc) return rc;
    o_d = stage_put(sg, nullptr, n * dir_bytes);
    o_t = stage_put(sg, nullptr, n_tasks * sizeof(ll::SpliceTask));
    o_w = stage_put(sg, nullptr, n * sizeof(ll::TableWrite));
    o_p = stage_put(sg, nullptr, static_cast<size_t>(n_entries) * 4);
    ddirs = reinterpret_cast<ll::SpliceDir*>(sg->host + o_d);
    gdirs = reinterpret_cast<ll::GqaDir*>(sg->host + o_d);
    move_out = reinterpret_cast<ll::SpliceTask*>(sg->host + o_t);
    rot_out = move_out + n_move_tasks;
    writes = reinterpret_cast<ll::TableWrite*>(sg->host + o_w);
    packed = reinterpret_cast<int32_t*>(sg->host + o_p);
    dev_base = sg->dev;
  }

  ProfRec rec{};
  ll::Stamp ts;
  auto launch_rows = [&]() -> ll_status {
    hipError_t e;
    if (p->gqa) {
      ll::GqaSpliceLaunch a{};
      a.planes = reinterpret_cast<const ll::chunk_t* const*>(p->d_layers);
      a.num_layers = p->desc.num_layers;
      a.page_shift = p->page_shift;
      a.row_chunks = static_cast<int32_t>(row_chunks);
      a.head_chunks = p->head_chunks;
      a.rot_shift = p->rot_shift;
      a.heads = p->heads;
      a.tasks = reinterpret_cast<const ll::SpliceTask*>(dev_base + o_t);
      a.n_move_tasks = n_move_tasks;
      a.n_rot_tasks = n_rot_tasks;
      // one thread per two chunks in K and V planes (row_chunks is even:
      // head_dim is a multiple of 16)
      a.move_blocks_per_plane = ll::flat_blocks(n_move_tasks * P * (row_chunks / 2));
      a.rot_blocks_per_plane = ll::flat_blocks(n_rot_tasks * P * (p->heads << (p->rot_shift - 1)));
      a.dirs = reinterpret_cast<const ll::GqaDir*>(dev_base + o_d);
      a.twrites = reinterpret_cast<const ll::TableWrite*>(dev_base + o_w);
      a.tables = reinterpret_cast<const int32_t*>(dev_base + o_p);
      a.n_twrites = n;
      a.max_pages_per_seq = p->desc.max_pages_per_seq;
      a.page_table = p->desc.page_table;
      if (!noalloc && prof_pick(p, 0) && (rc = prof_begin(p, &rec, &ts))) return rc;
      const int64_t L = a.num_layers;
      if ((3 * a.move_blocks_per_plane + a.rot_blocks_per_plane) * L + n <= p->dispatch_items / ll::kFlatThreads) {
        e = ll::launch_gqa_splice(a, p->desc.rope_pairing, st, ts);
        if (e != hipSuccess) return device_fail(p, e, "gqa_splice_kernel launch");
      } else {
        // the in-place bands on their own, then ranges of whole move tasks
        // over the K and V planes of every layer; the table rewrites ride in
        // the last launch
        ll::GqaSpliceLaunch part = a;
        if (n_rot_tasks > 0) {
          part.move_blocks_per_plane = 0;
          part.n_twrites = n_move_tasks == 0 ? n : 0;
          e = ll::launch_gqa_splice(part, p->desc.rope_pairing, st, part_stamp(ts, true, n_move_tasks == 0));
          if (e != hipSuccess) return device_fail(p, e, "gqa_splice_kernel launch");
        }
        const int64_t units = P * (row_chunks / 2);
        const int64_t per = tasks_per_dispatch(p->dispatch_items, units, 3 * L, ll::kFlatThreads, ll::kFlatThreads, n);
        for (int64_t k0 = 0; k0 < n_move_tasks; k0 += per) {
          const int64_t cnt = std::min(per, n_move_tasks - k0);
          const bool last = k0 + cnt == n_move_tasks;
          part = a;
          part.tasks = a.tasks + k0;
          part.n_move_tasks = cnt;
          part.n_rot_tasks = 0;
          part.rot_blocks_per_plane = 0;
          part.move_blocks_per_plane = ll::flat_blocks(cnt * units);
          part.n_twrites = last ? n : 0;
          e = ll::launch_gqa_splice(part, p->desc.rope_pairing, st, part_stamp(ts, k0 == 0 && n_rot_tasks == 0, last));
          if (e != hipSuccess) return device_fail(p, e, "gqa_splice_kernel launch");
        }
      }
    } else {
      ll::SpliceLaunch a{};
      a.layers = reinterpret_cast<const ll::chunk_t* const*>(p->d_layers);
      a.num_layers = p->desc.num_layers;
      a.page_shift = p->page_shift;
      a.tasks = reinterpret_cast<const ll::SpliceTask*>(dev_base + o_t);
      a.n_move_tasks = n_move_tasks;
      a.n_rot_tasks = n_rot_tasks;
      a.move_blocks_per_layer = ll::flat_blocks(n_move_tasks * P * ll::kRowChunks, ll::kSpliceChunksPerThread);
      a.rot_blocks_per_layer = (n_rot_tasks * P + ll::kInPlaceRowsPerBlock - 1) / ll::kInPlaceRowsPerBlock;
      a.dirs = reinterpret_cast<const ll::SpliceDir*>(dev_base + o_d);
      a.twrites = reinterpret_cast<const ll::TableWrite*>(dev_base + o_w);
      a.tables = reinterpret_cast<const int32_t*>(dev_base + o_p);
      a.n_twrites = n;
      a.max_pages_per_seq = p->desc.max_pages_per_seq;
      a.page_table = p->desc.page_table;
      if (!noalloc && prof_pick(p, 0) && (rc = prof_begin(p, &rec, &ts))) return rc;
      const int64_t L = a.num_layers;
      if (a.move_blocks_per_layer * L + n <= p->dispatch_items / ll::kFlatThreads) {
        e = ll::launch_splice(a, p->desc.rope_pairing, st, ts);
        if (e != hipSuccess) return device_fail(p, e, "splice_kernel launch");
      } else {
        // as above: the in-place bands, then ranges of whole move tasks over
        // every layer, the table rewrites in the last launch
        ll::SpliceLaunch part = a;
        if (n_rot_tasks > 0) {
          part.move_blocks_per_layer = 0;
          part.n_twrites = n_move_tasks == 0 ? n : 0;
          e = ll::launch_splice(part, p->desc.rope_pairing, st, part_stamp(ts, true, n_move_tasks == 0));
          if (e != hipSuccess) return device_fail(p, e, "splice_inplace_kernel launch");
        }
        const int64_t units = P * ll::kRowChunks;
        const int64_t per = tasks_per_dispatch(p->dispatch_items, units, L, ll::kFlatThreads,
                                               int64_t{ll::kFlatThreads} * ll::kSpliceChunksPerThread, n);
        for (int64_t k0 = 0; k0 < n_move_tasks; k0 += per) {
          const int64_t cnt = std::min(per, n_move_tasks - k0);
          const bool last = k0 + cnt == n_move_tasks;
          part = a;
          part.tasks = a.tasks + k0;
          part.n_move_tasks = cnt;
          part.n_rot_tasks = 0;
          part.rot_blocks_per_layer = 0;
          part.move_blocks_per_layer = ll::flat_blocks(cnt * units, ll::kSpliceChunksPerThread);
          part.n_twrites = last ? n : 0;
          e = ll::launch_splice(part, p->desc.rope_pairing, st, part_stamp(ts, k0 == 0 && n_rot_tasks == 0, last));
          if (e != hipSuccess) return device_fail(p, e, "splice_kernel launch");
        }
      }
    }
    return LL_OK;
  };
  if (direct) {
    // the compact plan from per-directive counts; the launches go out before
    // the host's own tables and counters are made
    int64_t mb = 0, rb = 0, pk = 0;
    for (int32_t i = 0; i < n; ++i) {
      const ll_directive& d = dirs[i];
      const SplicePlan& pl = plans[i];
      const int64_t r = d.mode == LL_FORGET ? 0 : d.r_len;
      float* cos_out = da.trig + 2 * pairs * i;
      rope_table_from(p->theta, pl.delta, cos_out, cos_out + pairs);
      ll::DirectDir& dd = da.d[i];
      dd.stub = static_cast<const ll::chunk_t*>(d.mode == LL_FORGET ? nullptr : d.r_rows);
      dd.stub_layer_chunks = (d.r_layer_stride_bytes ? d.r_layer_stride_bytes : r * p->row_bytes) / 16;
      dd.stub_v = p->gqa ? static_cast<const ll::chunk_t*>(d.mode == LL_FORGET ? nullptr : d.r_rows_v) : nullptr;
      dd.stub_v_layer_chunks =
          p->gqa ? (d.r_layer_stride_bytes_v ? d.r_layer_stride_bytes_v : r * p->row_bytes) / 16 : 0;
      dd.seq = d.seq_id;
      dd.s_start = static_cast<int32_t>(d.s_start);
      dd.stub_end = static_cast<int32_t>(d.s_start + r);
      dd.delta = static_cast<int32_t>(pl.delta);
      dd.n_new = static_cast<int32_t>(pl.n_new);
      dd.old_pages = static_cast<int32_t>(p->seqs[d.seq_id].pages.size());
      dd.rotate = (d.mode == LL_AMORTIZE && pl.delta != 0) ? 1 : 0;
      dd.q_fresh0 = q_fresh0[i];
      dd.q_rot0 = q_rot0[i];
      dd.move_base = static_cast<int32_t>(mb);
      dd.rot_base = static_cast<int32_t>(rb);
      dd.fresh_base = static_cast<int32_t>(mb);
      dd.packed_off = static_cast<int32_t>(pk);
      mb += pl.fresh;
      rb += n_rot_of[i];
      pk += static_cast<int64_t>(pl.reuse.size());
    }
    da.n_dirs = n;
    da.page_shift = p->page_shift;
    da.pairs = pairs;
    da.n_runs = static_cast<int32_t>(run_page.size());
    da.max_pages_per_seq = p->desc.max_pages_per_seq;
    da.gqa = p->gqa ? 1 : 0;
    da.page_reuse = p->page_reuse ? 1 : 0;
    da.n_move_tasks = n_move_tasks;
    da.n_rot_tasks = n_rot_tasks;
    da.n_entries = n_entries;
    da.page_table = p->desc.page_table;
    da.tasks = reinterpret_cast<ll::SpliceTask*>(dev_base + o_t);
    da.dirs = dev_base + o_d;
    da.twrites = reinterpret_cast<ll::TableWrite*>(dev_base + o_w);
    da.tables = reinterpret_cast<int32_t*>(dev_base + o_p);
    for (size_t k = 0; k < run_page.size(); ++k) {
      da.run_page[k] = run_page[k];
      da.run_first[k] = run_first[k];
    }
    da.run_first[run_page.size()] = static_cast<int32_t>(fresh.size());
    int32_t max_new_pages = 0;
    for (const SplicePlan& pl : plans) max_new_pages = std::max(max_new_pages, static_cast<int32_t>(pl.reuse.size()));
    hipError_t e = ll::launch_splice_plan(da, max_new_pages, st);
    if (e != hipSuccess) return device_fail(p, e, "splice_plan_kernel launch");
    if ((rc = launch_rows())) return rc;
  }

  std::vector<std::vector<int32_t>> new_tables(static_cast<size_t>(n));
  ll_plan_stats stats{};
  size_t cursor = 0;
  int64_t packed_at = 0;
  for (int32_t i = 0; i < n; ++i) {
    const ll_directive& d = dirs[i];
    const SplicePlan& pl = plans[i];
    const SeqState& s = p->seqs[d.seq_id];
    const std::vector<int32_t>& T = s.pages;
    const int64_t old_pages = static_cast<int64_t>(T.size());
    const int64_t r = d.mode == LL_FORGET ? 0 : d.r_len;
    if (!direct) {
      rope_table_from(p->theta, pl.delta, p->gqa ? gdirs[i].cos_ : ddirs[i].cos_,
                      p->gqa ? gdirs[i].sin_ : ddirs[i].sin_);
      if (p->gqa) {
        gdirs[i].stub_v = static_cast<const ll::chunk_t*>(d.mode == LL_FORGET ? nullptr : d.r_rows_v);
        gdirs[i].stub_v_layer_chunks = (d.r_layer_stride_bytes_v ? d.r_layer_stride_bytes_v : r * p->row_bytes) / 16;
      }
    }
    ll::SpliceTask base{};
    base.dir = i;
    base.rotate = (d.mode == LL_AMORTIZE && pl.delta != 0) ? 1 : 0;
    base.s_start = static_cast<int32_t>(d.s_start);
    base.stub_end = static_cast<int32_t>(d.s_start + r);
    base.delta = static_cast<int32_t>(pl.delta);
    base.n_new = static_cast<int32_t>(pl.n_new);
    base.stub = static_cast<const ll::chunk_t*>(d.mode == LL_FORGET ? nullptr : d.r_rows);
    base.stub_layer_chunks = (d.r_layer_stride_bytes ? d.r_layer_stride_bytes : r * p->row_bytes) / 16;
    base.pre_page = base.down_page0 = base.down_page1 = -1;
    base.down_lp0 = -1;
    std::vector<int32_t>& nt = new_tables[i];
    nt.resize(pl.reuse.size());
    for (size_t q = 0; q < pl.reuse.size(); ++q) {
      const int64_t a = static_cast<int64_t>(q) * P, b = std::min(a + P, pl.n_new);
      if (pl.reuse[q] >= 0) {
        nt[q] = T[pl.reuse[q]];
        if (pl.inplace[q]) {
          if (!direct) {
            ll::SpliceTask t = base;
            t.q = static_cast<int32_t>(q);
            t.dst_page = nt[q];
            *rot_out++ = t;
          }
          stats.rows_rotated_inplace += b - a;
        }
        continue;
      }
      nt[q] = fresh[cursor++];
      stats.rows_moved += b - a;
      if (direct) continue;
      ll::SpliceTask t = base;
      t.q = static_cast<int32_t>(q);
      t.dst_page = nt[q];
      if (a < d.s_start && static_cast<int64_t>(q) < old_pages) t.pre_page = T[q];
      const int64_t jd = std::max(a, d.s_start + r);  // first downstream row of the page
      if (jd < b) {
        const int64_t lp0 = (jd - pl.delta) / P;
        t.down_lp0 = static_cast<int32_t>(lp0);
        t.down_page0 = T[lp0];
        t.down_page1 = lp0 + 1 < old_pages ? T[lp0 + 1] : -1;
      }
      *move_out++ = t;
    }
    if (!direct) {
      writes[i].src_off = packed_at;
      writes[i].seq = d.seq_id;
      writes[i].count = static_cast<int32_t>(nt.size());
      if (!nt.empty()) std::memcpy(packed + packed_at, nt.data(), nt.size() * 4);
    }
    packed_at += static_cast<int64_t>(nt.size());
  }
  stats.fresh_pages = need;
  stats.table_entries = n_entries;
  stats.planned_on_device = direct ? 1 : 0;
  // old pages no new page keeps: released once the call is committed
  std::vector<int32_t> released;
  for (int32_t i = 0; i < n; ++i) {
    const SeqState& s = p->seqs[dirs[i].seq_id];
    std::vector<char> kept(s.pages.size(), 0);
    for (int32_t x : plans[i].reuse)
      if (x >= 0) kept[x] = 1;
    for (size_t k = 0; k < kept.size(); ++k)
      if (!kept[k]) released.push_back(s.pages[k]);
  }
  stats.freed_pages = static_cast<int64_t>(released.size());
  const int64_t L = p->desc.num_layers;
  stats.alg_bytes = p->num_planes * 2 * p->row_bytes * stats.rows_moved + L * 2 * p->band_bytes * stats.rows_rotated_inplace;
  if (!direct) {
    if ((rc = upload(p, sg, st))) return rc;
    if ((rc = launch_rows())) return rc;
  }
  if (rec.start) {
    rec.bytes = stats.alg_bytes + 4 * stats.table_entries;
    prof_end(p, 0, rec);
  }
  if (direct) {
    p->last_stream = st;
    p->unevented = true;
  } else if ((rc = end_call(p, sg, st))) {
    return rc;
  }

  // --- commit host state
  for (int32_t pg : fresh) p->free.take(pg);
  p->free.advance_hint();
  for (int32_t pg : released) p->free.give(pg);
  for (int32_t i = 0; i < n; ++i) {
    SeqState& s = p->seqs[dirs[i].seq_id];
    s.pages = std::move(new_tables[i]);
    s.len = plans[i].n_new;
    s.next_pos = plans[i].next_pos;
  }
  p->last = stats;
  return LL_OK;
}

ll_status leyline_splice(ll_pool* p, const ll_directive* dirs, int32_t n, void* stream) try {
  return splice_impl(p, dirs, n, stream, false);
} catch (...) {
  return host_exception(p);
}

ll_status leyline_splice_noalloc(ll_pool* p, const ll_directive* dirs, int32_t n, void* stream) try {
  return splice_impl(p, dirs, n, stream, true);
} catch (...) {
  return host_exception(p);
}

ll_status kv_evict_compact(ll_pool* p, const int32_t* seq_ids, int32_t n, const uint8_t* keep_dev,
                           const int64_t* keep_offsets, void* stream) try {
  ll_status rc = enter(p);
  if (rc) return rc;
  if (n < 0 || (n > 0 && (!seq_ids || !keep_offsets))) return fail(LL_EINVAL, "bad arguments");
  if (n == 0) return LL_OK;
  std::vector<char> seen(static_cast<size_t>(p->desc.max_seqs), 0);
  int64_t total_rows = 0, total_pages = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = seq_ids[i];
    if (s < 0 || s >= p->desc.max_seqs || !p->seqs[s].used) return fail(LL_EINVAL, "entry %d: unknown sequence %d", i, s);
    if (seen[s]) return fail(LL_EINVAL, "entry %d: sequence %d appears twice", i, s);
    seen[s] = 1;
    if (keep_offsets[i] < 0) return fail(LL_EINVAL, "entry %d: negative mask offset", i);
    total_rows += p->seqs[s].len;
    total_pages += ceil_div(p->seqs[s].len, p->P);
  }
  if (total_rows > 0 && !keep_dev) return fail(LL_EINVAL, "keep mask is NULL");
  DeviceGuard g(p->desc.device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  std::vector<ll::EvictSeq> es(static_cast<size_t>(n));
  {
    int64_t ro = 0, so = 0;
    for (int32_t i = 0; i < n; ++i) {
      const SeqState& s = p->seqs[seq_ids[i]];
      es[i].mask_off = keep_offsets[i];
      es[i].n_old = s.len;
      es[i].src_off = so;
      es[i].reuse_off = ro;
      es[i].seq = seq_ids[i];
      so += s.len;
      ro += ceil_div(s.len, p->P);
    }
  }
  return evict_device_plan(p, seq_ids, n, keep_dev, es, total_rows, total_pages, st);
} catch (...) {
  return host_exception(p);
}

ll_status ll_ptable_reindex(ll_pool* p, int32_t seq, const int32_t* keep_pages, int32_t n_keep, void* stream) try {
  ll_status rc = enter(p);
  if (rc) return rc;
  if (seq < 0 || seq >= p->desc.max_seqs || !p->seqs[seq].used) return fail(LL_EINVAL, "unknown sequence %d", seq);
  if (n_keep < 0 || (n_keep > 0 && !keep_pages)) return fail(LL_EINVAL, "bad keep_pages");
  if ((rc = fresh_table(p, seq))) return rc;
  SeqState& s = p->seqs[seq];
  const int64_t P = p->P;
  const int64_t old_pages = static_cast<int64_t>(s.pages.size());
  const bool tail_partial = s.len % P != 0;
  int64_t new_len = 0;
  for (int32_t i = 0; i < n_keep; ++i) {
    const int32_t k = keep_pages[i];
    if (k < 0 || k >= old_pages) return fail(LL_EINVAL, "keep_pages[%d] = %d out of range", i, k);
    if (i > 0 && k <= keep_pages[i - 1]) return fail(LL_EINVAL, "keep_pages must be strictly increasing");
    if (tail_partial && k == old_pages - 1 && i != n_keep - 1)
      return fail(LL_EINVAL, "a partial tail page may only be kept last");
    new_len += std::min(P, s.len - k * P);
  }
  std::vector<int32_t> nt(static_cast<size_t>(n_keep));
  std::vector<char> kept(static_cast<size_t>(old_pages), 0);
  for (int32_t i = 0; i < n_keep; ++i) {
    nt[i] = s.pages[keep_pages[i]];
    kept[keep_pages[i]] = 1;
  }
  DeviceGuard g(p->desc.device);
  TablePlan tp;
  tp.add(seq, nt);
  if ((rc = write_tables(p, tp, static_cast<hipStream_t>(stream)))) return rc;
  ll_plan_stats stats{};
  for (int64_t k = 0; k < old_pages; ++k)
    if (!kept[k]) {
      p->free.give(s.pages[k]);
      ++stats.freed_pages;
    }
  stats.table_entries = n_keep;
  s.pages = std::move(nt);
  s.len = new_len;
  p->last = stats;
  return LL_OK;
} catch (...) {
  return host_exception(p);
}

ll_status ll_rope_rows(ll_pool* p, int32_t seq, int64_t row_begin, int64_t n_rows, const int64_t* angle_dev,
                       void* out_dev, int64_t out_layer_stride_bytes, void* stream) try {
  ll_status rc = enter(p);
  if (rc) return rc;
  if (seq < 0 || seq >= p->desc.max_seqs || !p->seqs[seq].used) return fail(LL_EINVAL, "unknown sequence %d", seq);
  if ((rc = fresh_table(p, seq))) return rc;
  const SeqState& s = p->seqs[seq];
  if (row_begin < 0 || n_rows < 0 || row_begin + n_rows > s.len)
    return fail(LL_EINVAL, "rows [%lld, %lld) outside the sequence's %lld rows", (long long)row_begin,
                (long long)(row_begin + n_rows), (long long)s.len);
  if (n_rows > 0 && !angle_dev) return fail(LL_EINVAL, "angle_dev is NULL");
  const int64_t L = p->desc.num_layers;
  if (out_dev) {
    if (reinterpret_cast<uintptr_t>(out_dev) & 15) return fail(LL_EINVAL, "out_dev is not 16-byte aligned");
    if (out_layer_stride_bytes < 0 || (out_layer_stride_bytes & 15) ||
        (out_layer_stride_bytes && L > 1 && out_layer_stride_bytes < n_rows * p->row_bytes))
      return fail(LL_EINVAL, "bad out_layer_stride_bytes");
  }
  ll::RowShape sh{};
  if (p->gqa) {
    sh.row_chunks = static_cast<int32_t>(p->row_bytes / 16);
    sh.heads = p->heads;
    sh.head_chunks = p->head_chunks;
    sh.band_off = 0;
    sh.band_shift = p->rot_shift;
  } else {
    sh.row_chunks = ll::kRowChunks;
    sh.heads = 1;
    sh.head_chunks = ll::kRowChunks;
    sh.band_off = ll::kKpeChunk0;
    sh.band_shift = 3;
  }
  sh.pairs = 4 << sh.band_shift;
  const int64_t per_row = out_dev ? sh.row_chunks / 2 : static_cast<int64_t>(sh.heads) << (sh.band_shift - 1);
  if (n_rows * per_row >= (int64_t{1} << 32) || n_rows >= (int64_t{1} << 31))
    return fail(LL_EUNSUPPORTED, "too many rows for one call");
  if (n_rows == 0) return LL_OK;

  DeviceGuard g(p->desc.device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((rc = begin_call(p, st))) return rc;
  // MLA rows turned in place: one kernel that evaluates its own cos/sin; the
  // other cases read a per-row table made by rope_table_kernel
  const bool inplace_mla = !out_dev && !p->gqa;
  const size_t tab_floats = inplace_mla ? 0 : static_cast<size_t>(n_rows) * 2 * sh.pairs;
  if (tab_floats > p->rowtab_cap) {
    if ((rc = wait_idle(p))) return rc;
    if (p->d_rowtab) (void)hipFree(p->d_rowtab);
    p->d_rowtab = nullptr;
    p->rowtab_cap = 0;
    if (hipMalloc(reinterpret_cast<void**>(&p->d_rowtab), tab_floats * sizeof(float)) != hipSuccess)
      return fail(LL_ENOMEM, "cannot allocate %zu bytes of rotation tables", tab_floats * sizeof(float));
    p->rowtab_cap = tab_floats;
  }
  const int64_t P = p->P;
  const int64_t first_page = row_begin / P;
  const int64_t last_page = (row_begin + n_rows - 1) / P;
  const int64_t n_pages = last_page - first_page + 1;
  Staging* sg = nullptr;
  if ((rc = stage_acquire(p, stage_bytes_for({sizeof(double) * sh.pairs, sizeof(int32_t) * n_pages}), &sg))) return rc;
  const size_t o_th = stage_put(sg, nullptr, sizeof(double) * sh.pairs);
  const size_t o_pg = stage_put(sg, s.pages.data() + first_page, sizeof(int32_t) * n_pages);
  double* theta = reinterpret_cast<double*>(sg->host + o_th);
  const int rope_dim = 2 * sh.pairs;
  for (int j = 0; j < sh.pairs; ++j) theta[j] = std::pow(p->desc.rope_base, -2.0 * j / rope_dim);
  if ((rc = upload(p, sg, st))) return rc;

  ll::RopeTableLaunch t{};
  t.angle = angle_dev;
  t.theta = reinterpret_cast<const double*>(sg->dev + o_th);
  t.tab = p->d_rowtab;
  t.n = n_rows;
  t.pairs = sh.pairs;
  ll::RopeRowsLaunch a{};
  a.planes = reinterpret_cast<const ll::chunk_t* const*>(p->d_layers);
  a.plane0 = static_cast<const ll::chunk_t*>(p->layer_ptrs[0]);
  a.plane_stride = p->plane_stride_chunks;
  a.num_planes = static_cast<int32_t>(L);  // MLA layers, or the K planes of a GQA pool
  a.page_shift = p->page_shift;
  a.shape = sh;
  a.pages = reinterpret_cast<const int32_t*>(sg->dev + o_pg);
  a.row_begin = row_begin;
  a.first_page = first_page;
  a.n = n_rows;
  a.tab = p->d_rowtab;
  a.out = static_cast<ll::chunk_t*>(out_dev);
  a.out_plane_chunks = (out_layer_stride_bytes ? out_layer_stride_bytes : n_rows * p->row_bytes) / 16;
  a.n_pages = n_pages;
  a.blocks_per_plane = ll::rope_rows_blocks_per_plane(a, per_row);
  a.angle = angle_dev;
  ProfRec rec{};
  ll::Stamp ts;
  if (prof_pick(p, 2) && (rc = prof_begin(p, &rec, &ts))) return rc;
  hipError_t e;
  if (inplace_mla) {
    e = ll::launch_rope_inplace_mla(a, t.theta, p->desc.rope_pairing, st, ts);
    if (e != hipSuccess) return device_fail(p, e, "rope_inplace_mla_kernel launch");
  } else {
    e = ll::launch_rope_table(t, st, ll::Stamp{ts.start, nullptr});
    if (e != hipSuccess) return device_fail(p, e, "rope_table_kernel launch");
    // ranges of whole planes, each within one dispatch
    const int64_t per = std::max<int64_t>(1, p->dispatch_items / 256 / std::max<int64_t>(1, a.blocks_per_plane));
    ll::RopeRowsLaunch part = a;
    for (int64_t l0 = 0; l0 < a.num_planes; l0 += per) {
      const int64_t cnt = std::min<int64_t>(per, a.num_planes - l0);
      part.planes = a.planes + l0;
      part.plane0 = static_cast<const ll::chunk_t*>(p->layer_ptrs[static_cast<size_t>(l0)]);
      part.num_planes = static_cast<int32_t>(cnt);
      part.out = a.out + l0 * a.out_plane_chunks;
      e = ll::launch_rope_rows(part, p->desc.rope_pairing, st, ll::Stamp{nullptr, l0 + cnt == a.num_planes ? ts.stop : nullptr});
      if (e != hipSuccess) return device_fail(p, e, "rope_rows_kernel launch");
    }
  }
  ll_plan_stats stats{};
  stats.alg_bytes = out_dev ? L * n_rows * 2 * p->row_bytes : L * n_rows * 2 * p->band_bytes;
  stats.rows_rotated_inplace = out_dev ? 0 : n_rows;
  if (rec.start) {
    rec.bytes = stats.alg_bytes;
    prof_end(p, 2, rec);
  }
  if ((rc = end_call(p, sg, st))) return rc;
  p->last = stats;
  return LL_OK;
} catch (...) {
  return host_exception(p);
}

ll_status ll_last_plan_stats(const ll_pool* p, ll_plan_stats* out) {
  if (!p || !out) return fail(LL_EINVAL, "NULL argument");
  ll_status rc = settle(const_cast<ll_pool*>(p));
  if (rc) return rc;
  *out = p->last;
  return LL_OK;
}

ll_status ll_last_plan_bytes(const ll_pool* p, int64_t* alg_bytes, int64_t* rows_moved,
                             int64_t* rows_rotated_inplace) {
  ll_plan_stats s{};
  if (ll_status rc = ll_last_plan_stats(p, &s)) return rc;
  if (alg_bytes) *alg_bytes = s.alg_bytes;
  if (rows_moved) *rows_moved = s.rows_moved;
  if (rows_rotated_inplace) *rows_rotated_inplace = s.rows_rotated_inplace;
  return LL_OK;
}

ll_status ll_seq_lengths(const ll_pool* p, const int32_t* seq_ids, int32_t n, int64_t* lengths_out) try {
  if (!p) return fail(LL_EINVAL, "pool is NULL");
  if (n < 0 || (n > 0 && (!seq_ids || !lengths_out))) return fail(LL_EINVAL, "bad arguments");
  ll_status rc = settle(const_cast<ll_pool*>(p));
  if (rc) return rc;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = seq_ids[i];
    if (s < 0 || s >= p->desc.max_seqs || !p->seqs[s].used) return fail(LL_EINVAL, "entry %d: unknown sequence %d", i, s);
    lengths_out[i] = p->seqs[s].len;
  }
  return LL_OK;
} catch (...) {
  return host_exception(const_cast<ll_pool*>(p));
}

ll_status ll_pool_set_splice_planner(ll_pool* p, int32_t planner) {
  if (!p) return fail(LL_EINVAL, "pool is NULL");
  if (planner != LL_SPLICE_PLAN_AUTO && planner != LL_SPLICE_PLAN_HOST)
    return fail(LL_EINVAL, "unknown splice planner %d", planner);
  p->splice_planner = planner;
  return LL_OK;
}

ll_status ll_pool_set_page_reuse(ll_pool* p, int32_t on) {
  if (ll_status rc = enter(p)) return rc;
  if (on != 0 && on != 1) return fail(LL_EINVAL, "page reuse must be 0 or 1, not %d", on);
  if (!on && p->P == 1) return fail(LL_EUNSUPPORTED, "at page size 1 a page is one row: there is nothing to compact");
  p->page_reuse = on != 0;
  return LL_OK;
}

ll_status ll_pool_set_dispatch_limit(ll_pool* p, int64_t max_items) {
  if (ll_status rc = enter(p)) return rc;
  if (max_items < 0 || max_items > kMaxDispatchItems)
    return fail(LL_EINVAL, "the dispatch limit must lie in [0, 2^32 - 1], not %lld", (long long)max_items);
  if (max_items != 0 && max_items < 1024)
    return fail(LL_EINVAL, "the dispatch limit must be at least 1024 work-items, not %lld", (long long)max_items);
  p->dispatch_items = max_items == 0 ? kMaxDispatchItems : max_items;
  return LL_OK;
}

ll_status ll_pool_set_profiling(ll_pool* p, int32_t enable) {
  if (!p) return fail(LL_EINVAL, "pool is NULL");
  p->prof_every = enable > 0 ? enable : 0;
  for (int64_t& t : p->prof_tick) t = 0;
  return LL_OK;
}

ll_status ll_profile_read(ll_pool* p, int32_t kernel, int64_t* launches, double* total_ms, int64_t* total_bytes,
                          float* each_ms, int64_t each_cap) try {
  if (!p || kernel < 0 || kernel > 2 || each_cap < 0 || (each_cap > 0 && !each_ms)) return fail(LL_EINVAL, "bad argument");
  if (ll_status rc = settle(p)) return rc;
  DeviceGuard g(p->desc.device);
  int64_t cnt = 0, bytes = 0;
  double ms = 0.0;
  for (ProfRec& r : p->prof[kernel]) {
    hipError_t e = hipEventSynchronize(r.stop);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.start, r.stop);
    if (e != hipSuccess) return fail(LL_EDEVICE, "profile events: %s", hipGetErrorString(e));
    ms += t;
    bytes += r.bytes;
    if (cnt < each_cap) each_ms[cnt] = t;
    ++cnt;
    p->spare_events.push_back(r.start);
    p->spare_events.push_back(r.stop);
  }
  p->prof[kernel].clear();
  if (launches) *launches = cnt;
  if (total_ms) *total_ms = ms;
  if (total_bytes) *total_bytes = bytes;
  return LL_OK;
} catch (...) {
  return host_exception(p);
}

}  // extern "C"
