// Host side of the KV-streams trainer-side attention mask (include/leyline.h,
// "KV-streams trainer mask" section): argument checks, the upload of the
// eviction logs, and the launches of kernels_kvs.hip.
//
// "KV-streams" ("how it works"): the trainer mirrors the engine's evictions
// with a custom attention mask so that one forward pass over a rollout lets
// every token see exactly the keys the cache held when it was generated.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "../../include/leyline.h"
#include "host_common.h"
#include "kvs_internal.h"

// One staging region of the event logs: pinned host memory, its device copy,
// and the event recorded after the replay kernel that reads it.
struct KvsStage {
  char* host = nullptr;
  char* dev = nullptr;
  size_t cap = 0;
  hipEvent_t done = nullptr;
  bool pending = false;
};

constexpr int kKvsStages = 4;

struct kvs_ctx {
  int32_t device = 0;
  KvsStage stage[kKvsStages];  // taken in turn; a call waits only if its region is still in flight
  int next_stage = 0;
  char* rank = nullptr;      // death-time scratch: rows kept per event, then the ranks of every mask row
  size_t rank_cap = 0;       // bytes
  hipEvent_t rank_done = nullptr;  // the last death-time call that used it has finished
  bool rank_pending = false;
  hipStream_t rank_stream = nullptr;
  int2* minmax = nullptr;    // block-mask scratch
  size_t minmax_cap = 0;     // elements
  hipEvent_t minmax_done = nullptr;
  bool minmax_pending = false;
  hipStream_t minmax_stream = nullptr;  // the stream of the call that recorded minmax_done
  char* events = nullptr;     // dense-mask scratch: distinct death times and key bit sets per rollout
  size_t events_cap = 0;      // bytes
  hipEvent_t events_done = nullptr;
  bool events_pending = false;
  hipStream_t events_stream = nullptr;  // the stream of the call that recorded events_done
};

namespace {

using ll::fail;

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

ll_status dev_fail(hipError_t e, const char* what) { return fail(LL_EDEVICE, "%s: %s", what, hipGetErrorString(e)); }

// No exception crosses the C ABI: an exported function that catches one (in
// practice std::bad_alloc) returns LL_ENOMEM.
ll_status host_exception(std::nullptr_t) noexcept { return fail(LL_ENOMEM, "host memory exhausted during the call"); }

int log2_exact(int32_t x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return (1 << s) == x ? s : -1;
}

}  // namespace

extern "C" {

ll_status kvs_ctx_create(int32_t device, kvs_ctx** out) try {
  if (!out) return fail(LL_EINVAL, "NULL argument");
  *out = nullptr;
  if (device < 0) return fail(LL_EINVAL, "device must be >= 0");
  DeviceGuard g(device);
  if (!g.ok()) return fail(LL_EDEVICE, "hipSetDevice(%d) failed", device);
  kvs_ctx* c = new kvs_ctx();
  c->device = device;
  hipError_t e = hipSuccess;
  for (int i = 0; i < kKvsStages && e == hipSuccess; ++i)
    e = hipEventCreateWithFlags(&c->stage[i].done, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->rank_done, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->minmax_done, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->events_done, hipEventDisableTiming);
  if (e != hipSuccess) {
    kvs_ctx_destroy(c);
    return dev_fail(e, "kvs_ctx_create");
  }
  *out = c;
  return LL_OK;
} catch (...) {
  return host_exception(nullptr);
}

void kvs_ctx_destroy(kvs_ctx* c) try {
  if (!c) return;
  DeviceGuard g(c->device);
  for (KvsStage& S : c->stage)
    if (S.pending) (void)hipEventSynchronize(S.done);
  if (c->rank_pending) (void)hipEventSynchronize(c->rank_done);
  if (c->minmax_pending) (void)hipEventSynchronize(c->minmax_done);
  if (c->events_pending) (void)hipEventSynchronize(c->events_done);
  for (KvsStage& S : c->stage) {
    if (S.done) (void)hipEventDestroy(S.done);
    if (S.host) (void)hipHostFree(S.host);
    if (S.dev) (void)hipFree(S.dev);
  }
  if (c->rank_done) (void)hipEventDestroy(c->rank_done);
  if (c->minmax_done) (void)hipEventDestroy(c->minmax_done);
  if (c->events_done) (void)hipEventDestroy(c->events_done);
  if (c->events) (void)hipFree(c->events);
  if (c->minmax) (void)hipFree(c->minmax);
  if (c->rank) (void)hipFree(c->rank);
  delete c;
} catch (...) {
  return;
}

ll_status kvs_death_times(kvs_ctx* c, const kvs_rollout_log* logs, int32_t n, int64_t n_pad, const uint8_t* keep_dev,
                          int32_t* death_dev, int32_t* status_dev, void* stream) try {
  if (!c) return fail(LL_EINVAL, "context is NULL");
  if (n < 0 || (n > 0 && (!logs || !death_dev || !status_dev))) return fail(LL_EINVAL, "bad arguments");
  if (n_pad < 1 || n_pad >= (int64_t{1} << 31) - 1) return fail(LL_EINVAL, "n_pad must be in [1, 2^31 - 2]");
  if (n == 0) return LL_OK;
  int64_t n_events = 0;
  bool any_mask = false;
  for (int32_t i = 0; i < n; ++i) {
    const kvs_rollout_log& l = logs[i];
    if (l.n_tokens < 0 || l.n_tokens > n_pad) return fail(LL_EINVAL, "rollout %d: n_tokens outside [0, n_pad]", i);
    if (l.n_events < 0 || (l.n_events > 0 && (!l.event_time || !l.mask_len)))
      return fail(LL_EINVAL, "rollout %d: bad event arrays", i);
    if (l.mask_offset < 0) return fail(LL_EINVAL, "rollout %d: negative mask_offset", i);
    int64_t prev = 0;
    for (int32_t e = 0; e < l.n_events; ++e) {
      const int64_t t = l.event_time[e];
      if (t <= prev || t > l.n_tokens)
        return fail(LL_EINVAL, "rollout %d, event %d: times must increase inside (0, n_tokens]", i, e);
      if (l.mask_len[e] < 0 || l.mask_len[e] > t)
        return fail(LL_EINVAL, "rollout %d, event %d: mask_len outside [0, time]", i, e);
      any_mask = any_mask || l.mask_len[e] > 0;
      prev = t;
    }
    n_events += l.n_events;
  }
  if (any_mask && !keep_dev) return fail(LL_EINVAL, "keep masks are NULL");
  if (n_events >= (int64_t{1} << 31)) return fail(LL_EUNSUPPORTED, "too many events");
  const int64_t chain_blocks = (n_pad + ll::kChainThreads - 1) / ll::kChainThreads;
  if (static_cast<int64_t>(n) * chain_blocks >= (int64_t{1} << 31))
    return fail(LL_EUNSUPPORTED, "n * ceil(n_pad / 256) must stay below 2^31");
  // the rank scratch: rows kept per event, then 8 bytes per group of 32 mask rows
  const size_t kept_bytes = (sizeof(int32_t) * static_cast<size_t>(n_events) + 255) / 256 * 256;
  size_t rank_groups = 0;
  for (int32_t i = 0; i < n; ++i)
    for (int32_t e = 0; e < logs[i].n_events; ++e) rank_groups += (static_cast<size_t>(logs[i].mask_len[e]) + 31) / 32;
  const size_t rank_need = kept_bytes + 8 * rank_groups;

  DeviceGuard g(c->device);
  if (!g.ok()) return fail(LL_EDEVICE, "hipSetDevice(%d) failed", c->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t roll_bytes = sizeof(ll::KvsRollout) * static_cast<size_t>(n);
  const size_t ev_off = (roll_bytes + 255) / 256 * 256;
  const size_t need = ev_off + sizeof(ll::KvsEvent) * static_cast<size_t>(std::max<int64_t>(n_events, 1));
  // The rank scratch: one call at a time may use it.  A call on another
  // stream waits on the device for the last one; growing it waits on the host.
  if (rank_need > c->rank_cap) {
    if (c->rank_pending) {
      hipError_t e = hipEventSynchronize(c->rank_done);
      if (e != hipSuccess) return dev_fail(e, "hipEventSynchronize(rank scratch)");
      c->rank_pending = false;
    }
    if (c->rank) (void)hipFree(c->rank);
    c->rank = nullptr;
    c->rank_cap = 0;
    const size_t cap = std::max<size_t>(rank_need + rank_need / 4, size_t{1} << 16);
    if (hipMalloc(reinterpret_cast<void**>(&c->rank), cap) != hipSuccess)
      return fail(LL_ENOMEM, "cannot allocate %zu bytes of death-time scratch", cap);
    c->rank_cap = cap;
  } else if (c->rank_pending && c->rank_stream != st) {
    hipError_t e = hipStreamWaitEvent(st, c->rank_done, 0);
    if (e != hipSuccess) return dev_fail(e, "hipStreamWaitEvent(rank scratch)");
  }
  // the staging region of this call: wait only while the call that used it
  // last (kKvsStages calls ago) has not finished
  KvsStage& S = c->stage[c->next_stage];
  if (S.pending) {
    hipError_t e = hipEventSynchronize(S.done);
    if (e != hipSuccess) return dev_fail(e, "hipEventSynchronize(staging)");
    S.pending = false;
  }
  if (need > S.cap) {
    if (S.host) (void)hipHostFree(S.host);
    if (S.dev) (void)hipFree(S.dev);
    S.host = nullptr;
    S.dev = nullptr;
    S.cap = 0;
    const size_t cap = std::max<size_t>(need * 2, size_t{1} << 16);
    if (hipHostMalloc(reinterpret_cast<void**>(&S.host), cap, hipHostMallocDefault) != hipSuccess ||
        hipMalloc(reinterpret_cast<void**>(&S.dev), cap) != hipSuccess)
      return fail(LL_ENOMEM, "cannot allocate %zu bytes of staging", cap);
    std::memset(S.host, 0, cap);  // fault the pinned pages in once
    S.cap = cap;
  }
  c->next_stage = (c->next_stage + 1) % kKvsStages;
  ll::KvsRollout* rolls = reinterpret_cast<ll::KvsRollout*>(S.host);
  ll::KvsEvent* evs = reinterpret_cast<ll::KvsEvent*>(S.host + ev_off);
  int64_t at = 0, rank_off = 0;
  for (int32_t i = 0; i < n; ++i) {
    const kvs_rollout_log& l = logs[i];
    rolls[i].n_tokens = l.n_tokens;
    rolls[i].first_event = static_cast<int32_t>(at);
    rolls[i].n_events = l.n_events;
    int64_t off = l.mask_offset;
    for (int32_t e = 0; e < l.n_events; ++e) {
      ll::KvsEvent& ev = evs[at++];
      ev.time = l.event_time[e];
      ev.mask_len = l.mask_len[e];
      ev.mask_off = off;
      ev.rank_off = rank_off;
      off += l.mask_len[e];
      rank_off += (l.mask_len[e] + 31) / 32;
    }
  }
  hipError_t e = hipMemcpyAsync(S.dev, S.host, need, hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return dev_fail(e, "hipMemcpyAsync(event log)");
  ll::KvsDeathLaunch a{};
  a.rollouts = reinterpret_cast<const ll::KvsRollout*>(S.dev);
  a.events = reinterpret_cast<const ll::KvsEvent*>(S.dev + ev_off);
  a.keep = keep_dev;
  a.death = death_dev;
  a.status = status_dev;
  a.kept = reinterpret_cast<int32_t*>(c->rank);
  a.rank = reinterpret_cast<uint2*>(c->rank + kept_bytes);
  a.n_pad = n_pad;
  a.chain_blocks = chain_blocks;
  a.n = n;
  a.n_events = static_cast<int32_t>(n_events);
  e = ll::launch_kvs_death(a, st);
  if (e != hipSuccess) return dev_fail(e, "kvs_rank_kernel / kvs_chain_kernel launch");
  e = hipEventRecord(S.done, st);
  if (e == hipSuccess) e = hipEventRecord(c->rank_done, st);
  if (e != hipSuccess) return dev_fail(e, "hipEventRecord");
  S.pending = true;
  c->rank_pending = true;
  c->rank_stream = st;
  return LL_OK;
} catch (...) {
  return host_exception(nullptr);
}

ll_status kvs_block_mask(kvs_ctx* c, const int32_t* death_dev, int32_t n, int64_t n_pad, int32_t block_q,
                         int32_t block_k, int32_t* partial_num, int32_t* partial_idx, int32_t* full_num,
                         int32_t* full_idx, void* stream) try {
  if (!c) return fail(LL_EINVAL, "context is NULL");
  if (n < 0 || (n > 0 && (!death_dev || !partial_num || !partial_idx || !full_num || !full_idx)))
    return fail(LL_EINVAL, "bad arguments");
  if (n_pad < 1 || n_pad >= (int64_t{1} << 31) - 1) return fail(LL_EINVAL, "n_pad must be in [1, 2^31 - 2]");
  const int bq = log2_exact(block_q), bk = log2_exact(block_k);
  if (bq < 4 || bq > 10 || bk < 4 || bk > 10)
    return fail(LL_EINVAL, "block_q and block_k must be powers of two in [16, 1024]");
  if (n == 0) return LL_OK;
  const int64_t nq = (n_pad + block_q - 1) / block_q;
  const int64_t nk = (n_pad + block_k - 1) / block_k;
  const size_t mm = static_cast<size_t>(n) * static_cast<size_t>(nk);
  DeviceGuard g(c->device);
  if (!g.ok()) return fail(LL_EDEVICE, "hipSetDevice(%d) failed", c->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (mm > c->minmax_cap) {
    if (c->minmax_pending) {
      hipError_t e = hipEventSynchronize(c->minmax_done);
      if (e != hipSuccess) return dev_fail(e, "hipEventSynchronize(scratch)");
      c->minmax_pending = false;
    }
    if (c->minmax) (void)hipFree(c->minmax);
    c->minmax = nullptr;
    c->minmax_cap = 0;
    if (hipMalloc(reinterpret_cast<void**>(&c->minmax), mm * 2 * sizeof(int2)) != hipSuccess)
      return fail(LL_ENOMEM, "cannot allocate block-mask scratch");
    c->minmax_cap = mm * 2;
  } else if (c->minmax_pending && st != c->minmax_stream) {  // same stream: already in order
    // the scratch is reused: order this call after the last one that used it
    hipError_t e = hipStreamWaitEvent(st, c->minmax_done, 0);
    if (e != hipSuccess) return dev_fail(e, "hipStreamWaitEvent(scratch)");
  }
  ll::KvsBlockLaunch a{};
  a.death = death_dev;
  a.minmax = c->minmax;
  a.partial_num = partial_num;
  a.partial_idx = partial_idx;
  a.full_num = full_num;
  a.full_idx = full_idx;
  a.n_pad = n_pad;
  a.n = n;
  a.bq_shift = bq;
  a.bk_shift = bk;
  a.nq = static_cast<int32_t>(nq);
  a.nk = static_cast<int32_t>(nk);
  hipError_t e = ll::launch_kvs_block(a, st);
  if (e != hipSuccess) return dev_fail(e, "kvs_block_kernel launch");
  e = hipEventRecord(c->minmax_done, st);
  if (e != hipSuccess) return dev_fail(e, "hipEventRecord");
  c->minmax_pending = true;
  c->minmax_stream = st;
  return LL_OK;
} catch (...) {
  return host_exception(nullptr);
}

ll_status kvs_dense_mask(kvs_ctx* c, const int32_t* death_dev, int32_t n, int64_t n_pad, uint32_t* bits_dev,
                         void* stream) try {
  if (!c) return fail(LL_EINVAL, "context is NULL");
  if (n < 0 || (n > 0 && (!death_dev || !bits_dev))) return fail(LL_EINVAL, "bad arguments");
  if (n_pad < 128 || n_pad % 128 || n_pad >= (int64_t{1} << 31) - 1)
    return fail(LL_EINVAL, "n_pad must be a positive multiple of 128 below 2^31");
  if (reinterpret_cast<uintptr_t>(bits_dev) & 15) return fail(LL_EINVAL, "bits_dev is not 16-byte aligned");
  if (n == 0) return LL_OK;
  DeviceGuard g(c->device);
  if (!g.ok()) return fail(LL_EDEVICE, "hipSetDevice(%d) failed", c->device);
  ll::KvsDenseLaunch a{};
  a.death = death_dev;
  a.bits = bits_dev;
  a.n_pad = n_pad;
  a.n = n;
  a.rows_per_thread = 128;
  const int64_t runs = (n_pad + a.rows_per_thread - 1) / a.rows_per_thread;
  const int64_t groups = (n_pad / 128 + 63) / 64;  // waves per run of rows
  // blocks of the rebuild-walk launch, and of the run-of-rows launch (four
  // runs of 8 rows per block) when the pre-pass applies
  if (static_cast<int64_t>(n) * runs * groups / 4 >= (int64_t{1} << 31) ||
      (n_pad <= ll::kDenseEvMaxPad && static_cast<int64_t>(n) * (n_pad / 32) >= (int64_t{1} << 31)))
    return fail(LL_EUNSUPPORTED, "dense mask too large for one launch");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool by_events = n_pad <= ll::kDenseEvMaxPad;
  if (by_events) {
    // per rollout its distinct death times (kvs_events_kernel), read by the
    // two mask kernels; the scratch is reused call after call
    // [n][kDenseEvStride] int32, then [n][5][n_pad / 32] uint32
    const size_t ev_bytes = (static_cast<size_t>(n) * ll::kDenseEvStride * sizeof(int32_t) + 255) / 256 * 256;
    const size_t need = ev_bytes + static_cast<size_t>(n) * 5 * static_cast<size_t>(n_pad / 8);
    if (need > c->events_cap) {
      if (c->events_pending) {
        hipError_t e = hipEventSynchronize(c->events_done);
        if (e != hipSuccess) return dev_fail(e, "hipEventSynchronize(scratch)");
        c->events_pending = false;
      }
      if (c->events) (void)hipFree(c->events);
      c->events = nullptr;
      c->events_cap = 0;
      if (hipMalloc(reinterpret_cast<void**>(&c->events), need) != hipSuccess)
        return fail(LL_ENOMEM, "cannot allocate dense-mask scratch");
      c->events_cap = need;
    } else if (c->events_pending && st != c->events_stream) {  // same stream: already in order
      hipError_t e = hipStreamWaitEvent(st, c->events_done, 0);
      if (e != hipSuccess) return dev_fail(e, "hipStreamWaitEvent(scratch)");
    }
    a.events = reinterpret_cast<int32_t*>(c->events);
    a.planes = reinterpret_cast<uint32_t*>(c->events + ev_bytes);
  }
  hipError_t e = ll::launch_kvs_dense(a, st);
  if (e != hipSuccess) return dev_fail(e, "kvs_dense_kernel launch");
  if (by_events) {
    e = hipEventRecord(c->events_done, st);
    if (e != hipSuccess) return dev_fail(e, "hipEventRecord");
    c->events_pending = true;
    c->events_stream = st;
  }
  return LL_OK;
} catch (...) {
  return host_exception(nullptr);
}

}  // extern "C"
