// Internal types of the KV-streams trainer-mask kernels (kernels_kvs.hip) and
// their host side (kvs_mask.cpp).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ll {

// One rollout of a death-time call.
struct alignas(16) KvsRollout {
  int64_t n_tokens;
  int32_t first_event;   // index into the event array
  int32_t n_events;
};

// One eviction event of a rollout.
struct alignas(16) KvsEvent {
  int64_t time;          // tokens generated when the event ran
  int64_t mask_len;      // rows the keep mask covers
  int64_t mask_off;      // bytes into the keep buffer
  int64_t pad;
};

struct KvsDeathLaunch {
  const KvsRollout* rollouts;
  const KvsEvent* events;
  const uint8_t* keep;
  int32_t* death;        // [n][n_pad]
  int32_t* status;       // [n]
  int32_t* list;         // scratch [n][n_pad]: token ids the cache holds
  int64_t n_pad;
  int32_t n;
};

struct KvsBlockLaunch {
  const int32_t* death;  // [n][n_pad]
  int2* minmax;          // scratch [n][nk]: min and max death time per key block
  int32_t* partial_num;  // [n][nq]
  int32_t* partial_idx;  // [n][nq][nk]
  int32_t* full_num;
  int32_t* full_idx;
  int64_t n_pad;
  int32_t n;
  int32_t bq_shift, bk_shift;
  int32_t nq, nk;
};

struct KvsDenseLaunch {
  const int32_t* death;  // [n][n_pad]
  uint32_t* bits;        // [n][n_pad][n_pad / 32]
  int64_t n_pad;
  int32_t n;
  int32_t rows_per_thread;
};

hipError_t launch_kvs_death(const KvsDeathLaunch& a, hipStream_t s);
hipError_t launch_kvs_block(const KvsBlockLaunch& a, hipStream_t s);
hipError_t launch_kvs_dense(const KvsDenseLaunch& a, hipStream_t s);

}  // namespace ll
