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
  int64_t rank_off;      // groups of 32 rows into the rank scratch
};

// Death times in two launches.  kvs_rank_kernel, one block per event: for
// each group g of 32 rows of the event's keep mask, rank[rank_off + g] =
// {kept rows before the group, the group's keep bits}, and kept[event] =
// rows kept.  kvs_chain_kernel, one
// thread per (rollout, token): the token's row at the first event after its
// birth is (rows kept by the event before) + (tokens generated since); at
// each event it either dies (d = the event's time) or moves to the row its
// rank gives in the next event's list, where the survivors come first.
struct KvsDeathLaunch {
  const KvsRollout* rollouts;
  const KvsEvent* events;
  const uint8_t* keep;
  int32_t* death;        // [n][n_pad]
  int32_t* status;       // [n]
  uint2* rank;           // scratch: per group of 32 event rows, as above
  int32_t* kept;         // scratch [n_events]
  int64_t n_pad;
  int64_t chain_blocks;  // blocks of kvs_chain_kernel per rollout: ceil(n_pad / 256)
  int32_t n;
  int32_t n_events;
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

// The dense mask of a rollout whose keys die at no more than kDenseMaxEvents
// distinct times is written by kvs_dense_ev_kernel from per-key death codes;
// other rollouts by the rebuild walk of kvs_dense_kernel, run by the same
// launch's waves of that rollout.  events: [n][kDenseEvStride] int32,
// entry 0 the number of distinct death times d with k < d < n_pad over the
// rollout's keys (kDenseMaxEvents + 1: more than that), entries 1.. those
// times in increasing order.  planes: per rollout five bit sets over its keys
// -- visible at some row (d_k > k), then bits 0..3 of the key's code, the
// index of d_k among those times (15: no death before n_pad).
constexpr int kDenseMaxEvents = 15;
constexpr int kDenseEvStride = 16;
constexpr int64_t kDenseEvMaxPad = 262144;  // the pre-pass keeps an n_pad-bit set in LDS

struct KvsDenseLaunch {
  const int32_t* death;  // [n][n_pad]
  uint32_t* bits;        // [n][n_pad][n_pad / 32]
  int64_t n_pad;
  int32_t n;
  int32_t rows_per_thread;
  int32_t* events;       // nullptr: kvs_dense_kernel alone, every rollout by the rebuild walk
  uint32_t* planes;      // [n][5][n_pad / 32]: per key, visible at some row, then code bits 0..3
};

hipError_t launch_kvs_death(const KvsDeathLaunch& a, hipStream_t s);
constexpr int kChainThreads = 256;
hipError_t launch_kvs_block(const KvsBlockLaunch& a, hipStream_t s);
hipError_t launch_kvs_dense(const KvsDenseLaunch& a, hipStream_t s);

}  // namespace ll
