// gfx950 kernels of the KV-streams trainer-side attention mask ("KV-streams",
// "how it works": the trainer reproduces the engine's evictions with a custom
// attention mask, so one forward pass over a rollout lets each token see the
// keys the cache held when that token was generated).
//
// Token k's death time d_k is the time of the eviction event that dropped it
// (n_pad if none, k for padding keys); query q sees key k iff k <= q < d_k.
//
//  * kvs_rank_kernel / kvs_chain_kernel: the eviction log replayed in
//    parallel.  One block per event ranks its keep mask (kept rows before
//    each group of 32 rows, by a block prefix scan, with the group's keep
//    bits); then one thread per token follows the
//    token's row from event to event -- the held rows of an event are the
//    survivors of the one before, in order, followed by the tokens generated
//    since -- until an event drops it (its death time) or the log ends.
//  * kvs_minmax_kernel / kvs_block_kernel: per key block the smallest and
//    largest death time, then per query block the sorted lists of partial and
//    full key blocks (FlexAttention-style block mask).
//  * kvs_events_kernel / kvs_dense_ev_kernel: the packed bit mask of rollouts
//    whose keys die at few distinct times: the distinct death times and per
//    key a 4-bit code (which of them), once per rollout; then one wave per
//    run of 8 whole rows, its bits built at the run's first row from the
//    codes and carried down the run -- added on the diagonal, cleared at each
//    death time, no vector loads in the row loop -- so the grid writes the
//    mask in address order.  The waves of a rollout with more death times
//    take the rebuild walk below instead, in the same launch.
//  * kvs_dense_kernel (rebuild walk; every rollout when n_pad is too large
//    for the pre-pass): one 16-byte store per lane and row; a wave carries
//    its 64 x 128 keys' bits down a run of rows, adds keys as the rows reach
//    them and rebuilds the bits (coalesced loads, ballots) only at rows where
//    one of its keys dies.
#include <algorithm>

#include "device_common.h"
#include "kvs_internal.h"

namespace ll {
namespace {

using word4 = chunk_t;


// Bit b of the result: byte b of the 16 is nonzero.
__device__ __forceinline__ uint32_t nonzero_bytes16(word4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t out = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if ((w[q] >> (8 * c)) & 0xFFu) out |= 1u << (4 * q + c);
  return out;
}

// One block per event.  Each thread takes a group of 32 mask rows per tile:
// the 16-byte-aligned lines that hold them (three at most, each holding at
// least one of the mask's bytes, so never a page the mask does not touch),
// their nonzero bytes as bits, shifted to the group's first row.  The counts
// (0..32) are scanned across the wave with one ballot per bit of the count,
// then across the waves through LDS.  Group g of the event gets {kept rows
// before it, its 32 keep bits}: a row's rank is the first plus the kept rows
// below it in the second.
constexpr int kRankThreads = 512;
constexpr int kRankWaves = kRankThreads / 64;

__global__ __launch_bounds__(kRankThreads) void kvs_rank_kernel(KvsDeathLaunch a) {
  __shared__ int32_t wave_total[kRankWaves];
  const KvsEvent ev = a.events[blockIdx.x];
  const uint8_t* m = a.keep + ev.mask_off;
  uint2* out = a.rank + ev.rank_off;
  const int64_t len = ev.mask_len;
  const uintptr_t end = reinterpret_cast<uintptr_t>(m) + static_cast<uintptr_t>(len);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint64_t lanes_below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int64_t carry = 0;
  for (int64_t base = 0; base < len; base += 32 * kRankThreads) {
    const int64_t i0 = base + 32 * static_cast<int64_t>(threadIdx.x);
    uint32_t bits = 0;
    if (i0 < len) {
      const uintptr_t start = reinterpret_cast<uintptr_t>(m + i0);
      const uintptr_t a0 = start & ~uintptr_t{15};
      const int sk = static_cast<int>(start & 15u);
      uint64_t nz = nonzero_bytes16(*reinterpret_cast<const word4*>(a0));
      if (a0 + 16 < end) nz |= static_cast<uint64_t>(nonzero_bytes16(*reinterpret_cast<const word4*>(a0 + 16))) << 16;
      if (sk && a0 + 32 < end) nz |= static_cast<uint64_t>(nonzero_bytes16(*reinterpret_cast<const word4*>(a0 + 32))) << 32;
      bits = static_cast<uint32_t>(nz >> sk);
      if (len - i0 < 32) bits &= (1u << (len - i0)) - 1u;
    }
    const int cnt = __popc(bits);
    int below = 0, total = 0;
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {
      const uint64_t bal = __ballot((cnt >> bit) & 1);
      below += __popcll(bal & lanes_below) << bit;
      total += __popcll(bal) << bit;
    }
    if (lane == 0) wave_total[wave] = total;
    __syncthreads();
    int wave_below = 0, block_total = 0;
#pragma unroll
    for (int w = 0; w < kRankWaves; ++w) {
      const int x = wave_total[w];
      wave_below += w < wave ? x : 0;
      block_total += x;
    }
    if (i0 < len) out[i0 >> 5] = make_uint2(static_cast<uint32_t>(carry + wave_below + below), bits);
    carry += block_total;
    __syncthreads();
  }
  if (threadIdx.x == 0) a.kept[blockIdx.x] = static_cast<int32_t>(carry);
}

constexpr int kChainLdsEvents = 128;

// A rollout's events, from LDS (LDS = true: staged by the block) or from the
// event array.
template <bool LDS>
struct ChainEvents {
  const KvsEvent* ev;
  const int32_t* kept;
  const int64_t* s_time;
  const int64_t* s_len;
  const int64_t* s_roff;
  const int32_t* s_kept;
  __device__ int64_t time(int e) const { return LDS ? s_time[e] : ev[e].time; }
  __device__ int64_t len(int e) const { return LDS ? s_len[e] : ev[e].mask_len; }
  __device__ int64_t roff(int e) const { return LDS ? s_roff[e] : ev[e].rank_off; }
  __device__ int64_t held_after(int e) const { return LDS ? s_kept[e] : kept[e]; }
};

template <bool LDS>
__device__ int32_t chain_death(const KvsDeathLaunch& a, const ChainEvents<LDS>& E, int n_events, int64_t k) {
  int lo = 0, hi = n_events;  // the first event with time > k
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (E.time(mid) > k)
      hi = mid;
    else
      lo = mid + 1;
  }
  if (lo >= n_events) return static_cast<int32_t>(a.n_pad);
  int64_t row = (lo ? E.held_after(lo - 1) : 0) + (k - (lo ? E.time(lo - 1) : 0));
  for (int e = lo; e < n_events; ++e) {
    if (row >= E.len(e)) break;
    const uint2 g = a.rank[E.roff(e) + (row >> 5)];
    const uint32_t below = g.y & ((1u << (row & 31)) - 1u);
    if (!((g.y >> (row & 31)) & 1u)) return static_cast<int32_t>(E.time(e));
    row = g.x + __popc(below);
  }
  return static_cast<int32_t>(a.n_pad);
}

__global__ __launch_bounds__(kChainThreads) void kvs_chain_kernel(KvsDeathLaunch a) {
  __shared__ int64_t s_time[kChainLdsEvents], s_len[kChainLdsEvents], s_roff[kChainLdsEvents];
  __shared__ int32_t s_kept[kChainLdsEvents];
  const int64_t r = blockIdx.x / a.chain_blocks;
  const int64_t kb = blockIdx.x - r * a.chain_blocks;
  const KvsRollout ro = a.rollouts[r];
  const KvsEvent* ev = a.events + ro.first_event;
  const int32_t* kept = a.kept + ro.first_event;
  // up to kChainLdsEvents events staged in LDS: the walk's event reads then
  // wait on LDS, not memory
  const bool staged = ro.n_events <= kChainLdsEvents;
  if (staged)
    for (int e = threadIdx.x; e < ro.n_events; e += kChainThreads) {
      const KvsEvent x = ev[e];
      s_time[e] = x.time;
      s_len[e] = x.mask_len;
      s_roff[e] = x.rank_off;
      s_kept[e] = kept[e];
    }
  __syncthreads();
  if (kb == 0) {  // the rollout's status: its threads check the events in turn
    bool bad = false;
    for (int e = threadIdx.x; e < ro.n_events; e += kChainThreads) {
      const int64_t held = e ? kept[e - 1] : 0;
      const int64_t t_prev = e ? ev[e - 1].time : 0;
      bad = bad || held + (ev[e].time - t_prev) != ev[e].mask_len;
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) a.status[r] = bad ? 1 : 0;
  }
  const int64_t k = kb * kChainThreads + threadIdx.x;
  if (k >= a.n_pad) return;
  int32_t d;
  if (k >= ro.n_tokens)
    d = static_cast<int32_t>(k);
  else if (staged)
    d = chain_death<true>(a, ChainEvents<true>{ev, kept, s_time, s_len, s_roff, s_kept}, ro.n_events, k);
  else
    d = chain_death<false>(a, ChainEvents<false>{ev, kept, nullptr, nullptr, nullptr, nullptr}, ro.n_events, k);
  a.death[r * a.n_pad + k] = d;
}

// Smallest and largest death time of each key block: one wave per block.
__global__ __launch_bounds__(256) void kvs_minmax_kernel(KvsBlockLaunch a) {
  const int64_t gw = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (gw >= static_cast<int64_t>(a.n) * a.nk) return;
  const int64_t roll = gw / a.nk;
  const int64_t j = gw - roll * a.nk;
  const int32_t* d = a.death + roll * a.n_pad;
  const int64_t k0 = j << a.bk_shift;
  const int64_t k1 = min(k0 + (int64_t{1} << a.bk_shift), a.n_pad);
  int32_t mn = INT32_MAX, mx = INT32_MIN;
  for (int64_t k = k0 + lane; k < k1; k += 64) {
    const int32_t x = d[k];
    mn = min(mn, x);
    mx = max(mx, x);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = min(mn, __shfl_xor(mn, o));
    mx = max(mx, __shfl_xor(mx, o));
  }
  if (lane == 0) a.minmax[gw] = make_int2(mn, mx);
}

// One wave per query block [q0, q1).  Key block j = [k0, k1) is
//   empty   if k0 > q1 - 1 (above the diagonal);
//   below the diagonal (k1 - 1 <= q0): full iff min d >= q1, empty iff
//           max d <= q0, else partial;
//   across the diagonal: never full; partial iff some key k < q1 of the
//           block has max(k, q0) < min(d_k, q1) (an exact scan of its keys).
// Lanes classify 64 key blocks at a time; ballots give each listed block its
// slot, so both lists come out in increasing order.
__global__ __launch_bounds__(256) void kvs_block_kernel(KvsBlockLaunch a) {
  const int64_t gw = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (gw >= static_cast<int64_t>(a.n) * a.nq) return;
  const int64_t roll = gw / a.nq;
  const int64_t i = gw - roll * a.nq;
  const int32_t* d = a.death + roll * a.n_pad;
  const int2* mm = a.minmax + roll * a.nk;
  const int64_t q0 = i << a.bq_shift;
  const int64_t q1 = min(q0 + (int64_t{1} << a.bq_shift), a.n_pad);
  const int64_t bk = int64_t{1} << a.bk_shift;
  const int32_t last = static_cast<int32_t>(min<int64_t>(a.nk, ((q1 - 1) >> a.bk_shift) + 1));
  int32_t* p_idx = a.partial_idx + gw * a.nk;
  int32_t* f_idx = a.full_idx + gw * a.nk;
  const uint64_t lanes_below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int32_t np_ = 0, nf = 0;
  for (int32_t j0 = 0; j0 < last; j0 += 64) {
    const int32_t j = j0 + lane;
    bool part = false, full = false;
    if (j < last) {
      const int64_t k0 = int64_t{j} * bk;
      const int64_t k1 = min(k0 + bk, a.n_pad);
      if (k1 - 1 <= q0) {
        const int2 x = mm[j];
        full = x.x >= q1;
        part = !full && x.y > q0;
      } else {
        const int64_t kend = min(k1, q1);
        for (int64_t k = k0; k < kend && !part; ++k) {
          const int64_t lo = k > q0 ? k : q0;
          const int64_t hi = min<int64_t>(d[k], q1);
          part = lo < hi;
        }
      }
    }
    const uint64_t bp = __ballot(part);
    const uint64_t bf = __ballot(full);
    if (part) p_idx[np_ + __popcll(bp & lanes_below)] = j;
    if (full) f_idx[nf + __popcll(bf & lanes_below)] = j;
    np_ += __popcll(bp);
    nf += __popcll(bf);
  }
  if (lane == 0) {
    a.partial_num[gw] = np_;
    a.full_num[gw] = nf;
  }
}

// The wave's 64 strips of 128 keys are the 8192 consecutive keys
// [wk0, wk0 + 8192).  Recompute every lane's 128 bits for row q, reading the
// death times with coalesced loads (lane = key) and packing them with ballots:
// iteration it covers keys wk0 + 64 it .. + 63, i.e. words 2 (it & 1) and
// 2 (it & 1) + 1 of the strip it / 2, staged through the wave's 1 KiB of LDS.
// Also returns the wave's next death row (the least d_k > q over its keys
// that are visible at some row, d_k > k; INT32_MAX if none) and, in *real,
// the lane's keys that are visible at some row, so that keys reached by the
// diagonal later can be added without another load.
__device__ __forceinline__ word4 wave_bits(const int32_t* d, int64_t n_pad, int64_t wk0, int64_t q,
                                           uint64_t* lds, int lane, int32_t* next, word4* real) {
  int32_t nd = INT32_MAX;
  for (int it = 0; it < 128; ++it) {
    const int64_t k = wk0 + 64 * it + lane;
    bool vis = false, ever = false;
    if (k < n_pad) {
      const int32_t x = d[k];
      vis = k <= q && q < x;
      ever = x > k;
      if (x > q && ever) nd = min(nd, x);
    }
    const uint64_t bv = __ballot(vis);
    const uint64_t be = __ballot(ever);
    if (lane == 0) {
      lds[it] = bv;
      lds[128 + it] = be;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) nd = min(nd, __shfl_xor(nd, o));
  *next = nd;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint64_t lo = lds[2 * lane], hi = lds[2 * lane + 1];
  const uint64_t elo = lds[128 + 2 * lane], ehi = lds[128 + 2 * lane + 1];
  __builtin_amdgcn_wave_barrier();  // the next recompute overwrites lds only after every lane has read it
  *real = word4{static_cast<uint32_t>(elo), static_cast<uint32_t>(elo >> 32), static_cast<uint32_t>(ehi),
                static_cast<uint32_t>(ehi >> 32)};
  return word4{static_cast<uint32_t>(lo), static_cast<uint32_t>(lo >> 32), static_cast<uint32_t>(hi),
               static_cast<uint32_t>(hi >> 32)};
}

// One wave per (rollout, run of rows, 64 consecutive strips of 128 keys);
// lane s writes strip s, so each row is written as 1 KiB runs of 16-byte
// stores.  The wave computes its bits at its first row and carries them down
// the run: on its diagonal, key q appears at row q (if d_q > q); at a row
// where one of its keys dies (death times take at most one value per eviction
// event) it recomputes them with wave_bits.  The row loop itself loads
// nothing, so its stores never wait behind a load.
// One wave of the rebuild walk: wave gw of the grid, its LDS stage of 256
// words.  Only wave-level steps (ballots, the wave's own LDS), so waves of one
// block may take different rollouts and either walk.
__device__ __forceinline__ void dense_rebuild_wave(const KvsDenseLaunch& a, int64_t gw, int lane, uint64_t* lds) {
  const int64_t strips = a.n_pad >> 7;
  const int64_t groups = (strips + 63) >> 6;
  const int64_t runs = (a.n_pad + a.rows_per_thread - 1) / a.rows_per_thread;
  const int64_t grp = gw % groups;
  const int64_t rest = gw / groups;
  const int64_t run = rest % runs;
  const int64_t roll = rest / runs;
  const int32_t* d = a.death + roll * a.n_pad;
  const int64_t s = grp * 64 + lane;
  const bool active = s < strips;
  const int64_t words = a.n_pad >> 5;
  word4* out = reinterpret_cast<word4*>(a.bits + roll * a.n_pad * words) + s;
  const int64_t pitch = words >> 2;  // word4 per row
  const int64_t wk0 = grp << 13;     // first key of the wave
  const int64_t k0 = s << 7;         // first key of the lane's strip
  const int64_t q_begin = run * a.rows_per_thread;
  const int64_t q_end = min(q_begin + a.rows_per_thread, a.n_pad);
  if (q_end - 1 < wk0) {  // the whole run lies above the wave's diagonal
    if (active)
      for (int64_t q = q_begin; q < q_end; ++q)
        __builtin_nontemporal_store(word4{0u, 0u, 0u, 0u}, out + q * pitch);
    return;
  }
  int32_t death;
  word4 real;
  word4 w = wave_bits(d, a.n_pad, wk0, q_begin, lds, lane, &death, &real);
  if (active) __builtin_nontemporal_store(w, out + q_begin * pitch);
  for (int64_t q = q_begin + 1; q < q_end; ++q) {
    if (q == death) {  // wave-uniform
      w = wave_bits(d, a.n_pad, wk0, q, lds, lane, &death, &real);
    } else if (q >= k0 && q < k0 + 128) {  // key q appears (if it is ever visible): no load needed
      const int b = static_cast<int>(q - k0);
      w[b >> 5] |= real[b >> 5] & (1u << (b & 31));
    }
    if (active) __builtin_nontemporal_store(w, out + q * pitch);
  }
}

__global__ __launch_bounds__(256) void kvs_dense_kernel(KvsDenseLaunch a) {
  __shared__ uint64_t stage[4][256];
  const int64_t strips = a.n_pad >> 7;
  const int64_t groups = (strips + 63) >> 6;
  const int64_t runs = (a.n_pad + a.rows_per_thread - 1) / a.rows_per_thread;
  const int64_t gw = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 6;
  if (gw >= static_cast<int64_t>(a.n) * runs * groups) return;
  dense_rebuild_wave(a, gw, threadIdx.x & 63, stage[threadIdx.x >> 6]);
}

// gridDim.y 1024-thread blocks per rollout, each of which builds the set of
// death times d with k < d < n_pad (the times at which a key that was visible
// dies) as an n_pad-bit set in LDS -- the whole rollout's, so that every block
// knows the times -- then its first kDenseMaxEvents members in increasing
// order and its size (capped at kDenseMaxEvents + 1; block 0 stores them);
// when it has at most kDenseMaxEvents members, the keys of every gridDim.y-th
// 1024 get their bits in the five bit sets (visible at some row, code bits
// 0..3), one ballot per set and 64 keys.
__global__ __launch_bounds__(1024) void kvs_events_kernel(KvsDenseLaunch a) {
  extern __shared__ uint32_t set[];
  __shared__ int32_t part[1024];
  __shared__ int32_t times[kDenseMaxEvents];
  const int64_t n_pad = a.n_pad;
  const int32_t* d = a.death + static_cast<int64_t>(blockIdx.x) * n_pad;
  const int64_t words = n_pad >> 5;
  for (int64_t w = threadIdx.x; w < words; w += 1024) set[w] = 0u;
  __syncthreads();
  // eight loads in flight per thread, then their set bits; n_pad is a
  // multiple of 128, so a key's validity is uniform over its wave
  for (int64_t base = 0; base < n_pad; base += 8 * 1024) {
    int32_t x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t k = base + j * 1024 + threadIdx.x;
      x[j] = k < n_pad ? d[k] : 0;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t k = base + j * 1024 + threadIdx.x;
      if (k >= n_pad) break;
      // neighbouring keys mostly die together: one LDS atomic per run of
      // equal times in the wave rather than one per lane on the same word
      const int32_t left = __shfl_up(x[j], 1);
      if (x[j] > k && x[j] < n_pad && ((threadIdx.x & 63) == 0 || left != x[j]))
        atomicOr(&set[x[j] >> 5], 1u << (x[j] & 31));
    }
  }
  __syncthreads();
  // thread t owns words [t * per, (t + 1) * per): its count, then an
  // exclusive scan of the counts in LDS gives each member its rank
  const int64_t per = (words + 1023) / 1024;
  const int64_t w0 = threadIdx.x * per;
  const int64_t w1 = w0 + per < words ? w0 + per : words;
  int32_t cnt = 0;
  for (int64_t w = w0; w < w1; ++w) cnt += __popc(set[w]);
  part[threadIdx.x] = cnt;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive scan, Hillis-Steele
    const int32_t v = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int32_t* ev = a.events + static_cast<int64_t>(blockIdx.x) * kDenseEvStride;
  int32_t rank = part[threadIdx.x] - cnt;
  for (int64_t w = w0; w < w1 && rank < kDenseMaxEvents; ++w) {
    uint32_t bitsw = set[w];
    while (bitsw && rank < kDenseMaxEvents) {
      const int b = __builtin_ctz(bitsw);
      bitsw &= bitsw - 1u;
      const int32_t t = static_cast<int32_t>((w << 5) + b);
      times[rank] = t;
      if (blockIdx.y == 0) ev[1 + rank] = t;
      ++rank;
    }
  }
  if (threadIdx.x == 1023 && blockIdx.y == 0) ev[0] = part[1023] > kDenseMaxEvents ? kDenseMaxEvents + 1 : part[1023];
  const int32_t total = part[1023];
  if (total > kDenseMaxEvents) return;  // the rollout takes the rebuild walk
  // every member is in `times`; give each of the block's keys its visible
  // bit and code bits, 64 keys per wave and ballot
  __syncthreads();
  int32_t evs[kDenseMaxEvents];
#pragma unroll
  for (int e = 0; e < kDenseMaxEvents; ++e) evs[e] = e < total ? times[e] : INT32_MAX;
  uint32_t* pl = a.planes + static_cast<int64_t>(blockIdx.x) * 5 * words;
  const int lane = threadIdx.x & 63;
  for (int64_t base = (static_cast<int64_t>(blockIdx.y) * 16 + (threadIdx.x >> 6)) * 64; base < n_pad;
       base += int64_t{1024} * gridDim.y) {
    const int64_t k = base + lane;  // n_pad is a multiple of 128: no tail
    const int32_t x = d[k];
    const bool ever = x > k;
    int code = 15;
    if (ever && x < n_pad) {
      code = 0;
#pragma unroll
      for (int e = 0; e < kDenseMaxEvents; ++e) code += evs[e] < x ? 1 : 0;
    }
    const uint64_t m[5] = {__ballot(ever), __ballot(code & 1), __ballot(code & 2), __ballot(code & 4),
                           __ballot(code & 8)};
    if (lane < 10) {  // lane 2p + h writes word h of plane p
      const int p = lane >> 1, h = lane & 1;
      pl[p * words + (base >> 5) + h] = static_cast<uint32_t>(m[p] >> (32 * h));
    }
  }
}

// Bits [lo, hi] (strip-relative, may reach outside 0..127) of 32-bit word
// `word` (bits 32 word .. 32 word + 31) of a 128-bit strip.
__device__ __forceinline__ uint32_t range_word(int32_t lo, int32_t hi, int word) {
  const int32_t a = lo - 32 * word > 0 ? lo - 32 * word : 0;
  const int32_t b = hi - 32 * word < 31 ? hi - 32 * word : 31;
  if (a > b) return 0u;
  return (0xFFFFFFFFu >> (31 - b)) & (0xFFFFFFFFu << a);
}

// Rows per wave of kvs_dense_ev_kernel, and the groups of 64 strips whose
// bits a lane holds at once.
constexpr int kDenseRun = 8;
constexpr int kDenseHold = 4;

// One wave per (rollout, run of kDenseRun consecutive rows): the wave writes
// whole rows, so a block's four waves fill 4 * kDenseRun consecutive rows and
// the grid's write front moves through the mask in address order.  Lane l
// holds strips l, l + 64, ... (128 keys each) of up to kDenseHold groups of 64
// strips.  From the five bit sets of kvs_events_kernel (visible at some row;
// the 4-bit code, the index of d_k among the rollout's distinct death times)
// it builds a strip's bits at the run's first row q0 -- visible, k <= q0, and
// not dead: code >= the number of death times <= q0, a bit-serial compare of
// the code planes -- then walks the run's rows adding key q on the diagonal
// and clearing, at each death time passed, the keys with that code.  The row
// loop loads nothing but scalar event times, so its stores never wait behind
// a vector load.  A rollout with more than kDenseMaxEvents death times is
// written by the rebuild walk, dealt over the same rollout's waves.
__global__ __launch_bounds__(256) void kvs_dense_ev_kernel(KvsDenseLaunch a) {
  __shared__ uint64_t stage[4][256];  // the rebuild walk's
  const int lane = threadIdx.x & 63;
  const int64_t strips = a.n_pad >> 7;
  const int64_t groups = (strips + 63) >> 6;
  const int64_t runs = a.n_pad / kDenseRun;  // waves per rollout
  // the wave index, made visibly wave-uniform: the rollout, rows and the
  // death-time list then live in scalar registers and scalar loads
  const uint64_t gw_any = (static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x) >> 6;
  const int64_t gw = static_cast<int64_t>(
      (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(gw_any >> 32))) << 32) |
      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(gw_any)));
  if (gw >= static_cast<int64_t>(a.n) * runs) return;
  const int64_t run = gw % runs;
  const int32_t roll = static_cast<int32_t>(gw / runs);
  using cptr = const __attribute__((address_space(4))) int32_t*;
  const cptr ev = reinterpret_cast<cptr>(reinterpret_cast<uintptr_t>(a.events + int64_t{roll} * kDenseEvStride));
  const int32_t n_ev = ev[0];
  if (n_ev > kDenseMaxEvents) {  // too many death times for the codes: the rebuild walk
    const int64_t rb_waves = (a.n_pad + a.rows_per_thread - 1) / a.rows_per_thread * groups;
    for (int64_t j = run; j < rb_waves; j += runs)
      dense_rebuild_wave(a, int64_t{roll} * rb_waves + j, lane, stage[threadIdx.x >> 6]);
    return;
  }
  const int64_t words = a.n_pad >> 5;
  const int64_t row_bytes = a.n_pad >> 3;
  // rows and keys are below n_pad < 2^31
  const int32_t q0 = static_cast<int32_t>(run * kDenseRun);
  const char* out = reinterpret_cast<const char*>(a.bits) + (int64_t{roll} * a.n_pad + q0) * row_bytes;
  const uint32_t* pl_roll = a.planes + static_cast<int64_t>(roll) * 5 * words;
  int32_t e0 = 0;  // death times at or before q0
#pragma unroll
  for (int e = 0; e < kDenseMaxEvents; ++e) e0 += (e < n_ev && ev[1 + e] <= q0) ? 1 : 0;
  for (int64_t g0 = 0; g0 < groups; g0 += kDenseHold) {
    uint32_t vis[kDenseHold][4], code[kDenseHold][4][4];
    int32_t k0[kDenseHold];
#pragma unroll
    for (int h = 0; h < kDenseHold; ++h) {
      const int64_t s = (g0 + h) * 64 + lane;
      k0[h] = static_cast<int32_t>(s << 7);
      word4 p[5] = {};
      if (s < strips) {
#pragma unroll
        for (int c = 0; c < 5; ++c) p[c] = *reinterpret_cast<const word4*>(pl_roll + c * words + 4 * s);
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        vis[h][x] = p[0][x];
#pragma unroll
        for (int b = 0; b < 4; ++b) code[h][b][x] = p[1 + b][x];
      }
    }
    uint32_t w[kDenseHold][4];
#pragma unroll
    for (int h = 0; h < kDenseHold; ++h)
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        // dead at q0: code < e0, compared from the top bit down
        uint32_t lt = 0u, eq = 0xFFFFFFFFu;
#pragma unroll
        for (int b = 3; b >= 0; --b) {
          if ((e0 >> b) & 1) {
            lt |= eq & ~code[h][b][x];
            eq &= code[h][b][x];
          } else {
            eq &= ~code[h][b][x];
          }
        }
        w[h][x] = vis[h][x] & range_word(0, q0 - k0[h], x) & ~lt;
      }
    int32_t e_next = e0;
    int32_t t_next = e0 < n_ev ? ev[1 + e0] : INT32_MAX;
    for (int j = 0; j < kDenseRun; ++j) {
      const int32_t q = q0 + j;
      if (j > 0) {
        // key q joins (if it is ever visible)
#pragma unroll
        for (int h = 0; h < kDenseHold; ++h) {
          const int32_t b = q - k0[h];
          if (b >= 0 && b < 128) {
#pragma unroll
            for (int x = 0; x < 4; ++x) w[h][x] |= vis[h][x] & ((b >> 5) == x ? 1u << (b & 31) : 0u);
          }
        }
        // keys whose death time has come leave (times in increasing order)
        while (t_next <= q) {
          const int e = e_next++;
#pragma unroll
          for (int h = 0; h < kDenseHold; ++h)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              const uint32_t mk = ((e & 1) ? code[h][0][x] : ~code[h][0][x]) &
                                  ((e & 2) ? code[h][1][x] : ~code[h][1][x]) &
                                  ((e & 4) ? code[h][2][x] : ~code[h][2][x]) &
                                  ((e & 8) ? code[h][3][x] : ~code[h][3][x]);
              w[h][x] &= ~mk;
            }
          t_next = e_next < n_ev ? ev[1 + e_next] : INT32_MAX;
        }
      }
#pragma unroll
      for (int h = 0; h < kDenseHold; ++h) {
        const int64_t g = g0 + h;
        if (g < groups)
          // sc0 | nt | sc1 through a descriptor on the wave's 1 KiB of the row:
          // lanes past the row's last strip store nothing
          store_chunk_policy(word4{w[h][0], w[h][1], w[h][2], w[h][3]},
                             reinterpret_cast<const chunk_t*>(out + j * row_bytes + g * 1024), lane * 16,
                             static_cast<uint32_t>(min<int64_t>(64, strips - g * 64) * 16));
      }
    }
  }
}

}  // namespace

hipError_t launch_kvs_death(const KvsDeathLaunch& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  if (a.n_events > 0) {
    kvs_rank_kernel<<<dim3(static_cast<unsigned>(a.n_events)), dim3(kRankThreads), 0, s>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  kvs_chain_kernel<<<dim3(static_cast<unsigned>(a.n * a.chain_blocks)), dim3(kChainThreads), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_kvs_block(const KvsBlockLaunch& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  const int64_t w1 = static_cast<int64_t>(a.n) * a.nk;
  kvs_minmax_kernel<<<dim3(static_cast<unsigned>((w1 + 3) / 4)), dim3(256), 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t w2 = static_cast<int64_t>(a.n) * a.nq;
  kvs_block_kernel<<<dim3(static_cast<unsigned>((w2 + 3) / 4)), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_kvs_dense(const KvsDenseLaunch& a, hipStream_t s) {
  if (a.n == 0) return hipSuccess;
  if (a.events) {
    // blocks per rollout: enough to fill the chip's CUs, none without keys
    const int64_t split = std::min<int64_t>(std::max<int64_t>(1, 512 / a.n), (a.n_pad + 1023) / 1024);
    kvs_events_kernel<<<dim3(static_cast<unsigned>(a.n), static_cast<unsigned>(split)), dim3(1024),
                        static_cast<size_t>(a.n_pad >> 3), s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // four runs of kDenseRun rows per block: n_pad / kDenseRun is a multiple of 16
    const int64_t run_waves = static_cast<int64_t>(a.n) * (a.n_pad / kDenseRun);
    kvs_dense_ev_kernel<<<dim3(static_cast<unsigned>(run_waves / 4)), dim3(256), 0, s>>>(a);
    return hipGetLastError();
  }
  const int64_t runs = (a.n_pad + a.rows_per_thread - 1) / a.rows_per_thread;
  const int64_t groups = ((a.n_pad >> 7) + 63) >> 6;
  const int64_t waves = static_cast<int64_t>(a.n) * runs * groups;
  kvs_dense_kernel<<<dim3(static_cast<unsigned>((waves + 3) / 4)), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace ll
