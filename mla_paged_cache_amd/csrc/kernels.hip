// gfx950 kernels of the splice / evict path on a paged MLA cache.
//
//  * splice_kernel: writes the rows of fresh destination pages (prefix rows of
//    a boundary page, the stub rows R, and downstream rows moved by Delta with
//    their k_pe turned by R(Delta)) and rewrites the page-table rows
//    ("Leyline: KV Cache Directives for Agentic Inference", sections 2.1-2.3).
//  * splice_inplace_kernel: rotates the k_pe band of reused downstream pages
//    in place (Delta a multiple of the page size), before splice_kernel or,
//    with no page to move, with the page-table rewrite itself.
//  * keep_scan_kernel: per-sequence exclusive prefix sum of a keep mask built
//    from wave64 ballots, giving each kept row its new index and physical
//    source row, plus the per-new-page reuse test and the bitmap of the old
//    pages no new page keeps ("KV-streams", "how it works").  It serves every
//    pool kind.
//  * evict_move_kernel: copies kept rows into fresh pages, no rotation, and
//    rewrites the page-table rows.
//  * table_write_kernel: page-table row rewrites on their own.
//
// The row kernels are bound by HBM bandwidth (0.08 flop per byte), so they
// are flat 16-byte gathers, one chunk per thread, each block inside one layer
// (splice: 256-thread blocks; eviction: one wave per block), one 64-byte
// descriptor load before the data load, non-temporal loads, and stores with
// the streaming cache policy through a buffer descriptor on the wave's
// destination page (page size >= 8; smaller pages: non-temporal stores).  The
// in-place band rotation keeps plain stores.  Only k_pe chunks (8 of every
// 72) do arithmetic.
#include <mutex>

#include "device_common.h"

namespace ll {
namespace {

// Turn the k_pe chunk `v` (chunk kc = 0..7 of the band) by the directive's
// table.  Every lane of the wave must call this (the half-split layout trades
// chunks between lanes kc and kc ^ 4 of the same row); `on` selects the lanes
// whose chunk really turns.
template <int PAIRING>
__device__ __forceinline__ chunk_t rotate_kpe(chunk_t v, bool on, int kc, const SpliceDir* d) {
  if constexpr (PAIRING == 0) {
    if (on) {
      float cs[4], sn[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cs[e] = d->cos_[4 * kc + e];
        sn[e] = d->sin_[4 * kc + e];
      }
      v = rotate_interleaved(v, cs, sn);
    }
    return v;
  } else {
    const chunk_t other = shfl_xor4(v);
    if (on) {
      float cs[8], sn[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        cs[e] = d->cos_[8 * (kc & 3) + e];
        sn[e] = d->sin_[8 * (kc & 3) + e];
      }
      v = rotate_half(v, other, kc < 4, cs, sn);
    }
    return v;
  }
}

// The first 16 bytes of a splice task: dst_page, q, n_new, dir.  A scalar
// load when the index is wave-uniform (as load_task).
template <bool WAVE_TASK>
__device__ __forceinline__ chunk_t load_task_head(const SpliceTask* tasks, int64_t i) {
  if constexpr (WAVE_TASK) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(i));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(i) >> 32));
    const int64_t u = static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
    using word_ptr = const __attribute__((address_space(4))) chunk_t*;
    return *reinterpret_cast<word_ptr>(reinterpret_cast<uintptr_t>(tasks + u));
  } else {
    return *reinterpret_cast<const chunk_t*>(tasks + i);
  }
}

// Rotate the k_pe band of reused downstream rows in place: blocks
// [0, L * rot_blocks_per_layer), then (when the launch has them) the
// page-table rewrites.  A wave owns kInPlaceGroups groups of 8 rows of the
// rotate-task list (lane = 8 * row in group + band chunk), so each load
// instruction reads the whole 128-byte band line of 8 rows; the wave's
// stores follow all of its loads.  Rows are 1152 bytes apart, so these
// lines are scattered: loads are non-temporal, stores are plain (measured
// best for this pattern).  With page size >= 8 a group's 8 rows lie in one
// page and its task head is a scalar load.
template <int PAIRING, bool WAVE_TASK>
__global__ __launch_bounds__(kFlatThreads) void splice_inplace_kernel(SpliceLaunch a) {
  constexpr int R = kInPlaceGroups;
  const int64_t bb = blockIdx.x;
  const int64_t rot_blocks = a.rot_blocks_per_layer * a.num_layers;
  if (bb >= rot_blocks) {
    table_write_block(a.twrites, a.tables, a.page_table, a.max_pages_per_seq, bb - rot_blocks);
    return;
  }
  const int l = static_cast<int>(bb / a.rot_blocks_per_layer);
  const int64_t blk = bb - static_cast<int64_t>(l) * a.rot_blocks_per_layer;
  const int lane = threadIdx.x & 63;
  const int kc = lane & 7;
  const int shift = a.page_shift;
  const uint32_t pmask = (1u << shift) - 1u;
  const uint32_t row0 = static_cast<uint32_t>(blk) * kInPlaceRowsPerBlock + (threadIdx.x >> 6) * (8 * R) + (lane >> 3);
  const uint32_t n_rows = static_cast<uint32_t>(a.n_rot_tasks) << shift;
  chunk_t* layer = const_cast<chunk_t*>(a.layers[l]);
  chunk_t v[R];
  chunk_t* ptr[R];
  bool live[R];
  int dir[R];
  // Each group's task head is read just before its band load, and a lane
  // past the rows loads nothing: the compiler then keeps only about two band
  // loads of the wave in flight at a time.  For these scattered lines that
  // measured faster (28 us against 32 us for the 32k x 27 downstream) than
  // issuing all eight loads at once.
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const uint32_t rf = row0 + 8 * i;
    const bool in = rf < n_rows;  // uniform over the 8 rows of a group when P >= 8
    // head: x dst_page, y q, z n_new, w dir
    const chunk_t t = load_task_head<WAVE_TASK>(a.tasks, a.n_move_tasks + (in ? (rf >> shift) : 0));
    const uint32_t r = rf & pmask;
    live[i] = in && (static_cast<int32_t>(t.y) << shift) + static_cast<int32_t>(r) < static_cast<int32_t>(t.z);
    ptr[i] = layer + ((static_cast<int64_t>(static_cast<int32_t>(t.x)) << shift) + r) * kRowChunks + kKpeChunk0 + kc;
    dir[i] = static_cast<int32_t>(t.w);
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    v[i] = chunk_t{0u, 0u, 0u, 0u};
    if (live[i]) v[i] = __builtin_nontemporal_load(ptr[i]);
  }
#pragma unroll
  for (int i = 0; i < R; ++i) v[i] = rotate_kpe<PAIRING>(v[i], live[i], kc, a.dirs + dir[i]);
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (live[i]) *ptr[i] = v[i];
}

// Flat gather, one chunk per thread: block k of a layer covers chunks 256 k ..
// 256 k + 255.  (Two chunks per thread, both loads issued before either store,
// measured slower with the streaming stores: 182-184 us against 180.5 us for
// the 32k x 27 splice.)  Blocks [0, L * move_blocks_per_layer) move rows of
// fresh pages.  Within one page-task of P rows the 72 * P chunks are ordered
// c_kv first (chunk 64 * row + k, k < 64) and then k_pe (64 * P + 8 * row + k,
// k < 8): for P >= 8 every wave is then either a pure copy wave or a pure
// rotate wave, and the rotation code is skipped by the copy waves.  The
// remaining blocks rewrite page-table rows (no block reads the table).
// PAIRING: 0 interleaved, 1 half-split.  WAVE_TASK: page size >= 8.
template <int PAIRING, bool WAVE_TASK>
__global__ __launch_bounds__(kFlatThreads) void splice_kernel(SpliceLaunch a) {
  constexpr int CPT = kSpliceChunksPerThread;
  const int64_t b = blockIdx.x;
  const int64_t bpl = a.move_blocks_per_layer;
  const int64_t move_blocks = bpl * a.num_layers;
  if (b >= move_blocks) {
    table_write_block(a.twrites, a.tables, a.page_table, a.max_pages_per_seq, b - move_blocks);
    return;
  }
  const int64_t bb = b;
  const int l = static_cast<int>(bb / bpl);
  const uint32_t c0 = static_cast<uint32_t>((bb - static_cast<int64_t>(l) * bpl) * kFlatThreads * CPT + threadIdx.x);
  const int shift = a.page_shift;
  const uint32_t pmask = (1u << shift) - 1u;
  constexpr uint32_t kKpeChunks = kRowChunks - kKpeChunk0;
  const chunk_t* layer = a.layers[l];
  chunk_t v[CPT];
  const chunk_t* srcs[CPT];
  int64_t dsts[CPT];
  const chunk_t* dpage[CPT];
  uint32_t doff[CPT];
  bool lives[CPT], rots[CPT];
  int kcs[CPT], dirs[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const uint32_t c = c0 + u * kFlatThreads;
    uint32_t r, col;
    const uint32_t task = (c / kRowChunks) >> shift;
    const uint32_t lc = c - task * (static_cast<uint32_t>(kRowChunks) << shift);
    const uint32_t ckv_chunks = static_cast<uint32_t>(kKpeChunk0) << shift;
    if (lc < ckv_chunks) {
      r = lc / kKpeChunk0;
      col = lc - r * kKpeChunk0;
    } else {
      const uint32_t k = lc - ckv_chunks;
      r = k / kKpeChunks;
      col = kKpeChunk0 + (k - r * kKpeChunks);
    }
    const int64_t ti = static_cast<int64_t>(task);
    bool live = ti < a.n_move_tasks;
    const SpliceTask t = load_task<WAVE_TASK>(a.tasks, live ? ti : 0);
    const int32_t j = (t.q << shift) + static_cast<int32_t>(r);
    live = live && j < t.n_new;
    const int64_t dst_row = (static_cast<int64_t>(t.dst_page) << shift) + r;
    const chunk_t* src;
    bool rot = false;
    if (j < t.s_start) {
      src = layer + ((static_cast<int64_t>(t.pre_page) << shift) + (j & pmask)) * kRowChunks;
    } else if (j < t.stub_end) {
      src = t.stub + l * t.stub_layer_chunks + static_cast<int64_t>(j - t.s_start) * kRowChunks;
    } else {
      const int32_t o = j - t.delta;
      const int32_t pg = ((o >> shift) == t.down_lp0) ? t.down_page0 : t.down_page1;
      src = layer + ((static_cast<int64_t>(pg) << shift) + (o & pmask)) * kRowChunks;
      rot = t.rotate != 0;
    }
    srcs[u] = src + col;
    dsts[u] = dst_row * kRowChunks + col;
    dpage[u] = layer + (static_cast<int64_t>(t.dst_page) << shift) * kRowChunks;
    doff[u] = (r * kRowChunks + col) * 16u;
    lives[u] = live;
    rots[u] = rot;
    kcs[u] = static_cast<int>(col) - kKpeChunk0;
    dirs[u] = t.dir;
  }
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    v[u] = chunk_t{0u, 0u, 0u, 0u};
    if (lives[u]) v[u] = __builtin_nontemporal_load(srcs[u]);
  }
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    if (!WAVE_TASK || kcs[u] >= 0)
      v[u] = rotate_kpe<PAIRING>(v[u], lives[u] && rots[u] && kcs[u] >= 0, kcs[u], a.dirs + dirs[u]);
    if constexpr (WAVE_TASK) {  // the destination page is wave-uniform
      if (lives[u]) store_chunk_policy(v[u], dpage[u], doff[u], (static_cast<uint32_t>(kRowChunks) << shift) * 16u);
    } else {
      if (lives[u]) __builtin_nontemporal_store(v[u], const_cast<chunk_t*>(layer) + dsts[u]);
    }
  }
}

// Flat copy of the kept rows that land in fresh pages (rotation off), then
// the page-table rewrites in the blocks after the row blocks.
template <bool WAVE_TASK>
__global__ __launch_bounds__(kEvictThreads) void evict_move_kernel(EvictLaunch a) {
  const int64_t b = blockIdx.x;
  const int64_t bpl = a.blocks_per_layer;
  const int64_t move_blocks = bpl * a.num_layers;
  if (b >= move_blocks) {
    table_write_block(a.twrites, a.tables, a.page_table, a.max_pages_per_seq, b - move_blocks);
    return;
  }
  const int l = static_cast<int>(b / bpl);
  const uint32_t c = static_cast<uint32_t>((b - static_cast<int64_t>(l) * bpl) * kEvictThreads + threadIdx.x);
  const int shift = a.page_shift;
  const uint32_t row_flat = c / kRowChunks;
  const uint32_t col = c - row_flat * kRowChunks;
  const int64_t ti = row_flat >> shift;
  if (ti >= a.n_tasks) return;
  const EvictTask t = load_task<WAVE_TASK>(a.tasks, ti);
  const uint32_t r = row_flat & ((1u << shift) - 1u);
  if (static_cast<int32_t>(r) >= t.rows) return;
  int64_t src_row;
  if (t.src_off0 >= 0) {
    const int32_t o = t.src_off0 + static_cast<int32_t>(r);
    const int32_t P = 1 << shift;
    src_row = o < P ? (static_cast<int64_t>(t.src0) << shift) + o : (static_cast<int64_t>(t.src1) << shift) + (o - P);
  } else {
    src_row = a.src_rows[static_cast<int64_t>(t.src0) + r];
  }
  const chunk_t* layer = a.layers[l];
  const chunk_t v = __builtin_nontemporal_load(layer + src_row * kRowChunks + col);
  if constexpr (WAVE_TASK) {  // the destination page is wave-uniform
    store_chunk_policy(v, layer + (static_cast<int64_t>(t.dst_page) << shift) * kRowChunks, (r * kRowChunks + col) * 16u,
                       (static_cast<uint32_t>(kRowChunks) << shift) * 16u);
  } else {
    __builtin_nontemporal_store(v, const_cast<chunk_t*>(layer) +
                                       ((static_cast<int64_t>(t.dst_page) << shift) + r) * kRowChunks + col);
  }
}

__global__ __launch_bounds__(256) void table_write_kernel(TableLaunch a) {
  table_write_block(a.twrites, a.tables, a.page_table, a.max_pages_per_seq, blockIdx.x);
}

// Physical page of fresh index f: run r holds fresh indices
// run_first[r] .. run_first[r + 1] - 1 on pages run_page[r], run_page[r] + 1, ...
__device__ __forceinline__ int32_t fresh_page(const DirectPlanArgs& a, int32_t f) {
  int lo = 0, hi = a.n_runs - 1;  // the last run r with run_first[r] <= f
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.run_first[mid] <= f)
      lo = mid;
    else
      hi = mid - 1;
  }
  return a.run_page[lo] + (f - a.run_first[lo]);
}

// Expands a splice batch planned on the device (blockIdx.y = directive, one
// thread per new page) into
// the per-page tasks, rotation tables and new page-table rows of the row
// kernels.  Per new page q the rule is the closed form of the page plan: q
// keeps old page p iff all its live rows are old rows of page p at unchanged
// offsets -- pure prefix pages keep q, pure downstream pages keep
// (q * P - Delta) / P when Delta is a multiple of P, a page holding R rows, or
// prefix and downstream rows with Delta != 0, is fresh.  Old entries are read
// from the page table, which the row kernel rewrites only after this launch.
__global__ __launch_bounds__(256) void splice_plan_kernel(DirectPlanArgs a) {
  const int di = blockIdx.y;
  const DirectDir& D = a.d[di];
  const int shift = a.page_shift;
  const int32_t P = 1 << shift;
  const int32_t* T = a.page_table + static_cast<int64_t>(D.seq) * a.max_pages_per_seq;
  const int32_t pages = (D.n_new + P - 1) >> shift;
  const int32_t s0 = D.s_start, se = D.stub_end, delta = D.delta;
  const int32_t q = static_cast<int32_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q < pages) {
    const int32_t lo = q << shift;
    const int32_t hi = min(lo + P, D.n_new);
    const bool has_pre = lo < s0;
    const bool has_stub = se > s0 && lo < se && hi > s0;
    const bool has_down = hi > se;
    int32_t reuse;
    if (has_stub)
      reuse = -1;
    else if (has_pre && has_down)
      reuse = delta == 0 ? q : -1;
    else if (has_pre)
      reuse = q;
    else
      reuse = ((lo - delta) & (P - 1)) == 0 ? (lo - delta) >> shift : -1;
    if (!a.page_reuse) reuse = -1;  // page reuse off: every new page is fresh
    // the host checked that its plan puts fresh and rotated pages in the
    // ranges it sent; the guards only keep every access inside the buffers
    if (reuse >= D.old_pages) reuse = D.old_pages - 1;
    const int32_t f = D.fresh_base + (q - D.q_fresh0);
    const bool no_page = reuse < 0 && (a.n_runs == 0 || f < 0 || f >= a.run_first[a.n_runs]);
    const int32_t page = reuse >= 0 ? T[reuse] : (no_page ? 0 : fresh_page(a, f));
    if (D.packed_off + q < a.n_entries) a.tables[D.packed_off + q] = page;
    const bool in_place = reuse >= 0 && has_down && D.rotate != 0;
    SpliceTask t;
    t.dst_page = page;
    t.pre_page = -1;
    t.down_page0 = -1;
    t.down_page1 = -1;
    t.q = q;
    t.down_lp0 = -1;
    t.dir = di;
    t.rotate = D.rotate;
    t.s_start = s0;
    t.stub_end = se;
    t.delta = delta;
    t.n_new = no_page ? 0 : D.n_new;  // no live rows: the row kernel skips the task
    t.stub = D.stub;
    t.stub_layer_chunks = D.stub_layer_chunks;
    if (in_place) {
      const int64_t k = D.rot_base + (q - D.q_rot0);
      if (k >= 0 && k < a.n_rot_tasks) a.tasks[a.n_move_tasks + k] = t;
    } else if (reuse < 0) {
      if (has_pre && q < D.old_pages) t.pre_page = T[q];
      const int32_t jd = max(lo, se);  // first downstream row of the page
      if (jd < hi && ((jd - delta) >> shift) < D.old_pages) {
        const int32_t lp0 = (jd - delta) >> shift;
        t.down_lp0 = lp0;
        t.down_page0 = T[lp0];
        t.down_page1 = lp0 + 1 < D.old_pages ? T[lp0 + 1] : -1;
      }
      const int64_t k = D.move_base + (q - D.q_fresh0);
      if (k >= 0 && k < a.n_move_tasks) a.tasks[k] = t;
    }
  }
  if (blockIdx.x != 0) return;
  if (threadIdx.x == 0) {
    TableWrite w;
    w.src_off = D.packed_off;
    w.seq = D.seq;
    w.count = pages;
    a.twrites[di] = w;
  }
  const float* trig = a.trig + 2 * a.pairs * di;
  if (a.gqa) {
    GqaDir* g = static_cast<GqaDir*>(a.dirs) + di;
    if (threadIdx.x == 0) {
      g->stub_v = D.stub_v;
      g->stub_v_layer_chunks = D.stub_v_layer_chunks;
    }
    for (int j = threadIdx.x; j < a.pairs; j += blockDim.x) {
      g->cos_[j] = trig[j];
      g->sin_[j] = trig[a.pairs + j];
    }
  } else {
    SpliceDir* s = static_cast<SpliceDir*>(a.dirs) + di;
    for (int j = threadIdx.x; j < a.pairs; j += blockDim.x) {
      s->cos_[j] = trig[j];
      s->sin_[j] = trig[a.pairs + j];
    }
  }
}

constexpr int kScanThreads = 1024;
constexpr int kScanWaves = kScanThreads / 64;

// One block per sequence.  Each thread takes 16 mask bytes per tile; the
// count of kept bytes (0..16) is scanned across the wave with one ballot per
// bit of the count, then across the 16 waves through LDS.  Kept row i of the
// sequence gets new index = number of kept rows before it; its logical index
// i and its physical source row (old page table) are stored there.
__global__ __launch_bounds__(kScanThreads) void keep_scan_kernel(ScanLaunch a) {
  __shared__ int32_t wave_total[kScanWaves];
  const EvictSeq e = a.seqs[blockIdx.x];
  const uint8_t* m = a.keep + e.mask_off;
  int32_t* out = a.src_rows + e.src_off;
  int32_t* out_logical = a.src_logical + e.src_off;
  const int32_t* table = a.page_table + static_cast<int64_t>(e.seq) * a.max_pages_per_seq;
  const int shift = a.page_shift;
  const int64_t pmask = (int64_t{1} << shift) - 1;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint64_t lanes_below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int64_t carry = 0;
  for (int64_t base = 0; base < e.n_old; base += 16 * kScanThreads) {
    const int64_t i0 = base + 16 * static_cast<int64_t>(threadIdx.x);
    // page size 1: the 16 rows' pages, read with the mask (four 16-byte
    // loads when the row lies whole and aligned in the table)
    int32_t pg16[16];
    if (shift == 0) {
      if (i0 + 16 <= e.n_old && (reinterpret_cast<uintptr_t>(table + i0) & 15u) == 0) {
        const chunk_t* t4 = reinterpret_cast<const chunk_t*>(table + i0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const chunk_t v = t4[q];
          pg16[4 * q] = static_cast<int32_t>(v.x);
          pg16[4 * q + 1] = static_cast<int32_t>(v.y);
          pg16[4 * q + 2] = static_cast<int32_t>(v.z);
          pg16[4 * q + 3] = static_cast<int32_t>(v.w);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 16; ++c) pg16[c] = i0 + c < e.n_old ? table[i0 + c] : 0;
      }
    }
    uint32_t bits = 0;
    if (i0 + 16 <= e.n_old && (reinterpret_cast<uintptr_t>(m + i0) & 15u) == 0) {
      const chunk_t v = *reinterpret_cast<const chunk_t*>(m + i0);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if ((w[q] >> (8 * c)) & 0xFFu) bits |= 1u << (4 * q + c);
    } else {
      for (int c = 0; c < 16; ++c)
        if (i0 + c < e.n_old && m[i0 + c]) bits |= 1u << c;
    }
    const int cnt = __popc(bits);
    int below = 0, total = 0;
#pragma unroll
    for (int bit = 0; bit < 5; ++bit) {
      const uint64_t bal = __ballot((cnt >> bit) & 1);
      below += __popcll(bal & lanes_below) << bit;
      total += __popcll(bal) << bit;
    }
    if (lane == 0) wave_total[wave] = total;
    __syncthreads();
    int wave_below = 0, block_total = 0;
#pragma unroll
    for (int w = 0; w < kScanWaves; ++w) {
      const int x = wave_total[w];
      wave_below += w < wave ? x : 0;
      block_total += x;
    }
    int64_t pos = carry + wave_below + below;
    if (shift == 0) {
      // page size 1: the row's page is the row; a dropped row frees it
      for (int c = 0; c < 16; ++c) {
        const int64_t i = i0 + c;
        if (i >= e.n_old) break;
        const int32_t pg = pg16[c];
        if ((bits >> c) & 1u)
          out[pos++] = pg;
        else
          a.freed_bytes[pg] = 1;
      }
    } else {
      for (int c = 0; c < 16; ++c)
        if ((bits >> c) & 1u) {
          const int64_t i = i0 + c;
          out_logical[pos] = static_cast<int32_t>(i);
          out[pos++] = static_cast<int32_t>((static_cast<int64_t>(table[i >> shift]) << shift) + (i & pmask));
        }
    }
    carry += block_total;
    __syncthreads();
  }
  // Per new page: reusable iff its live rows are the old rows f .. f+k-1 with
  // f on a page boundary -- one old page, rows at their old offsets.  The old
  // pages no new page keeps go into the freed bitmap.
  const int64_t P = int64_t{1} << shift;
  const int64_t n_new = carry;
  if (shift == 0) {
    if (threadIdx.x == 0) a.counts[blockIdx.x] = n_new;
    return;
  }
  const int64_t pages = (n_new + P - 1) >> shift;
  const int64_t old_pages = (e.n_old + P - 1) >> shift;
  int32_t* reuse = a.reuse + e.reuse_off;
  uint8_t* kept = a.kept + e.reuse_off;
  for (int64_t k = threadIdx.x; k < old_pages; k += kScanThreads) kept[k] = 0;
  __syncthreads();
  for (int64_t q = threadIdx.x; q < pages; q += kScanThreads) {
    const int64_t k = (n_new - (q << shift)) < P ? (n_new - (q << shift)) : P;
    const int64_t f = out_logical[q << shift];
    const int64_t l = out_logical[(q << shift) + k - 1];
    const bool keep = a.page_reuse && (f & pmask) == 0 && l - f == k - 1;
    reuse[q] = keep ? static_cast<int32_t>(f >> shift) : -1;
    if (keep) kept[f >> shift] = 1;
  }
  __syncthreads();
  for (int64_t k = threadIdx.x; k < old_pages; k += kScanThreads)
    if (!kept[k]) {
      const uint32_t pg = static_cast<uint32_t>(table[k]);
      atomicOr(a.freed + (pg >> 6), 1ull << (pg & 63u));
    }
  if (threadIdx.x == 0) a.counts[blockIdx.x] = n_new;
}

__global__ __launch_bounds__(256) void unit_page_kernel(UnitPageLaunch a) {
  const int64_t b = blockIdx.x;
  if (b < a.n) {
    const EvictSeq e = a.seqs[b];
    const int64_t n_new = a.counts[b];
    int32_t* dst = a.page_table + static_cast<int64_t>(e.seq) * a.max_pages_per_seq;
    const int32_t* src = a.src_rows + e.src_off;
    for (int64_t q = threadIdx.x; q < n_new; q += 256) dst[q] = src[q];
    if (b == 0 && threadIdx.x < 4) a.info[threadIdx.x] = 0;
    return;
  }
  const int64_t w = (b - a.n) * 256 + threadIdx.x;
  if (w >= a.n_words) return;
  const chunk_t* src = reinterpret_cast<const chunk_t*>(a.freed_bytes + 64 * w);
  unsigned long long word = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const chunk_t v = src[k];
    const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if ((x[m] >> (8 * c)) & 0xFFu) word |= 1ull << (16 * k + 4 * m + c);
  }
  a.freed[w] = word;
}

}  // namespace

// The in-place band rotation is a kernel of its own (its deeper loads need
// more registers than the row moves, which then keep their occupancy).  It
// goes first; the page-table rewrite rides on the last launch.  The two
// launches touch disjoint pages.
hipError_t launch_unit_page(const UnitPageLaunch& a, hipStream_t s, const Stamp& t) {
  const int64_t grid = a.n + (a.n_words + 255) / 256;
  if (grid == 0) return stamp_empty(s, t);
  return dispatch(unit_page_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), s, t, true, true, a);
}

hipError_t launch_splice(const SpliceLaunch& a, int pairing, hipStream_t s, const Stamp& t) {
  const int64_t move = a.move_blocks_per_layer * a.num_layers;
  const int64_t rot = a.rot_blocks_per_layer * a.num_layers;
  if (move + rot + a.n_twrites == 0) return stamp_empty(s, t);
  const bool wave_task = a.page_shift >= 3;
  const dim3 blk(kFlatThreads);
  const bool moves = move > 0;
  if (rot > 0 || !moves) {
    void (*k)(SpliceLaunch);
    if (pairing == 0)
      k = wave_task ? splice_inplace_kernel<0, true> : splice_inplace_kernel<0, false>;
    else
      k = wave_task ? splice_inplace_kernel<1, true> : splice_inplace_kernel<1, false>;
    const int64_t grid = rot + (moves ? 0 : a.n_twrites);
    hipError_t e = dispatch(k, dim3(static_cast<unsigned>(grid)), blk, s, t, true, !moves, a);
    if (e != hipSuccess || !moves) return e;
  }
  void (*k)(SpliceLaunch);
  if (pairing == 0)
    k = wave_task ? splice_kernel<0, true> : splice_kernel<0, false>;
  else
    k = wave_task ? splice_kernel<1, true> : splice_kernel<1, false>;
  return dispatch(k, dim3(static_cast<unsigned>(move + a.n_twrites)), blk, s, t, rot == 0, true, a);
}

hipError_t launch_evict_move(const EvictLaunch& a, hipStream_t s, const Stamp& t) {
  const int64_t grid = a.blocks_per_layer * a.num_layers + a.n_twrites;
  if (grid == 0) return stamp_empty(s, t);
  void (*k)(EvictLaunch) = a.page_shift >= 3 ? evict_move_kernel<true> : evict_move_kernel<false>;
  return dispatch(k, dim3(static_cast<unsigned>(grid)), dim3(kEvictThreads), s, t, true, true, a);
}

hipError_t launch_table_write(const TableLaunch& a, hipStream_t s) {
  if (a.n_twrites == 0) return hipSuccess;
  table_write_kernel<<<dim3(a.n_twrites), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- scratch --
// Plan space of the splice that allocates nothing (leyline_splice_noalloc).
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address comes from hipGetSymbolAddress, per device, and only that
// address is ever handed to kernels or copies.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch_init(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device]) return hipSuccess;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_scratch_ptr[device] = ptr;
  return hipSuccess;
}

void* noalloc_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return g_scratch_ptr[device];
}

hipError_t launch_splice_plan(const DirectPlanArgs& a, int32_t max_new_pages, hipStream_t s) {
  if (a.n_dirs <= 0) return hipSuccess;
  const unsigned bx = static_cast<unsigned>(std::max(1, (max_new_pages + 255) / 256));
  splice_plan_kernel<<<dim3(bx, a.n_dirs), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_keep_scan(const ScanLaunch& a, hipStream_t s, const Stamp& t) {
  if (a.n_seqs == 0) return stamp_empty(s, t);
  return dispatch(keep_scan_kernel, dim3(a.n_seqs), dim3(kScanThreads), s, t, true, true, a);
}

}  // namespace ll
