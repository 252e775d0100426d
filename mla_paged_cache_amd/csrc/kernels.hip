// gfx950 kernels of the splice / evict path on a paged MLA cache.
//
//  * splice_kernel: writes the rows of fresh destination pages (prefix rows of
//    a boundary page, the stub rows R, and downstream rows moved by Delta with
//    their k_pe turned by R(Delta)), rotates the k_pe band of reused
//    downstream pages in place, and rewrites the page-table rows -- one
//    launch ("Leyline: KV Cache Directives for Agentic Inference", sections
//    2.1-2.3).
//  * keep_scan_kernel: per-sequence exclusive prefix sum of a keep mask built
//    from wave64 ballots, giving each kept row its new index and physical
//    source row, plus the per-new-page reuse test ("KV-streams", "how it
//    works").
//  * evict_move_kernel: copies kept rows into fresh pages, no rotation, and
//    rewrites the page-table rows.
//  * gqa_splice_kernel / plane_evict_kernel: the same two row kernels on GQA /
//    MHA pools (separate K and V planes, a RoPE band per K head).
//  * table_write_kernel: page-table row rewrites on their own.
//
// The row kernels are bound by HBM bandwidth (0.08 flop per byte), so they
// are flat 16-byte gathers: one chunk per thread, 256-thread blocks, each
// block inside one layer, one 64-byte descriptor load before the data load,
// non-temporal loads and stores.  Only k_pe chunks (8 of every 72) do
// arithmetic.
#include "leyline_internal.h"

namespace ll {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) | 0x40u) & 0xFFFFu;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// x' = x c - y s, y' = x s + y c: every product and the sum rounded to float32
// on its own (no contraction), then bf16.
__device__ __forceinline__ float rot_x(float x, float y, float c, float s) {
#pragma clang fp contract(off)
  const float xc = x * c;
  const float ys = y * s;
  return xc - ys;
}
__device__ __forceinline__ float rot_y(float x, float y, float c, float s) {
#pragma clang fp contract(off)
  const float xs = x * s;
  const float yc = y * c;
  return xs + yc;
}

// Interleaved pairs: word m of k_pe chunk k holds pair 4k+m, x in the low
// half, y in the high half.
__device__ __forceinline__ uint32_t rot_word(uint32_t w, float c, float s) {
  const float x = bf16_lo(w), y = bf16_hi(w);
  return to_bf16(rot_x(x, y, c, s)) | (to_bf16(rot_y(x, y, c, s)) << 16);
}

__device__ __forceinline__ chunk_t rotate_interleaved(chunk_t v, const float* c, const float* s) {
  v.x = rot_word(v.x, c[0], s[0]);
  v.y = rot_word(v.y, c[1], s[1]);
  v.z = rot_word(v.z, c[2], s[2]);
  v.w = rot_word(v.w, c[3], s[3]);
  return v;
}

// Half-split pairs: chunk k < 4 holds x of pairs 8k..8k+7, chunk k+4 holds
// their y.  `own` is this lane's chunk, `other` the partner lane's chunk.
__device__ __forceinline__ uint32_t rot_half_word(uint32_t own, uint32_t other, bool x_side,
                                                  const float* c, const float* s, int m) {
  const float a0 = bf16_lo(own), a1 = bf16_hi(own);
  const float b0 = bf16_lo(other), b1 = bf16_hi(other);
  const int e0 = 2 * m, e1 = 2 * m + 1;
  float r0, r1;
  if (x_side) {
    r0 = rot_x(a0, b0, c[e0], s[e0]);
    r1 = rot_x(a1, b1, c[e1], s[e1]);
  } else {
    r0 = rot_y(b0, a0, c[e0], s[e0]);
    r1 = rot_y(b1, a1, c[e1], s[e1]);
  }
  return to_bf16(r0) | (to_bf16(r1) << 16);
}

__device__ __forceinline__ chunk_t rotate_half(chunk_t own, chunk_t other, bool x_side, const float* c,
                                               const float* s) {
  chunk_t r;
  r.x = rot_half_word(own.x, other.x, x_side, c, s, 0);
  r.y = rot_half_word(own.y, other.y, x_side, c, s, 1);
  r.z = rot_half_word(own.z, other.z, x_side, c, s, 2);
  r.w = rot_half_word(own.w, other.w, x_side, c, s, 3);
  return r;
}

__device__ __forceinline__ chunk_t shfl_xor4(chunk_t v) {
  chunk_t r;
  r.x = __shfl_xor(v.x, 4);
  r.y = __shfl_xor(v.y, 4);
  r.z = __shfl_xor(v.z, 4);
  r.w = __shfl_xor(v.w, 4);
  return r;
}

__device__ __forceinline__ void table_write_block(const TableWrite* tw, const int32_t* tables,
                                                  int32_t* page_table, int32_t max_pages, int64_t i) {
  const TableWrite w = tw[i];
  int32_t* dst = page_table + static_cast<int64_t>(w.seq) * max_pages;
  for (int e = threadIdx.x; e < w.count; e += blockDim.x) dst[e] = tables[w.src_off + e];
}

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

// Descriptor load: when every lane of the wave needs the same task (page size
// >= 8: a page is 72 * P chunks, a multiple of 64, and waves start on multiples
// of 64), the index is made wave-uniform and read through the constant
// address space, i.e. with one scalar load instead of a 64-byte load per lane.
template <bool WAVE_TASK, typename T>
__device__ __forceinline__ T load_task(const T* tasks, int64_t i) {
  if constexpr (WAVE_TASK) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(i));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(i) >> 32));
    const int64_t u = static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
    static_assert(sizeof(T) % 16 == 0, "descriptors are whole 16-byte words");
    using word_ptr = const __attribute__((address_space(4))) chunk_t*;
    const word_ptr src = reinterpret_cast<word_ptr>(reinterpret_cast<uintptr_t>(tasks + u));
    T out;
    chunk_t* dst = reinterpret_cast<chunk_t*>(&out);
#pragma unroll
    for (int k = 0; k < static_cast<int>(sizeof(T) / 16); ++k) dst[k] = src[k];
    return out;
  } else {
    return tasks[i];
  }
}

// Flat gather.  Blocks [0, L * move_blocks_per_layer) move rows of fresh
// pages.  Within one page-task of P rows the 72 * P chunks are ordered c_kv
// first (chunk 64 * row + k, k < 64) and then k_pe (64 * P + 8 * row + k,
// k < 8): for P >= 8 every wave is then either a pure copy wave or a pure
// rotate wave, and the rotation code is skipped by the copy waves.  The next
// L * rot_blocks_per_layer blocks rotate k_pe in place (chunk 8 * row + k of
// the rotate-task list).  The remaining blocks rewrite page-table rows (no
// block reads the table).  PAIRING: 0 interleaved, 1 half-split.
// WAVE_TASK: page size >= 8.
template <int PAIRING, bool WAVE_TASK>
__global__ __launch_bounds__(kFlatThreads) void splice_kernel(SpliceLaunch a) {
  const int64_t b = blockIdx.x;
  const int64_t move_blocks = a.move_blocks_per_layer * a.num_layers;
  const int64_t rot_blocks = a.rot_blocks_per_layer * a.num_layers;
  if (b >= move_blocks + rot_blocks) {
    table_write_block(a.twrites, a.tables, a.page_table, a.max_pages_per_seq, b - move_blocks - rot_blocks);
    return;
  }
  const bool in_place = b >= move_blocks;
  const int64_t bb = in_place ? b - move_blocks : b;
  const int64_t bpl = in_place ? a.rot_blocks_per_layer : a.move_blocks_per_layer;
  const int l = static_cast<int>(bb / bpl);
  const uint32_t c = static_cast<uint32_t>((bb - static_cast<int64_t>(l) * bpl) * kFlatThreads + threadIdx.x);
  const int shift = a.page_shift;
  const uint32_t pmask = (1u << shift) - 1u;
  constexpr uint32_t kKpeChunks = kRowChunks - kKpeChunk0;

  uint32_t task, r, col;
  if (in_place) {
    const uint32_t row_flat = c / kKpeChunks;
    task = row_flat >> shift;
    r = row_flat & pmask;
    col = kKpeChunk0 + (c - row_flat * kKpeChunks);
  } else {
    task = (c / kRowChunks) >> shift;
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
  }
  const int64_t ti = static_cast<int64_t>(task) + (in_place ? a.n_move_tasks : 0);
  const int64_t t_end = in_place ? a.n_move_tasks + a.n_rot_tasks : a.n_move_tasks;
  bool live = ti < t_end;
  const SpliceTask t = load_task<WAVE_TASK>(a.tasks, live ? ti : 0);
  const int32_t j = (t.q << shift) + static_cast<int32_t>(r);
  live = live && j < t.n_new;

  const chunk_t* layer = a.layers[l];
  const int64_t dst_row = (static_cast<int64_t>(t.dst_page) << shift) + r;
  const chunk_t* src;
  bool rot = false;
  if (in_place) {
    src = layer + dst_row * kRowChunks;
    rot = true;
  } else if (j < t.s_start) {
    src = layer + ((static_cast<int64_t>(t.pre_page) << shift) + (j & pmask)) * kRowChunks;
  } else if (j < t.stub_end) {
    src = t.stub + l * t.stub_layer_chunks + static_cast<int64_t>(j - t.s_start) * kRowChunks;
  } else {
    const int32_t o = j - t.delta;
    const int32_t pg = ((o >> shift) == t.down_lp0) ? t.down_page0 : t.down_page1;
    src = layer + ((static_cast<int64_t>(pg) << shift) + (o & pmask)) * kRowChunks;
    rot = t.rotate != 0;
  }
  chunk_t v = chunk_t{0u, 0u, 0u, 0u};
  if (live) v = __builtin_nontemporal_load(src + col);
  const int kc = static_cast<int>(col) - kKpeChunk0;
  if (!WAVE_TASK || kc >= 0) {
    // k_pe waves (or mixed waves at page sizes below 8)
    v = rotate_kpe<PAIRING>(v, live && rot && kc >= 0, kc, a.dirs + t.dir);
  }
  if (live) __builtin_nontemporal_store(v, const_cast<chunk_t*>(layer) + dst_row * kRowChunks + col);
}

// Flat copy of the kept rows that land in fresh pages (rotation off), then
// the page-table rewrites in the blocks after the row blocks.
template <bool WAVE_TASK>
__global__ __launch_bounds__(kFlatThreads) void evict_move_kernel(EvictLaunch a) {
  const int64_t b = blockIdx.x;
  const int64_t move_blocks = a.blocks_per_layer * a.num_layers;
  if (b >= move_blocks) {
    table_write_block(a.twrites, a.tables, a.page_table, a.max_pages_per_seq, b - move_blocks);
    return;
  }
  const int l = static_cast<int>(b / a.blocks_per_layer);
  const uint32_t c = static_cast<uint32_t>((b - static_cast<int64_t>(l) * a.blocks_per_layer) * kFlatThreads +
                                           threadIdx.x);
  const int shift = a.page_shift;
  const uint32_t row_flat = c / kRowChunks;
  const uint32_t col = c - row_flat * kRowChunks;
  const int64_t ti = row_flat >> shift;
  if (ti >= a.n_tasks) return;
  const EvictTask t = load_task<WAVE_TASK>(a.tasks, ti);
  const uint32_t r = row_flat & ((1u << shift) - 1u);
  const int64_t j = (static_cast<int64_t>(t.q) << shift) + r;
  if (j >= t.n_new) return;
  const int64_t src_row = a.src_rows[t.src_off + j];
  const chunk_t* layer = a.layers[l];
  const chunk_t v = __builtin_nontemporal_load(layer + src_row * kRowChunks + col);
  __builtin_nontemporal_store(v, const_cast<chunk_t*>(layer) +
                                     ((static_cast<int64_t>(t.dst_page) << shift) + r) * kRowChunks + col);
}

// ---------------------------------------------------------------- GQA / MHA
// The same flat gather on pools of K and V planes ("Leyline", section 5).  A
// K head's RoPE band spans 2^rot_shift chunks starting at a multiple of that
// count (rotary_dim is a power of two dividing head_dim), so a band never
// straddles a wave and the half-split partner of band chunk kc is lane
// xor (band chunks / 2).

__device__ __forceinline__ chunk_t shfl_xor_n(chunk_t v, int m) {
  chunk_t r;
  r.x = __shfl_xor(v.x, m);
  r.y = __shfl_xor(v.y, m);
  r.z = __shfl_xor(v.z, m);
  r.w = __shfl_xor(v.w, m);
  return r;
}

// Turn band chunk kc (0 .. 2*half-1) of a K head.  Every lane of the wave
// calls this (half-split trades chunks between lanes); `on` selects the lanes
// whose chunk turns.
template <int PAIRING>
__device__ __forceinline__ chunk_t rotate_band(chunk_t v, bool on, int kc, int half, const GqaDir* d) {
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
    const chunk_t other = shfl_xor_n(v, half);
    if (on) {
      const int p0 = 8 * (kc & (half - 1));
      float cs[8], sn[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        cs[e] = d->cos_[p0 + e];
        sn[e] = d->sin_[p0 + e];
      }
      v = rotate_half(v, other, kc < half, cs, sn);
    }
    return v;
  }
}

// Blocks [0, 2L * move_blocks_per_plane) write the rows of fresh pages, plane
// by plane (K planes, then V planes); each row is row_chunks consecutive
// chunks.  The next L * rot_blocks_per_plane blocks turn the RoPE bands of
// reused pages' downstream rows in place (K planes only; chunk (row, head,
// kc) of the band list).  The remaining blocks rewrite page-table rows.
// WAVE_TASK: every wave lies inside one page task in both block ranges.
template <int PAIRING, bool WAVE_TASK>
__global__ __launch_bounds__(kFlatThreads) void gqa_splice_kernel(GqaSpliceLaunch a) {
  const int64_t b = blockIdx.x;
  const int64_t move_blocks = a.move_blocks_per_plane * 2 * a.num_layers;
  const int64_t rot_blocks = a.rot_blocks_per_plane * a.num_layers;
  if (b >= move_blocks + rot_blocks) {
    table_write_block(a.twrites, a.tables, a.page_table, a.max_pages_per_seq, b - move_blocks - rot_blocks);
    return;
  }
  const bool in_place = b >= move_blocks;
  const int64_t bb = in_place ? b - move_blocks : b;
  const int64_t bpp = in_place ? a.rot_blocks_per_plane : a.move_blocks_per_plane;
  const int plane = static_cast<int>(bb / bpp);
  const uint32_t c = static_cast<uint32_t>((bb - static_cast<int64_t>(plane) * bpp) * kFlatThreads + threadIdx.x);
  const int shift = a.page_shift;
  const uint32_t pmask = (1u << shift) - 1u;
  const uint32_t rc = static_cast<uint32_t>(a.row_chunks);
  const uint32_t hc = static_cast<uint32_t>(a.head_chunks);
  const int rs = a.rot_shift;
  const uint32_t band = 1u << rs;
  const bool k_plane = plane < a.num_layers;

  uint32_t row_flat, col;
  int kc;  // chunk within the head's RoPE band, or -1
  if (in_place) {
    const uint32_t per_row = static_cast<uint32_t>(a.heads) << rs;
    row_flat = c / per_row;
    const uint32_t w = c - row_flat * per_row;
    kc = static_cast<int>(w & (band - 1u));
    col = (w >> rs) * hc + static_cast<uint32_t>(kc);
  } else {
    row_flat = c / rc;
    col = c - row_flat * rc;
    const uint32_t in_head = col - (col / hc) * hc;
    kc = in_head < band ? static_cast<int>(in_head) : -1;
  }
  const uint32_t task = row_flat >> shift;
  const uint32_t r = row_flat & pmask;
  const int64_t ti = static_cast<int64_t>(task) + (in_place ? a.n_move_tasks : 0);
  const int64_t t_end = in_place ? a.n_move_tasks + a.n_rot_tasks : a.n_move_tasks;
  bool live = ti < t_end;
  const SpliceTask t = load_task<WAVE_TASK>(a.tasks, live ? ti : 0);
  const int32_t j = (t.q << shift) + static_cast<int32_t>(r);
  live = live && j < t.n_new;
  const GqaDir* dir = a.dirs + t.dir;

  const chunk_t* layer = a.planes[plane];
  const int64_t dst_row = (static_cast<int64_t>(t.dst_page) << shift) + r;
  const chunk_t* src;
  bool rot = false;
  if (in_place) {
    src = layer + dst_row * rc;
    rot = true;
  } else if (j < t.s_start) {
    src = layer + ((static_cast<int64_t>(t.pre_page) << shift) + (j & pmask)) * rc;
  } else if (j < t.stub_end) {
    const chunk_t* stub = k_plane ? t.stub + plane * t.stub_layer_chunks
                                  : dir->stub_v + (plane - a.num_layers) * dir->stub_v_layer_chunks;
    src = stub + static_cast<int64_t>(j - t.s_start) * rc;
  } else {
    const int32_t o = j - t.delta;
    const int32_t pg = ((o >> shift) == t.down_lp0) ? t.down_page0 : t.down_page1;
    src = layer + ((static_cast<int64_t>(pg) << shift) + (o & pmask)) * rc;
    rot = t.rotate != 0;
  }
  chunk_t v = chunk_t{0u, 0u, 0u, 0u};
  if (live) v = __builtin_nontemporal_load(src + col);
  if (k_plane) v = rotate_band<PAIRING>(v, live && rot && kc >= 0, kc, static_cast<int>(band >> 1), dir);
  if (live) __builtin_nontemporal_store(v, const_cast<chunk_t*>(layer) + dst_row * rc + col);
}

// Eviction on K / V planes: flat copy of the kept rows that land in fresh
// pages, then the page-table rewrites.
template <bool WAVE_TASK>
__global__ __launch_bounds__(kFlatThreads) void plane_evict_kernel(PlaneEvictLaunch a) {
  const int64_t b = blockIdx.x;
  const int64_t move_blocks = a.blocks_per_plane * a.num_planes;
  if (b >= move_blocks) {
    table_write_block(a.twrites, a.tables, a.page_table, a.max_pages_per_seq, b - move_blocks);
    return;
  }
  const int plane = static_cast<int>(b / a.blocks_per_plane);
  const uint32_t c = static_cast<uint32_t>((b - static_cast<int64_t>(plane) * a.blocks_per_plane) * kFlatThreads +
                                           threadIdx.x);
  const int shift = a.page_shift;
  const uint32_t rc = static_cast<uint32_t>(a.row_chunks);
  const uint32_t row_flat = c / rc;
  const uint32_t col = c - row_flat * rc;
  const int64_t ti = row_flat >> shift;
  if (ti >= a.n_tasks) return;
  const EvictTask t = load_task<WAVE_TASK>(a.tasks, ti);
  const uint32_t r = row_flat & ((1u << shift) - 1u);
  const int64_t j = (static_cast<int64_t>(t.q) << shift) + r;
  if (j >= t.n_new) return;
  const int64_t src_row = a.src_rows[t.src_off + j];
  const chunk_t* layer = a.planes[plane];
  const chunk_t v = __builtin_nontemporal_load(layer + src_row * rc + col);
  __builtin_nontemporal_store(v, const_cast<chunk_t*>(layer) + ((static_cast<int64_t>(t.dst_page) << shift) + r) * rc + col);
}

__global__ __launch_bounds__(256) void table_write_kernel(TableLaunch a) {
  table_write_block(a.twrites, a.tables, a.page_table, a.max_pages_per_seq, blockIdx.x);
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
    for (int c = 0; c < 16; ++c)
      if ((bits >> c) & 1u) {
        const int64_t i = i0 + c;
        out_logical[pos] = static_cast<int32_t>(i);
        out[pos++] = static_cast<int32_t>((static_cast<int64_t>(table[i >> shift]) << shift) + (i & pmask));
      }
    carry += block_total;
    __syncthreads();
  }
  // Per new page: reusable iff its live rows are the old rows f .. f+k-1 with
  // f on a page boundary -- one old page, rows at their old offsets.
  const int64_t P = int64_t{1} << shift;
  const int64_t n_new = carry;
  const int64_t pages = (n_new + P - 1) >> shift;
  int32_t* reuse = a.reuse + e.reuse_off;
  for (int64_t q = threadIdx.x; q < pages; q += kScanThreads) {
    const int64_t k = (n_new - (q << shift)) < P ? (n_new - (q << shift)) : P;
    const int64_t f = out_logical[q << shift];
    const int64_t l = out_logical[(q << shift) + k - 1];
    reuse[q] = ((f & pmask) == 0 && l - f == k - 1) ? static_cast<int32_t>(f >> shift) : -1;
  }
  if (threadIdx.x == 0) a.counts[blockIdx.x] = n_new;
}

}  // namespace

hipError_t launch_splice(const SpliceLaunch& a, int pairing, hipStream_t s) {
  const int64_t grid = (a.move_blocks_per_layer + a.rot_blocks_per_layer) * a.num_layers + a.n_twrites;
  if (grid == 0) return hipSuccess;
  const dim3 g(static_cast<unsigned>(grid)), blk(kFlatThreads);
  const bool wave_task = a.page_shift >= 3;
  if (pairing == 0) {
    if (wave_task) splice_kernel<0, true><<<g, blk, 0, s>>>(a);
    else splice_kernel<0, false><<<g, blk, 0, s>>>(a);
  } else {
    if (wave_task) splice_kernel<1, true><<<g, blk, 0, s>>>(a);
    else splice_kernel<1, false><<<g, blk, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_evict_move(const EvictLaunch& a, hipStream_t s) {
  const int64_t grid = a.blocks_per_layer * a.num_layers + a.n_twrites;
  if (grid == 0) return hipSuccess;
  if (a.page_shift >= 3)
    evict_move_kernel<true><<<dim3(static_cast<unsigned>(grid)), dim3(kFlatThreads), 0, s>>>(a);
  else
    evict_move_kernel<false><<<dim3(static_cast<unsigned>(grid)), dim3(kFlatThreads), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gqa_splice(const GqaSpliceLaunch& a, int pairing, hipStream_t s) {
  const int64_t grid = a.move_blocks_per_plane * 2 * a.num_layers + a.rot_blocks_per_plane * a.num_layers + a.n_twrites;
  if (grid == 0) return hipSuccess;
  const dim3 g(static_cast<unsigned>(grid)), blk(kFlatThreads);
  // one task per wave when a page's chunks are a whole number of waves in
  // both the move and the in-place ranges
  const int64_t move_chunks = int64_t{a.row_chunks} << a.page_shift;
  const int64_t band_chunks = (int64_t{a.heads} << a.rot_shift) << a.page_shift;
  const bool wave_task = move_chunks % 64 == 0 && band_chunks % 64 == 0;
  if (pairing == 0) {
    if (wave_task) gqa_splice_kernel<0, true><<<g, blk, 0, s>>>(a);
    else gqa_splice_kernel<0, false><<<g, blk, 0, s>>>(a);
  } else {
    if (wave_task) gqa_splice_kernel<1, true><<<g, blk, 0, s>>>(a);
    else gqa_splice_kernel<1, false><<<g, blk, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_plane_evict(const PlaneEvictLaunch& a, hipStream_t s) {
  const int64_t grid = a.blocks_per_plane * a.num_planes + a.n_twrites;
  if (grid == 0) return hipSuccess;
  if ((int64_t{a.row_chunks} << a.page_shift) % 64 == 0)
    plane_evict_kernel<true><<<dim3(static_cast<unsigned>(grid)), dim3(kFlatThreads), 0, s>>>(a);
  else
    plane_evict_kernel<false><<<dim3(static_cast<unsigned>(grid)), dim3(kFlatThreads), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_table_write(const TableLaunch& a, hipStream_t s) {
  if (a.n_twrites == 0) return hipSuccess;
  table_write_kernel<<<dim3(a.n_twrites), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_keep_scan(const ScanLaunch& a, hipStream_t s) {
  if (a.n_seqs == 0) return hipSuccess;
  keep_scan_kernel<<<dim3(a.n_seqs), dim3(kScanThreads), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace ll
