// gfx950 kernels of the splice / evict path on paged GQA / MHA caches
// ("Leyline: KV Cache Directives for Agentic Inference", section 5: the
// directive carries over to GQA and MHA caches, only the rotation step
// changes).  Each layer has a K plane and a V plane of rows H x D bf16.
//
//  * gqa_splice_kernel: the splice's flat gather over all K and V planes (two
//    16-byte chunks per thread in K planes, one in V planes), turning the
//    RoPE band of every K head of
//    downstream rows by R(Delta), plus in-place band rotation of reused pages
//    and the page-table rewrites.
//  * plane_evict_kernel: the eviction's copy of kept rows into fresh pages
//    over all planes (no rotation), plus the page-table rewrites.
#include "device_common.h"

namespace ll {
namespace {

// The same flat gather on pools of K and V planes ("Leyline", section 5).  A
// K head's RoPE band spans 2^rot_shift chunks starting at a multiple of that
// count (rotary_dim is a power of two dividing head_dim), so a band never
// straddles a wave and the half-split partner of band chunk kc is lane
// xor (band chunks / 2).

// Turn a pair of band chunks of one K head with the directive's cos/sin table
// (in LDS or global memory): `xa` is band chunk w, `xb` band chunk w + half
// (w < half).  Interleaved pairs: chunk k holds pairs 4k..4k+3.  Half-split
// pairs: chunk w holds the x of pairs 8w..8w+7 and chunk w + half their y, so
// one thread holds both halves of its pairs and no lanes trade data.
template <int PAIRING, typename Tab>
__device__ __forceinline__ void rotate_pair(chunk_t& xa, chunk_t& xb, int w, int half, Tab cos_t, Tab sin_t) {
  if constexpr (PAIRING == 0) {
    float cs[4], sn[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cs[e] = cos_t[4 * w + e];
      sn[e] = sin_t[4 * w + e];
    }
    xa = rotate_interleaved(xa, cs, sn);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cs[e] = cos_t[4 * (w + half) + e];
      sn[e] = sin_t[4 * (w + half) + e];
    }
    xb = rotate_interleaved(xb, cs, sn);
  } else {
    float cs[8], sn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      cs[e] = cos_t[8 * w + e];
      sn[e] = sin_t[8 * w + e];
    }
    const chunk_t x = xa, y = xb;
    xa = rotate_half(x, y, true, cs, sn);
    xb = rotate_half(y, x, false, cs, sn);
  }
}

// In a K plane each thread moves one unit of two chunks of a row: unit w of
// head h is band chunks (w, w + half) for w < half, else two chunks of the
// head's non-band part, one from each of its halves, so each load instruction
// of a wave reads whole 128-byte runs.  In a V plane (a plain copy) each
// thread moves one chunk.
//
// Blocks [0, 3 L * move_blocks_per_plane) write the rows of fresh pages in
// groups of three: one block in a layer's K plane, then two in its V plane
// (a K block that turns first stages its table behind a barrier; the V blocks
// keep the memory streams busy meanwhile), the next L * rot_blocks_per_plane
// turn the RoPE bands of reused pages' downstream rows in place (K planes
// only; units (row, head, w < half)), and the remaining blocks rewrite
// page-table rows.
// WAVE_TASK: every wave lies inside one page task in every block range.
// BLOCK_TASK: so does every block; a K-plane block whose task turns then
// stages the directive's cos/sin table in LDS once.
template <int PAIRING, bool WAVE_TASK, bool BLOCK_TASK>
__global__ __launch_bounds__(kFlatThreads) void gqa_splice_kernel(GqaSpliceLaunch a) {
  __shared__ float tab[2 * kMaxBandPairs];
  const int64_t b = blockIdx.x;
  const int64_t move_blocks = 3 * a.move_blocks_per_plane * a.num_layers;
  const int64_t rot_blocks = a.rot_blocks_per_plane * a.num_layers;
  if (b >= move_blocks + rot_blocks) {
    table_write_block(a.twrites, a.tables, a.page_table, a.max_pages_per_seq, b - move_blocks - rot_blocks);
    return;
  }
  const bool in_place = b >= move_blocks;
  // move range: groups of three blocks, one of the layer's K plane and two
  // of its V plane (a V block covers half the chunks of a K block)
  bool v_move = false;
  int64_t bb = b - move_blocks;
  if (!in_place) {
    const int64_t grp = b / 3, m = b - grp * 3;
    v_move = m != 0;
    bb = v_move ? 2 * grp + m - 1 : grp;
  }
  const int64_t bpp = in_place ? a.rot_blocks_per_plane : (v_move ? 2 : 1) * a.move_blocks_per_plane;
  const int plane = static_cast<int>(bb / bpp) + (v_move ? a.num_layers : 0);
  const uint32_t u = static_cast<uint32_t>((bb - static_cast<int64_t>(bb / bpp) * bpp) * kFlatThreads + threadIdx.x);
  const int shift = a.page_shift;
  const uint32_t pmask = (1u << shift) - 1u;
  const uint32_t rc = static_cast<uint32_t>(a.row_chunks);
  const uint32_t hc = static_cast<uint32_t>(a.head_chunks);
  const int hs = a.rot_shift - 1;  // log2(half)
  const uint32_t band = 1u << a.rot_shift;
  const uint32_t half = band >> 1;
  const bool k_plane = plane < a.num_layers;

  uint32_t row_flat, col_a, col_b, w = 0;
  bool band_unit = false;
  if (in_place) {
    const uint32_t per_row = static_cast<uint32_t>(a.heads) << hs;
    row_flat = u / per_row;
    const uint32_t x = u - row_flat * per_row;
    w = x & (half - 1u);
    col_a = (x >> hs) * hc + w;
    col_b = col_a + half;
    band_unit = true;
  } else if (v_move) {
    row_flat = u / rc;
    col_a = u - row_flat * rc;
    col_b = col_a;
  } else {
    const uint32_t ru = rc >> 1;
    row_flat = u / ru;
    const uint32_t cu = u - row_flat * ru;
    {
      const uint32_t hu = hc >> 1;
      const uint32_t h = cu / hu;
      w = cu - h * hu;
      if (w < half) {
        col_a = h * hc + w;
        col_b = col_a + half;
        band_unit = true;
      } else {
        col_a = h * hc + band + (w - half);
        col_b = col_a + ((hc - band) >> 1);
      }
    }
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
  chunk_t va = chunk_t{0u, 0u, 0u, 0u}, vb = va;
  if (live) {
    va = __builtin_nontemporal_load(src + col_a);
    if (!v_move) vb = __builtin_nontemporal_load(src + col_b);
  }
  if (k_plane) {
    const bool on = live && rot && band_unit;
    if constexpr (BLOCK_TASK) {
      if (t.rotate) {  // the same task, hence the same answer, in the whole block
        const int pairs = static_cast<int>(band) * 4;
        for (int e = threadIdx.x; e < 2 * pairs; e += kFlatThreads)
          tab[e] = e < pairs ? dir->cos_[e] : dir->sin_[e - pairs];
        __syncthreads();
        if (on)
          rotate_pair<PAIRING>(va, vb, static_cast<int>(w), static_cast<int>(half), static_cast<const float*>(tab),
                               static_cast<const float*>(tab) + pairs);
      }
    } else if (on) {
      rotate_pair<PAIRING>(va, vb, static_cast<int>(w), static_cast<int>(half), static_cast<const float*>(dir->cos_),
                           static_cast<const float*>(dir->sin_));
    }
  }
  if (live) {
    chunk_t* dst = const_cast<chunk_t*>(layer) + dst_row * rc;
    __builtin_nontemporal_store(va, dst + col_a);
    if (!v_move) __builtin_nontemporal_store(vb, dst + col_b);
  }
}

// Eviction on K / V planes: flat copy of the kept rows that land in fresh
// pages, then the page-table rewrites.
template <bool WAVE_TASK>
__global__ __launch_bounds__(kEvictThreads) void plane_evict_kernel(PlaneEvictLaunch a) {
  const int64_t b = blockIdx.x;
  const int64_t bpp = a.blocks_per_plane;
  const int64_t move_blocks = bpp * a.num_planes;
  if (b >= move_blocks) {
    table_write_block(a.twrites, a.tables, a.page_table, a.max_pages_per_seq, b - move_blocks);
    return;
  }
  const int plane = static_cast<int>(b / bpp);
  const uint32_t c = static_cast<uint32_t>((b - static_cast<int64_t>(plane) * bpp) * kEvictThreads + threadIdx.x);
  const int shift = a.page_shift;
  const uint32_t rc = static_cast<uint32_t>(a.row_chunks);
  const uint32_t row_flat = c / rc;
  const uint32_t col = c - row_flat * rc;
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
  const chunk_t* layer = a.planes[plane];
  const chunk_t v = __builtin_nontemporal_load(layer + src_row * rc + col);
  if constexpr (WAVE_TASK) {  // the destination page is wave-uniform
    store_chunk_policy(v, layer + (static_cast<int64_t>(t.dst_page) << shift) * rc, (r * rc + col) * 16u,
                       (rc << shift) * 16u);
  } else {
    __builtin_nontemporal_store(v, const_cast<chunk_t*>(layer) + ((static_cast<int64_t>(t.dst_page) << shift) + r) * rc + col);
  }
}

}  // namespace

hipError_t launch_gqa_splice(const GqaSpliceLaunch& a, int pairing, hipStream_t s, const Stamp& t) {
  const int64_t grid = (3 * a.move_blocks_per_plane + a.rot_blocks_per_plane) * a.num_layers + a.n_twrites;
  if (grid == 0) return stamp_empty(s, t);
  const dim3 g(static_cast<unsigned>(grid)), blk(kFlatThreads);
  // one task per wave (per block) when a page's units are a whole number of
  // waves (blocks) in both the move and the in-place ranges (a V page's
  // chunks are twice a K page's units, so then they are too)
  const int64_t move_units = int64_t{a.row_chunks / 2} << a.page_shift;
  const int64_t band_units = (int64_t{a.heads} << (a.rot_shift - 1)) << a.page_shift;
  const bool wave_task = move_units % 64 == 0 && band_units % 64 == 0;
  const bool block_task = move_units % kFlatThreads == 0 && band_units % kFlatThreads == 0;
  void (*k)(GqaSpliceLaunch);
  if (pairing == 0)
    k = block_task ? gqa_splice_kernel<0, true, true>
        : wave_task ? gqa_splice_kernel<0, true, false> : gqa_splice_kernel<0, false, false>;
  else
    k = block_task ? gqa_splice_kernel<1, true, true>
        : wave_task ? gqa_splice_kernel<1, true, false> : gqa_splice_kernel<1, false, false>;
  return dispatch(k, g, blk, s, t, true, true, a);
}

hipError_t launch_plane_evict(const PlaneEvictLaunch& a, hipStream_t s, const Stamp& t) {
  const int64_t grid = a.blocks_per_plane * a.num_planes + a.n_twrites;
  if (grid == 0) return stamp_empty(s, t);
  void (*k)(PlaneEvictLaunch) =
      (int64_t{a.row_chunks} << a.page_shift) % 64 == 0 ? plane_evict_kernel<true> : plane_evict_kernel<false>;
  return dispatch(k, dim3(static_cast<unsigned>(grid)), dim3(kEvictThreads), s, t, true, true, a);
}

}  // namespace ll
