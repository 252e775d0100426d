// gfx950 kernels of the splice / evict path on a paged MLA cache.
//
//  * splice_kernel: writes the rows of fresh destination pages (prefix rows of
//    a boundary page, the stub rows R, and downstream rows moved by Delta with
//    their k_pe turned by R(Delta)), rotates the k_pe band of reused
//    downstream pages in place, and rewrites the page-table rows -- one
//    launch ("Leyline: KV Cache Directives for Agentic Inference", sections
//    2.1-2.3).
//  * keep_scan_kernel: per-sequence exclusive prefix sum of a keep mask built
//    from wave64 ballots, giving each kept row its new index, plus the
//    per-new-page reuse test ("KV-streams", "how it works").
//  * evict_move_kernel: copies kept rows into fresh pages, no rotation.
//  * table_write_kernel: page-table row rewrites.
//
// The row kernels are bound by HBM bandwidth (0.08 flop per byte), so they
// are plain 16-byte vector copies: a block is 8 rows x 72 chunks = 576
// threads, each thread owns one 16-byte column for the whole launch, loads of
// all the layers it carries are issued before any store, and only the 8 k_pe
// columns do arithmetic.
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

// PAIRING: 0 interleaved, 1 half-split.
template <int LPB, int PAIRING>
__global__ __launch_bounds__(kMoveThreads) void splice_kernel(SpliceLaunch a) {
  const int64_t b = blockIdx.x;
  if (b >= a.n_move_blocks) {
    table_write_block(a.twrites, a.tables, a.page_table, a.max_pages_per_seq, b - a.n_move_blocks);
    return;
  }
  const int64_t lg = b / a.n_slabs;
  const int64_t slab = b - lg * a.n_slabs;
  const int tid = threadIdx.x;
  const int srow = tid / kRowChunks;
  const int col = tid - srow * kRowChunks;
  const int shift = a.page_shift;
  const int64_t pmask = (int64_t{1} << shift) - 1;

  // Row `flat` of the task list: task flat >> shift, row flat & pmask.  For
  // page sizes >= 8 a slab lies inside one task, so `t` is block-uniform.
  const int64_t flat = slab * kSlabRows + srow;
  const int64_t ti = flat >> shift;
  const bool in_range = ti < a.n_tasks;
  const SpliceTask t = a.tasks[in_range ? ti : 0];
  const SpliceDir& d = a.dirs[t.dir];
  const int64_t r = flat & pmask;
  const int64_t j = (static_cast<int64_t>(t.q) << shift) + r;
  const bool live = in_range && j < d.n_new;
  const bool kpe = col >= kKpeChunk0;

  bool active = live;
  bool from_stub = false;
  bool rot = false;
  int64_t src_row = 0;
  if (t.kind == kRotateInPlace) {
    active = live && kpe;
    src_row = (static_cast<int64_t>(t.dst_page) << shift) + r;
    rot = true;
  } else if (j < d.s_start) {
    src_row = (static_cast<int64_t>(t.pre_page) << shift) + (j & pmask);
  } else if (j < d.s_start + d.r_len) {
    from_stub = true;
    src_row = j - d.s_start;
  } else {
    const int64_t o = j - d.delta;
    const int32_t pg = ((o >> shift) == t.down_lp0) ? t.down_page0 : t.down_page1;
    src_row = (static_cast<int64_t>(pg) << shift) + (o & pmask);
    rot = d.rotate != 0;
  }
  const int64_t src_chunk = src_row * kRowChunks + col;
  const int64_t dst_chunk = ((static_cast<int64_t>(t.dst_page) << shift) + r) * kRowChunks + col;

  constexpr int NC = PAIRING == 0 ? 4 : 8;
  float cs[NC], sn[NC];
  const int k = col - kKpeChunk0;
  if (kpe) {
    const int j0 = PAIRING == 0 ? 4 * k : 8 * (k & 3);
#pragma unroll
    for (int e = 0; e < NC; ++e) {
      cs[e] = d.cos_[j0 + e];
      sn[e] = d.sin_[j0 + e];
    }
  }

  const int l0 = static_cast<int>(lg) * LPB;
  chunk_t v[LPB];
#pragma unroll
  for (int i = 0; i < LPB; ++i) {
    const int l = l0 + i;
    v[i] = chunk_t{0u, 0u, 0u, 0u};
    if (active && l < a.num_layers) {
      const chunk_t* base = from_stub ? d.stub + l * d.stub_layer_chunks : a.layers[l];
      v[i] = __builtin_nontemporal_load(base + src_chunk);
    }
  }
  const bool do_rot = active && rot && kpe;
#pragma unroll
  for (int i = 0; i < LPB; ++i) {
    if (PAIRING == 0) {
      if (do_rot) v[i] = rotate_interleaved(v[i], cs, sn);
    } else {
      // every lane takes part in the exchange; the partner of a k_pe lane is
      // the k_pe lane 4 columns away in the same row (same wave, same flags)
      const chunk_t other = shfl_xor4(v[i]);
      if (do_rot) v[i] = rotate_half(v[i], other, k < 4, cs, sn);
    }
  }
#pragma unroll
  for (int i = 0; i < LPB; ++i) {
    const int l = l0 + i;
    if (active && l < a.num_layers) {
      chunk_t* base = const_cast<chunk_t*>(a.layers[l]);
      __builtin_nontemporal_store(v[i], base + dst_chunk);
    }
  }
}

template <int LPB>
__global__ __launch_bounds__(kMoveThreads) void evict_move_kernel(EvictLaunch a) {
  const int64_t b = blockIdx.x;
  const int64_t lg = b / a.n_slabs;
  const int64_t slab = b - lg * a.n_slabs;
  const int tid = threadIdx.x;
  const int srow = tid / kRowChunks;
  const int col = tid - srow * kRowChunks;
  const int shift = a.page_shift;
  const int64_t pmask = (int64_t{1} << shift) - 1;
  const int64_t flat = slab * kSlabRows + srow;
  const int64_t ti = flat >> shift;
  const bool in_range = ti < a.n_tasks;
  const EvictTask t = a.tasks[in_range ? ti : 0];
  const int64_t r = flat & pmask;
  const int64_t j = (static_cast<int64_t>(t.q) << shift) + r;
  const bool live = in_range && j < t.n_new;
  int64_t src_row = 0;
  if (live) {
    const int64_t o = a.src_of_dst[t.src_off + j];
    const int32_t pg = a.page_table[static_cast<int64_t>(t.seq) * a.max_pages_per_seq + (o >> shift)];
    src_row = (static_cast<int64_t>(pg) << shift) + (o & pmask);
  }
  const int64_t src_chunk = src_row * kRowChunks + col;
  const int64_t dst_chunk = ((static_cast<int64_t>(t.dst_page) << shift) + r) * kRowChunks + col;
  const int l0 = static_cast<int>(lg) * LPB;
  chunk_t v[LPB];
#pragma unroll
  for (int i = 0; i < LPB; ++i) {
    const int l = l0 + i;
    v[i] = chunk_t{0u, 0u, 0u, 0u};
    if (live && l < a.num_layers) v[i] = __builtin_nontemporal_load(a.layers[l] + src_chunk);
  }
#pragma unroll
  for (int i = 0; i < LPB; ++i) {
    const int l = l0 + i;
    if (live && l < a.num_layers) {
      chunk_t* base = const_cast<chunk_t*>(a.layers[l]);
      __builtin_nontemporal_store(v[i], base + dst_chunk);
    }
  }
}

__global__ __launch_bounds__(256) void table_write_kernel(TableLaunch a) {
  table_write_block(a.twrites, a.tables, a.page_table, a.max_pages_per_seq, blockIdx.x);
}

constexpr int kScanThreads = 1024;
constexpr int kScanWaves = kScanThreads / 64;

// One block per sequence.  Each thread takes 16 mask bytes per tile; the
// count of kept bytes (0..16) is scanned across the wave with one ballot per
// bit of the count, then across the 16 waves through LDS.
__global__ __launch_bounds__(kScanThreads) void keep_scan_kernel(ScanLaunch a) {
  __shared__ int32_t wave_total[kScanWaves];
  const EvictSeq e = a.seqs[blockIdx.x];
  const uint8_t* m = a.keep + e.mask_off;
  int32_t* out = a.src_of_dst + e.src_off;
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
      if ((bits >> c) & 1u) out[pos++] = static_cast<int32_t>(i0 + c);
    carry += block_total;
    __syncthreads();
  }
  // Per new page: reusable iff its live rows are old rows f .. f+k-1 with f
  // on a page boundary (so one old page, same offsets).
  const int shift = a.page_shift;
  const int64_t P = int64_t{1} << shift;
  const int64_t n_new = carry;
  const int64_t pages = (n_new + P - 1) >> shift;
  int32_t* reuse = a.reuse + e.reuse_off;
  for (int64_t q = threadIdx.x; q < pages; q += kScanThreads) {
    const int64_t k = (n_new - (q << shift)) < P ? (n_new - (q << shift)) : P;
    const int64_t f = out[q << shift];
    const int64_t l = out[(q << shift) + k - 1];
    reuse[q] = ((f & (P - 1)) == 0 && l - f == k - 1) ? static_cast<int32_t>(f >> shift) : -1;
  }
  if (threadIdx.x == 0) a.counts[blockIdx.x] = n_new;
}

template <int LPB>
hipError_t launch_splice_lpb(const SpliceLaunch& a, int pairing, hipStream_t s) {
  const int64_t grid = a.n_move_blocks + a.n_twrites;
  if (grid == 0) return hipSuccess;
  if (pairing == 0)
    splice_kernel<LPB, 0><<<dim3(static_cast<unsigned>(grid)), dim3(kMoveThreads), 0, s>>>(a);
  else
    splice_kernel<LPB, 1><<<dim3(static_cast<unsigned>(grid)), dim3(kMoveThreads), 0, s>>>(a);
  return hipGetLastError();
}

template <int LPB>
hipError_t launch_evict_lpb(const EvictLaunch& a, hipStream_t s) {
  if (a.n_move_blocks == 0) return hipSuccess;
  evict_move_kernel<LPB><<<dim3(static_cast<unsigned>(a.n_move_blocks)), dim3(kMoveThreads), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

int64_t layer_groups(int num_layers, int layers_per_block) {
  return (num_layers + layers_per_block - 1) / layers_per_block;
}

hipError_t launch_splice(const SpliceLaunch& a, int layers_per_block, int pairing, hipStream_t s) {
  switch (layers_per_block) {
    case 1: return launch_splice_lpb<1>(a, pairing, s);
    case 2: return launch_splice_lpb<2>(a, pairing, s);
    case 3: return launch_splice_lpb<3>(a, pairing, s);
    case 4: return launch_splice_lpb<4>(a, pairing, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_evict_move(const EvictLaunch& a, int layers_per_block, hipStream_t s) {
  switch (layers_per_block) {
    case 1: return launch_evict_lpb<1>(a, s);
    case 2: return launch_evict_lpb<2>(a, s);
    case 3: return launch_evict_lpb<3>(a, s);
    case 4: return launch_evict_lpb<4>(a, s);
    default: return hipErrorInvalidValue;
  }
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
