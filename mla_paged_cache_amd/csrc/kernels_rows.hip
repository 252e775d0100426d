// gfx950 kernels of the per-row-angle RoPE rotation: every row of a range of
// a sequence turns its RoPE bands by its own angle steps a_i, e.g. back by its
// position so that a static map can reconstruct V from the position-free key
// ("VECTOR", gist.science summary, method: keys are inverse-rotated before
// the OLS reconstruction).  The rotation of one pair is the same float32
// arithmetic as the splice's delta-rotation ("Leyline", section 2.2).
//
//  * rope_table_kernel: per row and pair, the float64 angle a_i * theta_j and
//    its float64 cos and sin (argument reduction in float64 on the device),
//    rounded to float32 -- computed once per call, read by every layer.
//  * rope_rows_kernel: the flat gather of the rows (gather mode: whole rows
//    to a dense buffer; in place: the bands only), two chunks per thread so a
//    thread holds both halves of its pairs in half-split layout.
//  * rope_gather_mla_kernel: the gather of MLA rows at page size >= 8, page
//    by page in the splice kernel's chunk order (copy waves and turn waves).
//  * rope_inplace_mla_kernel: MLA rows turned in place, each wave owning 8
//    rows over all layers and evaluating their cos/sin itself.
#include "device_common.h"
#include "rows_internal.h"

namespace ll {
namespace {

__global__ __launch_bounds__(256) void rope_table_kernel(RopeTableLaunch a) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= a.n * a.pairs) return;
  const int64_t i = t / a.pairs;
  const int j = static_cast<int>(t - i * a.pairs);
  const double ang = static_cast<double>(a.angle[i]) * a.theta[j];
  double s, c;
  sincos(ang, &s, &c);
  float* row = a.tab + i * 2 * a.pairs;
  row[j] = static_cast<float>(c);
  row[a.pairs + j] = static_cast<float>(s);
}

// Chunk of non-band index x (0 .. head_chunks - band_chunks - 1) of a head.
__device__ __forceinline__ uint32_t nonband_chunk(uint32_t x, uint32_t band_off, uint32_t band) {
  return x < band_off ? x : x + band;
}

// Thread = (plane, row, unit).  Gather: a row has row_chunks / 2 units; unit
// w of a head is band chunks (w, w + half) for w < half, else two non-band
// chunks, one from each half of the head's non-band part.  In place: a row
// has heads * half units, band pairs only.
template <int PAIRING>
__global__ __launch_bounds__(256) void rope_rows_kernel(RopeRowsLaunch a) {
  const int64_t b = blockIdx.x;
  const int plane = static_cast<int>(b / a.blocks_per_plane);
  const uint32_t u = static_cast<uint32_t>((b - static_cast<int64_t>(plane) * a.blocks_per_plane) * 256 + threadIdx.x);
  const RowShape sh = a.shape;
  const uint32_t band = 1u << sh.band_shift;
  const uint32_t half = band >> 1;
  const uint32_t hc = static_cast<uint32_t>(sh.head_chunks);
  const uint32_t boff = static_cast<uint32_t>(sh.band_off);
  const bool gather = a.out != nullptr;
  const uint32_t per_row = gather ? static_cast<uint32_t>(sh.row_chunks) >> 1 : static_cast<uint32_t>(sh.heads) * half;
  const uint32_t i = u / per_row;
  if (i >= a.n) return;
  const uint32_t x = u - i * per_row;
  uint32_t ca, cb, w = 0;
  bool band_unit;
  if (gather) {
    const uint32_t hu = hc >> 1;
    const uint32_t h = x / hu;
    w = x - h * hu;
    band_unit = w < half;
    if (band_unit) {
      ca = h * hc + boff + w;
      cb = ca + half;
    } else {
      const uint32_t v = w - half;
      const uint32_t nb2 = (hc - band) >> 1;
      ca = h * hc + nonband_chunk(v, boff, band);
      cb = h * hc + nonband_chunk(v + nb2, boff, band);
    }
  } else {
    const uint32_t h = x >> (sh.band_shift - 1);
    w = x & (half - 1u);
    ca = h * hc + boff + w;
    cb = ca + half;
    band_unit = true;
  }
  const int shift = a.page_shift;
  const int64_t j = a.row_begin + i;
  const int64_t phys = (static_cast<int64_t>(a.pages[(j >> shift) - a.first_page]) << shift) + (j & ((int64_t{1} << shift) - 1));
  const uint32_t rc = static_cast<uint32_t>(sh.row_chunks);
  chunk_t* src = const_cast<chunk_t*>(a.planes[plane]) + phys * rc;
  chunk_t va = __builtin_nontemporal_load(src + ca);
  chunk_t vb = __builtin_nontemporal_load(src + cb);
  if (band_unit) {
    const float* cs = a.tab + static_cast<int64_t>(i) * 2 * sh.pairs;
    const float* sn = cs + sh.pairs;
    if constexpr (PAIRING == 0) {
      float c4[4], s4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c4[e] = cs[4 * w + e];
        s4[e] = sn[4 * w + e];
      }
      va = rotate_interleaved(va, c4, s4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c4[e] = cs[4 * (w + half) + e];
        s4[e] = sn[4 * (w + half) + e];
      }
      vb = rotate_interleaved(vb, c4, s4);
    } else {
      float c8[8], s8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        c8[e] = cs[8 * w + e];
        s8[e] = sn[8 * w + e];
      }
      const chunk_t xv = va, yv = vb;
      va = rotate_half(xv, yv, true, c8, s8);
      vb = rotate_half(yv, xv, false, c8, s8);
    }
  }
  chunk_t* dst = gather ? a.out + plane * a.out_plane_chunks + static_cast<int64_t>(i) * rc : src;
  __builtin_nontemporal_store(va, dst + ca);
  __builtin_nontemporal_store(vb, dst + cb);
}

// MLA rows gathered page by page.  Within one logical page of P rows the 64
// c_kv chunks of every row come first, then the 8 k_pe chunks of every row,
// so that (P >= 8) every wave either only copies (one row's c_kv, 1 KiB
// contiguous per load instruction) or only turns k_pe chunks; a turning lane
// reads its row's float32 table.  Two chunks per thread, 256 apart, both loads
// issued before either store.  The page of a wave is one scalar load.
template <int PAIRING>
__global__ __launch_bounds__(256) void rope_gather_mla_kernel(RopeRowsLaunch a) {
  constexpr int CPT = 2;
  constexpr uint32_t kRow = kRowChunks;                 // 72
  constexpr uint32_t kKpe = kRowChunks - kKpeChunk0;   // 8
  const int64_t b = blockIdx.x;
  const int plane = static_cast<int>(b / a.blocks_per_plane);
  const uint32_t c0 = static_cast<uint32_t>((b - static_cast<int64_t>(plane) * a.blocks_per_plane) * 256 * CPT +
                                            threadIdx.x);
  const int shift = a.page_shift;
  const int64_t row_end = a.row_begin + a.n;
  const chunk_t* layer = a.planes[plane];
  chunk_t* out = a.out + plane * a.out_plane_chunks;
  chunk_t v[CPT];
  const chunk_t* srcs[CPT];
  int64_t dsts[CPT];
  bool lives[CPT];
  int kcs[CPT];
  int64_t tabs[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const uint32_t c = c0 + u * 256;
    // wave-uniform: a page is 72 P chunks, a multiple of 64
    const uint32_t task = __builtin_amdgcn_readfirstlane((c / kRow) >> shift);
    const uint32_t lc = c - task * (kRow << shift);
    uint32_t r, col;
    if (lc < (static_cast<uint32_t>(kKpeChunk0) << shift)) {
      r = lc / kKpeChunk0;
      col = lc - r * kKpeChunk0;
    } else {
      const uint32_t k = lc - (static_cast<uint32_t>(kKpeChunk0) << shift);
      r = k / kKpe;
      col = kKpeChunk0 + (k - r * kKpe);
    }
    const bool in_range = task < a.n_pages;
    using cptr = const __attribute__((address_space(4))) int32_t*;
    // n_pages >= 1; past the last page the lanes are dead and read page 0's entry
    const int32_t page = *reinterpret_cast<cptr>(reinterpret_cast<uintptr_t>(a.pages + (in_range ? task : 0)));
    const int64_t j = ((a.first_page + task) << shift) + r;
    lives[u] = in_range && j >= a.row_begin && j < row_end;
    srcs[u] = layer + ((static_cast<int64_t>(page) << shift) + r) * kRow + col;
    const int64_t i = j - a.row_begin;
    dsts[u] = i * kRow + col;
    kcs[u] = static_cast<int>(col) - kKpeChunk0;
    tabs[u] = i * 2 * kHalfPairs;
  }
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    v[u] = chunk_t{0u, 0u, 0u, 0u};
    if (lives[u]) v[u] = __builtin_nontemporal_load(srcs[u]);
  }
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    if (kcs[u] >= 0) {  // a turn wave: every lane takes part (half-split lanes trade chunks)
      const int kc = kcs[u];
      const float* cs = a.tab + (lives[u] ? tabs[u] : 0);
      const float* sn = cs + kHalfPairs;
      if constexpr (PAIRING == 0) {
        if (lives[u]) {
          float c4[4], s4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            c4[e] = cs[4 * kc + e];
            s4[e] = sn[4 * kc + e];
          }
          v[u] = rotate_interleaved(v[u], c4, s4);
        }
      } else {
        const chunk_t other = shfl_xor4(v[u]);
        if (lives[u]) {
          float c8[8], s8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            c8[e] = cs[8 * (kc & 3) + e];
            s8[e] = sn[8 * (kc & 3) + e];
          }
          v[u] = rotate_half(v[u], other, kc < 4, c8, s8);
        }
      }
    }
    if (lives[u]) __builtin_nontemporal_store(v[u], out + dsts[u]);
  }
}

// MLA rows turned in place, the float64 cos/sin computed here (no table
// kernel).  A wave owns 8 rows (lane = 8 * row + band chunk: each load
// instruction reads the 128-byte k_pe line of 8 rows) over every layer, in
// batches of kInPlaceLayerBatch layers whose loads are all issued before their
// stores; the pairs' float64 cos and sin (the same device sincos as
// rope_table_kernel, so the same float32 values) are evaluated while the
// first batch is in flight.  Plain loads and stores: for these lines, 1152
// bytes apart, that measured best.  STRIDE: the layers are one allocation,
// layer l at plane0 + l * plane_stride (no per-layer pointer load before a
// band load: 55 us against 58 us for the 32k x 27 rows).
template <int PAIRING, bool STRIDE>
__global__ __launch_bounds__(256) void rope_inplace_mla_kernel(RopeRowsLaunch a, const double* theta) {
  constexpr int LB = kInPlaceLayerBatch;
  constexpr int NP = PAIRING == 0 ? 4 : 8;  // pairs a lane turns
  const int lane = threadIdx.x & 63;
  const int kc = lane & 7;
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * 8 + (lane >> 3);
  const bool live = i < a.n;
  const int shift = a.page_shift;
  const int L = a.num_planes;
  // pair p0 + e, e < NP: interleaved chunk kc holds pairs 4 kc .. 4 kc + 3;
  // half-split chunks kc and kc ^ 4 hold x and y of pairs 8 (kc & 3) ..
  const int p0 = PAIRING == 0 ? 4 * kc : 8 * (kc & 3);
  // The angle and theta loads go first, then the first batch's plane
  // pointers and band loads (a lane past the rows reads row row_begin, in
  // bounds): the sincos below then waits only for its own inputs, and no
  // branch separates the band loads.
  const double ang = static_cast<double>(a.angle[live ? i : 0]);
  double th[NP];
#pragma unroll
  for (int e = 0; e < NP; ++e) th[e] = theta[p0 + e];
  const int64_t j = a.row_begin + (live ? i : 0);
  const int64_t phys = (static_cast<int64_t>(a.pages[(j >> shift) - a.first_page]) << shift) +
                       (j & ((int64_t{1} << shift) - 1));
  const int64_t off = phys * kRowChunks + kKpeChunk0 + kc;
  // band chunk of layer l (a lane past the rows reads row row_begin's)
  auto band = [&](int l) -> chunk_t* {
    if constexpr (STRIDE)
      return const_cast<chunk_t*>(a.plane0) + l * a.plane_stride + off;
    else
      return const_cast<chunk_t*>(a.planes[l]) + off;
  };
  chunk_t v[LB];
#pragma unroll
  for (int k = 0; k < LB; ++k) v[k] = *band(k < L ? k : L - 1);
  float c[NP], sn[NP];
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    double sd, cd;
    sincos(ang * th[e], &sd, &cd);
    c[e] = static_cast<float>(cd);
    sn[e] = static_cast<float>(sd);
  }
  for (int l0 = 0; l0 < L; l0 += LB) {
#pragma unroll
    for (int k = 0; k < LB; ++k) {
      chunk_t r;
      if constexpr (PAIRING == 0) {
        r = rotate_interleaved(v[k], c, sn);
      } else {
        const chunk_t other = shfl_xor4(v[k]);
        r = rotate_half(v[k], other, kc < 4, c, sn);
      }
      if (live && l0 + k < L) *band(l0 + k) = r;
    }
    if (l0 + LB < L) {
#pragma unroll
      for (int k = 0; k < LB; ++k) {
        const int l = l0 + LB + k;
        v[k] = *band(l < L ? l : L - 1);
      }
    }
  }
}

}  // namespace

hipError_t launch_rope_inplace_mla(const RopeRowsLaunch& a, const double* theta, int pairing, hipStream_t s,
                                   const Stamp& t) {
  const int64_t waves = (a.n + 7) / 8;
  if (waves == 0 || a.num_planes == 0) return stamp_empty(s, t);
  void (*k)(RopeRowsLaunch, const double*);
  if (a.plane_stride != 0)
    k = pairing == 0 ? rope_inplace_mla_kernel<0, true> : rope_inplace_mla_kernel<1, true>;
  else
    k = pairing == 0 ? rope_inplace_mla_kernel<0, false> : rope_inplace_mla_kernel<1, false>;
  const dim3 g(static_cast<unsigned>((waves + 3) / 4)), b(256);
  hipEvent_t start = t.start, stop = t.stop;
  if (start || stop)
    hipExtLaunchKernelGGL(k, g, b, 0, s, start, stop, 0, a, theta);
  else
    k<<<g, b, 0, s>>>(a, theta);
  return hipGetLastError();
}

hipError_t launch_rope_table(const RopeTableLaunch& a, hipStream_t s, const Stamp& t) {
  const int64_t pairs = a.n * a.pairs;
  if (pairs == 0) return stamp_empty(s, t);
  return dispatch(rope_table_kernel, dim3(static_cast<unsigned>((pairs + 255) / 256)), dim3(256), s, t, true, true, a);
}

bool rope_gather_by_page(const RopeRowsLaunch& a) {
  const RowShape& sh = a.shape;
  return a.out != nullptr && a.page_shift >= 3 && sh.heads == 1 && sh.row_chunks == kRowChunks &&
         sh.band_off == kKpeChunk0 && (1 << sh.band_shift) == kRowChunks - kKpeChunk0;
}

int64_t rope_rows_blocks_per_plane(const RopeRowsLaunch& a, int64_t per_row) {
  if (rope_gather_by_page(a)) return flat_blocks(a.n_pages * (int64_t{kRowChunks} << a.page_shift), 2);
  return flat_blocks(a.n * per_row);
}

hipError_t launch_rope_rows(const RopeRowsLaunch& a, int pairing, hipStream_t s, const Stamp& t) {
  const int64_t grid = a.blocks_per_plane * a.num_planes;
  if (grid == 0) return stamp_empty(s, t);
  void (*k)(RopeRowsLaunch);
  if (rope_gather_by_page(a))
    k = pairing == 0 ? rope_gather_mla_kernel<0> : rope_gather_mla_kernel<1>;
  else
    k = pairing == 0 ? rope_rows_kernel<0> : rope_rows_kernel<1>;
  return dispatch(k, dim3(static_cast<unsigned>(grid)), dim3(256), s, t, true, true, a);
}

}  // namespace ll
