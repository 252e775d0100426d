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

}  // namespace

hipError_t launch_rope_table(const RopeTableLaunch& a, hipStream_t s, const Stamp& t) {
  const int64_t pairs = a.n * a.pairs;
  if (pairs == 0) return stamp_empty(s, t);
  return dispatch(rope_table_kernel, dim3(static_cast<unsigned>((pairs + 255) / 256)), dim3(256), s, t, true, true, a);
}

hipError_t launch_rope_rows(const RopeRowsLaunch& a, int pairing, hipStream_t s, const Stamp& t) {
  const int64_t grid = a.blocks_per_plane * a.num_planes;
  if (grid == 0) return stamp_empty(s, t);
  void (*k)(RopeRowsLaunch) = pairing == 0 ? rope_rows_kernel<0> : rope_rows_kernel<1>;
  return dispatch(k, dim3(static_cast<unsigned>(grid)), dim3(256), s, t, true, true, a);
}

}  // namespace ll
