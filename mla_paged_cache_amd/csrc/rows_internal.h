// Internal types of the per-row-angle RoPE kernels (kernels_rows.hip) and
// their host side (pool.cpp).  Not part of the C ABI.
#pragma once

#include "leyline_internal.h"

namespace ll {

// Row shape shared by MLA rows and GQA / MHA K rows: `heads` heads of
// head_chunks chunks; each head's RoPE band is band_chunks chunks starting at
// chunk band_off of the head (MLA: one head of 72 chunks, band 64..71; GQA:
// band 0..rotary/8-1 of every head).
struct RowShape {
  int32_t row_chunks;
  int32_t heads;
  int32_t head_chunks;
  int32_t band_off;
  int32_t band_shift;   // log2(band_chunks)
  int32_t pairs;        // RoPE pairs per band = 4 * band_chunks
};

struct RopeTableLaunch {
  const int64_t* angle;   // [n] angle steps of each row
  const double* theta;    // [pairs] float64 theta_j
  float* tab;             // [n][2][pairs]: float32 cos, then sin
  int64_t n;
  int32_t pairs;
};

struct RopeRowsLaunch {
  const chunk_t* const* planes;  // device array: the planes that carry bands come first
  const int64_t* angle;          // [n] angle steps of each row (read by the in-place MLA kernel)
  const chunk_t* plane0;         // plane 0 (host copy of planes[0])
  int64_t plane_stride;          // chunks between consecutive planes when uniform, else 0
  int32_t num_planes;            // planes taking part (MLA: L; GQA: the L K planes)
  int32_t page_shift;
  RowShape shape;
  const int32_t* pages;          // physical pages of logical pages first_page ..
  int64_t row_begin;             // first logical row
  int64_t first_page;            // row_begin >> page_shift
  int64_t n;                     // rows
  const float* tab;              // [n][2][pairs]
  chunk_t* out;                  // gather target, or nullptr for in place
  int64_t out_plane_chunks;      // chunks between planes of out
  int64_t blocks_per_plane;
  int64_t n_pages;               // logical pages the rows touch (first_page ..)
};

// Layers whose loads rope_inplace_mla_kernel issues before their stores.
constexpr int kInPlaceLayerBatch = 9;

hipError_t launch_rope_table(const RopeTableLaunch& a, hipStream_t s, const Stamp& t = Stamp{});
// MLA rows in place (a.out == nullptr, MLA row shape): one kernel that also
// evaluates the rows' float64 cos/sin from theta (device [32] float64).
hipError_t launch_rope_inplace_mla(const RopeRowsLaunch& a, const double* theta, int pairing, hipStream_t s,
                                   const Stamp& t = Stamp{});
hipError_t launch_rope_rows(const RopeRowsLaunch& a, int pairing, hipStream_t s, const Stamp& t = Stamp{});
// Blocks per plane of the launch launch_rope_rows picks for `a` (all fields
// but blocks_per_plane set); per_row: threads per row of the row-unit kernel.
int64_t rope_rows_blocks_per_plane(const RopeRowsLaunch& a, int64_t per_row);

}  // namespace ll
