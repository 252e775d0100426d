// Device helpers shared by the gfx950 row kernels (kernels.hip for MLA pools,
// kernels_gqa.hip for GQA / MHA pools): bf16 <-> float32, the float32
// delta-rotation of one RoPE pair ("Leyline: KV Cache Directives for Agentic
// Inference", section 2.2), the wave-uniform descriptor load and the
// page-table row rewrite.
#pragma once

#include <hip/hip_ext.h>

#include "leyline_internal.h"

namespace ll {
namespace {

// Launch `k` on `s`.  With events to stamp (the stamp's start if this is the
// launcher's first kernel, its stop if the last) the launch goes through the
// extended form, which takes them from this dispatch's own packet.
template <typename A>
hipError_t dispatch(void (*k)(A), dim3 g, dim3 b, hipStream_t s, const Stamp& t, bool first, bool last,
                    const A& a) {
  hipEvent_t start = first ? t.start : nullptr;
  hipEvent_t stop = last ? t.stop : nullptr;
  if (start || stop)
    hipExtLaunchKernelGGL(k, g, b, 0, s, start, stop, 0, a);
  else
    k<<<g, b, 0, s>>>(a);
  return hipGetLastError();
}

// A launcher with nothing to launch still leaves its events recorded.
inline hipError_t stamp_empty(hipStream_t s, const Stamp& t) {
  hipError_t e = hipSuccess;
  if (t.start) e = hipEventRecord(t.start, s);
  if (e == hipSuccess && t.stop) e = hipEventRecord(t.stop, s);
  return e;
}

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

// Cache policy of the row kernels' streamed stores: sc0 | nt | sc1 (gfx950
// bits 1, 2 and 16 of a buffer instruction's cache-policy operand).  A global
// store can carry only the nt bit; with all three, copies of the kind these
// kernels do measured 2-3% faster on MI355X (sc1 alone: slower).
constexpr int kStreamStore = 19;

// 16-byte store through a buffer descriptor based at `base`, `bytes` long,
// with cache policy AUX.  `base` must be wave-uniform (it is read from the
// first active lane); `byte_off` is the lane's offset from it.
template <int AUX = kStreamStore>
__device__ __forceinline__ void store_chunk_policy(chunk_t v, const chunk_t* base, uint32_t byte_off, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
  void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(ub, 0, static_cast<int>(bytes), 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(byte_off), 0, AUX);
}

}  // namespace
}  // namespace ll
