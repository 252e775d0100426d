// gfx950 kernels of the eviction's device-side page allocator: the same
// lowest-free-first page plan the host makes, computed on the device so that
// kv_evict_compact never waits for the keep scan ("KV-streams", "how it
// works": evicted entries are reclaimed inside the engine, kept entries are
// left as they were).
//
//  * fresh_rank_kernel: per sequence, a block scan over its new pages numbers
//    the ones that cannot reuse an old page (fresh pages).
//  * alloc_scan_kernel: one block; exclusive scans of the fresh counts over
//    the batch and of the free bitmap's word popcounts; the verdict (fresh
//    pages, or "short of pages").
//  * alloc_tables_kernel: per new page, its physical page: the reused old page,
//    or fresh page f = the f-th lowest free page (binary search over the word
//    prefix, then the bit inside the word); fresh pages also get a move task.
//  * table_copy_kernel: the new page-table rows, written after every read of
//    the old ones.
// The row moves into fresh pages are evict_move_kernel (kernels.hip) or
// plane_evict_kernel (kernels_gqa.hip), launched by the host on the exact
// grid once it has read the verdict.
#include "alloc_internal.h"
#include "device_common.h"

namespace ll {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kScanWaves = kScanThreads / 64;

// Exclusive scan of one int per thread across a 1024-thread block; *total gets
// the block's sum.  Uses `lds` (kScanWaves ints); all threads must call it.
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds[wave] = x;
  __syncthreads();
  int before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kScanWaves; ++w) {
    const int t = lds[w];
    before += w < wave ? t : 0;
    sum += t;
  }
  __syncthreads();  // lds is reused by the next call
  *total = sum;
  return before + x - v;
}

__global__ __launch_bounds__(kScanThreads) void fresh_rank_kernel(AllocLaunch a) {
  __shared__ int lds[kScanWaves];
  const EvictSeq e = a.seqs[blockIdx.x];
  const int64_t P = int64_t{1} << a.page_shift;
  const int64_t n_new = a.counts[blockIdx.x];
  const int64_t pages = (n_new + P - 1) >> a.page_shift;
  int carry = 0, moved = 0;
  for (int64_t base = 0; base < pages; base += kScanThreads) {
    const int64_t q = base + threadIdx.x;
    const bool fresh = q < pages && a.reuse[e.reuse_off + q] < 0;
    const int64_t live = fresh ? n_new - (q << a.page_shift) : 0;
    int total, rows_total;
    const int r = block_exclusive_scan(fresh ? 1 : 0, lds, &total);
    (void)block_exclusive_scan(static_cast<int>(live < P ? live : P), lds, &rows_total);
    if (q < pages) a.rank[e.reuse_off + q] = carry + r;
    carry += total;
    moved += rows_total;
  }
  if (threadIdx.x == 0) {
    a.fresh_count[blockIdx.x] = carry;
    a.moved_count[blockIdx.x] = moved;
  }
}

// info[2..3]: the rows written to fresh pages, as one 64-bit count.
__device__ __forceinline__ unsigned long long* moved_rows(const AllocLaunch& a) {
  return reinterpret_cast<unsigned long long*>(a.info + 2);
}

__global__ __launch_bounds__(kScanThreads) void alloc_scan_kernel(AllocLaunch a) {
  __shared__ int lds[kScanWaves];
  int carry = 0;
  for (int base = 0; base < a.n; base += kScanThreads) {
    const int i = base + threadIdx.x;
    const int v = i < a.n ? a.fresh_count[i] : 0;
    int total;
    const int r = block_exclusive_scan(v, lds, &total);
    if (i < a.n) a.fresh_base[i] = carry + r;
    carry += total;
  }
  const int fresh = carry;
  // rows written to fresh pages, over the batch (64-bit)
  unsigned long long moved = 0;
  for (int i = threadIdx.x; i < a.n; i += kScanThreads) moved += static_cast<unsigned long long>(a.moved_count[i]);
  for (int o = 32; o > 0; o >>= 1) moved += __shfl_down(moved, o);
  __shared__ unsigned long long wave_moved[kScanWaves];
  if ((threadIdx.x & 63) == 0) wave_moved[threadIdx.x >> 6] = moved;
  __syncthreads();
  carry = 0;
  for (int base = 0; base < a.n_words; base += kScanThreads) {
    const int w = base + threadIdx.x;
    const int v = w < a.n_words ? __popcll(a.free_words[w]) : 0;
    int total;
    const int r = block_exclusive_scan(v, lds, &total);
    if (w < a.n_words) a.word_base[w] = carry + r;
    carry += total;
  }
  if (threadIdx.x == 0) {
    const bool short_of_pages = fresh > carry;
    a.info[0] = short_of_pages ? 0 : fresh;
    a.info[1] = short_of_pages ? 1 : 0;
    unsigned long long sum = 0;
    for (int w = 0; w < kScanWaves; ++w) sum += wave_moved[w];
    *moved_rows(a) = short_of_pages ? 0ull : sum;
  }
}

// The f-th (0-based) lowest free page: the last word whose prefix is <= f,
// then the (f - prefix)-th set bit of that word.
__device__ __forceinline__ int32_t select_free(const AllocLaunch& a, int32_t f) {
  int lo = 0, hi = a.n_words - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.word_base[mid] <= f) lo = mid;
    else hi = mid - 1;
  }
  uint64_t w = a.free_words[lo];
  for (int k = f - a.word_base[lo]; k > 0; --k) w &= w - 1;
  return static_cast<int32_t>(lo * 64 + __builtin_ctzll(w));
}

__global__ __launch_bounds__(256) void alloc_tables_kernel(AllocLaunch a) {
  if (a.info[1]) return;  // not enough free pages: nothing changes
  const EvictSeq e = a.seqs[blockIdx.x];
  const int64_t P = int64_t{1} << a.page_shift;
  const int64_t n_new = a.counts[blockIdx.x];
  const int64_t pages = (n_new + P - 1) >> a.page_shift;
  const int32_t* old_t = a.page_table + static_cast<int64_t>(e.seq) * a.max_pages_per_seq;
  const int32_t base = a.fresh_base[blockIdx.x];
  for (int64_t q = threadIdx.x; q < pages; q += 256) {
    const int32_t r = a.reuse[e.reuse_off + q];
    int32_t page;
    if (r >= 0) {
      page = old_t[r];
    } else {
      const int32_t f = base + a.rank[e.reuse_off + q];
      page = select_free(a, f);
      // src_rows entries of one call number less than the pool's rows (< 2^31)
      const int64_t j0 = q << a.page_shift;
      const int64_t k = n_new - j0 < P ? n_new - j0 : P;
      EvictTask t{};
      t.dst_page = page;
      t.rows = static_cast<int16_t>(k);
      t.src_off0 = -1;
      t.src0 = static_cast<int32_t>(e.src_off + j0);
      t.src1 = -1;
      if (a.src_logical) {
        // live rows that are consecutive old rows lie in at most two old
        // pages: the row kernel then needs no per-row source lookup
        const int32_t first = a.src_logical[e.src_off + j0];
        const int32_t last = a.src_logical[e.src_off + j0 + k - 1];
        if (last - first == k - 1) {
          const int32_t off = first & static_cast<int32_t>(P - 1);
          t.src0 = old_t[first >> a.page_shift];
          t.src1 = off + k > P ? old_t[(first >> a.page_shift) + 1] : -1;
          t.src_off0 = static_cast<int16_t>(off);
        }
      }
      a.tasks[f] = t;
    }
    a.new_table[e.reuse_off + q] = page;
  }
}

__global__ __launch_bounds__(256) void zero_words_kernel(unsigned long long* w, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256)
    w[i] = 0ull;
}

__global__ __launch_bounds__(256) void table_copy_kernel(AllocLaunch a) {
  if (a.info[1]) return;
  const EvictSeq e = a.seqs[blockIdx.x];
  const int64_t P = int64_t{1} << a.page_shift;
  const int64_t pages = (a.counts[blockIdx.x] + P - 1) >> a.page_shift;
  int32_t* t = const_cast<int32_t*>(a.page_table) + static_cast<int64_t>(e.seq) * a.max_pages_per_seq;
  for (int64_t q = threadIdx.x; q < pages; q += 256) t[q] = a.new_table[e.reuse_off + q];
}

}  // namespace

hipError_t launch_alloc_scan(const AllocLaunch& a, hipStream_t s, const Stamp& t) {
  hipError_t e = dispatch(fresh_rank_kernel, dim3(a.n), dim3(kScanThreads), s, t, true, false, a);
  if (e != hipSuccess) return e;
  return dispatch(alloc_scan_kernel, dim3(1), dim3(kScanThreads), s, t, false, true, a);
}

hipError_t launch_alloc_tables(const AllocLaunch& a, hipStream_t s, const Stamp& t) {
  hipError_t e = dispatch(alloc_tables_kernel, dim3(a.n), dim3(256), s, t, true, false, a);
  if (e != hipSuccess) return e;
  return dispatch(table_copy_kernel, dim3(a.n), dim3(256), s, t, false, true, a);
}

hipError_t launch_zero_words(unsigned long long* w, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  zero_words_kernel<<<dim3(static_cast<unsigned>(blocks < 1024 ? blocks : 1024)), dim3(256), 0, s>>>(w, n);
  return hipGetLastError();
}

}  // namespace ll
