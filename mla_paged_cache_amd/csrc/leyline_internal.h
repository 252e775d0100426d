// Internal types shared by the host planner (pool.cpp) and the gfx950 kernels
// (kernels.hip).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ll {

// 16 bytes of a row, as one native vector so loads and stores are dwordx4.
typedef uint32_t chunk_t __attribute__((ext_vector_type(4)));

// One MLA cache row: c_kv (512 bf16) then k_pe (64 bf16) = 1152 bytes
// = 72 chunks of 16 bytes; k_pe is chunks 64..71.
constexpr int kKvLoraRank = 512;
constexpr int kRopeDim = 64;
constexpr int kRowElems = kKvLoraRank + kRopeDim;
constexpr int kRowBytes = kRowElems * 2;
constexpr int kRowChunks = kRowBytes / 16;
constexpr int kKpeChunk0 = kKvLoraRank * 2 / 16;
constexpr int kHalfPairs = kRopeDim / 2;

// The row-moving kernel works on slabs of 8 rows: 8 * 72 = 576 threads, so
// every thread keeps one 16-byte column of the row for the whole launch.
constexpr int kSlabRows = 8;
constexpr int kMoveThreads = kSlabRows * kRowChunks;

enum TaskKind : int32_t {
  kMoveRows = 0,        // fresh page: write every live row
  kRotateInPlace = 1,   // reused page: rotate the k_pe band of its live rows
};

// One splice directive as the kernel sees it.
struct alignas(16) SpliceDir {
  const chunk_t* stub;           // R rows of layer 0, in 16-byte chunks
  int64_t stub_layer_chunks;   // chunks between layers of R
  int64_t s_start;
  int64_t r_len;
  int64_t delta;
  int64_t n_new;
  int32_t rotate;              // 1 when downstream k_pe turns (AMORTIZE, delta != 0)
  int32_t pad0;
  int64_t pad1;
  float cos_[kHalfPairs];      // float32 of float64 cos(delta * theta_j)
  float sin_[kHalfPairs];
};

// One destination page of a splice.  Sources are given as physical pages so
// the kernel never reads the page table it rewrites.
struct alignas(16) SpliceTask {
  int32_t dir;         // index into the SpliceDir array
  int32_t q;           // new logical page
  int32_t dst_page;    // physical page written
  int32_t kind;        // TaskKind
  int32_t pre_page;    // physical page of old logical page q (prefix rows), or -1
  int32_t down_lp0;    // first old logical page feeding downstream rows
  int32_t down_page0;  // its physical page
  int32_t down_page1;  // physical page of down_lp0 + 1, or -1
};

// One page-table row rewrite: count entries from the packed table array.
struct alignas(16) TableWrite {
  int64_t src_off;
  int32_t seq;
  int32_t count;
};

// One sequence of an eviction, as the keep-mask scan sees it.
struct alignas(16) EvictSeq {
  int64_t mask_off;    // bytes into the keep buffer
  int64_t n_old;       // rows before the eviction (= mask length)
  int64_t src_off;     // entries into src_of_dst
  int64_t reuse_off;   // entries into the per-new-page reuse array
};

// One fresh destination page of an eviction.
struct alignas(16) EvictTask {
  int64_t src_off;     // where this sequence's src_of_dst starts
  int32_t seq;         // page-table row of the sequence (old table still there)
  int32_t q;           // new logical page
  int32_t dst_page;    // physical page written
  int32_t n_new;       // rows after the eviction
  int32_t pad[2];
};

struct SpliceLaunch {
  const chunk_t* const* layers;  // device array [num_layers] of pool bases
  int32_t num_layers;
  int32_t page_shift;          // log2(page_size)
  const SpliceTask* tasks;
  int64_t n_tasks;
  int64_t n_slabs;             // ceil(n_tasks * page_size / 8)
  int64_t n_move_blocks;       // n_slabs * layer groups
  const SpliceDir* dirs;
  const TableWrite* twrites;   // run by the blocks after the move blocks
  const int32_t* tables;
  int32_t n_twrites;
  int32_t max_pages_per_seq;
  int32_t* page_table;
};

struct EvictLaunch {
  const chunk_t* const* layers;
  int32_t num_layers;
  int32_t page_shift;
  const EvictTask* tasks;
  int64_t n_tasks;
  int64_t n_slabs;
  int64_t n_move_blocks;
  const int32_t* src_of_dst;
  const int32_t* page_table;   // read-only here (old table)
  int32_t max_pages_per_seq;
};

struct TableLaunch {
  const TableWrite* twrites;
  const int32_t* tables;
  int32_t n_twrites;
  int32_t max_pages_per_seq;
  int32_t* page_table;
};

struct ScanLaunch {
  const uint8_t* keep;
  const EvictSeq* seqs;
  int32_t n_seqs;
  int32_t page_shift;
  int32_t* src_of_dst;
  int64_t* counts;     // [n_seqs]
  int32_t* reuse;      // per new page: reused old logical page, or -1
};

// Launchers (kernels.hip).  layers_per_block is how many layers one block
// carries (loads of all of them are issued before any store).
hipError_t launch_splice(const SpliceLaunch& a, int layers_per_block, int pairing, hipStream_t s);
hipError_t launch_evict_move(const EvictLaunch& a, int layers_per_block, hipStream_t s);
hipError_t launch_table_write(const TableLaunch& a, hipStream_t s);
hipError_t launch_keep_scan(const ScanLaunch& a, hipStream_t s);

int64_t layer_groups(int num_layers, int layers_per_block);

}  // namespace ll
