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

// The row kernels are flat gathers: one 16-byte chunk per thread, blocks of
// 256 threads, every block inside one layer.
constexpr int kFlatThreads = 256;

enum TaskKind : int32_t {
  kMoveRows = 0,        // fresh page: write every live row
  kRotateInPlace = 1,   // reused page: rotate the k_pe band of its live rows
};

// One destination page of a splice, self-contained (64 bytes) so that a
// thread needs one descriptor load before its data load.  Sources are
// physical pages, so the kernel never reads the page table it rewrites.  Row
// indices fit in 32 bits (the pool checks max_pages_per_seq * page_size).
// The first 16 bytes are all a rotate-in-place task needs.
struct alignas(16) SpliceTask {
  int32_t dst_page;    // physical page written (or rotated in place)
  int32_t q;           // new logical page
  int32_t n_new;       // rows of the sequence after the splice
  int32_t dir;         // index into the SpliceDir array (cos/sin)
  int32_t pre_page;    // physical page of old logical page q (prefix rows), or -1
  int32_t down_page0;  // physical page of old logical page down_lp0
  int32_t down_page1;  // physical page of down_lp0 + 1, or -1
  int32_t down_lp0;    // first old logical page feeding downstream rows
  int32_t rotate;      // 1 when downstream k_pe turns (AMORTIZE, delta != 0)
  int32_t s_start;
  int32_t stub_end;    // s_start + r_len
  int32_t delta;
  const chunk_t* stub;         // R rows of layer 0, in 16-byte chunks
  int64_t stub_layer_chunks;   // chunks between layers of R
};
static_assert(sizeof(SpliceTask) == 64, "a splice task is four 16-byte words");

// The rotation table of a directive, read only by k_pe chunks.
struct alignas(16) SpliceDir {
  float cos_[kHalfPairs];      // float32 of float64 cos(delta * theta_j)
  float sin_[kHalfPairs];
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
  int64_t src_off;     // entries into src_rows
  int64_t reuse_off;   // entries into the per-new-page reuse array
  int32_t seq;         // page-table row of the sequence
  int32_t pad[3];
};

// One fresh destination page of an eviction: 16 bytes, so that the copy
// kernels' task reads (every XCD reads every task on every layer pass) take
// half the lines a 32-byte task did.
struct alignas(16) EvictTask {
  int32_t dst_page;  // physical page written
  int16_t rows;      // live rows of the page (1..P)
  // when the page's live rows are consecutive old rows: src_off0 = the first
  // row's offset in its old page src0, src1 = the next old page (-1 when
  // they all lie in src0); src_off0 = -1: row r of the page reads its source
  // row from src_rows[src0 + r]
  int16_t src_off0;
  int32_t src0;
  int32_t src1;
};
static_assert(sizeof(EvictTask) == 16, "an eviction task is one 16-byte word");

struct SpliceLaunch {
  const chunk_t* const* layers;  // device array [num_layers] of pool bases
  int32_t num_layers;
  int32_t page_shift;          // log2(page_size)
  const SpliceTask* tasks;     // move tasks, then rotate-in-place tasks
  int64_t n_move_tasks;
  int64_t n_rot_tasks;
  int64_t move_blocks_per_layer;
  int64_t rot_blocks_per_layer;   // kInPlaceRowsPerBlock rotate-task rows per block
  const SpliceDir* dirs;
  const TableWrite* twrites;   // run by the blocks after the row blocks
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
  int64_t blocks_per_layer;
  const int32_t* src_rows;     // physical source row of every kept row
  const TableWrite* twrites;   // run by the blocks after the row blocks
  const int32_t* tables;
  int32_t n_twrites;
  int32_t max_pages_per_seq;
  int32_t* page_table;
};

struct TableLaunch {
  const TableWrite* twrites;
  const int32_t* tables;
  int32_t n_twrites;
  int32_t max_pages_per_seq;
  int32_t* page_table;
};

// GQA / MHA pools.  A K or V row is H heads of D bf16 = H * D / 8 chunks; the
// RoPE band of a K head is its first rotary_dim values = 2^rot_shift chunks.
constexpr int kMaxBandPairs = 128;  // rotary_dim <= 256

// The rotation table of a directive on a GQA pool and its V stub rows (the K
// stub rows are in the task).
struct alignas(16) GqaDir {
  const chunk_t* stub_v;       // V rows of R, layer 0
  int64_t stub_v_layer_chunks;
  float cos_[kMaxBandPairs];   // float32 of float64 cos(delta * theta_j)
  float sin_[kMaxBandPairs];
};

struct GqaSpliceLaunch {
  const chunk_t* const* planes;  // device array [2L]: K of layers 0..L-1, then V
  int32_t num_layers;
  int32_t page_shift;
  int32_t row_chunks;          // H * D / 8
  int32_t head_chunks;         // D / 8
  int32_t rot_shift;           // log2(rotary_dim / 8)
  int32_t heads;
  const SpliceTask* tasks;     // move tasks, then rotate-in-place tasks
  int64_t n_move_tasks;
  int64_t n_rot_tasks;
  int64_t move_blocks_per_plane;  // per K plane (one thread per 2 chunks); a V plane takes twice as many
  int64_t rot_blocks_per_plane;   // per K plane, one thread per 2 band chunks
  const GqaDir* dirs;
  const TableWrite* twrites;
  const int32_t* tables;
  int32_t n_twrites;
  int32_t max_pages_per_seq;
  int32_t* page_table;
};

// Eviction on pools whose rows are not MLA rows: every plane (K and V of
// every layer) has rows of row_chunks chunks.
struct PlaneEvictLaunch {
  const chunk_t* const* planes;
  int32_t num_planes;
  int32_t page_shift;
  int32_t row_chunks;
  const EvictTask* tasks;
  int64_t n_tasks;
  int64_t blocks_per_plane;
  const int32_t* src_rows;
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
  const int32_t* page_table;   // old tables (read)
  int32_t max_pages_per_seq;
  int32_t* src_rows;           // out: physical source row of each kept row
  int32_t* src_logical;        // out: old logical index of each kept row
  int64_t* counts;             // out: [n_seqs] rows kept
  int32_t* reuse;              // out: per new page, the old logical page it keeps, or -1
  // page size > 1: the reuse test, and the old pages no new page keeps
  // OR-ed into `freed` (zeroed before the scan), using `kept` as scratch
  uint8_t* kept;               // scratch: per old page (at reuse_off), 1 if a new page keeps it
  unsigned long long* freed;   // out: bitmap over physical pages
  // page size 1: every kept row keeps its page, so no reuse test and no
  // src_logical; a dropped row's page gets freed_bytes[page] = 1 (each page
  // has one writer; zeroed before the scan)
  uint8_t* freed_bytes;
  int32_t page_reuse;          // 0: no new page keeps an old one (every new page is fresh)
};

// Page size 1, after the keep scan: blocks [0, n) write each sequence's new
// page-table row (its kept rows' pages, i.e. its src_rows, in order); the
// other blocks pack freed_bytes into the freed bitmap, 64 pages a word.
struct UnitPageLaunch {
  const EvictSeq* seqs;
  int32_t n;
  const int64_t* counts;
  const int32_t* src_rows;
  int32_t* page_table;
  int32_t max_pages_per_seq;
  const uint8_t* freed_bytes;  // [64 * n_words]
  unsigned long long* freed;   // [n_words]
  int64_t n_words;
  int32_t* info;               // zeroed (no fresh page, no row moved)
};

// A splice batch planned on the device.  The host sends the compact plan as
// kernel arguments (no staging, no host-to-device copy): per directive its
// fields and the ranges of its fresh and rotate-in-place pages, the fresh
// physical pages as runs of consecutive ids, and the cos/sin tables.
// splice_plan_kernel expands it, reading the old page tables on the device,
// into the SpliceTask / SpliceDir (GqaDir) / TableWrite / table arrays the row
// kernels take, so that the row kernel that follows is the same as on the
// host-planned path.  The limits keep the arguments under 8 KiB (this stack
// passes kernel arguments of 12 KiB intact).
constexpr int kDirectMaxDirs = 16;
constexpr int kDirectMaxRuns = 256;
constexpr int kDirectTrigFloats = 1024;  // cos and sin of every directive

struct DirectDir {
  const chunk_t* stub;         // K (MLA: whole) rows of R, layer 0
  int64_t stub_layer_chunks;
  const chunk_t* stub_v;       // GQA: V rows of R
  int64_t stub_v_layer_chunks;
  int32_t seq;
  int32_t s_start;
  int32_t stub_end;            // s_start + rows of R inserted (FORGET: s_start)
  int32_t delta;               // FORGET: 0
  int32_t n_new;
  int32_t old_pages;           // pages of the old table
  int32_t rotate;              // 1: downstream bands turn (AMORTIZE, delta != 0)
  int32_t q_fresh0;            // fresh pages are new pages q_fresh0 .. + fresh - 1
  int32_t q_rot0;              // rotate-in-place pages are q_rot0 .. + n_rot - 1
  int32_t move_base;           // index of its first fresh page among the move tasks
  int32_t rot_base;            // ... among the rotate tasks
  int32_t fresh_base;          // index of its first fresh page in the fresh runs
  int32_t packed_off;          // where its new table goes in the table array
  int32_t pad[3];
};

struct DirectPlanArgs {
  int32_t n_dirs;
  int32_t page_shift;
  int32_t pairs;               // RoPE pairs per table (MLA 32; GQA rotary_dim / 2)
  int32_t n_runs;
  int32_t max_pages_per_seq;
  int32_t gqa;
  int32_t page_reuse;          // 0: every new page is fresh
  int32_t pad0;
  int64_t n_move_tasks;
  int64_t n_rot_tasks;
  int64_t n_entries;           // length of the packed table array
  const int32_t* page_table;   // old tables (read only)
  SpliceTask* tasks;           // out: move tasks, then rotate tasks
  void* dirs;                  // out: SpliceDir[n_dirs] or GqaDir[n_dirs]
  TableWrite* twrites;         // out: one per directive
  int32_t* tables;             // out: packed new tables
  int32_t run_page[kDirectMaxRuns];       // first physical page of run r
  int32_t run_first[kDirectMaxRuns + 1];  // fresh index of run r's first page
  DirectDir d[kDirectMaxDirs];
  float trig[kDirectTrigFloats];  // directive i: cos at 2*pairs*i, sin at 2*pairs*i + pairs
};
static_assert(sizeof(DirectPlanArgs) <= 8192, "the direct splice plan must fit in 8 KiB of kernel arguments");

// Timing events a launcher stamps from the dispatch packets themselves (no
// marker packets of their own on the stream): `start` gets the start time of
// the first kernel it launches, `stop` the end time of the last one.  Null
// events are left alone.  A launcher that has no work records both at once.
struct Stamp {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Launchers (kernels.hip).
hipError_t launch_splice(const SpliceLaunch& a, int pairing, hipStream_t s, const Stamp& t = Stamp{});
hipError_t launch_evict_move(const EvictLaunch& a, hipStream_t s, const Stamp& t = Stamp{});
hipError_t launch_table_write(const TableLaunch& a, hipStream_t s);
hipError_t launch_keep_scan(const ScanLaunch& a, hipStream_t s, const Stamp& t = Stamp{});
hipError_t launch_unit_page(const UnitPageLaunch& a, hipStream_t s, const Stamp& t = Stamp{});
hipError_t launch_gqa_splice(const GqaSpliceLaunch& a, int pairing, hipStream_t s, const Stamp& t = Stamp{});
hipError_t launch_plane_evict(const PlaneEvictLaunch& a, hipStream_t s, const Stamp& t = Stamp{});
hipError_t launch_splice_plan(const DirectPlanArgs& a, int32_t max_new_pages, hipStream_t s);

// The plan space of leyline_splice_noalloc: a file-scope device array in
// kernels.hip (every device the library runs on holds one copy until the
// process ends).  noalloc_scratch_init looks up its address on `device` (the
// current device) once and keeps it; noalloc_scratch returns that address, or
// nullptr when the lookup has not succeeded on `device`.
constexpr size_t kNoAllocScratchBytes = size_t{4} << 20;
hipError_t noalloc_scratch_init(int device);
void* noalloc_scratch(int device);

// Chunks each thread of splice_kernel moves.
constexpr int kSpliceChunksPerThread = 1;

// Threads per block of the eviction's row copies (evict_move_kernel,
// plane_evict_kernel): one wave per block.
constexpr int kEvictThreads = 64;

// splice_inplace_kernel: groups of 8 rows per wave (one 128-byte k_pe line
// per row and lane group), and rows per 256-thread block.
constexpr int kInPlaceGroups = 8;
constexpr int kInPlaceRowsPerBlock = kFlatThreads / 64 * 8 * kInPlaceGroups;

// Blocks of `threads` threads that cover `chunks` chunks of one layer, each
// thread taking `per_thread` of them.
inline int64_t flat_blocks(int64_t chunks, int per_thread = 1, int threads = kFlatThreads) {
  const int64_t per_block = int64_t{threads} * per_thread;
  return (chunks + per_block - 1) / per_block;
}

}  // namespace ll
