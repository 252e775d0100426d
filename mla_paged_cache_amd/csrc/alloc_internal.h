// Internal types of the device-side page allocator of the eviction
// (kernels_alloc.hip) and its host side (pool.cpp).  Not part of the C ABI.
#pragma once

#include "leyline_internal.h"

namespace ll {

struct AllocLaunch {
  const EvictSeq* seqs;
  int32_t n;
  int32_t page_shift;
  const int64_t* counts;      // rows kept per sequence (keep scan)
  const int32_t* reuse;       // per new page: old logical page kept, or -1 (keep scan)
  const int32_t* page_table;  // old tables (read only)
  int32_t max_pages_per_seq;
  int32_t n_words;            // words of the free bitmap
  const uint64_t* free_words; // the free set at the call's start (bit set = free)
  int32_t* rank;              // per new page: its index among the sequence's fresh pages
  int32_t* fresh_count;       // [n]
  int32_t* fresh_base;        // [n]: fresh pages of the sequences before
  int32_t* moved_count;       // [n]: rows of each sequence's fresh pages
  int32_t* word_base;         // [n_words]: free pages in the words before
  int32_t* new_table;         // per sequence at reuse_off: the new page table
  EvictTask* tasks;           // [fresh pages], in (sequence, page) order
  const int32_t* src_logical; // old logical row of every kept row (keep scan), or null: tasks
                              // then always point at src_rows
  int32_t* info;              // [0] fresh pages, [1] 1 if they exceed the free pages,
                              // [2..3] rows written to fresh pages (64-bit); 16-byte aligned
};


// fresh_rank + alloc_scan (ends with the verdict in info), then
// alloc_tables + table_copy (both do nothing when info[1] is set).
hipError_t launch_alloc_scan(const AllocLaunch& a, hipStream_t s, const Stamp& t = Stamp{});
hipError_t launch_alloc_tables(const AllocLaunch& a, hipStream_t s, const Stamp& t = Stamp{});
// Zero n 64-bit words (a kernel, so that it can sit in a captured graph).
hipError_t launch_zero_words(unsigned long long* w, int64_t n, hipStream_t s);

}  // namespace ll
