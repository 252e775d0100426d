// Stand-ins for the HIP runtime and for the library's device launches, so
// that the host side of libleyline (pool.cpp, kvs_mask.cpp: validation, page
// planning, the allocator, staging, the eviction's settle, the lazy page
// tables) runs on the CPU under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// "Device" memory is host memory.  Copies are synchronous, events and streams
// are tokens that are always complete.  Launches whose results the host reads
// back -- the eviction's keep scan, verdict, new tables and freed-page bitmap,
// and every page-table rewrite -- are done here on the CPU, the same
// operations the kernels perform, so that the library's books can be compared
// with an independent model.  Row contents are never produced (the host never
// reads them): row-moving launches do nothing.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../mla_paged_cache_amd/csrc/alloc_internal.h"
#include "../../mla_paged_cache_amd/csrc/kvs_internal.h"
#include "../../mla_paged_cache_amd/csrc/leyline_internal.h"
#include "../../mla_paged_cache_amd/csrc/rows_internal.h"

namespace {
int g_device = 0;
struct Token {
  int kind;
};
void* zalloc(size_t n) { return std::calloc(n ? n : 1, 1); }
}  // namespace

extern "C" {

hipError_t hipMalloc(void** p, size_t n) {
  *p = zalloc(n);
  return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void* p) {
  std::free(p);
  return hipSuccess;
}
hipError_t hipHostMalloc(void** p, size_t n, unsigned int) { return hipMalloc(p, n); }
hipError_t hipHostFree(void* p) { return hipFree(p); }
hipError_t hipMemcpy(void* d, const void* s, size_t n, hipMemcpyKind) {
  if (n) std::memmove(d, s, n);
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void* d, const void* s, size_t n, hipMemcpyKind k, hipStream_t) { return hipMemcpy(d, s, n, k); }
hipError_t hipEventCreate(hipEvent_t* e) {
  *e = reinterpret_cast<hipEvent_t>(new Token{1});
  return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) { return hipEventCreate(e); }
hipError_t hipEventDestroy(hipEvent_t e) {
  delete reinterpret_cast<Token*>(e);
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t) { return e ? hipSuccess : hipErrorInvalidValue; }
hipError_t hipEventSynchronize(hipEvent_t e) { return e ? hipSuccess : hipErrorInvalidValue; }
hipError_t hipEventQuery(hipEvent_t e) { return e ? hipSuccess : hipErrorInvalidValue; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t a, hipEvent_t b) {
  if (!a || !b) return hipErrorInvalidValue;
  *ms = 0.f;
  return hipSuccess;
}
hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned int) {
  *s = reinterpret_cast<hipStream_t>(new Token{2});
  return hipSuccess;
}
hipError_t hipStreamDestroy(hipStream_t s) {
  delete reinterpret_cast<Token*>(s);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t e, unsigned int) { return e ? hipSuccess : hipErrorInvalidValue; }
hipError_t hipGetDevice(int* d) {
  *d = g_device;
  return hipSuccess;
}
hipError_t hipSetDevice(int d) {
  if (d < 0 || d > 7) return hipErrorInvalidDevice;
  g_device = d;
  return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "error in the HIP stand-in"; }
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int) {
  *v = attr == hipDeviceAttributeMaxSharedMemoryPerBlock ? 160 * 1024 : 0;
  return hipSuccess;
}

}  // extern "C"

namespace ll {

namespace {
// The page-table rows a launch rewrites.
void table_writes(const TableWrite* tw, const int32_t* tables, int32_t n, int32_t max_pages, int32_t* page_table) {
  for (int32_t i = 0; i < n; ++i) {
    int32_t* dst = page_table + static_cast<int64_t>(tw[i].seq) * max_pages;
    for (int32_t e = 0; e < tw[i].count; ++e) dst[e] = tables[tw[i].src_off + e];
  }
}
std::vector<char> g_scratch(kNoAllocScratchBytes);
}  // namespace

hipError_t noalloc_scratch_init(int) { return hipSuccess; }
void* noalloc_scratch(int) { return g_scratch.data(); }

hipError_t launch_splice(const SpliceLaunch& a, int, hipStream_t, const Stamp&) {
  table_writes(a.twrites, a.tables, a.n_twrites, a.max_pages_per_seq, a.page_table);
  return hipSuccess;
}
hipError_t launch_gqa_splice(const GqaSpliceLaunch& a, int, hipStream_t, const Stamp&) {
  table_writes(a.twrites, a.tables, a.n_twrites, a.max_pages_per_seq, a.page_table);
  return hipSuccess;
}
hipError_t launch_table_write(const TableLaunch& a, hipStream_t) {
  table_writes(a.twrites, a.tables, a.n_twrites, a.max_pages_per_seq, a.page_table);
  return hipSuccess;
}
hipError_t launch_evict_move(const EvictLaunch&, hipStream_t, const Stamp&) { return hipSuccess; }
hipError_t launch_plane_evict(const PlaneEvictLaunch&, hipStream_t, const Stamp&) { return hipSuccess; }

// The page plan of a device-planned splice: per directive and new page, the
// kept old page or the fresh page of its fresh index (runs of consecutive
// ids), the new table rows and their write records.
hipError_t launch_splice_plan(const DirectPlanArgs& a, int32_t, hipStream_t) {
  const int32_t P = 1 << a.page_shift;
  for (int di = 0; di < a.n_dirs; ++di) {
    const DirectDir& D = a.d[di];
    const int32_t* T = a.page_table + static_cast<int64_t>(D.seq) * a.max_pages_per_seq;
    const int32_t pages = (D.n_new + P - 1) / P;
    for (int32_t q = 0; q < pages; ++q) {
      const int32_t lo = q * P, hi = std::min(lo + P, D.n_new);
      const bool has_pre = lo < D.s_start;
      const bool has_stub = D.stub_end > D.s_start && lo < D.stub_end && hi > D.s_start;
      const bool has_down = hi > D.stub_end;
      int32_t reuse;
      if (has_stub)
        reuse = -1;
      else if (has_pre && has_down)
        reuse = D.delta == 0 ? q : -1;
      else if (has_pre)
        reuse = q;
      else
        reuse = ((lo - D.delta) % P) == 0 ? (lo - D.delta) / P : -1;
      if (!a.page_reuse) reuse = -1;
      int32_t page;
      if (reuse >= 0) {
        page = T[reuse];
      } else {
        const int32_t f = D.fresh_base + (q - D.q_fresh0);
        int r = 0;
        while (r + 1 < a.n_runs && a.run_first[r + 1] <= f) ++r;
        page = a.run_page[r] + (f - a.run_first[r]);
      }
      a.tables[D.packed_off + q] = page;
    }
    a.twrites[di] = TableWrite{D.packed_off, D.seq, pages};
  }
  return hipSuccess;
}

hipError_t launch_keep_scan(const ScanLaunch& a, hipStream_t, const Stamp&) {
  const int shift = a.page_shift;
  const int64_t P = int64_t{1} << shift;
  for (int32_t b = 0; b < a.n_seqs; ++b) {
    const EvictSeq& e = a.seqs[b];
    const uint8_t* m = a.keep + e.mask_off;
    const int32_t* table = a.page_table + static_cast<int64_t>(e.seq) * a.max_pages_per_seq;
    int64_t pos = 0;
    for (int64_t i = 0; i < e.n_old; ++i) {
      if (m[i]) {
        if (shift == 0) {
          a.src_rows[e.src_off + pos] = table[i];
        } else {
          a.src_logical[e.src_off + pos] = static_cast<int32_t>(i);
          a.src_rows[e.src_off + pos] = static_cast<int32_t>((static_cast<int64_t>(table[i >> shift]) << shift) + (i & (P - 1)));
        }
        ++pos;
      } else if (shift == 0) {
        a.freed_bytes[table[i]] = 1;
      }
    }
    a.counts[b] = pos;
    if (shift == 0) continue;
    const int64_t pages = (pos + P - 1) >> shift, old_pages = (e.n_old + P - 1) >> shift;
    std::vector<char> kept(static_cast<size_t>(old_pages), 0);
    for (int64_t q = 0; q < pages; ++q) {
      const int64_t k = std::min(P, pos - (q << shift));
      const int64_t f = a.src_logical[e.src_off + (q << shift)];
      const int64_t l = a.src_logical[e.src_off + (q << shift) + k - 1];
      const bool keep = a.page_reuse && (f & (P - 1)) == 0 && l - f == k - 1;
      a.reuse[e.reuse_off + q] = keep ? static_cast<int32_t>(f >> shift) : -1;
      if (keep) kept[f >> shift] = 1;
    }
    for (int64_t k = 0; k < old_pages; ++k)
      if (!kept[k]) a.freed[table[k] >> 6] |= 1ull << (table[k] & 63);
  }
  return hipSuccess;
}

hipError_t launch_zero_words(unsigned long long* w, int64_t n, hipStream_t) {
  if (n > 0) std::memset(w, 0, static_cast<size_t>(n) * 8);
  return hipSuccess;
}

hipError_t launch_alloc_scan(const AllocLaunch& a, hipStream_t, const Stamp&) {
  const int64_t P = int64_t{1} << a.page_shift;
  int32_t fresh = 0;
  unsigned long long moved = 0;
  for (int32_t b = 0; b < a.n; ++b) {
    const EvictSeq& e = a.seqs[b];
    const int64_t n_new = a.counts[b], pages = (n_new + P - 1) / P;
    int32_t rank = 0, rows = 0;
    for (int64_t q = 0; q < pages; ++q) {
      a.rank[e.reuse_off + q] = rank;
      if (a.reuse[e.reuse_off + q] < 0) {
        ++rank;
        rows += static_cast<int32_t>(std::min(P, n_new - q * P));
      }
    }
    a.fresh_count[b] = rank;
    a.moved_count[b] = rows;
    a.fresh_base[b] = fresh;
    fresh += rank;
    moved += static_cast<unsigned long long>(rows);
  }
  int32_t free_total = 0;
  for (int32_t w = 0; w < a.n_words; ++w) {
    a.word_base[w] = free_total;
    free_total += __builtin_popcountll(a.free_words[w]);
  }
  const bool short_of_pages = fresh > free_total;
  a.info[0] = short_of_pages ? 0 : fresh;
  a.info[1] = short_of_pages ? 1 : 0;
  *reinterpret_cast<unsigned long long*>(a.info + 2) = short_of_pages ? 0 : moved;
  return hipSuccess;
}

hipError_t launch_alloc_tables(const AllocLaunch& a, hipStream_t, const Stamp&) {
  if (a.info[1]) return hipSuccess;
  const int64_t P = int64_t{1} << a.page_shift;
  for (int32_t b = 0; b < a.n; ++b) {
    const EvictSeq& e = a.seqs[b];
    const int64_t n_new = a.counts[b], pages = (n_new + P - 1) / P;
    const int32_t* old_t = a.page_table + static_cast<int64_t>(e.seq) * a.max_pages_per_seq;
    for (int64_t q = 0; q < pages; ++q) {
      const int32_t r = a.reuse[e.reuse_off + q];
      int32_t page;
      if (r >= 0) {
        page = old_t[r];
      } else {
        int32_t f = a.fresh_base[b] + a.rank[e.reuse_off + q];
        page = -1;
        for (int32_t w = 0; w < a.n_words && page < 0; ++w) {
          const int c = __builtin_popcountll(a.free_words[w]);
          if (f >= c) {
            f -= c;
            continue;
          }
          uint64_t bits = a.free_words[w];
          for (; f > 0; --f) bits &= bits - 1;
          page = w * 64 + __builtin_ctzll(bits);
        }
        const int64_t rows = std::min<int64_t>(P, n_new - q * P);
        a.tasks[a.fresh_base[b] + a.rank[e.reuse_off + q]] =
            EvictTask{page, static_cast<int16_t>(rows), -1, static_cast<int32_t>(e.src_off + q * P), -1};
      }
      a.new_table[e.reuse_off + q] = page;
    }
  }
  for (int32_t b = 0; b < a.n; ++b) {
    const EvictSeq& e = a.seqs[b];
    const int64_t pages = (a.counts[b] + P - 1) / P;
    int32_t* t = const_cast<int32_t*>(a.page_table) + static_cast<int64_t>(e.seq) * a.max_pages_per_seq;
    for (int64_t q = 0; q < pages; ++q) t[q] = a.new_table[e.reuse_off + q];
  }
  return hipSuccess;
}

hipError_t launch_unit_page(const UnitPageLaunch& a, hipStream_t, const Stamp&) {
  for (int32_t b = 0; b < a.n; ++b) {
    int32_t* dst = a.page_table + static_cast<int64_t>(a.seqs[b].seq) * a.max_pages_per_seq;
    for (int64_t q = 0; q < a.counts[b]; ++q) dst[q] = a.src_rows[a.seqs[b].src_off + q];
  }
  for (int64_t w = 0; w < a.n_words; ++w) {
    unsigned long long word = 0;
    for (int k = 0; k < 64; ++k)
      if (a.freed_bytes[64 * w + k]) word |= 1ull << k;
    a.freed[w] = word;
  }
  for (int k = 0; k < 4; ++k) a.info[k] = 0;
  return hipSuccess;
}

hipError_t launch_rope_table(const RopeTableLaunch&, hipStream_t, const Stamp&) { return hipSuccess; }
hipError_t launch_rope_rows(const RopeRowsLaunch&, int, hipStream_t, const Stamp&) { return hipSuccess; }
hipError_t launch_rope_inplace_mla(const RopeRowsLaunch&, const double*, int, hipStream_t, const Stamp&) {
  return hipSuccess;
}
int64_t rope_rows_blocks_per_plane(const RopeRowsLaunch&, int64_t) { return 1; }

hipError_t launch_kvs_death(const KvsDeathLaunch& a, hipStream_t) {
  // the scratch must hold every event's groups of 32 rows behind the
  // per-event counts
  int64_t need = 0;
  for (int32_t e = 0; e < a.n_events; ++e) {
    if (a.events[e].rank_off != need) return hipErrorInvalidValue;
    need += (a.events[e].mask_len + 31) / 32;
  }
  if (a.n_events == 0) return hipSuccess;  // no event: neither scratch array is read
  return a.rank && a.kept && (reinterpret_cast<uintptr_t>(a.rank) & 15) == 0 ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_kvs_block(const KvsBlockLaunch&, hipStream_t) { return hipSuccess; }
hipError_t launch_kvs_dense(const KvsDenseLaunch&, hipStream_t) { return hipSuccess; }

}  // namespace ll
