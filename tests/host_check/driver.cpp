// Operation interpreter over the library's C ABI, for the host-side checks:
// built with hip_shim.cpp (HIP stand-ins, the device launches done on the
// CPU) under AddressSanitizer and UndefinedBehaviorSanitizer.  It reads one
// operation per line from stdin and prints one result line per operation;
// the test that drives it predicts every line from the oracle.
//
//   pool mla|gqa L P num_pages max_seqs max_pages [planner]  -> "pool <status>"
//   alloc n                                   -> "alloc <status> <seq>"
//   free s                                    -> "free <status>"
//   set s n k p_1 .. p_k                      -> "set <status>"
//   splice noalloc planner k (s mode s0 s1 r)*k  -> "splice <status> <fresh> <freed>"
//   evict k (s mask)*k   (mask: 0/1 string, "-" when empty)
//                                             -> "evict <status> <fresh> <freed>"
//   reindex s k p_1 .. p_k                    -> "reindex <status>"
//   reuse on                                  -> "reuse <status>"   (page reuse on / off)
//   rope s r0 n in_place                      -> "rope <status>"
//   books                                     -> "seq s <status> len pos k p_1 .. p_k" per row,
//                                                then "free <n>"
//   lengths k s_1 .. s_k                      -> "lengths <status> n_1 .. n_k"
//   kvs n_pad n (n_tokens e (t m)*e)*n        -> "kvs <status>"
//   kvsmask n n_pad bq bk dense               -> "kvsmask <block status> <dense status>"
//   misc                                      -> "misc <status> ..."  (assorted calls)
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "leyline.h"

namespace {

void* dev_alloc(size_t n) {
  void* p = nullptr;
  if (hipMalloc(&p, n) != hipSuccess) {
    std::fprintf(stderr, "stand-in hipMalloc failed\n");
    std::exit(2);
  }
  return p;
}

void dev_free(void* p) { static_cast<void>(hipFree(p)); }

struct Pool {
  ll_pool* pool = nullptr;
  bool gqa = false;
  int32_t L = 0, P = 0, num_pages = 0, max_seqs = 0, max_pages = 0;
  int64_t row_bytes = 0;
  std::vector<void*> k, v;
  int32_t* table = nullptr;
  void* stub = nullptr;    // K (MLA: whole) rows of R, all layers, zeros
  void* stub_v = nullptr;
  int64_t stub_rows = 0;
  int64_t* angles = nullptr;
  void* rope_out = nullptr;

  void reset() {
    if (pool) ll_pool_destroy(pool);
    pool = nullptr;
    for (void* p : k) dev_free(p);
    for (void* p : v) dev_free(p);
    k.clear();
    v.clear();
    for (void* p : {static_cast<void*>(table), stub, stub_v, static_cast<void*>(angles), rope_out}) dev_free(p);
    table = nullptr;
    stub = stub_v = rope_out = nullptr;
    angles = nullptr;
  }
};

Pool g;

int do_pool(std::istringstream& in) {
  std::string kind;
  int32_t planner = 0;
  in >> kind >> g.L >> g.P >> g.num_pages >> g.max_seqs >> g.max_pages;
  if (!(in >> planner)) planner = 0;
  g.reset();
  g.gqa = kind == "gqa";
  // GQA: 3 KV heads of 64, RoPE on the first 32 of each head
  g.row_bytes = g.gqa ? 3 * 64 * 2 : 576 * 2;
  const size_t plane = static_cast<size_t>(g.num_pages) * g.P * g.row_bytes;
  for (int l = 0; l < g.L; ++l) {
    g.k.push_back(dev_alloc(plane));
    if (g.gqa) g.v.push_back(dev_alloc(plane));
  }
  g.table = static_cast<int32_t*>(dev_alloc(static_cast<size_t>(g.max_seqs) * g.max_pages * 4));
  g.stub_rows = 4 * g.P + 8;
  g.stub = dev_alloc(static_cast<size_t>(g.L) * g.stub_rows * g.row_bytes);
  if (g.gqa) g.stub_v = dev_alloc(static_cast<size_t>(g.L) * g.stub_rows * g.row_bytes);
  const int64_t max_rows = static_cast<int64_t>(g.max_pages) * g.P;
  g.angles = static_cast<int64_t*>(dev_alloc(static_cast<size_t>(max_rows) * 8));
  g.rope_out = dev_alloc(static_cast<size_t>(g.L) * max_rows * g.row_bytes);
  ll_status st;
  if (g.gqa) {
    ll_gqa_pool_desc d{};
    d.num_layers = g.L;
    d.page_size = g.P;
    d.num_pages = g.num_pages;
    d.max_seqs = g.max_seqs;
    d.max_pages_per_seq = g.max_pages;
    d.num_kv_heads = 3;
    d.head_dim = 64;
    d.rotary_dim = 32;
    d.rope_pairing = LL_ROPE_HALF;
    d.rope_base = 500000.0;
    d.k_layer_base = g.k.data();
    d.v_layer_base = g.v.data();
    d.page_table = g.table;
    d.device = 0;
    st = ll_pool_create_gqa(&d, &g.pool);
  } else {
    ll_pool_desc d{};
    d.num_layers = g.L;
    d.page_size = g.P;
    d.num_pages = g.num_pages;
    d.max_seqs = g.max_seqs;
    d.max_pages_per_seq = g.max_pages;
    d.kv_lora_rank = 512;
    d.rope_dim = 64;
    d.rope_pairing = LL_ROPE_INTERLEAVED;
    d.rope_base = 10000.0;
    d.layer_base = g.k.data();
    d.page_table = g.table;
    d.device = 0;
    st = ll_pool_create(&d, &g.pool);
  }
  if (st == LL_OK && planner) st = ll_pool_set_splice_planner(g.pool, planner);
  return st;
}

void print_stats(const char* op, ll_status st) {
  ll_plan_stats s{};
  if (st == LL_OK) {
    const ll_status e = ll_last_plan_stats(g.pool, &s);
    if (e != LL_OK) {
      std::printf("%s stats-failed %d\n", op, e);
      return;
    }
  }
  std::printf("%s %d %lld %lld\n", op, st, static_cast<long long>(s.fresh_pages),
              static_cast<long long>(s.freed_pages));
}

void do_splice(std::istringstream& in) {
  int noalloc = 0, planner = 0, n = 0;
  in >> noalloc >> planner >> n;
  std::vector<ll_directive> d(static_cast<size_t>(n));
  for (auto& x : d) {
    int64_t r = 0;
    x = ll_directive{};
    in >> x.seq_id >> x.mode >> x.s_start >> x.s_end >> r;
    x.r_len = r;
    if (r > g.stub_rows) {
      std::fprintf(stderr, "stub of %lld rows exceeds the driver's %lld\n", static_cast<long long>(r),
                   static_cast<long long>(g.stub_rows));
      std::exit(2);
    }
    if (r > 0) {
      x.r_rows = g.stub;
      x.r_layer_stride_bytes = g.stub_rows * g.row_bytes;
      if (g.gqa) {
        x.r_rows_v = g.stub_v;
        x.r_layer_stride_bytes_v = g.stub_rows * g.row_bytes;
      }
    }
  }
  ll_status st = ll_pool_set_splice_planner(g.pool, planner);
  if (st == LL_OK)
    st = noalloc ? leyline_splice_noalloc(g.pool, d.data(), n, nullptr) : leyline_splice(g.pool, d.data(), n, nullptr);
  print_stats("splice", st);
}

void do_evict(std::istringstream& in) {
  int n = 0;
  in >> n;
  std::vector<int32_t> seqs(static_cast<size_t>(n));
  std::vector<int64_t> offs(static_cast<size_t>(n));
  std::string keep;
  for (int i = 0; i < n; ++i) {
    std::string m;
    in >> seqs[i] >> m;
    if (m == "-") m.clear();
    offs[i] = static_cast<int64_t>(keep.size());
    keep += m;
  }
  uint8_t* dev = static_cast<uint8_t*>(dev_alloc(keep.size() + 16));
  for (size_t i = 0; i < keep.size(); ++i) dev[i] = keep[i] == '1';
  const ll_status st = kv_evict_compact(g.pool, seqs.data(), n, dev, offs.data(), nullptr);
  print_stats("evict", st);
  dev_free(dev);
}

void do_books() {
  std::vector<int32_t> pages(static_cast<size_t>(g.max_pages));
  for (int32_t s = 0; s < g.max_seqs; ++s) {
    int64_t len = -1, pos = -1;
    int32_t np = -1;
    const ll_status st = ll_seq_get(g.pool, s, &len, &pos, pages.data(), g.max_pages, &np);
    std::printf("seq %d %d", s, st);
    if (st == LL_OK) {
      std::printf(" %lld %lld %d", static_cast<long long>(len), static_cast<long long>(pos), np);
      for (int32_t i = 0; i < np; ++i) std::printf(" %d", pages[i]);
      // the device table row must agree with the host copy
      for (int32_t i = 0; i < np; ++i)
        if (g.table[static_cast<int64_t>(s) * g.max_pages + i] != pages[i]) std::printf(" DEVICE-TABLE-DIFFERS");
    }
    std::printf("\n");
  }
  int64_t n_free = -1;
  const ll_status st = ll_pool_free_pages(g.pool, &n_free);
  std::printf("free %d %lld\n", st, static_cast<long long>(n_free));
}

void do_kvs(std::istringstream& in) {
  int64_t n_pad = 0;
  int n = 0;
  in >> n_pad >> n;
  std::vector<kvs_rollout_log> logs(static_cast<size_t>(n));
  std::vector<std::vector<int64_t>> times(static_cast<size_t>(n)), lens(static_cast<size_t>(n));
  int64_t mask_bytes = 0;
  for (int i = 0; i < n; ++i) {
    int e = 0;
    in >> logs[i].n_tokens >> e;
    logs[i].n_events = e;
    for (int j = 0; j < e; ++j) {
      int64_t t = 0, m = 0;
      in >> t >> m;
      times[i].push_back(t);
      lens[i].push_back(m);
    }
    logs[i].event_time = times[i].data();
    logs[i].mask_len = lens[i].data();
    logs[i].mask_offset = mask_bytes;
    for (int64_t m : lens[i]) mask_bytes += m > 0 ? m : 0;
  }
  kvs_ctx* ctx = nullptr;
  ll_status st = kvs_ctx_create(0, &ctx);
  if (st == LL_OK) {
    uint8_t* keep = static_cast<uint8_t*>(dev_alloc(static_cast<size_t>(mask_bytes) + 16));
    const int64_t pad = n_pad > 0 && n_pad < (int64_t{1} << 20) ? n_pad : 1;
    int32_t* death = static_cast<int32_t*>(dev_alloc(static_cast<size_t>(n > 0 ? n : 1) * pad * 4));
    int32_t* status = static_cast<int32_t*>(dev_alloc(static_cast<size_t>(n > 0 ? n : 1) * 4));
    st = kvs_death_times(ctx, logs.data(), n, n_pad, keep, death, status, nullptr);
    dev_free(keep);
    dev_free(death);
    dev_free(status);
    kvs_ctx_destroy(ctx);
  }
  std::printf("kvs %d\n", st);
}

void do_kvsmask(std::istringstream& in) {
  int n = 0, bq = 0, bk = 0;
  int64_t n_pad = 0;
  in >> n >> n_pad >> bq >> bk;
  kvs_ctx* ctx = nullptr;
  ll_status st = kvs_ctx_create(0, &ctx);
  if (st != LL_OK) {
    std::printf("kvsmask %d %d\n", st, st);
    return;
  }
  const int64_t nn = n > 0 ? n : 1, np = n_pad > 0 ? n_pad : 1;
  int32_t* death = static_cast<int32_t*>(dev_alloc(static_cast<size_t>(nn * np * 4)));
  const int64_t nq = bq > 0 ? (np + bq - 1) / bq : 1, nk = bk > 0 ? (np + bk - 1) / bk : 1;
  int32_t* pn = static_cast<int32_t*>(dev_alloc(static_cast<size_t>(nn * nq * 4)));
  int32_t* pi = static_cast<int32_t*>(dev_alloc(static_cast<size_t>(nn * nq * nk * 4)));
  int32_t* fn = static_cast<int32_t*>(dev_alloc(static_cast<size_t>(nn * nq * 4)));
  int32_t* fi = static_cast<int32_t*>(dev_alloc(static_cast<size_t>(nn * nq * nk * 4)));
  const ll_status sb = kvs_block_mask(ctx, death, n, n_pad, bq, bk, pn, pi, fn, fi, nullptr);
  uint32_t* bits = static_cast<uint32_t*>(dev_alloc(static_cast<size_t>(nn * np * ((np + 31) / 32) * 4)));
  const ll_status sd = kvs_dense_mask(ctx, death, n, n_pad, bits, nullptr);
  for (void* p : {static_cast<void*>(death), static_cast<void*>(pn), static_cast<void*>(pi),
                  static_cast<void*>(fn), static_cast<void*>(fi), static_cast<void*>(bits)})
    dev_free(p);
  kvs_ctx_destroy(ctx);
  std::printf("kvsmask %d %d\n", sb, sd);
}

// Calls whose results the test checks by their documented contract: the
// profiling record, the last plan's bytes, the delta table, error strings.
void do_misc() {
  ll_status st = ll_pool_set_profiling(g.pool, 1);
  int64_t launches = -1, bytes = -1, alg = -1, moved = -1, rot = -1;
  double ms = -1;
  float each[4];
  if (st == LL_OK) st = ll_profile_read(g.pool, 0, &launches, &ms, &bytes, each, 4);
  if (st == LL_OK) st = ll_pool_set_profiling(g.pool, 0);
  const ll_status sb = ll_last_plan_bytes(g.pool, &alg, &moved, &rot);
  float cs[32], sn[32];
  const ll_status sr = ll_rope_delta_table(10000.0, 64, 7, cs, sn);
  const ll_status bad = ll_rope_delta_table(10000.0, 63, 7, cs, sn);
  const char* msg = ll_last_error();
  const ll_status sk = ll_profile_read(g.pool, 9, nullptr, nullptr, nullptr, nullptr, 0);
  std::printf("misc %d %d %d %d %d %d %s\n", st, sb, sr, bad, sk, msg && *msg ? 1 : 0, ll_status_str(LL_ENOMEM));
}

}  // namespace

int main() {
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string op;
    if (!(in >> op)) continue;
    if (op == "pool") {
      std::printf("pool %d\n", do_pool(in));
    } else if (op == "alloc") {
      int64_t n = 0;
      in >> n;
      int32_t sid = -1;
      const ll_status st = ll_seq_alloc(g.pool, n, &sid, nullptr);
      std::printf("alloc %d %d\n", st, st == LL_OK ? sid : -1);
    } else if (op == "free") {
      int32_t s = 0;
      in >> s;
      std::printf("free %d\n", ll_seq_free(g.pool, s));
    } else if (op == "set") {
      int32_t s = 0, k = 0;
      int64_t n = 0;
      in >> s >> n >> k;
      std::vector<int32_t> pages(static_cast<size_t>(k));
      for (auto& p : pages) in >> p;
      std::printf("set %d\n", ll_seq_set_pages(g.pool, s, pages.data(), n, nullptr));
    } else if (op == "splice") {
      do_splice(in);
    } else if (op == "evict") {
      do_evict(in);
    } else if (op == "reindex") {
      int32_t s = 0, k = 0;
      in >> s >> k;
      std::vector<int32_t> keep(static_cast<size_t>(k));
      for (auto& p : keep) in >> p;
      std::printf("reindex %d\n", ll_ptable_reindex(g.pool, s, keep.data(), k, nullptr));
    } else if (op == "reuse") {
      int32_t on = 1;
      in >> on;
      std::printf("reuse %d\n", ll_pool_set_page_reuse(g.pool, on));
    } else if (op == "limit") {
      int64_t items = 0;
      in >> items;
      std::printf("limit %d\n", ll_pool_set_dispatch_limit(g.pool, items));
    } else if (op == "rope") {
      int32_t s = 0, in_place = 1;
      int64_t r0 = 0, n = 0;
      in >> s >> r0 >> n >> in_place;
      std::printf("rope %d\n", ll_rope_rows(g.pool, s, r0, n, g.angles, in_place ? nullptr : g.rope_out, 0, nullptr));
    } else if (op == "books") {
      do_books();
    } else if (op == "lengths") {
      int k = 0;
      in >> k;
      std::vector<int32_t> s(static_cast<size_t>(k));
      for (auto& x : s) in >> x;
      std::vector<int64_t> len(static_cast<size_t>(k), -1);
      const ll_status st = ll_seq_lengths(g.pool, s.data(), k, len.data());
      std::printf("lengths %d", st);
      if (st == LL_OK)
        for (int64_t x : len) std::printf(" %lld", static_cast<long long>(x));
      std::printf("\n");
    } else if (op == "kvs") {
      do_kvs(in);
    } else if (op == "kvsmask") {
      do_kvsmask(in);
    } else if (op == "misc") {
      do_misc();
    } else {
      std::fprintf(stderr, "unknown operation %s\n", op.c_str());
      return 2;
    }
    std::fflush(stdout);
  }
  g.reset();
  return 0;
}
