/*
 * leyline.h - C ABI of the MI355X (gfx950) splice / evict library for a paged
 * MLA KV cache.
 *
 * The operations come from two pages:
 *   [Leyline]    "Leyline: KV Cache Directives for Agentic Inference"
 *                (gist.science summary of paper 2606.01065);
 *   [KV-streams] "KV-streams" (onedev.kr summary of paper 273).
 *
 * Cache layout (the MLA split of [Leyline] section 2.2 into the position-free
 * latent K_nope / V and the RoPE band K_pe).  One token of one layer is a row
 * of kv_lora_rank + rope_dim bf16 values: c_kv[0..511] then k_pe[0..63],
 * 1152 bytes.  Each layer has its own pool, an array
 * [num_pages][page_size][row] of bf16 in device memory.  A sequence owns a
 * list of physical pages (its page table), shared by every layer: logical row
 * j of the sequence lives at page table[j / page_size], offset j % page_size.
 *
 * Ownership.  Every device buffer named below (layer pools, page-table array,
 * stub rows, keep masks) belongs to the caller and must stay valid until the
 * stream work of the call that uses it has finished (pools and the page-table
 * array: until ll_pool_destroy).  The library owns its host bookkeeping and a
 * few small device and pinned host staging buffers.
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL: the null stream).
 * Each call enqueues its device work on that stream and returns; the work of a
 * call is ordered after the work of the previous call on the same pool, also
 * across streams.  No call waits for the device, with three exceptions: a
 * kv_evict_compact whose host-made page plan needs one small device-to-host
 * copy first (see there); the first call after a device-planned
 * kv_evict_compact, which waits for that call's results (a small readback)
 * before it reads or changes the pool's bookkeeping; and a call that needs a
 * larger library buffer than any call before it (the staging ring, the
 * eviction scratch, the device-planned splice's plan space, the per-row
 * rotation tables), which waits once for the pool's earlier work before it
 * replaces the buffer, or that finds the 16 MiB staging ring still held by
 * uploads the device has not yet consumed.  A pool is not thread-safe.
 *
 * Errors.  Every function returns an ll_status.  All checks run before any
 * state changes, so a call that returns LL_EINVAL, LL_ERANGE, LL_ENOMEM or
 * LL_EUNSUPPORTED leaves the pool exactly as it was.  A HIP failure after
 * state has changed returns LL_EDEVICE and poisons the pool: every later call
 * on it returns LL_EPOISONED.  No C++ exception leaves the library: host
 * memory running out inside a call returns LL_ENOMEM and also poisons the
 * pool (the call may have stopped half-way).  ll_last_error() gives a message
 * for the calling thread's last failure.
 *
 * Page plan.  When a call rewrites a sequence, new logical page q reuses the
 * old physical page of logical page p iff every live row of q comes from old
 * page p at the same in-page offset; every other new page is fresh and takes
 * the lowest-numbered free page, in order of (position in the batch, q), from
 * the free set as it was when the call began; old pages that are not reused
 * return to the free set after the call.  Rows beyond a sequence's length and
 * rows of free pages hold unspecified values.
 *
 * GQA / MHA caches ([Leyline] section 5: the directive applies unchanged to
 * GQA and MHA caches; only the rotation step differs).  A pool made by
 * ll_pool_create_gqa has, per layer, a K pool and a V pool, each
 * [num_pages][page_size][num_kv_heads][head_dim] bf16 and indexed by the same
 * page table.  The first rotary_dim values of every K head are its RoPE band
 * (pairs interleaved or half-split inside the band); the rest of K and all of
 * V are position-free.  A splice copies V and the non-rotary part of K
 * bit-exactly and turns every downstream K band by R(Delta), with
 * theta_j = rope_base^(-2j/rotary_dim); an eviction moves both K and V rows
 * unchanged.  Every other rule above holds as written, with "row" meaning the
 * K row and the V row of a token together.
 */
#ifndef LEYLINE_H
#define LEYLINE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LL_OK = 0,
  LL_EINVAL = -1,       /* malformed request (bad span, unknown sequence, ...) */
  LL_ERANGE = -2,       /* a sequence would outgrow its page-table row */
  LL_ENOMEM = -3,       /* not enough free pages (or host memory) */
  LL_EUNSUPPORTED = -4, /* reserved mode or unsupported shape */
  LL_EDEVICE = -5,      /* a HIP call failed */
  LL_EPOISONED = -6     /* an earlier device failure left the pool unusable */
} ll_status;

/* Directive modes, [Leyline] section 2.1.  PIN, DECAY and SCRATCH are the
 * verbs that section 5 names for future work: reserved, LL_EUNSUPPORTED. */
enum { LL_AMORTIZE = 0, LL_FORGET = 1, LL_PIN = 2, LL_DECAY = 3, LL_SCRATCH = 4 };

/* RoPE pair layout of k_pe: interleaved pairs (2j, 2j+1), or half-split
 * pairs (j, j + rope_dim/2). */
enum { LL_ROPE_INTERLEAVED = 0, LL_ROPE_HALF = 1 };

typedef struct ll_pool ll_pool;

typedef struct {
  int32_t num_layers;        /* >= 1 */
  int32_t page_size;         /* rows per page: a power of two, 1 .. 256 */
  int32_t num_pages;         /* physical pages per layer pool */
  int32_t max_seqs;          /* page-table rows */
  int32_t max_pages_per_seq; /* page-table columns */
  int32_t kv_lora_rank;      /* c_kv width: must be 512 */
  int32_t rope_dim;          /* k_pe width: must be 64 */
  int32_t rope_pairing;      /* LL_ROPE_INTERLEAVED or LL_ROPE_HALF */
  double rope_base;          /* theta_j = rope_base^(-2j/rope_dim), e.g. 10000 */
  void* const* layer_base;   /* host array [num_layers] of device pointers, each
                                16-byte aligned, to [num_pages][page_size][row] bf16 */
  int32_t* page_table;       /* device int32 [max_seqs][max_pages_per_seq]; the
                                library writes row s for sequence s */
  int32_t device;            /* HIP device ordinal that holds all of the above */
} ll_pool_desc;

/* D = (s_start, s_end, R, m) for one sequence, [Leyline] section 2.1. */
typedef struct {
  int32_t seq_id;
  int32_t mode;              /* LL_AMORTIZE or LL_FORGET */
  int64_t s_start;           /* span [s_start, s_end), 0-based logical rows,
                                0 <= s_start <= s_end <= length */
  int64_t s_end;
  int64_t r_len;             /* |R| >= 0 stub rows */
  const void* r_rows;        /* device bf16 [num_layers][r_len][row], rows already
                                prefilled at their final positions; NULL iff r_len == 0;
                                16-byte aligned.  Ignored by LL_FORGET. */
  int64_t r_layer_stride_bytes; /* bytes between layers of r_rows; 0 means
                                   r_len * row bytes; a multiple of 16 otherwise */
  const void* r_rows_v;      /* GQA / MHA pools: r_rows holds the K rows of R,
                                [num_layers][r_len][num_kv_heads][head_dim], and this
                                the V rows, same shape; NULL iff r_len == 0; 16-byte
                                aligned.  MLA pools: must be NULL. */
  int64_t r_layer_stride_bytes_v; /* bytes between layers of r_rows_v, as above */
} ll_directive;

/* What the last splice / evict / reindex call on a pool did. */
typedef struct {
  int64_t alg_bytes;            /* row bytes the call must move, all layers:
                                   read + write of every live row of a fresh
                                   page, plus read + write of the RoPE bands of
                                   each row rotated in place (MLA: 2*1152 and
                                   2*128 bytes per row and layer; GQA: 2*2*H*D*2
                                   and 2*H*rotary_dim*2) */
  int64_t rows_moved;           /* live rows written to fresh pages (per layer) */
  int64_t rows_rotated_inplace; /* downstream rows of reused pages (per layer) */
  int64_t fresh_pages;
  int64_t freed_pages;
  int64_t table_entries;        /* page-table entries written */
  int64_t planned_on_device;    /* 1: the device made or expanded the page plan
                                   (device-planned eviction, or a splice planned
                                   from kernel arguments); 0: the host did */
} ll_plan_stats;

/* [Leyline] section 3: agent edits become block-level operations on a paged
 * KV store; this is that store.  Create a pool over caller-owned device
 * memory.  Checks the descriptor,
 * copies the layer pointer array to the device and allocates staging.  All
 * pages start free and no sequence exists.  Errors: LL_EINVAL (bad field or
 * NULL pointer), LL_EUNSUPPORTED (row shape other than 512 + 64),
 * LL_EDEVICE. */
ll_status ll_pool_create(const ll_pool_desc* desc, ll_pool** out);

/* A GQA / MHA cache (MHA: num_kv_heads = number of attention heads);
 * [Leyline] section 5: the directive carries over to GQA and MHA caches. */
typedef struct {
  int32_t num_layers;        /* >= 1 */
  int32_t page_size;         /* rows per page: a power of two, 1 .. 256 */
  int32_t num_pages;
  int32_t max_seqs;
  int32_t max_pages_per_seq;
  int32_t num_kv_heads;      /* >= 1 */
  int32_t head_dim;          /* a multiple of 8; num_kv_heads * head_dim <= 32768 */
  int32_t rotary_dim;        /* RoPE band of each K head: a power of two in
                                [16, 256] that divides head_dim */
  int32_t rope_pairing;      /* LL_ROPE_INTERLEAVED or LL_ROPE_HALF, inside the band */
  double rope_base;          /* theta_j = rope_base^(-2j/rotary_dim) */
  void* const* k_layer_base; /* host arrays [num_layers] of device pointers, each */
  void* const* v_layer_base; /*   16-byte aligned, to [num_pages][page_size][H][D] bf16 */
  int32_t* page_table;       /* device int32 [max_seqs][max_pages_per_seq] */
  int32_t device;
} ll_gqa_pool_desc;

/* [Leyline] section 5 (GQA / MHA) over the block store of section 3.
 * Create a GQA / MHA pool over caller-owned device memory; the same calls as
 * for an MLA pool then apply to it.  Errors: LL_EINVAL (bad field or NULL
 * pointer), LL_EUNSUPPORTED (head_dim, rotary_dim or row width outside the
 * ranges above), LL_EDEVICE. */
ll_status ll_pool_create_gqa(const ll_gqa_pool_desc* desc, ll_pool** out);

/* [Leyline] section 3 (block-level KV store): end of a pool's life.
 * Wait for the pool's device work and free what the library allocated.  The
 * caller's buffers are not touched.  NULL is ignored. */
void ll_pool_destroy(ll_pool* pool);

/* [Leyline] section 3 (block-level KV store): a sequence's pages.
 * New sequence of n_tokens >= 0 rows: the lowest free sequence id and the
 * ceil(n_tokens / page_size) lowest free pages; next position = n_tokens.
 * Row contents are the caller's to write (prefill).  Errors: LL_EINVAL,
 * LL_ERANGE, LL_ENOMEM (no free id or pages). */
ll_status ll_seq_alloc(ll_pool* pool, int64_t n_tokens, int32_t* seq_id_out, void* stream);

/* [Leyline] section 3 (block-level KV store): a sequence's page table.
 * Give sequence seq_id (new or existing) an explicit page table: `pages` is a
 * host array of ceil(n_tokens / page_size) distinct physical pages, each free
 * or already owned by seq_id.  Pages the sequence held and no longer lists are
 * freed; next position = n_tokens.  Errors: LL_EINVAL, LL_ERANGE. */
ll_status ll_seq_set_pages(ll_pool* pool, int32_t seq_id, const int32_t* pages,
                           int64_t n_tokens, void* stream);

/* [Leyline] section 3 (block-level KV store): release a sequence and all of
 * its pages.  Errors: LL_EINVAL. */
ll_status ll_seq_free(ll_pool* pool, int32_t seq_id);

/* [Leyline] section 2.2 (positions move by Delta) and [KV-streams] "how it
 * works" (eviction keeps positions), read back from the block store of
 * [Leyline] section 3.
 * Host copy of a sequence's state: length, next RoPE position and up to `cap`
 * page-table entries (pages_out may be NULL when cap == 0); *n_pages_out gets
 * the page count.  Errors: LL_EINVAL. */
ll_status ll_seq_get(const ll_pool* pool, int32_t seq_id, int64_t* len, int64_t* next_position,
                     int32_t* pages_out, int32_t cap, int32_t* n_pages_out);

/* [Leyline] section 3 (block-level KV store): number of free pages.
 * Errors: LL_EINVAL. */
ll_status ll_pool_free_pages(const ll_pool* pool, int64_t* n_free);

/* Apply n directives, at most one per sequence ([Leyline] sections 2.1-2.3).
 *
 * LL_AMORTIZE: the sequence becomes old[0, s_start) ++ R ++ old[s_end, n),
 * n' = n + Delta with Delta = r_len - (s_end - s_start) (section 2.2).
 * Prefix rows and the R rows are copied bit-exactly.  Every downstream row
 * keeps its c_kv bit-exactly and gets k_pe_new = R(Delta) k_pe: each pair
 * (x, y) turns by the angle Delta*theta_j, with cos/sin evaluated in float64
 * and rounded to float32, then x' = x*c - y*s and y' = x*s + y*c in float32
 * (no fused multiply-add) and rounded to bf16, nearest-even.  The next
 * position moves by Delta.  On a GQA / MHA pool the K and V rows of R are
 * copied, V and the non-rotary K values of downstream rows stay bit-exact and
 * each K head's RoPE band turns as k_pe does.
 * LL_FORGET: the sequence is cut to its first s_start rows (the caller then
 * re-prefills, section 2.1); the next position moves back by n - s_start.
 *
 * The host makes the page plan.  With the default planner
 * (ll_pool_set_splice_planner) a batch of at most 16 directives (GQA / MHA
 * pools: at most 1024 / rotary_dim) whose fresh pages form at most 256 runs of
 * consecutive page ids travels as kernel arguments: a small kernel expands it
 * into per-page tasks and new page-table rows, reading the old rows from the
 * device page table, and the row kernel (fresh pages, in-place rotation and
 * the page-table rewrite in one launch) follows on the same stream; nothing
 * is copied to the device and the call records no event of its own.  Other
 * batches, and every batch under LL_SPLICE_PLAN_HOST, have their tasks written
 * by the host into pinned staging and uploaded (one host-to-device copy, on
 * the pool's copy stream when earlier work is queued) before the same row
 * kernel.  Both planners give the same result.  n == 0 is a no-op.  Errors:
 * LL_EINVAL (bad span, unknown or repeated sequence, r_rows (GQA: or
 * r_rows_v) NULL with r_len > 0, r_rows_v given to an MLA pool, misaligned
 * pointer or stride), LL_EUNSUPPORTED (reserved mode, or a call that would
 * write 2^32 or more 16-byte chunks into one layer: 64 GiB of rows per
 * layer), LL_ERANGE (n' exceeds max_pages_per_seq pages), LL_ENOMEM (too
 * few free pages), LL_EDEVICE.  A call may move more than 2^32 chunks over
 * all its layers (ll_pool_set_dispatch_limit). */
ll_status leyline_splice(ll_pool* pool, const ll_directive* dirs, int32_t n, void* stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * splice as leyline_splice (same arguments, results and errors), with the
 * page plan expanded on the device into a library-owned static device array
 * of 4 MiB per device instead of the pool's growable plan space: the call
 * allocates no device or pinned memory, creates no event and times no
 * launch (ll_pool_set_profiling does not apply to it).  Only batches the
 * device plans itself qualify -- at most 16 directives (GQA / MHA pools:
 * 1024 / rotary_dim), fresh pages in at most 256 runs of consecutive ids,
 * and a plan of at most 4 MiB (about 60 000 page tasks, 64 bytes each, plus
 * the new page-table rows) -- whatever ll_pool_set_splice_planner says;
 * other batches return LL_EUNSUPPORTED with nothing changed.  Every call on
 * a device uses that device's one array and leaves its contents there for
 * the next call to overwrite: calls on one pool are ordered by the pool, but
 * calls on different pools of the same device that can overlap in time (on
 * streams with no ordering between them) race on the array. */
ll_status leyline_splice_noalloc(ll_pool* pool, const ll_directive* dirs, int32_t n, void* stream);

/* KV-streams eviction ([KV-streams] "how it works"): for each of the n
 * sequences seq_ids[i], keep exactly the rows whose keep byte is nonzero, in
 * order, unchanged (no rotation, no position reset: the next position stays).
 * keep_dev is a device uint8 buffer; sequence i's mask is its length-many
 * bytes starting at keep_dev + keep_offsets[i] (keep_offsets is a host
 * array).  A device prefix scan gives each kept row its new index; rows move
 * only where a new page cannot reuse an old one (at page size 1 none move).
 *
 * Page plan, always made on the device: fresh pages are the lowest free
 * pages in (batch position, page) order, found by rank/select on the free
 * bitmap.  Page size > 1: the call waits once for a small device-to-host
 * copy of the device's verdict (fresh pages needed, and whether they exceed
 * the free ones); a shortage returns LL_ENOMEM with nothing changed,
 * otherwise the rows move and the tables are rewritten on the device and the
 * call returns without waiting for them.  Page size 1 (nothing moves, no
 * page is fresh): the call returns without waiting at all, and the pool's
 * host bookkeeping (lengths, free set, ll_last_plan_stats) catches up when
 * the pool is next used.  Host copies of the rewritten page tables are
 * fetched from the device only when read (ll_seq_get, a later call on that
 * sequence).  Errors: LL_EINVAL, LL_EUNSUPPORTED (the sequences' pages
 * hold 2^32 or more 16-byte chunks per layer: 64 GiB of rows per layer),
 * LL_ENOMEM, LL_EDEVICE. */
ll_status kv_evict_compact(ll_pool* pool, const int32_t* seq_ids, int32_t n,
                           const uint8_t* keep_dev, const int64_t* keep_offsets, void* stream);

/* Page-table re-index: page-granular eviction without row moves
 * ([Leyline] section 3, edits decomposed into block-level operations;
 * [KV-streams] "how it works").  keep_pages is a host array of n_keep strictly
 * increasing logical pages of the sequence; the new table lists their physical
 * pages in that order and the new length is the sum of their live rows; a
 * partial last page may only be kept last.  Other pages are freed; the next
 * position stays.  Errors: LL_EINVAL. */
ll_status ll_ptable_reindex(ll_pool* pool, int32_t seq_id, const int32_t* keep_pages,
                            int32_t n_keep, void* stream);

/* Per-row-angle RoPE rotation of the rows [row_begin, row_begin + n_rows) of a
 * sequence: row row_begin + i has every RoPE band (MLA: k_pe; GQA / MHA: the
 * rotary part of each K head) turned by R(a_i), a_i = angle_dev[i] (device
 * int64 [n_rows]).  An angle of minus the row's position turns a stored key
 * back to its position-free form -- the step VECTOR takes before its static
 * K -> V reconstruction ("VECTOR", gist.science summary of paper 2605.23258,
 * method: reconstructability through OLS).  Per row and pair the float64
 * angle a_i * theta_j and its float64 cos and sin (argument reduction on the
 * device) are rounded to float32; the pair then turns with the float32
 * arithmetic of leyline_splice.
 *
 * out_dev == NULL: in place, only the bands are written.  Otherwise the rows
 * are gathered, bands turned, into out_dev (device, 16-byte aligned):
 * [num_layers][n_rows][row] bf16 (MLA rows of 576; GQA: the K rows, H x D),
 * layers out_layer_stride_bytes apart (0: n_rows * row bytes); the pool is
 * not written.  V planes never take part.  Errors: LL_EINVAL (unknown
 * sequence, rows outside it, NULL angles, misaligned output or stride),
 * LL_EUNSUPPORTED, LL_ENOMEM, LL_EDEVICE. */
ll_status ll_rope_rows(ll_pool* pool, int32_t seq_id, int64_t row_begin, int64_t n_rows,
                       const int64_t* angle_dev, void* out_dev, int64_t out_layer_stride_bytes,
                       void* stream);

/* The float32 cos/sin table of the delta-rotation ([Leyline] section 2.2):
 * for j < rope_dim/2, the float64 angle delta * base^(-2j/rope_dim), its
 * float64 cos and sin, each rounded to float32.  cos_out and sin_out are host
 * arrays of rope_dim/2 floats.  Errors: LL_EINVAL. */
ll_status ll_rope_delta_table(double base, int32_t rope_dim, int64_t delta,
                              float* cos_out, float* sin_out);

/* Library bookkeeping, no passage of the pages defines it: counters of the
 * last splice / evict / reindex / per-row rotation call.  Errors: LL_EINVAL. */
ll_status ll_last_plan_stats(const ll_pool* pool, ll_plan_stats* out);

/* Library bookkeeping, no passage of the pages defines it: the first three
 * counters of ll_last_plan_stats -- the algorithmic row bytes of the last
 * call, the rows it wrote to fresh pages (per layer) and the rows it turned in
 * place (per layer).  Any output pointer may be NULL.  Errors: LL_EINVAL. */
ll_status ll_last_plan_bytes(const ll_pool* pool, int64_t* alg_bytes, int64_t* rows_moved,
                             int64_t* rows_rotated_inplace);

/* Library bookkeeping, no passage of the pages defines it: the current length
 * of each of n sequences seq_ids[i] into lengths_out[i] (host arrays), e.g. to
 * size keep masks for kv_evict_compact.  Errors: LL_EINVAL (unknown
 * sequence). */
ll_status ll_seq_lengths(const ll_pool* pool, const int32_t* seq_ids, int32_t n, int64_t* lengths_out);

/* Library bookkeeping, no passage of the pages defines it.
 * Who expands a splice batch's page plan (see leyline_splice):
 * LL_SPLICE_PLAN_AUTO (the default) lets the device do it when the batch
 * fits in kernel arguments; LL_SPLICE_PLAN_HOST always stages and uploads the
 * host's tasks.  Results do not depend on the choice.  Errors: LL_EINVAL. */
typedef enum { LL_SPLICE_PLAN_AUTO = 0, LL_SPLICE_PLAN_HOST = 1 } ll_splice_planner;
ll_status ll_pool_set_splice_planner(ll_pool* pool, int32_t planner);

/* Library setting, no passage of the pages defines it: the page plan's reuse
 * rule ([Leyline] section 2.3 decomposes an edit into block-level operations;
 * keeping an old page whose rows stay at their offsets is this library's).
 * on = 1 (the default): a new page keeps an old one when all its live rows are
 * rows of that page at unchanged offsets, as described at the top of this
 * file.  on = 0: no new page keeps an old one -- every page of a sequence that
 * leyline_splice (AMORTIZE or FORGET), leyline_splice_noalloc or
 * kv_evict_compact rewrites is fresh (lowest free pages first, in batch
 * order), every live row is written into it (downstream k_pe turned as
 * always) and every old page of the sequence is freed; row values, lengths
 * and positions are the same as with reuse on, only the physical pages differ
 * (a compaction of the sequence into the lowest free pages).  Such calls need
 * as many free pages as the new pages of their sequences.  Applies to calls
 * made after it; ll_ptable_reindex moves no rows and is not affected.
 * Errors: LL_EINVAL (on not 0 or 1), LL_EUNSUPPORTED (on = 0 on a pool of
 * page size 1, where a page is one row). */
ll_status ll_pool_set_page_reuse(ll_pool* pool, int32_t on);

/* Library setting, no passage of the pages defines it.
 * Work-items one dispatch of a row-moving kernel may hold.  A dispatch packet
 * counts them in 32 bits, so 0 (the default) means 2^32 - 1.  A splice,
 * eviction or per-row gather whose grid would hold more is issued as several
 * dispatches in order on the same stream: the splice's in-place band
 * rotation on its own, then ranges of whole page tasks over every layer (the
 * page-table rewrites in the last one); the gather by ranges of whole layers.
 * Results do not depend on the split.  A smaller limit (at least 1024) splits
 * smaller launches the same way; it exists to exercise the split.  Applies to
 * calls made after it.  Errors: LL_EINVAL (out of range). */
ll_status ll_pool_set_dispatch_limit(ll_pool* pool, int64_t max_items);

/* Library bookkeeping, no passage of the pages defines it.
 * Kernel timing.  `enable` = n > 0 times every n-th launch (counted from
 * this call; 1: every launch) of the row-moving kernel (kernel 0; on the
 * device-planned eviction path its page-plan kernels too), of the keep-mask
 * scan (kernel 1) and of the per-row rotation (kernel 2: its table and row
 * kernels together); 0 stops timing.  A timed launch gets a pair of HIP
 * events that it stamps from its own dispatch packets (the start of its
 * first kernel, the end of its last); the stamps still cost the stream a few
 * microseconds per timed launch, hence the sampling.
 * ll_profile_read waits for the recorded events, returns the launch count,
 * the summed milliseconds and the summed algorithmic bytes of `kernel`, puts
 * the milliseconds of the first each_cap timed launches, in launch order,
 * into each_ms (host floats; NULL when each_cap is 0), and clears the
 * record.  Any other output pointer may be NULL.  Errors: LL_EINVAL,
 * LL_EDEVICE. */
ll_status ll_pool_set_profiling(ll_pool* pool, int32_t enable);
ll_status ll_profile_read(ll_pool* pool, int32_t kernel, int64_t* launches, double* total_ms,
                          int64_t* total_bytes, float* each_ms, int64_t each_cap);

/* ------------------------------------------------------------------------
 * KV-streams trainer-side attention mask ([KV-streams] "how it works": the
 * trainer reproduces the engine's evictions with a custom attention mask, so
 * that one forward pass over a whole rollout lets every token see exactly the
 * keys the cache held when that token was generated).
 *
 * A rollout is n_tokens tokens in generation order.  An eviction event
 * (time t, keep) ran after t tokens had been generated and before token t:
 * keep is the keep mask over the rows the cache held then, in order -- the
 * mask the engine passed to kv_evict_compact.  The death time d_k of token k
 * is the time of the event that dropped it (n_pad if none; k for padding keys
 * k >= n_tokens of a batch padded to n_pad), and query q sees key k iff
 * k <= q < d_k.  Positions are the original token indices (no reset).
 *
 * The calls below take a context (staging and scratch on one device) and
 * enqueue their work on `stream`; a context is not thread-safe.  All buffers
 * are caller-owned device memory and must stay valid until the work is done.
 */
typedef struct kvs_ctx kvs_ctx;

typedef struct {
  int64_t n_tokens;          /* rollout length, <= n_pad */
  int32_t n_events;
  const int64_t* event_time; /* host [n_events]: strictly increasing, in (0, n_tokens] */
  const int64_t* mask_len;   /* host [n_events]: rows the cache held at each event */
  int64_t mask_offset;       /* bytes into keep_dev of the rollout's first keep mask;
                                its other masks follow back to back */
} kvs_rollout_log;

/* [KV-streams] "how it works" (the trainer's mask).  Create / destroy a
 * context on HIP device `device`.  Errors: LL_EINVAL, LL_EDEVICE. */
ll_status kvs_ctx_create(int32_t device, kvs_ctx** out);
void kvs_ctx_destroy(kvs_ctx* ctx);

/* [KV-streams] "how it works": the engine's eviction pattern, replayed.
 * Death times of n rollouts: death_dev is int32 [n][n_pad] (rollout i at
 * i * n_pad), status_dev int32 [n].  The logs are replayed on the device:
 * the rows held at an event are the tokens held after the previous event
 * followed by the tokens generated since, and the token of row i dies at the
 * event's time when keep byte i is 0.  status_dev[i] is
 * 0, or 1 when some event's mask_len differs from the number of rows the
 * cache held at that time (the rollout's death times are then unspecified).
 * The host arrays are read before the call returns.  The context stages
 * the logs in four regions taken in turn; a call waits on the host only when
 * its region's last user (the call four calls earlier) has not finished.
 * The replay keeps 8 bytes per 32 mask rows and 4 per event in a
 * context-owned scratch: a call on another stream waits on the device for
 * the last call,
 * and one that must grow the scratch waits on the host for it.
 * Errors: LL_EINVAL
 * (n_pad outside [1, 2^31 - 2], n_tokens > n_pad, event times not increasing
 * inside (0, n_tokens], mask_len outside [0, time], NULL pointers),
 * LL_EUNSUPPORTED (n * ceil(n_pad / 256) of 2^31 or more), LL_ENOMEM,
 * LL_EDEVICE. */
ll_status kvs_death_times(kvs_ctx* ctx, const kvs_rollout_log* logs, int32_t n, int64_t n_pad,
                          const uint8_t* keep_dev, int32_t* death_dev, int32_t* status_dev, void* stream);

/* [KV-streams] "how it works": the trainer's custom attention mask, as tiles.
 * Block mask from death times: the n_pad x n_pad mask of each rollout cut
 * into block_q x block_k tiles (powers of two in [16, 1024]; edge tiles are
 * cut at n_pad).  A tile is full when every entry is visible, empty when none
 * is, partial otherwise.  With nq = ceil(n_pad / block_q) and
 * nk = ceil(n_pad / block_k): partial_num / full_num are int32 [n][nq] and
 * partial_idx / full_idx int32 [n][nq][nk]; row (i, b) lists the partial
 * (full) key blocks of query block b in increasing order, the entries past
 * the count are left as they were.  An attention kernel skips empty tiles,
 * needs no mask on full tiles and applies k <= q < d_k on partial ones.
 * Errors: LL_EINVAL, LL_ENOMEM, LL_EDEVICE. */
ll_status kvs_block_mask(kvs_ctx* ctx, const int32_t* death_dev, int32_t n, int64_t n_pad,
                         int32_t block_q, int32_t block_k, int32_t* partial_num, int32_t* partial_idx,
                         int32_t* full_num, int32_t* full_idx, void* stream);

/* [KV-streams] "how it works": the trainer's custom attention mask, as bits.
 * Dense bit mask from death times: bits_dev is uint32 [n][n_pad][n_pad / 32]
 * (16-byte aligned; n_pad a multiple of 128); bit b of word w of row q of
 * rollout i is 1 iff query q sees key 32 w + b, i.e. k <= q < d_k for any
 * int32 death times (values at or below k, or at or beyond n_pad, included).
 * For n_pad <= 262144 the call keeps a context-owned device scratch of
 * n * (64 + 5 * n_pad / 8) bytes (plus 256 of alignment), reused call after
 * call: a later call on another stream waits on the device for the last one,
 * and a call that must grow the scratch first waits on the host for the last
 * call to finish.  Errors: LL_EINVAL, LL_ENOMEM, LL_EDEVICE, and
 * LL_EUNSUPPORTED when one launch cannot cover the mask: n * n_pad / 32
 * blocks (n_pad <= 262144), or n * ceil(n_pad / 128) * ceil(n_pad / 8192) / 4
 * blocks, reach 2^31. */
ll_status kvs_dense_mask(kvs_ctx* ctx, const int32_t* death_dev, int32_t n, int64_t n_pad,
                         uint32_t* bits_dev, void* stream);

/* Library bookkeeping, no passage of the pages defines it: message for the
 * calling thread's last failure ("" if none). */
const char* ll_last_error(void);

/* Library bookkeeping, no passage of the pages defines it: name of a status
 * code. */
const char* ll_status_str(ll_status status);

#ifdef __cplusplus
}
#endif

#endif /* LEYLINE_H */
