/*
 * duo.h -- C ABI of libduo: attention over a per-KV-head mixed KV cache on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (DuoAttention): each KV head of each layer is either a retrieval
 * head, which keeps every token and attends over the whole context, or a
 * streaming head, which keeps only S attention-sink tokens plus the W most
 * recent tokens and attends over those ("DuoAttention: Dual Retrieval &
 * Streaming Heads Guide", section "2. DuoAttention Cache Partitioning
 * Mechanics"; the static binary mask M of section "3. Automated Head
 * Identification via Lightweight Optimization").  The mask lives at KV-head
 * granularity so that grouped query heads share their KV head's role (same
 * guide, "Practical Deployment Checklist for Enterprise AI Serving").
 *
 * Notation: L layers, B batch rows, n_q query heads, n_kv KV heads,
 * g = n_q / n_kv, d = d_head, S = sink, W = recent, T_cap = most tokens a
 * retrieval head can hold.  Query head h reads KV head h / g (the
 * repeat_interleave mapping of "Attention Variants and Memory Efficiency",
 * "Multi-Query and Grouped-Query Attention").  Positions are 0-based.
 *
 * Conventions for every entry point:
 *   - Ownership: the caller owns every device buffer (arena, inputs, outputs,
 *     workspace).  The library never allocates or frees device memory; the
 *     only thing it allocates is the small host-side handle.
 *   - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the
 *     default stream) with no implicit synchronisation.  Calls on one cache
 *     must be issued in order on one stream.
 *   - Token counts are kept twice.  The host-side count of each (layer, batch
 *     row) advances when a call is enqueued and is what the library validates
 *     against.  The device-side count, in the arena, is what the kernels read
 *     when they run: an append or a fused decode-append stores its tokens at
 *     the row's device count and advances it, so a step captured in a HIP
 *     graph ("DuoAttention: Dual Retrieval & Streaming Heads Guide",
 *     "Production Advantages and Deployment Considerations", item 1: static
 *     execution graphs) replays as the next step, at the next position.
 *     Replays do not move the host count: call duo_cache_sync before the next
 *     call that is not a replay.  A captured call must be replayed only while
 *     every row holds at least the tokens it held when the call was captured
 *     (replays only move counts forward, so this holds for replays of steps).
 *     A replayed append or decode-append that finds no room (T_cap, or a paged
 *     row past its reserved pages, see duo_cache_reserve) stores nothing,
 *     does not advance, and sets a flag duo_cache_sync reports.  Prefill
 *     chunks and forks set the device counts to the host's values: replaying
 *     one repeats it.
 *   - Errors: 0 (DUO_OK) or a negative DUO_E* code.  Every argument is
 *     validated before anything is enqueued, so a failing call changes no
 *     state.  duo_last_error() returns a message for the calling thread.
 *   - Layout: all tensors are dense row-major in the cache dtype; d is the
 *     fastest axis.
 */
#ifndef DUO_H_
#define DUO_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DUO_OK 0
#define DUO_EINVAL (-1)        /* bad argument, shape, pointer or layer index     */
#define DUO_EUNSUPPORTED (-2)  /* d_head, dtype or group size not built           */
#define DUO_ECAPACITY (-3)     /* seq_len + n_new would exceed T_cap, or no free page */
#define DUO_EEMPTY (-4)        /* decode of a batch row that holds no token       */
#define DUO_EWORKSPACE (-5)    /* workspace missing or smaller than required      */
#define DUO_EHIP (-6)          /* a HIP call or kernel launch failed              */

typedef enum { DUO_F32 = 0, DUO_BF16 = 1 } duo_dtype;

/* How the cache stores K and V rows.  DUO_KV_NATIVE: in the cache dtype.
 * DUO_KV_FP8: as 8-bit E4M3 codes (OCP format: bias 7, largest finite 448)
 * with one fp32 scale per stored row, K and V separately: s = max|x| / 448,
 * code_i = E4M3(x_i / s) rounded to nearest even (a zero row: s = 0, codes 0);
 * attention sees code value * s.  Low-bit KV rows cut the cache to half the
 * bytes on top of the head split ("DuoAttention: Dual Retrieval & Streaming
 * Heads Guide", "Production Advantages and Deployment Considerations", item 2;
 * "Attention Variants and Memory Efficiency", "What the Inference Runtime Can
 * Change": cache precision changes the bytes per stored element, not the
 * attention rule).
 * DUO_KV_INT4: as 4-bit integer codes with one fp32 scale per stored row, K
 * and V separately: s = max|x| / 7, c_i = x_i / s rounded to the nearest
 * integer (ties to even, |c_i| <= 7), stored as the nibble c_i + 8, two per
 * byte (element 2k in the low nibble of byte k); a zero row: s = 0, c = 0;
 * attention sees c_i * s (the same guide item: 4 bits per element).
 * Both are built for dtype bf16 and d_head 128; queries, new tokens and
 * outputs stay bf16. */
typedef enum { DUO_KV_NATIVE = 0, DUO_KV_FP8 = 1, DUO_KV_INT4 = 2 } duo_kv_format;

/* Cache configuration.  d_head in {64, 128}; g = n_q / n_kv any integer from 1
 * to 16 for bf16 with d_head 128 (every kv_format: the scores run on the
 * matrix cores, one query per column of a 16-column tile), from 1 to 8 for
 * fp32 or d_head 64 (the vector-ALU decode); n_kv <= 128; 1 <= B <= 64; S >= 0; W >= 1;
 * 1 <= T_cap <= 2^31 - 4097.  Each batch row keeps
 * its own token count and attends over what it holds (a ragged batch).
 * retrieval_mask is a host array uint8 [L][n_kv] (1 = retrieval head,
 * 0 = streaming head); it is copied.
 *
 * Retrieval rows are stored one of two ways.  page_rows = 0: contiguous, T_cap
 * rows per retrieval head and batch row.  page_rows > 0 (a power of two of at
 * least 64 rows and at least one decode round, 32 KB of stored K rows: 128
 * rows for bf16 at d_head 128, 256 for bf16 at d_head 64 and for DUO_KV_FP8,
 * 512 for DUO_KV_INT4, 64 for fp32 at d_head 128, 128 for fp32 at d_head 64;
 * smaller is DUO_EUNSUPPORTED): paged ("Attention Variants and Memory Efficiency", "What the
 * Inference Runtime Can Change": the runtime may cut a request's rows into
 * equal blocks placed anywhere and shared between requests; "A Closer Look at
 * Attention Memory": a ragged batch then holds only what each request needs).
 * Each layer has a pool of n_pages pages; a page holds page_rows consecutive
 * positions of every retrieval head of one batch row, and a row takes a page
 * from the pool when it grows past its last page.  T_cap still bounds each
 * row (it sizes the page tables).  Streaming heads keep their S + W slots per
 * batch row either way.
 *
 * rope_theta > 0 applies rotary position embedding at each token's logical
 * position, not at the slot a ring buffer gives it ("Attention Variants and
 * Memory Efficiency", "Sliding-Window and Mixed Attention"; "What the
 * Inference Runtime Can Change": the kernel applies the checkpoint's
 * positional treatment).  The rotation is the one of Su et al., "RoFormer:
 * Enhanced Transformer with Rotary Position Embedding": dimensions i and
 * i + d/2 (i < d/2) turn by the angle p * rope_theta^(-2i/d) at position p.
 * Keys are stored rotated (appends, prefill commits, fused appends); queries
 * are rotated at their own position by decode and prefill.  Values are never
 * rotated.  The angle is formed from rope_theta^(-2/d) held to about 104
 * bits and reduced modulo 2 pi in three parts, so that its cosine and sine
 * are within a few double roundings of the exact ones at every position up
 * to 2^31 (see duo_rope_apply); keys are rotated in double and rounded once
 * to the cache dtype, queries are rotated in fp32.
 * rope_theta = 0: queries and keys are used as given. */
typedef struct {
  int32_t L, B, n_q, n_kv, d_head;
  int64_t T_cap;
  int32_t sink, recent;
  int32_t dtype; /* duo_dtype: Q, K, V and outputs; accumulation is fp32 */
  const uint8_t* retrieval_mask;
  int32_t kv_format; /* duo_kv_format of the stored K/V rows (0 = native) */
  int32_t page_rows; /* 0: contiguous retrieval rows; else rows per page (power of two, >= one decode round) */
  int32_t n_pages;   /* paged: pages per layer (>= 1); ignored when page_rows = 0 */
  float rope_theta;  /* 0: no rotary embedding; else its base (> 1, e.g. 10000) */
} duo_config;

typedef struct duo_cache duo_cache; /* opaque host handle */

/* Sizes (host only, no device work).  *arena_bytes: the device arena for
 * duo_cache_init.  It holds, per layer, K and V as [B][n_ret][T_cap][d] for
 * the retrieval heads and [B][n_str][S+W][d] for the streaming heads (the two
 * buffer kinds of the guide's section 2), an int32 position per streaming
 * slot, and for DUO_KV_FP8 an fp32 scale per stored K and V row.  A paged
 * cache holds instead K and V pools [n_pages][n_ret][page_rows][d] (scales
 * [n_pages][n_ret][page_rows]) and an int32 page table
 * [B][ceil(T_cap / page_rows)] per layer.
 * *workspace_bytes: the device scratch that duo_decode, duo_decode_append and
 * duo_prefill_chunk need (partial softmax results; for DUO_KV_FP8 also room
 * for one layer's held rows in bf16, which prefill reads; a prefill with
 * rotary positions needs more, see duo_prefill_workspace_bytes).  Either
 * output pointer may be NULL.  Returns DUO_OK or DUO_EINVAL/DUO_EUNSUPPORTED. */
int duo_cache_bytes(const duo_config* cfg, size_t* arena_bytes, size_t* workspace_bytes);

/* K+V payload bytes of the arena (the KV-cache size the guide's section 2
 * formula counts: retrieval heads T_cap rows, streaming heads S+W rows; for
 * DUO_KV_FP8 the codes plus the row scales; for a paged cache the pools,
 * n_pages * page_rows rows per retrieval head, in place of B * T_cap). */
int duo_cache_payload_bytes(const duo_config* cfg, size_t* payload_bytes);

/* Bind a cache to a caller-owned device arena of at least duo_cache_bytes()
 * bytes, 256-byte aligned.  Enqueues the zeroing of the positions on
 * `stream`; every layer starts empty.  On success *out receives a handle that
 * must be released with duo_cache_free (the arena must outlive it). */
int duo_cache_init(const duo_config* cfg, void* arena, size_t arena_bytes, void* stream,
                   duo_cache** out);

/* Append n_new >= 1 tokens to every batch row of `layer`, row b at positions
 * len_b .. len_b+n_new-1 where len_b is its token count.  k, v: device
 * [B][n_kv][n_new][d].  A retrieval head stores position p in
 * row p.  A streaming head stores p in slot p while p < S, and otherwise in
 * ring slot S + ((p - S) mod W) (sinks fill first, then the window of the
 * guide's section 2; the ring slot rule of "Attention Variants and Memory
 * Efficiency", "Sliding-Window and Mixed Attention"); tokens of the batch that
 * would be evicted before the call ends are not written.  Each written
 * streaming slot records p in its position array.  DUO_ECAPACITY if
 * some row would exceed T_cap, or a paged layer has fewer free pages than the
 * rows' growth needs. */
int duo_append(duo_cache* c, int layer, const void* k, const void* v, int64_t n_new, void* stream);

/* duo_append for batch row `row` alone: k, v device [1][n_kv][n_new][d],
 * positions len_row .. len_row+n_new-1.  With it and duo_prefill_chunk_row
 * the rows of a batch grow independently (a ragged batch: the cache a request
 * needs is its own rows, "Attention Variants and Memory Efficiency", "A
 * Closer Look at Attention Memory"). */
int duo_append_row(duo_cache* c, int layer, int row, const void* k, const void* v, int64_t n_new, void* stream);

/* One decode step on `layer`: the query of every head of batch row b is the
 * token at position len_b-1 (its row's token count less one), which the
 * caller has appended; rows may hold different counts.  q, out: device
 * [B][n_q][d].  Retrieval heads attend over positions 0..len_b-1; streaming
 * heads over their min(len_b, S+W) held tokens (exactly the sinks and the W
 * most recent positions the query may see).  out = softmax(scale * q K^T) V
 * over those keys, accumulated in fp32 and rounded to the cache dtype.
 * ws: device workspace of ws_bytes >= duo_cache_bytes' workspace_bytes.
 * DUO_EEMPTY if a row holds no token. */
int duo_decode(duo_cache* c, int layer, const void* q, void* out, float scale, void* ws,
               size_t ws_bytes, void* stream);

/* One generation step in a single launch: append one token to every batch
 * row (at that row's own count) and decode the query at its position.  Same
 * result and cache state as duo_append(k, v, 1) followed by duo_decode(q)
 * (also for a row that held no token yet): the new token attends to the
 * cached keys of the
 * earlier tokens and to its own, and appending leaves the earlier cached
 * states unchanged ("Attention Variants and KV-Cache Compression", "When Is
 * Reuse Exact?").  Fusing the two neighbouring operations saves a launch per
 * layer and step ("Attention Variants and Memory Efficiency", "What the
 * Inference Runtime Can Change").  The token is written to its row or ring
 * slot while the held rows are read; a streaming slot whose token it evicts
 * is left out of the attention.  k, v: device [B][n_kv][1][d]; q, out: device
 * [B][n_q][d]; ws as for duo_decode.  DUO_ECAPACITY if some row is full
 * (or, paged, no page is free for a row that starts one);
 * other errors as duo_append and duo_decode.  Every row advances by one
 * token. */
int duo_decode_append(duo_cache* c, int layer, const void* k, const void* v, const void* q, void* out,
                      float scale, void* ws, size_t ws_bytes, void* stream);

/* duo_decode_append for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same launch, result and cache state, but the partial
 * softmax records go to a device array inside the library instead of a
 * caller workspace.  That array holds 8 MiB on each GPU the library runs on
 * (it is part of the loaded code object and stays until the process ends);
 * a call whose partial records need more (one per work item, and one per
 * row of a share group for each shared work item: about 2,000 records at
 * g = 8, d_head = 128) fails with DUO_EWORKSPACE and changes no state, and
 * duo_decode_append with a workspace serves it.  The call allocates nothing.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind (no call reads what an earlier one left): calls that may run at the
 * same time on one GPU (other streams, other caches, other threads) race on
 * it and must be ordered by the caller.  Other errors as duo_decode_append. */
int duo_decode_append_noalloc(duo_cache* c, int layer, const void* k, const void* v, const void* q, void* out,
                              float scale, void* stream);

/* Chunked prefill of C >= 1 tokens on `layer`, at positions P .. P+C-1 with
 * P = the rows' token count, equal in every row (DUO_EINVAL otherwise)
 * ("Attention Variants and KV-Cache Compression", "When Is Reuse
 * Exact?": chunk row i attends through absolute key position P + i, and
 * evicted tokens keep their original positions).  q, out: device
 * [B][n_q][C][d]; k, v: device [B][n_kv][C][d].  Retrieval heads: causal
 * attention over positions 0 .. P+i.  Streaming heads: the sink+window mask,
 * key j visible to row i iff j <= P+i and (j < S or j >= P+i-W+1), with keys
 * taken from the held sink and ring slots and from the chunk.  The chunk is
 * attended first and then appended as by duo_append.  With DUO_KV_FP8 the held
 * rows are read as stored (code value * scale) and the chunk's own rows as
 * given, and ws must hold duo_cache_bytes' workspace_bytes (DUO_EWORKSPACE
 * otherwise); a native cache needs no workspace here.  With rope_theta > 0
 * the chunk's queries and keys are rotated at positions P + i into the
 * workspace first (ws must then hold duo_prefill_workspace_bytes for B rows
 * and C tokens).  DUO_ECAPACITY if P + C > T_cap or (paged) the chunk needs
 * more pages than are free. */
int duo_prefill_chunk(duo_cache* c, int layer, const void* q, const void* k, const void* v,
                      int64_t C, void* out, float scale, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes duo_prefill_chunk (rows = B) or duo_prefill_chunk_row
 * (rows = 1) needs for a chunk of C tokens: 0 for a native cache without
 * rotary positions; the decode workspace for DUO_KV_FP8; with rotary
 * positions the decode workspace plus room for the rotated chunk. */
int duo_prefill_workspace_bytes(const duo_cache* c, int rows, int64_t C, size_t* bytes);

/* duo_prefill_chunk for batch row `row` alone, at P = that row's token count:
 * q, out device [1][n_q][C][d]; k, v device [1][n_kv][C][d]. */
int duo_prefill_chunk_row(duo_cache* c, int layer, int row, const void* q, const void* k, const void* v, int64_t C,
                          void* out, float scale, void* ws, size_t ws_bytes, void* stream);

/* Host-side token count of a layer whose rows hold equal counts (advanced at
 * enqueue time); DUO_EINVAL if the rows differ. */
int duo_cache_seq_len(const duo_cache* c, int layer, int64_t* out);

/* Host-side token count of one batch row of a layer. */
int duo_cache_row_len(const duo_cache* c, int layer, int row, int64_t* out);

/* Where one KV head's rows live, for bit-exact inspection of the layout.
 * For a retrieval head of a paged cache, *k_base / *v_base are the head's
 * rows in page 0, *n_slots = page_rows and *head_stride_bytes the distance
 * between consecutive pages; position p of batch row b is then row
 * p mod page_rows of page duo_cache_row_pages(b)[p / page_rows].
 * *k_base / *v_base: device address of the head's first row (batch row b at
 * + b * head_stride_bytes); *pos: device int32 [n_slots] slot positions of a
 * streaming head (NULL for a retrieval head, whose row index is the
 * position); *n_slots: T_cap or S+W; *row_bytes: d * element size;
 * *head_stride_bytes: distance between consecutive batch rows of this head;
 * *pos_stride: int32 elements between consecutive batch rows of *pos. */
int duo_cache_head_view(const duo_cache* c, int layer, int kv_head, int* is_retrieval,
                        void** k_base, void** v_base, int32_t** pos, int64_t* n_slots,
                        int64_t* row_bytes, int64_t* head_stride_bytes, int64_t* pos_stride);

/* Shape of a head-gated forward: one whole sequence of N tokens at positions
 * 0 .. N-1, no cache.  d_head in {64, 128}; n_q a multiple of n_kv (any group
 * size); S = sink >= 0; W = recent >= 1; N >= 1 and N + max(W, 64) < 2^31. */
typedef struct {
  int32_t B, n_q, n_kv, d_head;
  int64_t N;
  int32_t sink, recent;
  int32_t dtype; /* duo_dtype of q, k, v and out; accumulation is fp32 */
} duo_gated_shape;

/* Head-gated attention forward, the pass through which head identification
 * trains its gates ("DuoAttention: Dual Retrieval & Streaming Heads Guide",
 * section 3, item 2: a continuous gate per head mixes full attention and
 * streaming attention over the same queries, keys and values).  For query
 * head h of KV head k = h / g and the row at position t:
 *   out = alpha[k] * A_full + (1 - alpha[k]) * A_stream,
 * where A_full = softmax(scale q K^T) V over the keys j <= t (causal) and
 * A_stream the same over the keys j <= t with j < S or j >= t - W + 1 (the
 * sinks and the window the cache keeps for a streaming head).  One gate per
 * KV head: the roles it relaxes are per KV head.  q, out: device
 * [B][n_q][N][d]; k, v: device [B][n_kv][N][d]; alpha: device float32
 * [n_kv], used as given (not clipped to [0, 1]).  Needs no cache and no
 * workspace; enqueued on `stream`. */
int duo_gated_attention(const duo_gated_shape* shape, const void* q, const void* k, const void* v,
                        const float* alpha, void* out, float scale, void* stream);

/* The rotary position embedding the cache applies (rope_theta in
 * duo_config), on its own: row c of x[b][h] is rotated at position
 * p0[b] + c, dimensions i and i + d/2 turning by the angle
 * (p0[b] + c) * theta^(-2i/d), in double, and rounded once to the dtype.
 * For callers that rotate queries or keys outside the cache so that they
 * agree with the keys it stores, and for checking the angle arithmetic at
 * positions up to the largest a cache row can reach.  x, out: device
 * [B][H][C][d] of `dtype` (duo_dtype); out may be x.  p0: host array of B
 * starting positions, 0 <= p0[b] and p0[b] + C <= 2^31.  1 <= B <= 64,
 * H >= 1, C >= 0, d even with 2 <= d <= 256, theta finite and > 0
 * (DUO_EINVAL otherwise).  Enqueued on `stream`. */
int duo_rope_apply(float theta, int dtype, int B, int H, int64_t C, int d, const int64_t* p0, const void* x,
                   void* out, void* stream);

/* Row scales of one KV head of a DUO_KV_FP8 cache: *k_scale / *v_scale
 * receive the device float [n_slots] scales of batch row 0 (batch row b at
 * + b * *scale_stride floats), in the slot order of duo_cache_head_view (a
 * paged retrieval head: the scales of its rows in page 0, page i at
 * + i * *scale_stride floats).  For
 * a native cache both are set to NULL.  For bit-exact inspection. */
int duo_cache_head_scales(const duo_cache* c, int layer, int kv_head, float** k_scale, float** v_scale,
                          int64_t* scale_stride);

/* Forget batch row `row` of `layer`: its token count becomes 0 and the pages
 * it alone held return to the layer's pool (a finished request of a ragged
 * batch leaves room for the next).  Host only: the device-side count and
 * page-table entries are written ahead of the next call on the layer that
 * takes a stream (or by duo_cache_sync); later calls on the row see an empty
 * row.  Captured calls that involve the row must be captured again. */
int duo_cache_reset_row(duo_cache* c, int layer, int row);

/* How duo_decode / duo_decode_append would cut `layer`'s rows into work
 * items as the rows stand now: *n_items in one launch, *n_shared of them
 * shared items that read the pages a group of forked rows holds in common
 * once for the whole group ("Attention Variants and Memory Efficiency",
 * "What the Inference Runtime Can Change": a matching prefix is stored once;
 * the decode also reads it once).  Groups are consecutive batch rows that
 * hold the same physical pages from position 0 (rows forked from one
 * prefix, see duo_cache_fork_row), at most 16 / g rows each, in bf16 caches
 * of d_head = 128 with g = 4 or 8.  Host only. */
int duo_decode_plan(const duo_cache* c, int layer, int* n_items, int* n_shared);

/* Prefix sharing: batch row dst (which must hold no token) becomes a copy of
 * batch row src of `layer`, with src's token count ("Attention Variants and
 * Memory Efficiency", "What the Inference Runtime Can Change": matching
 * prefixes need not be stored twice).  In a paged cache the full pages of src
 * are shared, not copied: both rows' tables name them, and since a row only
 * ever writes positions past its own count, a full page is never written
 * again.  src's last page, if partly filled, is copied to a page of dst's own;
 * so are the streaming heads' slots, positions and scales.  A contiguous cache
 * copies every held row.  Enqueued on `stream`.  DUO_ECAPACITY if no page is
 * free for the copy.  Decodes read the shared pages once for all the rows
 * holding them when those rows are consecutive batch rows (bf16 queries,
 * d_head = 128, g = 4 or 8, up to 16 / g rows a group; see duo_decode_plan). */
int duo_cache_fork_row(duo_cache* c, int layer, int src_row, int dst_row, void* stream);

/* Bring the host-side token counts up to date with the device-side counts
 * after replays of captured calls: waits for `stream`, then reads every
 * layer's counts back (also writes the counts a duo_cache_reset_row left
 * pending).  DUO_ECAPACITY if some replayed append or decode-append found no
 * room for its tokens since the last sync (it stored nothing and its count
 * did not advance); the flag is then cleared.  Not to be captured. */
int duo_cache_sync(duo_cache* c, void* stream);

/* Give every batch row of `layer` room for n_tokens more tokens now, so that
 * replays of captured steps can advance that far: on a paged layer the pages
 * they will need are taken from the pool (DUO_ECAPACITY if the pool has too
 * few, nothing taken); on a contiguous one the rows already have their T_cap.
 * DUO_ECAPACITY if some row would exceed T_cap. */
int duo_cache_reserve(duo_cache* c, int layer, int64_t n_tokens, void* stream);

/* Pages of `layer` not held by any row (0 for a contiguous cache). */
int duo_cache_free_pages(const duo_cache* c, int layer, int64_t* out);

/* The page table of batch row `row` of a paged layer, as the host keeps it:
 * *n receives the number of pages the row holds (ceil(count / page_rows));
 * the first min(*n, cap) page numbers are written to the host array pages. */
int duo_cache_row_pages(const duo_cache* c, int layer, int row, int32_t* pages, int64_t cap, int64_t* n);

/* Release the host handle (device memory is the caller's). NULL is ignored. */
void duo_cache_free(duo_cache* c);

/* Message for the most recent failing call on this thread ("" if none). */
const char* duo_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DUO_H_ */
