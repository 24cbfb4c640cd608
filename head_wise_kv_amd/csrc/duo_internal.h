// Internal declarations shared by the host library (duo_host.cpp) and the HIP
// kernels (duo_kernels.hip, duo_prefill.hip, duo_gated.hip).  Not part of the
// public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace duo {

constexpr int kMaxKV = 128;        // KV heads per layer the head maps can hold
constexpr int kMaxRows = 64;       // batch rows per cache (each row keeps its own token count)
constexpr int kMaxDecodeBlocks = 1024;  // decode work items per call at most
constexpr int kDecodeThreads = 512;  // 8 wavefronts of 64

// Per-layer head tables: role and compact index of each KV head, and the KV
// head behind each compact retrieval / streaming index.
struct HeadMap {
  int8_t kind[kMaxKV];      // kv head -> 1 retrieval, 0 streaming
  int8_t cidx[kMaxKV];      // kv head -> index among heads of its kind
  int8_t orig_ret[kMaxKV];  // compact retrieval index -> kv head
  int8_t orig_str[kMaxKV];  // compact streaming index -> kv head
};

// Device addresses of one layer inside the arena.
struct LayerPtrs {
  char* k_ret;     // [B][n_ret][cap_ret][d]; paged: [n_pages][n_ret][page rows][d]
  char* v_ret;
  char* k_str;     // [B][n_str][cap_str][d]
  char* v_str;
  int32_t* pos;    // [B][n_str][cap_str]
  // FP8 rows only (else null): one fp32 scale per stored row
  float* ksc_ret;  // [B][n_ret][cap_ret]
  float* vsc_ret;
  float* ksc_str;  // [B][n_str][cap_str]
  float* vsc_str;
  // Paged retrieval rows (table null: contiguous).  table[b * max_pages + i]
  // is the page holding positions [i << page_shift, (i + 1) << page_shift)
  // of every retrieval head of batch row b.
  int32_t* table;
  int32_t max_pages;
  int32_t page_shift;
  // Token count of each batch row ([B], device), read by the kernels when they
  // run and advanced by the appends: a step captured in a HIP graph replays
  // as the next step.  `status` (one word per cache): bit 0 is set when a
  // step found no room for its tokens (it then stored nothing and the count
  // did not advance).
  int32_t* len;
  int32_t* status;
  int64_t cap;     // T_cap: positions a row may hold
};


// Rotary position embedding (on = 0: keys and queries are used as given).
// Pair i of a head's dimensions, (i, i + d/2), turns by p * theta^(-2i/d) at
// position p.  b_k = theta^(-2 * 2^k / d) as double-doubles
// (hi[k] + lo[k]) for k < kRopeBits, from make_rope, so that the frequency
// of pair i is the product of the b_k of i's set bits; on = 0 for none.
constexpr int kRopeBits = 7;  // pairs i < 128 (d <= 256)
struct Rope {
  double hi[kRopeBits], lo[kRopeBits];
  int on;
};

// int32 words written before the kernels that read them (same stream): page
// table entries, and token counts set by the host (prefill, fork, reset).
constexpr int kMaxTableUpdates = 240;
struct TableUpdateArgs {
  int32_t* table;
  int n;
  int32_t index[kMaxTableUpdates];
  int32_t page[kMaxTableUpdates];
};

// Advance the token counts of rows [0, B) of a layer by n after an append
// that read them (each row only if it had room, else the status bit).
struct AdvanceArgs {
  LayerPtrs lp;
  int B;
  int64_t n;
};

// Device copies of byte ranges: segment i copies `count` blocks of `bytes`
// (a multiple of 4) from src + j * src_stride to dst + j * dst_stride.
constexpr int kMaxCopySegments = 12;
struct CopySegment {
  const char* src;
  char* dst;
  int64_t bytes, count, src_stride, dst_stride;
};
struct CopyArgs {
  int n;
  CopySegment seg[kMaxCopySegments];
};

struct AppendArgs {
  // p0 from the device: each row's first position is its count in lp.len
  // at execution (duo_append, duo_append_row), else p0[] (a prefill commit,
  // which then sets the counts to p0 + n_new).
  int p0_from_device;
  const char* k;   // [B][n_kv][n_new][d]
  const char* v;
  LayerPtrs lp;
  HeadMap map;
  int B, n_kv, n_ret, n_str;
  int row_bytes;      // bytes per stored row
  int in_row_bytes;   // bytes per input row (equal unless the rows are stored as FP8)
  int64_t cap_ret, cap_str;
  int64_t n_new;          // tokens per batch row
  int32_t p0[kMaxRows];   // first position of each batch row (its token count before the call)
  int S, W;
  int dtype;              // 0 = fp32, 1 = bf16 (of the inputs)
  int d;
  Rope rope;              // K rows are rotated at their position before they are stored
};

// Per batch row of a decode: the rows it held when the call was planned and
// its work items.  The kernel reads the row's count (lp.len) when it runs:
// the last work item of a head ends at the rows held then, and a fused
// append's new token goes to that position, so a replayed step that finds
// more tokens than were planned for covers them.
struct DecodeRow {
  int32_t rows_ret, rows_str;    // rows per retrieval / streaming head at planning (before a fused append)
  int32_t nb_ret, nb_str;        // work items per retrieval / streaming head of this row (each >= 1)
  int32_t first_ret, first_str;  // index of the first work item of the row's retrieval / streaming heads
};

// A row of a share group: the rows of its retrieval heads that shared items
// read for it (the full pages it shares with the other rows of its group;
// 0: none).  The row's own retrieval items cover positions sh_rows ..
// rows_ret; the shared items' sh_nb partial records for its retrieval head r
// are records sh_rec + r * sh_nb + part.
struct DecodeRowShare {
  int32_t sh_rows, sh_rec, sh_nb;
};

// Rows R of a share group (batch rows b0 .. b0 + R - 1, forked from one
// prefix) hold the same physical pages for positions 0 .. rows - 1.  Shared
// work items read those rows once and attend every row's queries to them:
// nb items per retrieval head, head r's at first + r * nb.  Item (head r,
// part p) writes a record for each row i of the group: record
// rec + (i * n_ret + r) * nb + p.
constexpr int kMaxShares = 16;
struct DecodeShare {
  int32_t first, b0, R, rows, nb, rec;
};
// Partial records of one decode at most: one per work item, and up to four
// per shared item (one per row of its group).
constexpr int64_t kMaxDecodeRecords = 5 * (int64_t)kMaxDecodeBlocks;

struct DecodeArgs {
  const void* q;   // [B][n_q][d]
  void* out;       // [B][n_q][d]
  LayerPtrs lp;
  HeadMap map;
  float* ws1;      // partial records [work item][g][d + 2]
  int B, n_q, n_kv, n_ret, n_str;
  int64_t cap_ret, cap_str;     // rows reserved per head
  int32_t items_ret;            // work items of all retrieval heads (they come first)
  int32_t multi;                // nonzero if some head spans several work items
  int32_t S, W;
  float scale_log2;             // softmax scale * log2(e)
  // Fused append (decode of a token appended by the same call); new_k is
  // null for a plain decode.  The rows counts are then those held before the
  // append; the last work item of every head adds the new token and writes
  // it to the cache.
  const char* new_k;            // [B][n_kv][d]
  const char* new_v;
  DecodeRow rows[kMaxRows];     // items ordered: row 0's retrieval heads, row 1's, ..., then streaming likewise
  // Queries (and a fused append's new K row) are rotated at the query's
  // position: the row's count for a fused append, the count - 1 otherwise.
  // Last: it is read after the first loads are issued, and the fields before
  // it keep the argument lines the item lookup reads (moving them measured
  // up to 1% slower decode steps).
  Rope rope;
  // Share groups, read only by the kernels launched for a plan that has
  // some (kept after the fields above so that those keep their places).
  // Shared items come after the streaming items, from items_sh; records end
  // at n_records.
  int32_t items_sh, n_share, n_records;
  DecodeShare share[kMaxShares];
  DecodeRowShare rsh[kMaxRows];
};

struct PrefillArgs {
  const void* q;     // [B][n_q][C][d]
  const void* k;     // [B][n_kv][C][d]
  const void* v;
  void* out;         // [B][n_q][C][d]
  LayerPtrs lp;
  HeadMap map;
  int B, n_q, n_kv, n_ret, n_str;
  int64_t cap_ret, cap_str;
  int64_t P;          // tokens cached before the chunk
  int64_t C;          // chunk length
  int64_t held_str;   // streaming slots holding a token before the chunk: min(P, S+W)
  int S, W;
  float scale_log2;
  int q_tiles;        // ceil(C / rows per work item)
  int items_ret;      // B * n_ret * (g / heads per item) * q_tiles (retrieval items come first)
};

// Head-gated forward over one whole sequence (no cache): row t of query head
// h gets alpha[h / g] * causal attention + (1 - alpha[h / g]) * sink + window
// attention.
struct GatedArgs {
  const void* q;       // [B][n_q][N][d]
  const void* k;       // [B][n_kv][N][d]
  const void* v;
  const float* alpha;  // [n_kv]
  void* out;           // [B][n_q][N][d]
  int B, n_q, n_kv, S, W;
  int64_t N;           // tokens, positions 0 .. N-1
  float scale_log2;
  int q_tiles;         // ceil(N / rows per work item)
};

// Prefill with rotary positions: the chunk's queries and keys rotated at
// positions p0[b] + i into the workspace (same layouts), before the attention.
struct RopeArgs {
  const void* q;   // [B][n_q][C][d]
  const void* k;   // [B][n_kv][C][d]
  void* q_out;
  void* k_out;
  int B, n_q, n_kv, d, dtype;
  int64_t C;
  int32_t p0[kMaxRows];
  Rope rope;
};

// The allocation-free decode's partial records live in a file-scope device
// array of this many bytes (duo_kernels.hip), one copy per device.
constexpr size_t kStaticScratchBytes = size_t{8} << 20;
// Device address of that array on the current device (looked up once per
// device, then cached).
hipError_t static_scratch(void** ptr);

// Launchers (duo_kernels.hip, duo_prefill.hip, duo_gated.hip).  dtype: 0 = fp32, 1 = bf16.
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_fill_ones(void* p, size_t bytes, hipStream_t s);  // every byte 0xFF (int32 -1)
hipError_t launch_advance(const AdvanceArgs& a, hipStream_t s);
hipError_t launch_table_update(const TableUpdateArgs& a, hipStream_t s);
hipError_t launch_copy(const CopyArgs& a, hipStream_t s);
hipError_t launch_rope(const RopeArgs& a, hipStream_t s);
// kvfmt: 0 = rows in the cache dtype, 1 = FP8 codes, 2 = INT4 codes (with row scales).
hipError_t launch_append(const AppendArgs& a, int dtype, int d, int kvfmt, hipStream_t s);
// FP8 caches: the held rows of one layer, dequantized to bf16 for prefill.
struct DequantArgs {
  LayerPtrs src;               // codes and scales in the arena
  LayerPtrs dst;               // bf16 rows (k/v pointers only), [B][n_ret][cap_ret_dst][d] and [B][n_str][cap_str][d]
  int64_t heads_ret, heads_str;  // B * n_ret, B * n_str
  int64_t cap_ret_src, cap_ret_dst, rows_ret;
  int64_t cap_str, rows_str;
  int d;
  int n_ret;
  int int4;                    // rows are INT4 codes (two per byte) rather than FP8
};
hipError_t launch_dequant(const DequantArgs& a, hipStream_t s);
// Split phase over `blocks` work items (retrieval heads' items first), then
// the combine of heads cut into several items.
hipError_t launch_decode(const DecodeArgs& a, int dtype, int d, int g, int kvfmt, int blocks, hipStream_t s);
// Rows one round of the decode kernel covers (a work item should span at least one).
int64_t decode_round_rows(int dtype, int d, int g, int kvfmt);
hipError_t launch_prefill(const PrefillArgs& a, int dtype, int d, int g, hipStream_t s);
// Query rows and query heads one prefill work item covers.
void prefill_plan(int dtype, int d, int g, int* rows_per_item, int* heads_per_item);
hipError_t launch_gated(const GatedArgs& a, int dtype, int d, int g, hipStream_t s);
// Query rows one gated-forward work item covers.
int gated_rows_per_item(int dtype, int g);

}  // namespace duo
