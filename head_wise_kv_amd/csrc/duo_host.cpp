// libduo host side: the C ABI of include/duo.h.  Validates arguments, plans
// the arena layout and the decode work split, keeps the per-layer token
// counts, and enqueues the HIP kernels of duo_kernels.hip.  It never allocates
// device memory: the arena and workspace belong to the caller.
#include "duo.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "duo_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return DUO_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(DUO_EHIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct LayerPlan {
  int n_ret = 0, n_str = 0;
  size_t off_kr = 0, off_vr = 0, off_ks = 0, off_vs = 0, off_pos = 0;
  size_t off_tab = 0;  // paged caches: int32 page table [B][max_pages]
  // FP8 caches: per-row scales of K and V (retrieval, then streaming heads)
  size_t off_skr = 0, off_svr = 0, off_sks = 0, off_svs = 0;
  duo::HeadMap map{};
};

struct Plan {
  size_t off_status = 0, off_len = 0;  // int32 status word, int32 token counts [L][B]
  std::vector<LayerPlan> layers;
  size_t arena = 0, workspace = 0, payload = 0;
  size_t ws_records = 0;  // decode partial records at the start of the workspace
  size_t ws_dequant = 0;  // FP8 caches: one layer's held rows in bf16 for prefill (after the records)
};

// Group sizes the decode kernels are built for: 1 .. 16 where scores run on
// the matrix cores (bf16 queries, d_head 128, every K/V row format), 1 .. 8
// on the vector ALU (fp32, or d_head 64).
int max_group(const duo_config* c) { return (c->dtype == DUO_BF16 && c->d_head == 128) ? 16 : 8; }

int validate(const duo_config* c) {
  if (!c) return fail(DUO_EINVAL, "config is NULL");
  if (c->L < 1 || c->B < 1 || c->n_q < 1 || c->n_kv < 1)
    return fail(DUO_EINVAL, "L, B, n_q, n_kv must be >= 1 (got %d, %d, %d, %d)", c->L, c->B, c->n_q, c->n_kv);
  if (c->n_q % c->n_kv != 0) return fail(DUO_EINVAL, "n_q (%d) must be a multiple of n_kv (%d)", c->n_q, c->n_kv);
  if (c->n_kv > duo::kMaxKV) return fail(DUO_EUNSUPPORTED, "n_kv %d > %d", c->n_kv, duo::kMaxKV);
  if (c->B > duo::kMaxRows) return fail(DUO_EUNSUPPORTED, "B %d > %d batch rows", c->B, duo::kMaxRows);
  if (c->d_head != 64 && c->d_head != 128) return fail(DUO_EUNSUPPORTED, "d_head %d not built (64, 128)", c->d_head);
  if (c->dtype != DUO_F32 && c->dtype != DUO_BF16) return fail(DUO_EUNSUPPORTED, "dtype %d", c->dtype);
  if (c->n_q / c->n_kv > max_group(c))
    return fail(DUO_EUNSUPPORTED, "group size g = %d not built (1 .. %d for this dtype and d_head)", c->n_q / c->n_kv,
                max_group(c));
  if (c->kv_format != DUO_KV_NATIVE && c->kv_format != DUO_KV_FP8 && c->kv_format != DUO_KV_INT4)
    return fail(DUO_EUNSUPPORTED, "kv_format %d", c->kv_format);
  if (c->kv_format != DUO_KV_NATIVE && (c->dtype != DUO_BF16 || c->d_head != 128))
    return fail(DUO_EUNSUPPORTED, "FP8 and INT4 K/V rows are built for bf16 and d_head 128");
  if (c->T_cap < 1) return fail(DUO_EINVAL, "T_cap must be >= 1");
  // positions are int32, and the decode's row arithmetic runs a few rounds
  // past a head's end in int32
  if (c->T_cap > INT32_MAX - 4096) return fail(DUO_EINVAL, "T_cap must be at most 2^31 - 4097 (positions are int32)");
  if (c->page_rows != 0) {
    if (c->page_rows < 64 || c->page_rows > (1 << 20) || (c->page_rows & (c->page_rows - 1)) != 0)
      return fail(DUO_EINVAL, "page_rows %d must be 0 or a power of two in [64, 2^20]", c->page_rows);
    if (c->n_pages < 1) return fail(DUO_EINVAL, "a paged cache needs n_pages >= 1 (got %d)", c->n_pages);
    // a decode round of rows (32 KB of stored K rows: 128 bf16 rows of d_head
    // 128, 256 FP8 rows, 512 INT4 rows) must lie within one page
    const int64_t round = duo::decode_round_rows(c->dtype, c->d_head, c->n_q / c->n_kv, c->kv_format);
    if (c->page_rows < round)
      return fail(DUO_EUNSUPPORTED, "pages of this row format hold at least %lld rows, one decode round (got %d)",
                  (long long)round, c->page_rows);
  } else if ((uint64_t)c->T_cap * (uint64_t)c->d_head * (c->dtype == DUO_BF16 ? 2u : 4u) > 0xffffffffull) {
    return fail(DUO_EUNSUPPORTED, "one head's rows (T_cap * d_head * element size) must fit 4 GiB");
  }
  if (c->sink < 0 || c->recent < 1) return fail(DUO_EINVAL, "need sink >= 0 and recent >= 1");
  if (!std::isfinite(c->rope_theta) || c->rope_theta < 0.f || (c->rope_theta > 0.f && c->rope_theta <= 1.f))
    return fail(DUO_EINVAL, "rope_theta must be 0 (off) or a finite base > 1 (got %g)", (double)c->rope_theta);
  if (!c->retrieval_mask) return fail(DUO_EINVAL, "retrieval_mask is NULL");
  for (int i = 0; i < c->L * c->n_kv; ++i)
    if (c->retrieval_mask[i] > 1) return fail(DUO_EINVAL, "retrieval_mask[%d] = %d, must be 0 or 1", i, c->retrieval_mask[i]);
  return DUO_OK;
}

int elem_bytes(const duo_config* c) { return c->dtype == DUO_BF16 ? 2 : 4; }

// (h, l) * (bh, bl) in double-double arithmetic (contraction off: a fused
// h = p + e would count the product's rounding error twice)
void dd_mul_host(double& h, double& l, double bh, double bl) {
#pragma clang fp contract(off)
  const double p = h * bh;
  double e = std::fma(h, bh, -p);
  e = std::fma(h, bl, std::fma(l, bh, e));
  h = p + e;
  l = e - (h - p);
}

// Rotary positions of base theta for heads of d dimensions: b = theta^(-2/d)
// as a double-double, to about 104 bits, and its squares b^(2^k).  A
// long-double estimate of b is refined by one Newton step on b^m theta = 1
// (m = d / 2) taken in double-double arithmetic: b <- b - b (b^m theta - 1) / m.
duo::Rope make_rope(float theta, int d) {
#pragma clang fp contract(off)
  duo::Rope r{};
  if (!(theta > 0.f)) return r;
  r.on = 1;
  const long double x = powl((long double)theta, -2.0L / (long double)d);
  double bh = (double)x, bl = (double)(x - (long double)bh);
  const int m = d / 2;
  double th = 1.0, tl = 0.0, ph = bh, pl = bl;  // b^m by binary powers
  for (int e = m; e != 0; e >>= 1) {
    if (e & 1) dd_mul_host(th, tl, ph, pl);
    if (e > 1) dd_mul_host(ph, pl, ph, pl);
  }
  const double tt = (double)theta;  // exact
  const double p = th * tt;
  const double pe = std::fma(th, tt, -p) + tl * tt;  // b^m theta = p + pe, p within an ulp of 1
  const double g = (p - 1.0) + pe;                  // p - 1 is exact
  const double lo = bl - bh * g / m;
  double h = bh + lo, l = lo - ((bh + lo) - bh);
  for (int k = 0; k < duo::kRopeBits; ++k) {
    r.hi[k] = h;
    r.lo[k] = l;
    dd_mul_host(h, l, h, l);
  }
  return r;
}
// bytes per stored K/V row: d elements in the cache dtype, d FP8 codes, or d
// INT4 codes two to a byte
int kv_row_bytes(const duo_config* c) {
  if (c->kv_format == DUO_KV_FP8) return c->d_head;
  if (c->kv_format == DUO_KV_INT4) return c->d_head / 2;
  return c->d_head * elem_bytes(c);
}

size_t decode_rec_floats(const duo_config* c) {  // acc[g][d], max[g], sum[g], padded to 16 bytes
  const int g = c->n_q / c->n_kv;
  return ((size_t)g * (c->d_head + 2) + 3) / 4 * 4;
}

void make_plan(const duo_config* c, Plan* p) {
  const size_t row = (size_t)kv_row_bytes(c);
  const bool lowbit = c->kv_format != DUO_KV_NATIVE;  // rows carry an fp32 scale each
  size_t dequant = 0;
  const int64_t cap_str = (int64_t)c->sink + c->recent;
  p->layers.assign(c->L, LayerPlan{});
  // header: the status word, then every layer's per-row token counts
  p->off_status = 0;
  p->off_len = sizeof(int32_t);
  size_t off = align_up(p->off_len + (size_t)c->L * c->B * sizeof(int32_t));
  p->payload = 0;
  for (int l = 0; l < c->L; ++l) {
    LayerPlan& lp = p->layers[l];
    std::memset(&lp.map, 0, sizeof lp.map);
    for (int h = 0; h < c->n_kv; ++h) {
      const bool ret = c->retrieval_mask[(size_t)l * c->n_kv + h] != 0;
      lp.map.kind[h] = ret ? 1 : 0;
      if (ret) {
        lp.map.cidx[h] = (int8_t)lp.n_ret;
        lp.map.orig_ret[lp.n_ret++] = (int8_t)h;
      } else {
        lp.map.cidx[h] = (int8_t)lp.n_str;
        lp.map.orig_str[lp.n_str++] = (int8_t)h;
      }
    }
    // retrieval rows per head: T_cap per batch row, or the page pool's rows
    const size_t ret_rows = c->page_rows ? (size_t)c->n_pages * c->page_rows : (size_t)c->B * c->T_cap;
    const size_t ret_bytes = ret_rows * lp.n_ret * row;
    const size_t str_bytes = (size_t)c->B * lp.n_str * cap_str * row;
    lp.off_kr = off; off = align_up(off + ret_bytes);
    lp.off_vr = off; off = align_up(off + ret_bytes);
    lp.off_ks = off; off = align_up(off + str_bytes);
    lp.off_vs = off; off = align_up(off + str_bytes);
    lp.off_pos = off; off = align_up(off + (size_t)c->B * lp.n_str * cap_str * sizeof(int32_t));
    if (c->page_rows) {
      lp.off_tab = off;
      off = align_up(off + (size_t)c->B * ceil_div(c->T_cap, c->page_rows) * sizeof(int32_t));
    }
    p->payload += 2 * (ret_bytes + str_bytes);
    if (lowbit) {
      const size_t ret_sc = ret_rows * lp.n_ret * sizeof(float);
      const size_t str_sc = (size_t)c->B * lp.n_str * cap_str * sizeof(float);
      lp.off_skr = off; off = align_up(off + ret_sc);
      lp.off_svr = off; off = align_up(off + ret_sc);
      lp.off_sks = off; off = align_up(off + str_sc);
      lp.off_svs = off; off = align_up(off + str_sc);
      p->payload += 2 * (ret_sc + str_sc);
      // prefill reads a layer's held rows dequantized to bf16: K and V of
      // every retrieval and streaming head
      const size_t bf_row = (size_t)c->d_head * 2;
      dequant = std::max(dequant, 2 * (align_up((size_t)c->B * lp.n_ret * c->T_cap * bf_row) +
                                       align_up((size_t)c->B * lp.n_str * cap_str * bf_row)));
    }
  }
  p->arena = off;
  // decode partial records: one per (work item, head) overlap, indexed by
  // first work item of the head + flat head index + segment
  const size_t rec = decode_rec_floats(c) * sizeof(float);
  p->ws_records = align_up(((size_t)duo::kMaxDecodeRecords + (size_t)c->B * c->n_kv) * rec);
  p->ws_dequant = dequant;
  p->workspace = p->ws_records + p->ws_dequant;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

struct duo_cache {
  duo_config cfg{};
  std::vector<uint8_t> mask;
  Plan plan;
  char* arena = nullptr;
  size_t arena_bytes = 0;
  std::vector<int64_t> row_len;  // tokens held by each (layer, batch row), advanced at enqueue time
  int num_cu = 256;  // compute units of the device current at init (decode work items per call)
  // Paged caches, per layer: the pages each batch row holds (in position
  // order), how many rows hold each page, and the free pages (a stack).
  struct Pages {
    std::vector<std::vector<int32_t>> rows;
    std::vector<int32_t> refs;
    std::vector<int32_t> free_list;
  };
  std::vector<Pages> pages;
  // Device words a host-only call (duo_cache_reset_row) left to write: per
  // layer, rows whose count becomes 0 and page-table entries that become -1.
  // Written ahead of the next call on the layer that takes a stream.
  std::vector<std::vector<int32_t>> pend_len, pend_tab;

  duo::LayerPtrs ptrs(int l) const {
    const LayerPlan& lp = plan.layers[l];
    duo::LayerPtrs p;
    p.k_ret = arena + lp.off_kr;
    p.v_ret = arena + lp.off_vr;
    p.k_str = arena + lp.off_ks;
    p.v_str = arena + lp.off_vs;
    p.pos = reinterpret_cast<int32_t*>(arena + lp.off_pos);
    const bool lb = cfg.kv_format != DUO_KV_NATIVE;
    p.ksc_ret = lb ? reinterpret_cast<float*>(arena + lp.off_skr) : nullptr;
    p.vsc_ret = lb ? reinterpret_cast<float*>(arena + lp.off_svr) : nullptr;
    p.ksc_str = lb ? reinterpret_cast<float*>(arena + lp.off_sks) : nullptr;
    p.vsc_str = lb ? reinterpret_cast<float*>(arena + lp.off_svs) : nullptr;
    p.table = paged(l) ? reinterpret_cast<int32_t*>(arena + lp.off_tab) : nullptr;
    p.max_pages = paged(l) ? (int32_t)max_pages() : 0;
    p.page_shift = paged(l) ? page_shift() : 0;
    p.len = reinterpret_cast<int32_t*>(arena + plan.off_len) + (size_t)l * cfg.B;
    p.status = reinterpret_cast<int32_t*>(arena + plan.off_status);
    p.cap = cfg.T_cap;
    return p;
  }
  // a layer stores paged retrieval rows (a layer with no retrieval head needs no pages)
  bool paged(int l) const { return cfg.page_rows != 0 && plan.layers[l].n_ret > 0; }
  int64_t max_pages() const { return ceil_div(cfg.T_cap, cfg.page_rows); }
  int page_shift() const {
    int sh = 0;
    while ((1 << sh) < cfg.page_rows) ++sh;
    return sh;
  }
  // pages a row of n tokens holds
  int64_t pages_for(int64_t n) const { return ceil_div(n, cfg.page_rows); }
  int64_t cap_str() const { return (int64_t)cfg.sink + cfg.recent; }
  int64_t len(int l, int b) const { return row_len[(size_t)l * cfg.B + b]; }
  int64_t& len(int l, int b) { return row_len[(size_t)l * cfg.B + b]; }
  // the common token count of a layer's rows, or -1 if they differ
  int64_t uniform_len(int l) const {
    for (int b = 1; b < cfg.B; ++b)
      if (len(l, b) != len(l, 0)) return -1;
    return len(l, 0);
  }
  int64_t max_len(int l) const {
    int64_t m = 0;
    for (int b = 0; b < cfg.B; ++b) m = std::max(m, len(l, b));
    return m;
  }
  // The layer seen as a cache of one batch row (row b): every region starts at
  // that row's part of the [B][...] arrays.
  duo::LayerPtrs row_ptrs(int l, int b) const {
    const LayerPlan& lp = plan.layers[l];
    duo::LayerPtrs p = ptrs(l);
    // a paged layer's pool is shared by the rows: only the table moves
    const size_t ret_rows = p.table ? 0 : (size_t)b * lp.n_ret * cfg.T_cap;
    const size_t str_rows = (size_t)b * lp.n_str * cap_str();
    const size_t rb = (size_t)row_bytes();
    p.k_ret += ret_rows * rb;
    p.v_ret += ret_rows * rb;
    p.k_str += str_rows * rb;
    p.v_str += str_rows * rb;
    p.pos += str_rows;
    if (p.ksc_ret) {
      p.ksc_ret += ret_rows;
      p.vsc_ret += ret_rows;
      p.ksc_str += str_rows;
      p.vsc_str += str_rows;
    }
    if (p.table) p.table += (size_t)b * p.max_pages;
    p.len += b;
    return p;
  }
  duo::Rope rope() const { return make_rope(cfg.rope_theta, cfg.d_head); }
  // prefill with rotary positions: the chunk's rotated queries and keys in the
  // workspace, after the decode records and the FP8 prefill copies
  size_t rope_ws_bytes(int64_t B, int64_t C) const {
    const size_t row = (size_t)cfg.d_head * elem_bytes(&cfg);
    return align_up((size_t)B * cfg.n_q * C * row) + align_up((size_t)B * cfg.n_kv * C * row);
  }
  int row_bytes() const { return kv_row_bytes(&cfg); }                  // stored K/V row
  int in_row_bytes() const { return cfg.d_head * elem_bytes(&cfg); }     // input / query row
  // low-bit rows (FP8 or INT4 codes with one fp32 scale per row)
  bool lowbit() const { return cfg.kv_format != DUO_KV_NATIVE; }
  int kvfmt() const { return cfg.kv_format; }
};

namespace {

int check_layer(const duo_cache* c, int layer) {
  if (!c) return fail(DUO_EINVAL, "cache handle is NULL");
  if (layer < 0 || layer >= c->cfg.L) return fail(DUO_EINVAL, "layer %d out of range [0, %d)", layer, c->cfg.L);
  return DUO_OK;
}

// Write the device words a host-only call left for `layer` (counts of reset
// rows, their released page-table entries), ahead of the call's own work.
int flush_pending(duo_cache* c, int layer, hipStream_t s) {
  if (c->pend_len.empty()) return DUO_OK;
  std::vector<int32_t>& pl = c->pend_len[layer];
  std::vector<int32_t>& pt = c->pend_tab[layer];
  const duo::LayerPtrs p = c->ptrs(layer);
  auto write = [&](int32_t* base, const std::vector<int32_t>& idx, int32_t value) -> hipError_t {
    duo::TableUpdateArgs u{};
    u.table = base;
    for (size_t i = 0; i < idx.size(); i += duo::kMaxTableUpdates) {
      u.n = (int)std::min<size_t>(duo::kMaxTableUpdates, idx.size() - i);
      for (int j = 0; j < u.n; ++j) {
        u.index[j] = idx[i + j];
        u.page[j] = value;
      }
      if (hipError_t e = duo::launch_table_update(u, s)) return e;
    }
    return hipSuccess;
  };
  if (!pt.empty()) {
    if (hipError_t e = write(p.table, pt, -1)) return hip_fail(e, "page table update launch");
    pt.clear();
  }
  if (!pl.empty()) {
    if (hipError_t e = write(p.len, pl, 0)) return hip_fail(e, "token count update launch");
    pl.clear();
  }
  return DUO_OK;
}

// Paged layers: give every growing row (row < 0: every batch row) the pages
// it needs to hold n_new more tokens, and enqueue the page-table writes ahead
// of the kernels that use them.  DUO_ECAPACITY (nothing taken) if the pool
// has too few free pages.  A row never holds fewer pages than its count
// needs; it may hold more after a later launch of the call fails (their
// table entries are written), which later growth reuses.
int reserve_pages(duo_cache* c, int layer, int row, int64_t n_new, hipStream_t s) {
  if (!c->paged(layer)) return DUO_OK;
  duo_cache::Pages& pg = c->pages[layer];
  const int b0 = row < 0 ? 0 : row, b1 = row < 0 ? c->cfg.B : row + 1;
  int64_t need = 0;
  for (int b = b0; b < b1; ++b)
    need += std::max<int64_t>(0, c->pages_for(c->len(layer, b) + n_new) - (int64_t)pg.rows[b].size());
  if (need > (int64_t)pg.free_list.size())
    return fail(DUO_ECAPACITY, "layer %d needs %lld more pages; %zu of %d are free", layer, (long long)need,
                pg.free_list.size(), c->cfg.n_pages);
  duo::TableUpdateArgs u{};
  u.table = c->ptrs(layer).table;
  // pages taken by this call whose table entries are not enqueued yet: given
  // back if a launch fails, so no row ever holds a page its table does not name
  std::vector<std::pair<int, int32_t>> pending;
  auto flush = [&]() -> int {
    const hipError_t e = duo::launch_table_update(u, s);
    u.n = 0;
    if (e != hipSuccess) {
      for (auto it = pending.rbegin(); it != pending.rend(); ++it) {
        pg.rows[it->first].pop_back();
        pg.refs[it->second] = 0;
        pg.free_list.push_back(it->second);
      }
      return hip_fail(e, "page table update launch");
    }
    pending.clear();
    return DUO_OK;
  };
  for (int b = b0; b < b1; ++b) {
    const int64_t want = c->pages_for(c->len(layer, b) + n_new);
    while ((int64_t)pg.rows[b].size() < want) {
      const int32_t page = pg.free_list.back();
      pg.free_list.pop_back();
      pg.refs[page] = 1;
      u.index[u.n] = (int32_t)((int64_t)b * c->max_pages() + (int64_t)pg.rows[b].size());
      u.page[u.n] = page;
      ++u.n;
      pg.rows[b].push_back(page);
      pending.emplace_back(b, page);
      if (u.n == duo::kMaxTableUpdates)
        if (int r = flush()) return r;
    }
  }
  return flush();
}

// Enqueue the append of n_new tokens to every batch row at its own token
// count, or (row >= 0) to that one row only, the inputs then being
// [1][n_kv][n_new][d] (no validation).
// With device_p0 each row's first position is its device count when the
// kernel runs, and an advance kernel follows (duo_append, duo_append_row);
// otherwise the positions start at the host count and the kernel sets the
// device counts to the host's new ones (a prefill commit).
hipError_t enqueue_append(duo_cache* c, int layer, const void* k, const void* v, int64_t n_new, hipStream_t s,
                          int row = -1, bool rotate = true, bool device_p0 = false) {
  const LayerPlan& lp = c->plan.layers[layer];
  duo::AppendArgs a{};
  a.p0_from_device = device_p0 ? 1 : 0;
  a.k = static_cast<const char*>(k);
  a.v = static_cast<const char*>(v);
  a.lp = row < 0 ? c->ptrs(layer) : c->row_ptrs(layer, row);
  a.map = lp.map;
  a.B = row < 0 ? c->cfg.B : 1;
  a.n_kv = c->cfg.n_kv;
  a.n_ret = lp.n_ret;
  a.n_str = lp.n_str;
  a.row_bytes = c->row_bytes();
  a.in_row_bytes = c->in_row_bytes();
  a.cap_ret = c->cfg.T_cap;
  a.cap_str = c->cap_str();
  for (int b = 0; b < a.B; ++b) a.p0[b] = (int32_t)c->len(layer, row < 0 ? b : row);
  a.n_new = n_new;
  a.S = c->cfg.sink;
  a.W = c->cfg.recent;
  a.dtype = c->cfg.dtype;
  a.d = c->cfg.d_head;
  if (rotate) a.rope = c->rope();  // else the keys come rotated already
  hipError_t e = duo::launch_append(a, c->cfg.dtype, c->cfg.d_head, c->kvfmt(), s);
  if (e != hipSuccess || !device_p0) return e;
  duo::AdvanceArgs adv{};
  adv.lp = a.lp;
  adv.B = a.B;
  adv.n = n_new;
  return duo::launch_advance(adv, s);
}

}  // namespace

extern "C" {

int duo_cache_bytes(const duo_config* cfg, size_t* arena_bytes, size_t* workspace_bytes) {
  if (int e = validate(cfg)) return e;
  Plan p;
  make_plan(cfg, &p);
  if (arena_bytes) *arena_bytes = p.arena;
  if (workspace_bytes) *workspace_bytes = p.workspace;
  return ok();
}

int duo_cache_payload_bytes(const duo_config* cfg, size_t* payload_bytes) {
  if (int e = validate(cfg)) return e;
  if (!payload_bytes) return fail(DUO_EINVAL, "payload_bytes is NULL");
  Plan p;
  make_plan(cfg, &p);
  *payload_bytes = p.payload;
  return ok();
}

int duo_cache_init(const duo_config* cfg, void* arena, size_t arena_bytes, void* stream, duo_cache** out) {
  if (int e = validate(cfg)) return e;
  if (!out) return fail(DUO_EINVAL, "out is NULL");
  if (!arena) return fail(DUO_EINVAL, "arena is NULL");
  if ((reinterpret_cast<uintptr_t>(arena) % kAlign) != 0) return fail(DUO_EINVAL, "arena must be 256-byte aligned");
  Plan p;
  make_plan(cfg, &p);
  if (arena_bytes < p.arena)
    return fail(DUO_EINVAL, "arena holds %zu bytes, %zu needed", arena_bytes, p.arena);
  duo_cache* c = new (std::nothrow) duo_cache;
  if (!c) return fail(DUO_EINVAL, "out of host memory");
  c->cfg = *cfg;
  c->mask.assign(cfg->retrieval_mask, cfg->retrieval_mask + (size_t)cfg->L * cfg->n_kv);
  c->cfg.retrieval_mask = c->mask.data();
  c->plan = p;
  c->arena = static_cast<char*>(arena);
  c->arena_bytes = arena_bytes;
  c->row_len.assign((size_t)cfg->L * cfg->B, 0);
  c->pend_len.assign(cfg->L, {});
  c->pend_tab.assign(cfg->L, {});
  if (cfg->page_rows) {
    c->pages.resize(cfg->L);
    for (int l = 0; l < cfg->L; ++l) {
      duo_cache::Pages& pg = c->pages[l];
      pg.rows.assign(cfg->B, {});
      pg.refs.assign(cfg->n_pages, 0);
      pg.free_list.resize(cfg->n_pages);
      for (int i = 0; i < cfg->n_pages; ++i) pg.free_list[i] = cfg->n_pages - 1 - i;  // page 0 is taken first
    }
  }
  {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      c->num_cu = n;
  }
  {
    // the allocation-free decode's scratch: its device address on this
    // device, resolved once per device
    void* scratch = nullptr;
    const hipError_t e = duo::static_scratch(&scratch);
    if (e != hipSuccess) {
      delete c;
      return hip_fail(e, "address of the library's device scratch");
    }
  }
  hipError_t s_err = hipSuccess;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the status word and every token count start at zero
  s_err = duo::launch_fill_zero(c->arena, p.off_len + (size_t)cfg->L * cfg->B * sizeof(int32_t), s);
  for (int l = 0; l < cfg->L && s_err == hipSuccess; ++l) {
    const LayerPlan& lp = p.layers[l];
    // positions start at zero (payload rows need no clearing)
    s_err = duo::launch_fill_zero(c->arena + lp.off_pos, (size_t)cfg->B * lp.n_str * c->cap_str() * sizeof(int32_t), s);
    // page-table entries start at -1: no page
    if (s_err == hipSuccess && c->paged(l))
      s_err = duo::launch_fill_ones(c->arena + lp.off_tab, (size_t)cfg->B * c->max_pages() * sizeof(int32_t), s);
  }
  if (s_err != hipSuccess) {
    delete c;
    return hip_fail(s_err, "initialising the arena");
  }
  *out = c;
  return ok();
}

int duo_append(duo_cache* c, int layer, const void* k, const void* v, int64_t n_new, void* stream) {
  if (int e = check_layer(c, layer)) return e;
  if (!k || !v) return fail(DUO_EINVAL, "k or v is NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(DUO_EINVAL, "k and v must be 16-byte aligned");
  if (n_new < 1) return fail(DUO_EINVAL, "n_new must be >= 1 (got %lld)", (long long)n_new);
  const int64_t pmax = c->max_len(layer);
  if (pmax + n_new > c->cfg.T_cap)
    return fail(DUO_ECAPACITY, "layer %d has a row of %lld tokens; %lld more exceed T_cap %lld", layer,
                (long long)pmax, (long long)n_new, (long long)c->cfg.T_cap);
  if (int r = flush_pending(c, layer, static_cast<hipStream_t>(stream))) return r;
  if (int r = reserve_pages(c, layer, -1, n_new, static_cast<hipStream_t>(stream))) return r;
  hipError_t e = enqueue_append(c, layer, k, v, n_new, static_cast<hipStream_t>(stream), -1, true, true);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  for (int b = 0; b < c->cfg.B; ++b) c->len(layer, b) += n_new;
  return ok();
}

int duo_append_row(duo_cache* c, int layer, int row, const void* k, const void* v, int64_t n_new, void* stream) {
  if (int e = check_layer(c, layer)) return e;
  if (row < 0 || row >= c->cfg.B) return fail(DUO_EINVAL, "row %d out of range [0, %d)", row, c->cfg.B);
  if (!k || !v) return fail(DUO_EINVAL, "k or v is NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(DUO_EINVAL, "k and v must be 16-byte aligned");
  if (n_new < 1) return fail(DUO_EINVAL, "n_new must be >= 1 (got %lld)", (long long)n_new);
  const int64_t p0 = c->len(layer, row);
  if (p0 + n_new > c->cfg.T_cap)
    return fail(DUO_ECAPACITY, "row %d of layer %d holds %lld tokens; %lld more exceed T_cap %lld", row, layer,
                (long long)p0, (long long)n_new, (long long)c->cfg.T_cap);
  if (int r = flush_pending(c, layer, static_cast<hipStream_t>(stream))) return r;
  if (int r = reserve_pages(c, layer, row, n_new, static_cast<hipStream_t>(stream))) return r;
  hipError_t e = enqueue_append(c, layer, k, v, n_new, static_cast<hipStream_t>(stream), row, true, true);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  c->len(layer, row) = p0 + n_new;
  return ok();
}

namespace {

// Checks shared by the decode entry points (the layer is already checked).
int check_decode_args(const duo_cache* c, const void* q, void* out, float scale, void* ws, size_t ws_bytes) {
  if (!q || !out) return fail(DUO_EINVAL, "q or out is NULL");
  if (!aligned16(q) || !aligned16(out)) return fail(DUO_EINVAL, "q and out must be 16-byte aligned");
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(DUO_EINVAL, "scale must be finite and > 0");
  if (!ws || ws_bytes < c->plan.ws_records)
    return fail(DUO_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", c->plan.ws_records, ws_bytes);
  if (!aligned16(ws)) return fail(DUO_EINVAL, "workspace must be 16-byte aligned");
  return DUO_OK;
}

// Plan the decode kernels over the rows each batch row holds (its token
// count); with new_k / new_v set, every row's next token (at its token count)
// is appended and attended by the same launch.  Fills *a (all but the
// workspace pointer) and returns the number of work items.  Host only.
int plan_decode(const duo_cache* c, int layer, const void* q, void* out, float scale, const void* new_k,
                const void* new_v, duo::DecodeArgs* ap) {
  const LayerPlan& lp = c->plan.layers[layer];
  const duo_config& cf = c->cfg;
  duo::DecodeArgs& a = *ap;
  a = duo::DecodeArgs{};
  a.q = q;
  a.out = out;
  a.lp = c->ptrs(layer);
  a.map = lp.map;
  a.B = cf.B;
  a.n_q = cf.n_q;
  a.n_kv = cf.n_kv;
  a.n_ret = lp.n_ret;
  a.n_str = lp.n_str;
  a.cap_ret = cf.T_cap;
  a.cap_str = c->cap_str();
  a.S = cf.sink;
  a.W = cf.recent;
  for (int b = 0; b < cf.B; ++b) {
    duo::DecodeRow& R = a.rows[b];
    const int64_t held = c->len(layer, b);
    R.rows_ret = (int32_t)held;
    R.rows_str = (int32_t)std::min<int64_t>(held, c->cap_str());
  }
  if (new_k) {
    a.new_k = static_cast<const char*>(new_k);
    a.new_v = static_cast<const char*>(new_v);
  }
  a.rope = c->rope();
  const int g = cf.n_q / cf.n_kv;
  const int64_t heads = (int64_t)cf.B * (lp.n_ret + lp.n_str);
  const int64_t slots = std::max<int64_t>(std::min(c->num_cu, duo::kMaxDecodeBlocks), heads);
  const int64_t R0 = duo::decode_round_rows(cf.dtype, cf.d_head, g, c->kvfmt());
  const bool paged = a.lp.table != nullptr;
  // Share groups ("Attention Variants and Memory Efficiency", "What the
  // Inference Runtime Can Change": a matching prefix is stored once; here it
  // is also read once).  Consecutive batch rows whose first pages are the
  // same physical pages -- rows forked from one prefix -- form a group of up
  // to 16 / g rows (their g queries each fill the 16 columns of one
  // matrix-core tile; bf16 queries of d = 128 and g >= 4, so that a row's
  // queries are whole 1 KB staging pieces).  The group's shared items attend
  // all its rows' queries to the shared rows; each row's own items cover the
  // rest of its rows.
  a.n_share = 0;
  if (paged && lp.n_ret > 0 && cf.dtype == DUO_BF16 && cf.d_head == 128 && (g == 4 || g == 8)) {
    const std::vector<std::vector<int32_t>>& pr = c->pages[layer].rows;
    // full pages that rows b0 and b hold at the same positions
    auto common = [&](int b0, int b) {
      const int64_t held = std::min(c->len(layer, b0), c->len(layer, b));
      const int64_t full = std::min<int64_t>(held / cf.page_rows, (int64_t)std::min(pr[b0].size(), pr[b].size()));
      int64_t k = 0;
      while (k < full && pr[b0][k] == pr[b][k]) ++k;
      return k;
    };
    const int rmax = 16 / g;
    for (int b0 = 0; b0 < cf.B && a.n_share < duo::kMaxShares;) {
      int n = 1;
      int64_t k = INT64_MAX;
      while (b0 + n < cf.B && n < rmax) {
        const int64_t kk = common(b0, b0 + n);
        if (kk < 1) break;
        k = std::min(k, kk);
        ++n;
      }
      if (n >= 2) {
        duo::DecodeShare& S = a.share[a.n_share++];
        S.b0 = b0;
        S.R = n;
        S.rows = (int32_t)(k * cf.page_rows);
        for (int b = b0; b < b0 + n; ++b) a.rsh[b].sh_rows = S.rows;
        b0 += n;
      } else {
        ++b0;
      }
    }
  }
  // Work items: contiguous row ranges of one head, at most one workgroup per
  // compute unit (or one per head if there are more heads), none shorter
  // than one round of the kernel where the head allows.  All heads are cut to
  // a common item length t, the smallest with which the items fit: the
  // launch ends with its longest item, so the items' lengths are balanced
  // across retrieval and streaming heads and across batch rows of different
  // lengths (e.g. a 1,088-row streaming head is cut in two when a 128k
  // retrieval head's items hold about 1,050 rows).
  auto items = [&](int64_t rows, int64_t t) { return std::max<int64_t>(1, ceil_div(rows, t)); };
  // A paged head's items start at multiples of R0 rows (the kernel rounds
  // its item length up to R0), so that each round of rows lies in one page.
  auto items_ret = [&](int64_t rows, int64_t t) { return items(rows, paged ? ceil_div(t, R0) * R0 : t); };
  auto count = [&](int64_t t) {
    int64_t n = 0;
    for (int b = 0; b < cf.B; ++b)
      n += lp.n_ret * items_ret(a.rows[b].rows_ret - a.rsh[b].sh_rows, t) + lp.n_str * items(a.rows[b].rows_str, t);
    for (int k = 0; k < a.n_share; ++k) n += lp.n_ret * items_ret(a.share[k].rows, t);
    return n;
  };
  int64_t longest = 1;
  for (int b = 0; b < cf.B; ++b) longest = std::max<int64_t>(longest, std::max(a.rows[b].rows_ret, a.rows[b].rows_str));
  if (a.n_share > 0 && count(longest) > slots) {  // one item per head already fills the launch
    a.n_share = 0;
    for (int b = 0; b < cf.B; ++b) a.rsh[b].sh_rows = 0;
  }
  int64_t lo = std::min(R0, longest), hi = longest;  // count(hi) <= heads <= slots
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo) / 2;
    if (count(mid) <= slots) hi = mid;
    else lo = mid + 1;
  }
  const int64_t t = lo;
  int32_t next = 0;
  a.multi = 0;
  for (int b = 0; b < cf.B; ++b) {  // retrieval items of every row, then streaming
    duo::DecodeRow& R = a.rows[b];
    const int64_t own = R.rows_ret - a.rsh[b].sh_rows;
    const int64_t nr = items_ret(own, t);
    // no empty item: contiguous heads are cut evenly; a paged head's items of
    // ceil(rows / nr) rows rounded up to R0 all hold rows (a row whose rows
    // are all shared keeps one empty item, which takes a fused append's token)
    R.nb_ret = (int32_t)(paged || own == 0 ? nr : ceil_div(own, ceil_div(own, nr)));
    R.first_ret = next;
    next += lp.n_ret * R.nb_ret;
    if (lp.n_ret > 0 && R.nb_ret > 1) a.multi = 1;
  }
  a.items_ret = next;
  for (int b = 0; b < cf.B; ++b) {
    duo::DecodeRow& R = a.rows[b];
    const int64_t ns = items(R.rows_str, t);
    R.nb_str = (int32_t)(R.rows_str > 0 ? ceil_div(R.rows_str, ceil_div(R.rows_str, ns)) : 1);
    R.first_str = next;
    next += lp.n_str * R.nb_str;
    if (lp.n_str > 0 && R.nb_str > 1) a.multi = 1;
  }
  a.items_sh = next;
  for (int k = 0; k < a.n_share; ++k) {
    duo::DecodeShare& S = a.share[k];
    S.nb = (int32_t)items_ret(S.rows, t);
    S.first = next;
    next += lp.n_ret * S.nb;
    a.multi = 1;
  }
  int32_t rec = next;  // records past the items': the shared items', group by group
  for (int k = 0; k < a.n_share; ++k) {
    duo::DecodeShare& S = a.share[k];
    S.rec = rec;
    for (int i = 0; i < S.R; ++i) {
      a.rsh[S.b0 + i].sh_rec = rec + i * lp.n_ret * S.nb;
      a.rsh[S.b0 + i].sh_nb = S.nb;
    }
    rec += S.R * lp.n_ret * S.nb;
  }
  a.n_records = rec;
  a.scale_log2 = scale * 1.4426950408889634f;
  return (int)next;
}

// Bytes of partial records a planned decode writes: one per work item, and
// with share groups one per (row of the group, shared item) after those.
size_t decode_records_bytes(const duo_cache* c, const duo::DecodeArgs& a, int blocks) {
  const size_t n = a.n_share > 0 ? (size_t)a.n_records : (size_t)blocks;
  return n * decode_rec_floats(&c->cfg) * sizeof(float);
}

hipError_t launch_planned_decode(const duo_cache* c, duo::DecodeArgs& a, int blocks, void* ws, hipStream_t stream) {
  a.ws1 = static_cast<float*>(ws);
  const int g = c->cfg.n_q / c->cfg.n_kv;
  return duo::launch_decode(a, c->cfg.dtype, c->cfg.d_head, g, c->kvfmt(), blocks, stream);
}

hipError_t enqueue_decode(duo_cache* c, int layer, const void* q, void* out, float scale, void* ws,
                          const void* new_k, const void* new_v, hipStream_t stream) {
  duo::DecodeArgs a;
  const int blocks = plan_decode(c, layer, q, out, scale, new_k, new_v, &a);
  return launch_planned_decode(c, a, blocks, ws, stream);
}

}  // namespace

int duo_decode(duo_cache* c, int layer, const void* q, void* out, float scale, void* ws, size_t ws_bytes,
               void* stream) {
  if (int e = check_layer(c, layer)) return e;
  if (int e = check_decode_args(c, q, out, scale, ws, ws_bytes)) return e;
  for (int b = 0; b < c->cfg.B; ++b)
    if (c->len(layer, b) < 1) return fail(DUO_EEMPTY, "row %d of layer %d holds no token", b, layer);
  if (int r = flush_pending(c, layer, static_cast<hipStream_t>(stream))) return r;
  hipError_t e = enqueue_decode(c, layer, q, out, scale, ws, nullptr, nullptr, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

int duo_decode_append(duo_cache* c, int layer, const void* k, const void* v, const void* q, void* out, float scale,
                      void* ws, size_t ws_bytes, void* stream) {
  if (int e = check_layer(c, layer)) return e;
  if (!k || !v) return fail(DUO_EINVAL, "k or v is NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(DUO_EINVAL, "k and v must be 16-byte aligned");
  if (int e = check_decode_args(c, q, out, scale, ws, ws_bytes)) return e;
  const int64_t pmax = c->max_len(layer);
  if (pmax + 1 > c->cfg.T_cap)
    return fail(DUO_ECAPACITY, "layer %d has a row of %lld tokens; one more exceeds T_cap %lld", layer,
                (long long)pmax, (long long)c->cfg.T_cap);
  // one launch: each row attends over what it holds and its new token, which
  // the kernel also stores (a row that holds nothing yet attends to the new
  // token alone)
  if (int r = flush_pending(c, layer, static_cast<hipStream_t>(stream))) return r;
  if (int r = reserve_pages(c, layer, -1, 1, static_cast<hipStream_t>(stream))) return r;
  hipError_t e = enqueue_decode(c, layer, q, out, scale, ws, k, v, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  for (int b = 0; b < c->cfg.B; ++b) c->len(layer, b) += 1;
  return ok();
}

int duo_decode_append_noalloc(duo_cache* c, int layer, const void* k, const void* v, const void* q, void* out,
                              float scale, void* stream) {
  if (int e = check_layer(c, layer)) return e;
  if (!k || !v) return fail(DUO_EINVAL, "k or v is NULL");
  if (!aligned16(k) || !aligned16(v)) return fail(DUO_EINVAL, "k and v must be 16-byte aligned");
  if (!q || !out) return fail(DUO_EINVAL, "q or out is NULL");
  if (!aligned16(q) || !aligned16(out)) return fail(DUO_EINVAL, "q and out must be 16-byte aligned");
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(DUO_EINVAL, "scale must be finite and > 0");
  const int64_t pmax = c->max_len(layer);
  if (pmax + 1 > c->cfg.T_cap)
    return fail(DUO_ECAPACITY, "layer %d has a row of %lld tokens; one more exceeds T_cap %lld", layer,
                (long long)pmax, (long long)c->cfg.T_cap);
  void* scratch = nullptr;
  const hipError_t se = duo::static_scratch(&scratch);
  if (se != hipSuccess) return hip_fail(se, "address of the library's device scratch");
  duo::DecodeArgs a;
  const int blocks = plan_decode(c, layer, q, out, scale, k, v, &a);
  const size_t need = decode_records_bytes(c, a, blocks);
  if (need > duo::kStaticScratchBytes)
    return fail(DUO_EWORKSPACE,
                "this decode writes %zu bytes of partial results (%d work items); the library's device scratch "
                "holds %zu: use duo_decode_append with a workspace",
                need, blocks, duo::kStaticScratchBytes);
  if (int r = flush_pending(c, layer, static_cast<hipStream_t>(stream))) return r;
  if (int r = reserve_pages(c, layer, -1, 1, static_cast<hipStream_t>(stream))) return r;
  const hipError_t e = launch_planned_decode(c, a, blocks, scratch, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  for (int b = 0; b < c->cfg.B; ++b) c->len(layer, b) += 1;
  return ok();
}

}  // extern "C"

namespace {

// Workspace a chunked prefill of B rows and C tokens needs: FP8 caches hold
// the dequantized rows after the decode records; rotary positions add the
// rotated chunk after those.  0 if none.
size_t prefill_ws_bytes(const duo_cache* c, int64_t B, int64_t C) {
  if (c->rope().on) return c->plan.workspace + c->rope_ws_bytes(B, C);
  return c->lowbit() ? c->plan.workspace : 0;
}

// Chunked prefill of every batch row (row < 0; the rows must hold equal
// counts) or of batch row `row` alone (inputs [1][...]).
int prefill_impl(duo_cache* c, int layer, int row, const void* q, const void* k, const void* v, int64_t C, void* out,
                 float scale, void* ws, size_t ws_bytes, void* stream) {
  if (int e = check_layer(c, layer)) return e;
  if (row >= c->cfg.B) return fail(DUO_EINVAL, "row %d out of range [0, %d)", row, c->cfg.B);
  if (!q || !k || !v || !out) return fail(DUO_EINVAL, "q, k, v or out is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(DUO_EINVAL, "q, k, v and out must be 16-byte aligned");
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(DUO_EINVAL, "scale must be finite and > 0");
  if (C < 1) return fail(DUO_EINVAL, "chunk length must be >= 1 (got %lld)", (long long)C);
  const size_t need = prefill_ws_bytes(c, row < 0 ? c->cfg.B : 1, C);
  if (need) {
    if (!ws || ws_bytes < need) return fail(DUO_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    if ((reinterpret_cast<uintptr_t>(ws) % kAlign) != 0) return fail(DUO_EINVAL, "workspace must be 256-byte aligned");
  }
  const int64_t P = row < 0 ? c->uniform_len(layer) : c->len(layer, row);
  if (P < 0)
    return fail(DUO_EINVAL, "the rows of layer %d hold different token counts; prefill them one at a time "
                "(duo_prefill_chunk_row)", layer);
  if (P + C > c->cfg.T_cap)
    return fail(DUO_ECAPACITY, "layer %d holds %lld tokens; a chunk of %lld exceeds T_cap %lld", layer,
                (long long)P, (long long)C, (long long)c->cfg.T_cap);
  const LayerPlan& lp = c->plan.layers[layer];
  const duo_config& cf = c->cfg;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  duo::PrefillArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lp = row < 0 ? c->ptrs(layer) : c->row_ptrs(layer, row);
  a.map = lp.map;
  a.B = row < 0 ? cf.B : 1;
  a.n_q = cf.n_q;
  a.n_kv = cf.n_kv;
  a.n_ret = lp.n_ret;
  a.n_str = lp.n_str;
  a.cap_ret = cf.T_cap;
  a.cap_str = c->cap_str();
  a.P = P;
  a.C = C;
  a.held_str = std::min<int64_t>(P, c->cap_str());
  a.S = cf.sink;
  a.W = cf.recent;
  a.scale_log2 = scale * 1.4426950408889634f;
  const int g = cf.n_q / cf.n_kv;
  int rows = 1, hpi = 1;
  duo::prefill_plan(cf.dtype, cf.d_head, g, &rows, &hpi);
  a.q_tiles = (int)ceil_div(C, rows);
  a.items_ret = a.B * lp.n_ret * (g / hpi) * a.q_tiles;
  if (int r = flush_pending(c, layer, s)) return r;
  // pages for the chunk's rows (the attention reads only the held rows)
  if (int r = reserve_pages(c, layer, row, C, s)) return r;
  hipError_t e = hipSuccess;
  if (c->lowbit()) {
    // the held rows, dequantized to bf16 in the workspace (after the decode
    // records), stand in for the cache's rows during the attention
    const int64_t cap_r = std::max<int64_t>(P, 1);
    const size_t bf_row = (size_t)cf.d_head * 2;
    char* base = static_cast<char*>(ws) + c->plan.ws_records;
    const size_t ret_b = align_up((size_t)a.B * lp.n_ret * cap_r * bf_row);
    const size_t str_b = align_up((size_t)a.B * lp.n_str * c->cap_str() * bf_row);
    duo::DequantArgs d{};
    d.src = a.lp;
    d.dst = duo::LayerPtrs{};
    d.dst.k_ret = base;
    d.dst.v_ret = base + ret_b;
    d.dst.k_str = base + 2 * ret_b;
    d.dst.v_str = base + 2 * ret_b + str_b;
    d.heads_ret = (int64_t)a.B * lp.n_ret;
    d.heads_str = (int64_t)a.B * lp.n_str;
    d.cap_ret_src = cf.T_cap;
    d.cap_ret_dst = cap_r;
    d.rows_ret = P;
    d.cap_str = c->cap_str();
    d.rows_str = a.held_str;
    d.d = cf.d_head;
    d.n_ret = lp.n_ret;
    d.int4 = cf.kv_format == DUO_KV_INT4 ? 1 : 0;
    e = duo::launch_dequant(d, s);
    if (e != hipSuccess) return hip_fail(e, "dequant launch");
    a.lp.k_ret = d.dst.k_ret;
    a.lp.v_ret = d.dst.v_ret;
    a.lp.k_str = d.dst.k_str;
    a.lp.v_str = d.dst.v_str;
    a.lp.table = nullptr;  // the copies are contiguous rows
    a.cap_ret = cap_r;
  }
  const duo::Rope rope = c->rope();
  if (rope.on) {
    // the chunk's queries and keys rotated at positions P + i, into the
    // workspace after the records and the FP8 copies
    duo::RopeArgs r{};
    char* base = static_cast<char*>(ws) + c->plan.workspace;
    r.q = q;
    r.k = k;
    r.q_out = base;
    r.k_out = base + align_up((size_t)a.B * cf.n_q * C * c->in_row_bytes());
    r.B = a.B;
    r.n_q = cf.n_q;
    r.n_kv = cf.n_kv;
    r.d = cf.d_head;
    r.dtype = cf.dtype;
    r.C = C;
    for (int b = 0; b < a.B; ++b) r.p0[b] = (int32_t)P;
    r.rope = rope;
    e = duo::launch_rope(r, s);
    if (e != hipSuccess) return hip_fail(e, "rotary launch");
    a.q = r.q_out;
    a.k = r.k_out;
  }
  e = duo::launch_prefill(a, cf.dtype, cf.d_head, g, s);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  // Commit the chunk after attention has read the cache (same stream); with
  // rotary positions its keys are the rotated copies.
  e = enqueue_append(c, layer, a.k, v, C, s, row, /*rotate=*/false);
  if (e != hipSuccess) return hip_fail(e, "prefill commit launch");
  if (row < 0)
    for (int b = 0; b < cf.B; ++b) c->len(layer, b) = P + C;
  else
    c->len(layer, row) = P + C;
  return ok();
}

}  // namespace

extern "C" {

int duo_prefill_chunk(duo_cache* c, int layer, const void* q, const void* k, const void* v, int64_t C, void* out,
                      float scale, void* ws, size_t ws_bytes, void* stream) {
  return prefill_impl(c, layer, -1, q, k, v, C, out, scale, ws, ws_bytes, stream);
}

int duo_prefill_chunk_row(duo_cache* c, int layer, int row, const void* q, const void* k, const void* v, int64_t C,
                          void* out, float scale, void* ws, size_t ws_bytes, void* stream) {
  if (row < 0) return fail(DUO_EINVAL, "row %d out of range", row);
  return prefill_impl(c, layer, row, q, k, v, C, out, scale, ws, ws_bytes, stream);
}

int duo_prefill_workspace_bytes(const duo_cache* c, int rows, int64_t C, size_t* bytes) {
  if (!c) return fail(DUO_EINVAL, "cache handle is NULL");
  if (rows < 1 || rows > c->cfg.B) return fail(DUO_EINVAL, "rows %d out of range [1, %d]", rows, c->cfg.B);
  if (C < 1) return fail(DUO_EINVAL, "chunk length must be >= 1 (got %lld)", (long long)C);
  if (!bytes) return fail(DUO_EINVAL, "bytes is NULL");
  *bytes = prefill_ws_bytes(c, rows, C);
  return ok();
}

int duo_cache_seq_len(const duo_cache* c, int layer, int64_t* out) {
  if (int e = check_layer(c, layer)) return e;
  if (!out) return fail(DUO_EINVAL, "out is NULL");
  const int64_t n = c->uniform_len(layer);
  if (n < 0) return fail(DUO_EINVAL, "the rows of layer %d hold different token counts (duo_cache_row_len)", layer);
  *out = n;
  return ok();
}

int duo_cache_row_len(const duo_cache* c, int layer, int row, int64_t* out) {
  if (int e = check_layer(c, layer)) return e;
  if (row < 0 || row >= c->cfg.B) return fail(DUO_EINVAL, "row %d out of range [0, %d)", row, c->cfg.B);
  if (!out) return fail(DUO_EINVAL, "out is NULL");
  *out = c->len(layer, row);
  return ok();
}

int duo_cache_reset_row(duo_cache* c, int layer, int row) {
  if (int e = check_layer(c, layer)) return e;
  if (row < 0 || row >= c->cfg.B) return fail(DUO_EINVAL, "row %d out of range [0, %d)", row, c->cfg.B);
  if (c->paged(layer)) {
    duo_cache::Pages& pg = c->pages[layer];
    for (size_t i = 0; i < pg.rows[row].size(); ++i) {
      const int32_t page = pg.rows[row][i];
      if (--pg.refs[page] == 0) pg.free_list.push_back(page);
      // the row's table entry names no page any more
      c->pend_tab[layer].push_back((int32_t)((int64_t)row * c->max_pages() + (int64_t)i));
    }
    pg.rows[row].clear();
  }
  c->len(layer, row) = 0;
  c->pend_len[layer].push_back(row);  // the device count, ahead of the next call on the layer
  return ok();
}

int duo_cache_fork_row(duo_cache* c, int layer, int src_row, int dst_row, void* stream) {
  if (int e = check_layer(c, layer)) return e;
  const duo_config& cf = c->cfg;
  if (src_row < 0 || src_row >= cf.B || dst_row < 0 || dst_row >= cf.B)
    return fail(DUO_EINVAL, "rows %d, %d out of range [0, %d)", src_row, dst_row, cf.B);
  if (src_row == dst_row) return fail(DUO_EINVAL, "src_row and dst_row are the same row");
  if (c->len(layer, dst_row) != 0)
    return fail(DUO_EINVAL, "row %d of layer %d holds %lld tokens; reset it before a fork", dst_row, layer,
                (long long)c->len(layer, dst_row));
  const int64_t n = c->len(layer, src_row);
  if (n == 0) return ok();
  const LayerPlan& lp = c->plan.layers[layer];
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (int r = flush_pending(c, layer, s)) return r;
  const duo::LayerPtrs src = c->row_ptrs(layer, src_row), dst = c->row_ptrs(layer, dst_row);
  const int64_t rb = c->row_bytes();
  duo::CopyArgs cp{};
  auto seg = [&](const void* from, void* to, int64_t bytes, int64_t count = 1, int64_t stride = 0) {
    if (bytes <= 0 || count <= 0) return;
    cp.seg[cp.n++] = duo::CopySegment{static_cast<const char*>(from), static_cast<char*>(to), bytes, count, stride,
                                      stride};
  };
  const bool f8 = c->lowbit();  // rows carry scales
  if (c->paged(layer)) {
    duo_cache::Pages& pg = c->pages[layer];
    for (int32_t page : pg.rows[dst_row])  // spares left by a failed launch
      if (--pg.refs[page] == 0) pg.free_list.push_back(page);
    pg.rows[dst_row].clear();
    const int64_t full = n / cf.page_rows;
    const bool partial = n % cf.page_rows != 0;
    if (partial && pg.free_list.empty())
      return fail(DUO_ECAPACITY, "layer %d has no free page for the copy of row %d's last page", layer, src_row);
    duo::TableUpdateArgs u{};
    u.table = c->ptrs(layer).table;
    std::vector<int32_t> pages(pg.rows[src_row].begin(), pg.rows[src_row].begin() + full);
    for (int32_t page : pages) ++pg.refs[page];
    if (partial) {
      const int32_t from = pg.rows[src_row][full];
      const int32_t page = pg.free_list.back();
      pg.free_list.pop_back();
      pg.refs[page] = 1;
      pages.push_back(page);
      // the whole page: every retrieval head's rows, K and V (and scales)
      const int64_t rows = (int64_t)lp.n_ret * cf.page_rows;
      const duo::LayerPtrs L = c->ptrs(layer);
      seg(L.k_ret + from * rows * rb, L.k_ret + page * rows * rb, rows * rb);
      seg(L.v_ret + from * rows * rb, L.v_ret + page * rows * rb, rows * rb);
      if (f8) {
        seg(L.ksc_ret + from * rows, L.ksc_ret + page * rows, rows * 4);
        seg(L.vsc_ret + from * rows, L.vsc_ret + page * rows, rows * 4);
      }
    }
    // the table entries go in launches of at most kMaxTableUpdates
    for (size_t i = 0; i < pages.size(); i += duo::kMaxTableUpdates) {
      u.n = (int)std::min<size_t>(duo::kMaxTableUpdates, pages.size() - i);
      for (int j = 0; j < u.n; ++j) {
        u.index[j] = (int32_t)((int64_t)dst_row * c->max_pages() + (int64_t)(i + j));
        u.page[j] = pages[i + j];
      }
      if (hipError_t e = duo::launch_table_update(u, s)) return hip_fail(e, "page table update launch");
    }
    pg.rows[dst_row] = pages;
  } else if (lp.n_ret > 0) {
    // held rows [0, n) of every retrieval head (heads T_cap rows apart)
    seg(src.k_ret, dst.k_ret, n * rb, lp.n_ret, cf.T_cap * rb);
    seg(src.v_ret, dst.v_ret, n * rb, lp.n_ret, cf.T_cap * rb);
    if (f8) {
      seg(src.ksc_ret, dst.ksc_ret, n * 4, lp.n_ret, cf.T_cap * 4);
      seg(src.vsc_ret, dst.vsc_ret, n * 4, lp.n_ret, cf.T_cap * 4);
    }
  }
  // the streaming heads' slots, positions and scales of the row
  const int64_t slots = (int64_t)lp.n_str * c->cap_str();
  seg(src.k_str, dst.k_str, slots * rb);
  seg(src.v_str, dst.v_str, slots * rb);
  seg(src.pos, dst.pos, slots * 4);
  if (f8) {
    seg(src.ksc_str, dst.ksc_str, slots * 4);
    seg(src.vsc_str, dst.vsc_str, slots * 4);
  }
  if (hipError_t e = duo::launch_copy(cp, s)) return hip_fail(e, "row copy launch");
  {  // the device count of dst
    duo::TableUpdateArgs u{};
    u.table = c->ptrs(layer).len;
    u.n = 1;
    u.index[0] = dst_row;
    u.page[0] = (int32_t)n;
    if (hipError_t e = duo::launch_table_update(u, s)) return hip_fail(e, "token count update launch");
  }
  c->len(layer, dst_row) = n;
  return ok();
}

int duo_cache_sync(duo_cache* c, void* stream) {
  if (!c) return fail(DUO_EINVAL, "cache handle is NULL");
  const hipStream_t s = static_cast<hipStream_t>(stream);
  for (int l = 0; l < c->cfg.L; ++l)
    if (int r = flush_pending(c, l, s)) return r;
  const size_t n = (size_t)c->cfg.L * c->cfg.B;
  std::vector<int32_t> host(n + 1);
  hipError_t e = hipMemcpyAsync(host.data(), c->arena + c->plan.off_status, (n + 1) * sizeof(int32_t),
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading the token counts back");
  // the layout puts the counts right after the status word
  static_assert(sizeof(int32_t) == 4, "int32 words");
  const int32_t status = host[0];
  for (size_t i = 0; i < n; ++i) c->row_len[i] = host[1 + i];
  if (status != 0) {
    e = duo::launch_fill_zero(c->arena + c->plan.off_status, sizeof(int32_t), s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "clearing the status word");
    return fail(DUO_ECAPACITY, "a step found no room for its tokens (T_cap reached, or a paged row without a "
                "reserved page): it stored nothing and its token count did not advance");
  }
  return ok();
}

int duo_cache_reserve(duo_cache* c, int layer, int64_t n_tokens, void* stream) {
  if (int e = check_layer(c, layer)) return e;
  if (n_tokens < 0) return fail(DUO_EINVAL, "n_tokens must be >= 0 (got %lld)", (long long)n_tokens);
  const int64_t pmax = c->max_len(layer);
  if (pmax + n_tokens > c->cfg.T_cap)
    return fail(DUO_ECAPACITY, "layer %d has a row of %lld tokens; %lld more exceed T_cap %lld", layer,
                (long long)pmax, (long long)n_tokens, (long long)c->cfg.T_cap);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (int r = flush_pending(c, layer, s)) return r;
  if (int r = reserve_pages(c, layer, -1, n_tokens, s)) return r;
  return ok();
}

int duo_cache_free_pages(const duo_cache* c, int layer, int64_t* out) {
  if (int e = check_layer(c, layer)) return e;
  if (!out) return fail(DUO_EINVAL, "out is NULL");
  if (c->cfg.page_rows == 0) *out = 0;
  else if (!c->paged(layer)) *out = c->cfg.n_pages;  // no retrieval head: no page is ever taken
  else *out = (int64_t)c->pages[layer].free_list.size();
  return ok();
}

int duo_cache_row_pages(const duo_cache* c, int layer, int row, int32_t* pages, int64_t cap, int64_t* n) {
  if (int e = check_layer(c, layer)) return e;
  if (row < 0 || row >= c->cfg.B) return fail(DUO_EINVAL, "row %d out of range [0, %d)", row, c->cfg.B);
  if (!n) return fail(DUO_EINVAL, "n is NULL");
  if (cap > 0 && !pages) return fail(DUO_EINVAL, "pages is NULL");
  if (!c->paged(layer)) {
    *n = 0;
    return ok();
  }
  const std::vector<int32_t>& rp = c->pages[layer].rows[row];
  const int64_t held = c->pages_for(c->len(layer, row));  // pages in use (a failed launch may have left spares)
  *n = held;
  for (int64_t i = 0; i < std::min(held, cap); ++i) pages[i] = rp[i];
  return ok();
}

int duo_cache_head_view(const duo_cache* c, int layer, int kv_head, int* is_retrieval, void** k_base, void** v_base,
                        int32_t** pos, int64_t* n_slots, int64_t* row_bytes, int64_t* head_stride_bytes,
                        int64_t* pos_stride) {
  if (int e = check_layer(c, layer)) return e;
  if (kv_head < 0 || kv_head >= c->cfg.n_kv) return fail(DUO_EINVAL, "kv_head %d out of range", kv_head);
  const LayerPlan& lp = c->plan.layers[layer];
  const duo::LayerPtrs p = c->ptrs(layer);
  const bool ret = lp.map.kind[kv_head] != 0;
  const int ci = lp.map.cidx[kv_head];
  const int64_t rb = c->row_bytes();
  // a paged head: its rows in page 0, pages n_ret * page_rows rows apart
  const int64_t slots = ret ? (c->paged(layer) ? c->cfg.page_rows : c->cfg.T_cap) : c->cap_str();
  const int n_kind = ret ? lp.n_ret : lp.n_str;
  if (is_retrieval) *is_retrieval = ret ? 1 : 0;
  if (n_slots) *n_slots = slots;
  if (row_bytes) *row_bytes = rb;
  if (head_stride_bytes) *head_stride_bytes = (int64_t)n_kind * slots * rb;
  if (pos_stride) *pos_stride = ret ? 0 : (int64_t)n_kind * slots;
  if (k_base) *k_base = (ret ? p.k_ret : p.k_str) + (size_t)ci * slots * rb;
  if (v_base) *v_base = (ret ? p.v_ret : p.v_str) + (size_t)ci * slots * rb;
  if (pos) *pos = ret ? nullptr : p.pos + (size_t)ci * slots;
  return ok();
}

int duo_gated_attention(const duo_gated_shape* shape, const void* q, const void* k, const void* v,
                        const float* alpha, void* out, float scale, void* stream) {
  if (!shape) return fail(DUO_EINVAL, "shape is NULL");
  const duo_gated_shape& sh = *shape;
  if (sh.B < 1 || sh.n_q < 1 || sh.n_kv < 1)
    return fail(DUO_EINVAL, "B, n_q, n_kv must be >= 1 (got %d, %d, %d)", sh.B, sh.n_q, sh.n_kv);
  if (sh.n_q % sh.n_kv != 0) return fail(DUO_EINVAL, "n_q (%d) must be a multiple of n_kv (%d)", sh.n_q, sh.n_kv);
  if (sh.d_head != 64 && sh.d_head != 128) return fail(DUO_EUNSUPPORTED, "d_head %d not built (64, 128)", sh.d_head);
  if (sh.dtype != DUO_F32 && sh.dtype != DUO_BF16) return fail(DUO_EUNSUPPORTED, "dtype %d", sh.dtype);
  if (sh.N < 1) return fail(DUO_EINVAL, "N must be >= 1 (got %lld)", (long long)sh.N);
  if (sh.sink < 0 || sh.recent < 1) return fail(DUO_EINVAL, "need sink >= 0 and recent >= 1");
  // positions and key-tile ends (N plus a 64-key tile) stay within int32
  if (sh.N + std::max<int64_t>(sh.recent, 64) > INT32_MAX)
    return fail(DUO_EINVAL, "N + max(recent, 64) must fit int32 (positions are int32)");
  if (!q || !k || !v || !alpha || !out) return fail(DUO_EINVAL, "q, k, v, alpha or out is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(DUO_EINVAL, "q, k, v and out must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(alpha) & 3u) != 0) return fail(DUO_EINVAL, "alpha must be 4-byte aligned");
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(DUO_EINVAL, "scale must be finite and > 0");
  const int g = sh.n_q / sh.n_kv;
  duo::GatedArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.out = out;
  a.B = sh.B;
  a.n_q = sh.n_q;
  a.n_kv = sh.n_kv;
  a.S = sh.sink;
  a.W = sh.recent;
  a.N = sh.N;
  a.scale_log2 = scale * 1.4426950408889634f;
  const int64_t rows = duo::gated_rows_per_item(sh.dtype, g);
  const int64_t q_tiles = ceil_div(sh.N, rows);
  if (q_tiles * sh.B * sh.n_q > INT32_MAX) return fail(DUO_EUNSUPPORTED, "too many work items for one launch");
  a.q_tiles = (int)q_tiles;
  const hipError_t e = duo::launch_gated(a, sh.dtype, sh.d_head, g, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gated forward launch");
  return ok();
}

int duo_cache_head_scales(const duo_cache* c, int layer, int kv_head, float** k_scale, float** v_scale,
                          int64_t* scale_stride) {
  if (int e = check_layer(c, layer)) return e;
  if (kv_head < 0 || kv_head >= c->cfg.n_kv) return fail(DUO_EINVAL, "kv_head %d out of range", kv_head);
  const LayerPlan& lp = c->plan.layers[layer];
  const duo::LayerPtrs p = c->ptrs(layer);
  const bool ret = lp.map.kind[kv_head] != 0;
  const int ci = lp.map.cidx[kv_head];
  const int64_t slots = ret ? (c->paged(layer) ? c->cfg.page_rows : c->cfg.T_cap) : c->cap_str();
  const int n_kind = ret ? lp.n_ret : lp.n_str;
  const bool f8 = c->lowbit();  // rows carry scales
  if (k_scale) *k_scale = f8 ? (ret ? p.ksc_ret : p.ksc_str) + (size_t)ci * slots : nullptr;
  if (v_scale) *v_scale = f8 ? (ret ? p.vsc_ret : p.vsc_str) + (size_t)ci * slots : nullptr;
  if (scale_stride) *scale_stride = f8 ? (int64_t)n_kind * slots : 0;
  return ok();
}

int duo_decode_plan(const duo_cache* c, int layer, int* n_items, int* n_shared) {
  if (int e = check_layer(c, layer)) return e;
  if (!n_items || !n_shared) return fail(DUO_EINVAL, "n_items or n_shared is NULL");
  duo::DecodeArgs a;
  const int blocks = plan_decode(c, layer, nullptr, nullptr, 1.f, nullptr, nullptr, &a);
  *n_items = blocks;
  *n_shared = blocks - a.items_sh;
  return ok();
}

int duo_rope_apply(float theta, int dtype, int B, int H, int64_t C, int d, const int64_t* p0, const void* x,
                   void* out, void* stream) {
  if (!std::isfinite(theta) || !(theta > 0.f)) return fail(DUO_EINVAL, "theta must be finite and > 0");
  if (dtype != DUO_F32 && dtype != DUO_BF16) return fail(DUO_EINVAL, "dtype %d is not a duo_dtype", dtype);
  if (B < 1 || B > duo::kMaxRows) return fail(DUO_EINVAL, "B = %d outside 1 .. %d", B, duo::kMaxRows);
  if (H < 1) return fail(DUO_EINVAL, "H = %d must be >= 1", H);
  if (C < 0) return fail(DUO_EINVAL, "C = %lld must be >= 0", (long long)C);
  if (d < 2 || d > 256 || d % 2 != 0) return fail(DUO_EINVAL, "d = %d must be even, 2 .. 256", d);
  if (!p0) return fail(DUO_EINVAL, "p0 is NULL");
  for (int b = 0; b < B; ++b)
    if (p0[b] < 0 || p0[b] + C > (int64_t{1} << 31))
      return fail(DUO_EINVAL, "p0[%d] = %lld: positions must lie in 0 .. 2^31 - 1", b, (long long)p0[b]);
  if (C == 0) return ok();
  if (!x || !out) return fail(DUO_EINVAL, "x or out is NULL");
  if ((double)B * H * C * d > 9.0e18) return fail(DUO_EINVAL, "tensor too large");
  duo::RopeArgs r{};
  r.q = x;
  r.q_out = out;
  r.B = B;
  r.n_q = H;
  r.n_kv = 0;  // no second tensor
  r.d = d;
  r.dtype = dtype;
  r.C = C;
  for (int b = 0; b < B; ++b) r.p0[b] = (int32_t)p0[b];
  r.rope = make_rope(theta, d);
  const hipError_t e = duo::launch_rope(r, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rotary launch");
  return ok();
}

void duo_cache_free(duo_cache* c) { delete c; }

const char* duo_last_error(void) { return g_err.c_str(); }

}  // extern "C"
