// Chunked prefill over a per-KV-head mixed KV cache, for gfx950 (CDNA4).
//
// A chunk of C tokens at absolute positions P .. P+C-1 attends over the keys
// the cache holds plus the chunk itself.  Retrieval heads use the causal mask
// (key j visible to the row at t iff j <= t); streaming heads use the
// sink + local-window mask (j <= t and (j < S or j >= t - W + 1)), with cached
// keys read from the sink and ring slots and their stored positions.  The
// chunk is committed to the cache by the append kernel afterwards.
//
// bf16: a dense contraction, tiled on MFMA (v_mfma_f32_32x32x16_bf16).
//   * Work item = one workgroup of eight wavefronts: four row wavefronts,
//     each owning 32 query rows of one query head (one 32-row MFMA N tile;
//     up to four heads of a GQA group, or row blocks of one head), times two
//     key halves that take the even and the odd key tiles of the same rows.
//     The halves merge their softmax states through LDS at the end.  Every
//     SIMD runs two wavefronts, so one's MFMA work overlaps the other's
//     softmax; 128 query rows share each K / V tile a workgroup loads, and
//     the LDS operand reads (1 KB per MFMA) stay under the LDS bandwidth.
//   * K and V tiles of 64 keys are brought into LDS with direct buffer->LDS
//     loads, double buffered per half: the next tile streams in while the
//     current one is consumed.  Rows are XOR-swizzled in 16-byte chunks (the
//     swizzle is applied on the global side of the copy) so operand reads are
//     free of bank conflicts.
//   * Scores S^T = K Q^T put keys on the MFMA M axis and queries on N, so each
//     lane holds one query's scores and the softmax needs one exchange with
//     the partner lane (v_permlane32_swap).  P^T then feeds O^T = V^T P^T from the
//     accumulator registers; the V^T operand comes straight from the
//     row-major V tile through LDS transpose reads (ds_read_b64_tr_b16).
//   * Streaming heads visit only the sink tiles, the ring tiles some row's
//     window reaches, and the local band of the chunk; retrieval heads the
//     causal prefix.  Tiles every row of the item sees in full skip the mask;
//     the rest test each key's visible-row interval with one compare.
//   * The online softmax rescales the O accumulators only when a row's
//     running max has grown by more than a fixed slack.
//   * Paged retrieval heads: a cached tile (64 keys from a multiple of 64)
//     lies in one page, found through the batch row's page table with a
//     scalar load when the tile is issued.  Rotary positions are applied
//     before this kernel (queries and the chunk's keys rotated into the
//     workspace), so it sees them as plain inputs.
//
// fp32: a plain vector-ALU path (one wavefront per query row) kept for
// completeness of the dtype surface; it is not tuned.
#include "duo_attn_tile.h"
#include "duo_internal.h"
#include "duo_rows.h"

#include <hip/hip_runtime.h>

#include <climits>

namespace duo {
namespace {

__device__ __forceinline__ bool visible(int64_t kp, int64_t t, bool ret, int S, int W) {
  return kp >= 0 && kp <= t && (ret || kp < S || kp >= t - W + 1);
}

// The rows of the chunk (absolute position P + i) that see the key at absolute
// position kp: i >= kp - P, for every later row under the causal mask alone
// (retrieval heads, sink keys) and for W rows otherwise (the local window).
// Keys that do not exist (kp < 0) are seen by no row.
__device__ __forceinline__ KeySpan key_span(int64_t kp, int64_t P, bool ret, int S, int W) {
  KeySpan k;
  if (kp < 0) {
    k.lo = -1;
    k.span = 0;
  } else {
    k.lo = (int32_t)(kp - P);
    k.span = (ret || kp < S) ? (uint32_t)0x7fffffff - (uint32_t)k.lo : (uint32_t)(W - 1);
  }
  return k;
}

// Key tile sources.
enum : int { SRC_CACHE_LINEAR = 0, SRC_CACHE_SLOTS = 1, SRC_CHUNK = 2 };

// Tile ranges (in units of kBN keys) a workgroup visits, per source.
struct TileRanges {
  int64_t cache_lo, cache_hi;                          // cache part
  int64_t chunk_lo0, chunk_hi0, chunk_lo1, chunk_hi1;  // up to two ranges of chunk tiles
};

__device__ __forceinline__ TileRanges plan_tiles(const PrefillArgs& a, bool ret, int64_t i0, int64_t i1) {
  // rows [i0, i1) of the chunk; query positions P+i0 .. P+i1-1
  TileRanges tr;
  const int64_t chunk_hi = (min64(i1, a.C) + kBN - 1) / kBN;  // causal: keys jj <= i < i1
  if (ret) {
    tr.cache_lo = 0;
    tr.cache_hi = (a.P + kBN - 1) / kBN;
    tr.chunk_lo0 = 0;
    tr.chunk_hi0 = chunk_hi;
    tr.chunk_lo1 = tr.chunk_hi1 = 0;
  } else {
    // cache slots: sinks always; ring slots only if some row's window reaches back before P
    const int64_t held = a.held_str;
    const bool ring_needed = (i0 < (int64_t)a.W - 1);
    const int64_t last_slot = ring_needed ? held : min64(held, a.S);
    tr.cache_lo = 0;
    tr.cache_hi = (last_slot + kBN - 1) / kBN;
    // chunk: sink keys (positions < S) and the band jj >= i0 - W + 1
    const int64_t sink_rows = max64(0, min64(a.C, (int64_t)a.S - a.P));
    const int64_t sink_tiles = (sink_rows + kBN - 1) / kBN;
    const int64_t band_lo = max64(0, i0 - a.W + 1) / kBN;
    if (band_lo <= sink_tiles) {
      tr.chunk_lo0 = 0;
      tr.chunk_hi0 = chunk_hi;
      tr.chunk_lo1 = tr.chunk_hi1 = 0;
    } else {
      tr.chunk_lo0 = 0;
      tr.chunk_hi0 = min64(sink_tiles, chunk_hi);
      tr.chunk_lo1 = band_lo;
      tr.chunk_hi1 = chunk_hi;
    }
  }
  return tr;
}

// ------------------------------------------------------------------ bf16 MFMA path

// Tile descriptors a workgroup keeps in LDS (16 bytes each): 16 KB at
// d = 128; 8 KB at d = 64, where two workgroups still share a CU.
template <int D>
constexpr int pf_tile_table() { return D >= 128 ? 1024 : 512; }

struct PfItem {
  int b, kvh, cidx, h_first, qt;
  bool ret;
};

// Work items: retrieval items first, then streaming.  Within a kind the
// index runs (b, head group, query tile, KV head) with the KV head fastest:
// workgroups are dealt to the XCDs in turn, so the items of one KV head land
// on the same XCDs and share its K and V in their L2; query tiles with the
// most keys come first.
__device__ __forceinline__ PfItem pf_item(const PrefillArgs& a, int g, int hpi) {
  PfItem w;
  int rem = blockIdx.x;
  int n_kind;
  if (rem < a.items_ret) {
    w.ret = true;
    n_kind = a.n_ret;
  } else {
    w.ret = false;
    rem -= a.items_ret;
    n_kind = a.n_str;
  }
  const int ngrp = g / hpi;
  w.cidx = rem % n_kind;
  rem /= n_kind;
  const int qt_rev = rem % a.q_tiles;
  rem /= a.q_tiles;
  const int hg = rem % ngrp;
  w.b = rem / ngrp;
  w.qt = a.q_tiles - 1 - qt_rev;
  w.kvh = w.ret ? a.map.orig_ret[w.cidx] : a.map.orig_str[w.cidx];
  w.h_first = w.kvh * g + hg * hpi;
  return w;
}


template <int D>
__global__ __launch_bounds__(kPfThreads) void prefill_mfma_kernel(PrefillArgs a, int g, int hpi) {
  using SH = PfShape<D>;
  constexpr int KSTEPS = SH::KSTEPS, DT = SH::DT;

  // [key half][buffer]
  __shared__ __attribute__((aligned(1024))) char k_lds[kPfHalves][2][SH::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds[kPfHalves][2][SH::TILE_BYTES];
  __shared__ int32_t klo_lds[kPfHalves][2][kBN];
  __shared__ uint32_t kspan_lds[kPfHalves][2][kBN];
  __shared__ int s_full[kPfHalves][2];
  constexpr int TT = pf_tile_table<D>();
  static_assert(TT / 2 <= kPfThreads, "half the table filled at once, one tile per thread");
  __shared__ uint4 tdesc[TT];

  const PfItem w = pf_item(a, g, hpi);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = wave / kPfRowWaves;   // key half: tiles kh, kh + 2, kh + 4, ...
  const int sub = wave % kPfRowWaves;  // row wavefront within the half
  const int n = lane & 31, hf = lane >> 5;
  // this wavefront's head and rows: hpi heads x (kPfRowWaves / hpi) row blocks
  const int h = w.h_first + (sub % hpi);
  const int rows_item = kPfRowsPerWave * (kPfRowWaves / hpi);
  const int64_t i0 = (int64_t)w.qt * rows_item;                       // item's first chunk row
  const int64_t i1 = min64(i0 + rows_item, a.C);
  const int64_t wr0 = i0 + (int64_t)(sub / hpi) * kPfRowsPerWave;    // wavefront's first row
  const size_t rowb = (size_t)D * 2;

  // Q^T operands: lane holds 8 consecutive d of query row (wr0 + 32*nt + n) per k-step.
  bf16x8_t qb[kPfNT][KSTEPS];
  int32_t iq[kPfNT];  // chunk row of the lane's query in tile nt
  bool qvalid[kPfNT];
#pragma unroll
  for (int nt = 0; nt < kPfNT; ++nt) {
    const int64_t qrow = wr0 + 32 * nt + n;
    qvalid[nt] = qrow < a.C;
    iq[nt] = (int32_t)qrow;
    const char* qp = static_cast<const char*>(a.q) + (((size_t)w.b * a.n_q + h) * a.C + (qvalid[nt] ? qrow : 0)) * rowb;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4_t v = qvalid[nt] ? *reinterpret_cast<const u32x4_t*>(qp + (ks * 16 + hf * 8) * 2) : u32x4_t{0, 0, 0, 0};
      qb[nt][ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // Key sources for this KV head.
  const char *kc, *vc;
  const int32_t* posc = nullptr;
  if (w.ret) {
    // the head's row 0 (contiguous), or its rows in page 0 (paged)
    const size_t off = (a.lp.table ? ((size_t)w.cidx << a.lp.page_shift)
                                   : ((size_t)w.b * a.n_ret + w.cidx) * a.cap_ret) * rowb;
    kc = a.lp.k_ret + off;
    vc = a.lp.v_ret + off;
  } else {
    const size_t hrow = ((size_t)w.b * a.n_str + w.cidx) * a.cap_str;
    kc = a.lp.k_str + hrow * rowb;
    vc = a.lp.v_str + hrow * rowb;
    posc = a.lp.pos + hrow;
  }
  const size_t chunk_off = ((size_t)w.b * a.n_kv + w.kvh) * a.C * rowb;
  const char* kn = static_cast<const char*>(a.k) + chunk_off;
  const char* vn = static_cast<const char*>(a.v) + chunk_off;

  // The item's key tiles: up to three runs of consecutive tiles (cache, then
  // one or two of the chunk), in 32-bit tile and row numbers (positions stay
  // below 2^31), held as wavefront-uniform values so that the per-tile
  // arithmetic below is a few scalar instructions without branches.
  const TileRanges tr = plan_tiles(a, w.ret, i0, i1);
  const int32_t n_cache = uniform32(tr.cache_hi - tr.cache_lo);
  const int32_t n_c0 = uniform32(tr.chunk_hi0 - tr.chunk_lo0);
  const int32_t n_c1 = uniform32(tr.chunk_hi1 - tr.chunk_lo1);
  const int32_t n_tiles = n_cache + n_c0 + n_c1;
  const int32_t cache_lo = uniform32(tr.cache_lo), c0_lo = uniform32(tr.chunk_lo0), c1_lo = uniform32(tr.chunk_lo1);
  const int32_t cache_rows = uniform32(w.ret ? a.P : a.held_str), chunk_rows = uniform32(a.C);
  const int32_t r0 = uniform32(i0), r1 = uniform32(i1);  // the item's chunk rows [r0, r1)
  const int32_t win_lo = r1 - a.W;                         // first chunk row in every row's window
  const int32_t sink_rows = uniform32(max64(-1, min64((int64_t)a.S - a.P, 1 << 30)));  // chunk rows that are sinks

  // per-lane byte offsets of this wavefront's first K / V piece within a tile
  const uint32_t koff = dma_offset<D, false>(sub, lane);
  const uint32_t voff = dma_offset<D, true>(sub, lane);
  // Rows past a source's end read as zero; clear both buffers once so no
  // stale bit pattern (which could be a NaN) ever meets a zero probability.
  {
    const u32x4_t z = {0, 0, 0, 0};
    for (int off = tid * 16; off < kPfHalves * 2 * SH::TILE_BYTES; off += kPfThreads * 16) {
      *reinterpret_cast<u32x4_t*>(&k_lds[0][0][0] + off) = z;
      *reinterpret_cast<u32x4_t*>(&v_lds[0][0][0] + off) = z;
    }
  }

  // Tile `it` -> (source, first row, row limit), as selects of per-run
  // constants (tile number = first tile of the run + offset within it).
  const int32_t skip0 = c0_lo - cache_lo - n_cache, skip1 = c1_lo - c0_lo - n_c0;
  auto tile_src = [&](int32_t it, int& src, int32_t& base, int32_t& limit) {
    const bool in_cache = it < n_cache, in_c0 = it < n_cache + n_c0;
    base = (cache_lo + it + (in_cache ? 0 : skip0) + (in_c0 ? 0 : skip1)) * kBN;
    limit = in_cache ? cache_rows : chunk_rows;
    src = in_cache ? (w.ret ? SRC_CACHE_LINEAR : SRC_CACHE_SLOTS) : SRC_CHUNK;
  };
  // Whether every row of the item sees every key of tile `it`, decided from
  // scalars where the keys' positions follow from their rows (a retrieval
  // head's cached rows, the chunk's rows); the cached slots of a streaming
  // head, whose positions are read from the cache, take the per-key test.
  // A tile that passes needs no mask and no per-key bookkeeping.
  auto tile_full = [&](int32_t it) -> bool {
    int src;
    int32_t base, limit;
    tile_src(it, src, base, limit);
    const bool whole = base + kBN <= limit;  // no key past the end of the source
    // chunk keys: causal for the item's first row; for a streaming head also
    // all sinks (chunk rows below S - P), or all inside the window of the
    // item's last row
    const bool chunk_ok = base + kBN - 1 <= r0 && (w.ret || base + kBN - 1 < sink_rows || base >= win_lo);
    // a retrieval head's cached positions (< P) are seen by every chunk row
    return whole && (src == SRC_CACHE_LINEAR || (src == SRC_CHUNK && chunk_ok));
  };
  // Tile descriptors, one per tile of the item, computed once by the whole
  // workgroup (one tile per thread) into an LDS table: the byte offset of the
  // tile's first row in its source (after the page lookup of a paged head),
  // the tile's first row number, its byte count, source and whether it needs
  // no mask.  Every wavefront of a key half then reads the descriptor of its
  // next tile instead of working it out in scalar code each step.  The table
  // holds TT tiles; an item with more tiles has the entries of tiles it has
  // passed refilled, well before they are read (see the loop).
  auto fill_desc = [&](int32_t t0) {  // tiles t0 .. t0 + TT / 2 - 1
    const int32_t it = t0 + tid;
    if (tid >= TT / 2 || it >= n_tiles) return;
    int src;
    int32_t base, limit;
    tile_src(it, src, base, limit);
    const int nbytes = min(limit - base, kBN) * (int)rowb;
    // a paged head's tile (64 rows from a multiple of 64) lies in one page
    const int64_t roff = (src == SRC_CACHE_LINEAR && a.lp.table)
                             ? paged_row(a.lp.table + (size_t)w.b * a.lp.max_pages, a.lp.page_shift,
                                         (int64_t)a.n_ret << a.lp.page_shift, base)
                             : base;
    const uint64_t boff = (uint64_t)roff * rowb;
    tdesc[it & (TT - 1)] =
        make_uint4((uint32_t)boff, (uint32_t)(boff >> 32), (uint32_t)base,
                   (uint32_t)nbytes | ((uint32_t)src << 16) | ((uint32_t)tile_full(it) << 18));
  };

  // Prepare tile `it` for buffer `buf` of this wavefront's key half: its key
  // visibility, for a tile that needs a mask, by plain stores (the half's
  // first wavefront) with a flag telling whether every row of the item sees
  // every key of the tile all the same (then the mask is skipped); and the
  // direct loads of its K/V pieces (split over the half's wavefronts), which
  // the caller issues.  `full` tells whether the tile needs no mask at all.
  auto prepare = [&](int32_t it, int buf, bool& full) -> TileLoads<D> {
    TileLoads<D> ld;
    ld.kdst = lds_addr(k_lds[kh][buf] + sub * 1024);
    ld.vdst = lds_addr(v_lds[kh][buf] + sub * 1024);
    ld.koff = koff;
    ld.voff = voff;
    full = true;
    if (it >= n_tiles) {
      ld.rk = ld.rv = dma_rsrc(kn, 0);
      return ld;
    }
    const uint4 dsc = tdesc[it & (TT - 1)];
    // (readfirstlane gives an int: each word goes through uint32_t so that
    // the low one is not sign-extended)
    const uint32_t meta = (uint32_t)__builtin_amdgcn_readfirstlane(dsc.w);
    const uint64_t boff = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(dsc.y) << 32) |
                          (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(dsc.x);
    const int src = (int)((meta >> 16) & 3u);
    full = ((meta >> 18) & 1u) != 0;
    const int nbytes = (int)(meta & 0xffffu);
    // The stored positions of a streaming head's slots are a global load:
    // it is waited for here, before any of the tile's direct loads is issued
    // (waits count loads in issue order).
    if (sub == 0 && !full) {  // one wavefront, all lanes: lane = key of the tile
      const int32_t base = (int32_t)__builtin_amdgcn_readfirstlane(dsc.z);
      const int32_t limit = src == SRC_CHUNK ? chunk_rows : cache_rows;
      const int32_t row = base + lane;
      int64_t kp = -1;  // past the end: never visible
      if (row < limit) {
        if (src == SRC_CACHE_LINEAR) kp = row;
        else if (src == SRC_CACHE_SLOTS) kp = posc[row];
        else kp = a.P + row;
      }
      const KeySpan sp = key_span(kp, a.P, w.ret, a.S, a.W);
      klo_lds[kh][buf][lane] = sp.lo;
      kspan_lds[kh][buf][lane] = sp.span;
      // the tile needs no mask iff every key is seen by the item's first and
      // last row (the visible rows of a key form an interval)
      const bool all = sees(r0, sp.lo, sp.span) && sees(r1 - 1, sp.lo, sp.span);
      const uint64_t bal = __builtin_amdgcn_ballot_w64(all);
      if (lane == 0) s_full[kh][buf] = (bal == ~0ull) ? 1 : 0;
    }
    const char* ks = (src == SRC_CHUNK) ? kn : kc;
    const char* vs = (src == SRC_CHUNK) ? vn : vc;
    ld.rk = dma_rsrc(ks + boff, nbytes);
    ld.rv = dma_rsrc(vs + boff, nbytes);
    return ld;
  };

  f32x16_t o[DT][kPfNT];
  float m_run[kPfNT], l_run[kPfNT];
#pragma unroll
  for (int nt = 0; nt < kPfNT; ++nt) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][nt][r] = 0.f;
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
  }

  // The two halves walk the tile list in lockstep, one barrier per step.
  // The next tile's loads are issued during the current tile's work.
  // The table starts with tiles [0, TT); the zero fill above and these
  // stores are published by one barrier.
  fill_desc(0);
  fill_desc(TT / 2);
  __syncthreads();
  const int32_t n_steps = (n_tiles + 1) / 2;
  bool full_cur;  // the current tile needs no mask
  prepare(kh, 0, full_cur).all();
  for (int32_t step = 0; step < n_steps; ++step) {
    const int buf = (int)(step & 1);
    // this wavefront's direct loads for the current tile have landed; after
    // the barrier every wavefront's have, and the previous tile is consumed.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // Every TT / 4 steps (tiles 2 step .. 2 step + TT / 2 - 1 are in the
    // table), the entries of the TT / 2 tiles before 2 step, all consumed,
    // take the tiles 2 step + TT / 2 onwards, which are first read
    // TT / 4 - 1 steps (and as many barriers) later.
    if (step > 0 && step % (TT / 4) == 0) fill_desc(2 * step + TT / 2);
    // this half has no tile left, and so no next one (wavefront-uniform)
    if (2 * step + kh >= n_tiles) continue;
    bool full_next;
    const TileLoads<D> next = prepare(2 * (step + 1) + kh, buf ^ 1, full_next);
    const char* kt = k_lds[kh][buf];
    const char* vt = v_lds[kh][buf];
    const bool masked = !full_cur && s_full[kh][buf] == 0;
    pf_tile<D>(o, m_run, l_run, qb, kt, vt, masked, klo_lds[kh][buf], kspan_lds[kh][buf], iq, a.scale_log2, lane,
               next);
    full_cur = full_next;
  }

  // ---- merge the odd half into the even half through LDS (the tile buffers
  // are free now): per lane, registers in order (dt, nt, r), then m and l.
  constexpr int NREG = DT * kPfNT * 16;
  static_assert(kPfRowWaves * NREG * 64 * 4 <= kPfHalves * 2 * SH::TILE_BYTES, "exchange fits the K buffers");
  static_assert(kPfRowWaves * 2 * kPfNT * 64 * 4 <= kPfHalves * 2 * SH::TILE_BYTES, "m, l fit the V buffers");
  float* xo = reinterpret_cast<float*>(&k_lds[0][0][0]) + sub * NREG * 64 + lane;
  float* xml = reinterpret_cast<float*>(&v_lds[0][0][0]) + sub * 2 * kPfNT * 64 + lane;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (kh == 1) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int nt = 0; nt < kPfNT; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[((dt * kPfNT + nt) * 16 + r) * 64] = o[dt][nt][r];
#pragma unroll
    for (int nt = 0; nt < kPfNT; ++nt) {
      xml[nt * 64] = m_run[nt];
      xml[(kPfNT + nt) * 64] = l_run[nt];
    }
  }
  __syncthreads();
  if (kh == 1) return;
#pragma unroll
  for (int nt = 0; nt < kPfNT; ++nt) {
    const float m2 = xml[nt * 64], l2 = xml[(kPfNT + nt) * 64];
    const float m_new = fmaxf(m_run[nt], m2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float a1 = fast_exp2(m_run[nt] - m_use), a2 = fast_exp2(m2 - m_use);
    l_run[nt] = l_run[nt] * a1 + l2 * a2;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][nt][r] = o[dt][nt][r] * a1 + xo[((dt * kPfNT + nt) * 16 + r) * 64] * a2;
  }

  // ---- normalise and store: lane holds d = dt*32 + 8*(r/4) + 4*hf + r%4 of query 32*nt + n
#pragma unroll
  for (int nt = 0; nt < kPfNT; ++nt) {
    const float l_tot = pair_sum(l_run[nt]);
    if (!qvalid[nt]) continue;
    const float inv = 1.f / l_tot;
    const int64_t qrow = wr0 + 32 * nt + n;
    uint16_t* op = static_cast<uint16_t*>(a.out) + (((size_t)w.b * a.n_q + h) * a.C + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = dt * 32 + 8 * r4 + 4 * hf;
        uint2 v;
        v.x = pack_bf16(o[dt][nt][4 * r4 + 0] * inv, o[dt][nt][4 * r4 + 1] * inv);
        v.y = pack_bf16(o[dt][nt][4 * r4 + 2] * inv, o[dt][nt][4 * r4 + 3] * inv);
        *reinterpret_cast<uint2*>(op + d0) = v;
      }
  }
}

// ------------------------------------------------------------------ fp32 path
// One wavefront per (batch, query head, chunk row); lanes own keys for the
// scores and d-chunks for the weighted sum.
template <int D>
__global__ __launch_bounds__(256) void prefill_f32_kernel(PrefillArgs a, int g) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t total = (int64_t)a.B * a.n_q * a.C;
  if (gw >= total) return;
  const int64_t qrow = gw % a.C;
  const int h = (int)((gw / a.C) % a.n_q);
  const int b = (int)(gw / ((int64_t)a.C * a.n_q));
  const int kvh = h / g;
  const bool ret = a.map.kind[kvh] != 0;
  const int ci = a.map.cidx[kvh];
  const int64_t t = a.P + qrow;
  const float* q = static_cast<const float*>(a.q) + (((size_t)b * a.n_q + h) * a.C + qrow) * D;
  // cache rows: row r of the head is row crow(r) of the layer's K / V array
  const float *kc, *vc;
  const int32_t* posc = nullptr;
  int64_t cache_rows;
  const size_t hrow = ((size_t)b * a.n_str + ci) * a.cap_str;
  if (ret) {
    kc = reinterpret_cast<const float*>(a.lp.k_ret);
    vc = reinterpret_cast<const float*>(a.lp.v_ret);
    cache_rows = a.P;
  } else {
    kc = reinterpret_cast<const float*>(a.lp.k_str);
    vc = reinterpret_cast<const float*>(a.lp.v_str);
    posc = a.lp.pos + hrow;
    cache_rows = a.held_str;
  }
  auto crow = [&](int64_t r) -> size_t {
    return ret ? (size_t)ret_row(a.lp, a.n_ret, a.cap_ret, b, ci, r) : hrow + (size_t)r;
  };
  const size_t coff = ((size_t)b * a.n_kv + kvh) * a.C * D;
  const float* kn = static_cast<const float*>(a.k) + coff;
  const float* vn = static_cast<const float*>(a.v) + coff;
  constexpr int EPL = D / 64;  // output elements per lane
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int64_t n_keys = cache_rows + qrow + 1;
  for (int64_t k0 = 0; k0 < n_keys; k0 += 64) {
    const int64_t kk = k0 + lane;
    float sv = -INFINITY;
    if (kk < n_keys) {
      const bool from_cache = kk < cache_rows;
      const int64_t row = from_cache ? kk : kk - cache_rows;
      const int64_t kp = from_cache ? (ret ? row : (int64_t)posc[row]) : a.P + row;
      if (visible(kp, t, ret, a.S, a.W)) {
        const float* kr = from_cache ? kc + crow(row) * D : kn + (size_t)row * D;
        float s = 0.f;
        for (int d = 0; d < D; ++d) s = fmaf(q[d], kr[d], s);
        sv = s * a.scale_log2;
      }
    }
    float mx = sv;
    for (int o2 = 32; o2 > 0; o2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o2));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    const float p = fast_exp2(sv - m_use);
    l_run = l_run * alpha + p;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
    const int nk = (int)min64(64, n_keys - k0);
    for (int j = 0; j < nk; ++j) {
      const float pj = __shfl(p, j);
      if (pj == 0.f) continue;
      const int64_t kj = k0 + j;
      const bool from_cache = kj < cache_rows;
      const int64_t row = from_cache ? kj : kj - cache_rows;
      const float* vr = from_cache ? vc + crow(row) * D : vn + (size_t)row * D;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pj, vr[lane + 64 * e], acc[e]);
    }
  }
  float l_tot = l_run;
  for (int o2 = 32; o2 > 0; o2 >>= 1) l_tot += __shfl_xor(l_tot, o2);
  float* op = static_cast<float*>(a.out) + (((size_t)b * a.n_q + h) * a.C + qrow) * D;
#pragma unroll
  for (int e = 0; e < EPL; ++e) op[lane + 64 * e] = acc[e] / l_tot;
}

}  // namespace

void prefill_plan(int dtype, int d, int g, int* rows_per_item, int* heads_per_item) {
  (void)d;
  if (dtype == 1) {
    // query heads per work item: four when 4 divides g, two when 2 does,
    // otherwise one (its four row wavefronts then take four row blocks)
    const int hpi = g % 4 == 0 ? 4 : g % 2 == 0 ? 2 : 1;
    *heads_per_item = hpi;
    *rows_per_item = kPfRowsPerWave * (kPfRowWaves / hpi);
  } else {
    *heads_per_item = 1;
    *rows_per_item = 1;
  }
}

hipError_t launch_prefill(const PrefillArgs& a, int dtype, int d, int g, hipStream_t s) {
  if (dtype == 1) {
    int rows, hpi;
    prefill_plan(dtype, d, g, &rows, &hpi);
    const int blocks = a.items_ret + a.B * a.n_str * (g / hpi) * a.q_tiles;
    if (blocks == 0) return hipSuccess;
    if (d == 128) prefill_mfma_kernel<128><<<blocks, kPfThreads, 0, s>>>(a, g, hpi);
    else if (d == 64) prefill_mfma_kernel<64><<<blocks, kPfThreads, 0, s>>>(a, g, hpi);
    else return hipErrorInvalidValue;
  } else {
    const int64_t waves = (int64_t)a.B * a.n_q * a.C;
    const int blocks = (int)((waves + 3) / 4);
    if (d == 128) prefill_f32_kernel<128><<<blocks, 256, 0, s>>>(a, g);
    else if (d == 64) prefill_f32_kernel<64><<<blocks, 256, 0, s>>>(a, g);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace duo
