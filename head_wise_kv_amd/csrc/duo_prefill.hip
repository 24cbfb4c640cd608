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
//   * Work item = one workgroup of two wavefronts; each wavefront owns 64
//     query rows of one query head (two 32-row MFMA N tiles), and the two
//     wavefronts share the K/V tiles of their KV head (two heads of a GQA
//     group, or two row blocks of one head).  64 query rows per wavefront is
//     what keeps LDS reads (K and V operands, re-read by every wavefront) under
//     the LDS bandwidth at full MFMA rate.
//   * K and V tiles of 64 keys are brought into LDS with direct global->LDS
//     loads, double buffered: the next tile streams in while the current one
//     is consumed.  Rows are XOR-swizzled in 16-byte chunks (the swizzle is
//     applied on the global side of the copy) so operand reads are free of
//     bank conflicts.
//   * Scores S^T = K Q^T put keys on the MFMA M axis and queries on N, so each
//     lane holds one query's scores and the softmax needs one exchange with
//     the partner lane.  P^T then feeds O^T = V^T P^T directly from the
//     accumulator registers; the V^T operand comes straight from the
//     row-major V tile through LDS transpose reads (ds_read_b64_tr_b16).
//   * Streaming heads visit only the sink tiles, the ring tiles some row's
//     window reaches, and the local band of the chunk; retrieval heads the
//     causal prefix.  Tiles every row sees in full skip the mask.
//
// fp32: a plain vector-ALU path (one wavefront per query row) kept for
// completeness of the dtype surface; it is not tuned.
#include "duo_internal.h"

#include <hip/hip_runtime.h>

#include <climits>

namespace duo {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr int kPfWaves = 2;                       // wavefronts per workgroup
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfRowsPerWave = 64;                // query rows per wavefront
constexpr int kBN = 64;                           // keys per tile

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  bf2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bool visible(int64_t kp, int64_t t, bool ret, int S, int W) {
  return kp >= 0 && kp <= t && (ret || kp < S || kp >= t - W + 1);
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
  const int64_t chunk_hi = (min(i1, a.C) + kBN - 1) / kBN;  // causal: keys jj <= i < i1
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
    const int64_t last_slot = ring_needed ? held : min<int64_t>(held, a.S);
    tr.cache_lo = 0;
    tr.cache_hi = (last_slot + kBN - 1) / kBN;
    // chunk: sink keys (positions < S) and the band jj >= i0 - W + 1
    const int64_t sink_rows = max<int64_t>(0, min<int64_t>(a.C, (int64_t)a.S - a.P));
    const int64_t sink_tiles = (sink_rows + kBN - 1) / kBN;
    const int64_t band_lo = max<int64_t>(0, i0 - a.W + 1) / kBN;
    if (band_lo <= sink_tiles) {
      tr.chunk_lo0 = 0;
      tr.chunk_hi0 = chunk_hi;
      tr.chunk_lo1 = tr.chunk_hi1 = 0;
    } else {
      tr.chunk_lo0 = 0;
      tr.chunk_hi0 = min(sink_tiles, chunk_hi);
      tr.chunk_lo1 = band_lo;
      tr.chunk_hi1 = chunk_hi;
    }
  }
  return tr;
}

// ------------------------------------------------------------------ bf16 MFMA path

template <int D>
struct PfShape {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int TILE_BYTES = kBN * D * 2;    // one K (or V) tile
  static constexpr int DMA_PER_TILE = TILE_BYTES / 1024;  // 1 KB per wavefront-wide direct load
  static constexpr int KSTEPS = D / 16;             // MFMA k-steps over d for S^T
  static constexpr int DT = D / 32;                 // 32-row tiles of O^T over d
  static_assert(DMA_PER_TILE % kPfWaves == 0, "tile loads split over the wavefronts");
  // K rows: chunk c of key r sits at chunk slot c ^ swz_k(r) (A-operand reads
  // of 16 consecutive keys at one chunk hit 16 distinct bank groups).
  __device__ static __forceinline__ int swz_k(int r) { return CPR == 16 ? (r & 15) : ((r >> 1) & 7); }
  // V rows: chunk c of key r at c ^ swz_v(r) (a transpose read of 4 rows x
  // 4 chunks by 32 lanes hits 16 distinct bank groups).
  __device__ static __forceinline__ int swz_v(int r) { return CPR == 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

struct PfItem {
  int b, kvh, cidx, h_first, qt;
  bool ret;
};

// Work items: retrieval items first (longest rows first), then streaming.
// Within a kind: (b, kv head, head group, query tile), query tile fastest.
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
  const int qt_rev = rem % a.q_tiles;
  rem /= a.q_tiles;
  const int hg = rem % ngrp;
  rem /= ngrp;
  w.cidx = rem % n_kind;
  w.b = rem / n_kind;
  w.qt = a.q_tiles - 1 - qt_rev;
  w.kvh = w.ret ? a.map.orig_ret[w.cidx] : a.map.orig_str[w.cidx];
  w.h_first = w.kvh * g + hg * hpi;
  return w;
}

// Direct global->LDS copy of one 64-row tile (K or V): wavefront `wave`
// issues every kPfWaves-th 1 KB piece.  Piece n covers LDS bytes
// [n*1024, n*1024+1024): lane i writes 16 bytes at n*1024 + i*16, i.e. row
// (n*1024 + i*16) / (16*CPR), chunk slot ((n*64 + i) % CPR); the global
// chunk it fetches is that slot XOR the row's swizzle.  Rows past `limit`
// are clamped to the last valid row (their keys are masked).
template <int D, bool IS_V>
__device__ __forceinline__ void dma_tile(char* lds_tile, const char* src, int64_t base, int64_t limit, int wave,
                                         int lane) {
  using SH = PfShape<D>;
#pragma unroll
  for (int n = wave; n < SH::DMA_PER_TILE; n += kPfWaves) {
    const int piece = n * 64 + lane;              // 16-byte slot index within the tile
    const int r = piece / SH::CPR;
    const int slot = piece % SH::CPR;
    const int c = slot ^ (IS_V ? SH::swz_v(r) : SH::swz_k(r));
    const int64_t row = min<int64_t>(base + r, limit - 1);
    const char* g = src + (size_t)row * (D * 2) + c * 16;
    __builtin_amdgcn_global_load_lds((const void*)g, (__attribute__((address_space(3))) void*)(lds_tile + n * 1024),
                                     16, 0, 0);
  }
}

template <int D>
__global__ __launch_bounds__(kPfThreads) void prefill_mfma_kernel(PrefillArgs a, int g, int hpi) {
  using SH = PfShape<D>;
  constexpr int CPR = SH::CPR, KSTEPS = SH::KSTEPS, DT = SH::DT;

  __shared__ __attribute__((aligned(1024))) char k_lds[2][SH::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds[2][SH::TILE_BYTES];
  __shared__ int64_t kpos_lds[2][kBN];
  __shared__ int s_full[2];

  const PfItem w = pf_item(a, g, hpi);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hf = lane >> 5;
  // this wavefront's head and rows: hpi heads x (kPfWaves / hpi) row blocks
  const int h = w.h_first + (wave % hpi);
  const int rows_item = kPfRowsPerWave * (kPfWaves / hpi);
  const int64_t i0 = (int64_t)w.qt * rows_item;                       // item's first chunk row
  const int64_t i1 = min<int64_t>(i0 + rows_item, a.C);
  const int64_t wr0 = i0 + (int64_t)(wave / hpi) * kPfRowsPerWave;   // wavefront's first row
  const size_t rowb = (size_t)D * 2;

  // Q^T operands: lane holds 8 consecutive d of query row (wr0 + 32*nt + n) per k-step.
  bf16x8_t qb[2][KSTEPS];
  int64_t tq[2];
  bool qvalid[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int64_t qrow = wr0 + 32 * nt + n;
    qvalid[nt] = qrow < a.C;
    tq[nt] = a.P + qrow;
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
    const size_t off = ((size_t)w.b * a.n_ret + w.cidx) * a.cap_ret * rowb;
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
  const int64_t cache_rows = w.ret ? a.P : a.held_str;

  const TileRanges tr = plan_tiles(a, w.ret, i0, i1);
  const int64_t n_cache = tr.cache_hi - tr.cache_lo;
  const int64_t n_c0 = tr.chunk_hi0 - tr.chunk_lo0;
  const int64_t n_c1 = tr.chunk_hi1 - tr.chunk_lo1;
  const int64_t n_tiles = n_cache + n_c0 + n_c1;
  // query positions the item covers (for the "every row sees every key" test)
  const int64_t t_lo = a.P + i0;

  // Tile `it` -> (source, first row, row limit).
  auto tile_src = [&](int64_t it, int& src, int64_t& base, int64_t& limit) {
    if (it < n_cache) {
      src = w.ret ? SRC_CACHE_LINEAR : SRC_CACHE_SLOTS;
      base = (tr.cache_lo + it) * kBN;
      limit = cache_rows;
    } else if (it < n_cache + n_c0) {
      src = SRC_CHUNK;
      base = (tr.chunk_lo0 + (it - n_cache)) * kBN;
      limit = a.C;
    } else {
      src = SRC_CHUNK;
      base = (tr.chunk_lo1 + (it - n_cache - n_c0)) * kBN;
      limit = a.C;
    }
  };
  // Issue tile `it` into buffer `buf`: K/V by direct loads, positions by plain
  // stores (thread < kBN), and a flag telling whether every row of the item
  // sees every key of the tile (then the mask is skipped).
  auto issue = [&](int64_t it, int buf) {
    int src;
    int64_t base, limit;
    tile_src(it, src, base, limit);
    const char* ks = (src == SRC_CHUNK) ? kn : kc;
    const char* vs = (src == SRC_CHUNK) ? vn : vc;
    dma_tile<D, false>(k_lds[buf], ks, base, limit, wave, lane);
    dma_tile<D, true>(v_lds[buf], vs, base, limit, wave, lane);
    if (tid < kBN) {
      const int64_t row = base + tid;
      int64_t kp = INT64_MIN;  // past the end: never visible
      if (row < limit) {
        if (src == SRC_CACHE_LINEAR) kp = row;
        else if (src == SRC_CACHE_SLOTS) kp = posc[row];
        else kp = a.P + row;
      }
      kpos_lds[buf][tid] = kp;
    }
    if (tid == 0) {
      // full iff all 64 rows exist and (retrieval: the last key precedes the
      // first query) -- streaming tiles are always masked (the window moves).
      const bool all_rows = base + kBN <= limit;
      int64_t last_pos;
      if (src == SRC_CACHE_LINEAR) last_pos = base + kBN - 1;
      else if (src == SRC_CHUNK) last_pos = a.P + base + kBN - 1;
      else last_pos = INT64_MAX;
      s_full[buf] = (w.ret && all_rows && last_pos <= t_lo) ? 1 : 0;
    }
  };

  f32x16_t o[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][nt][r] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  if (n_tiles > 0) issue(0, 0);
  for (int64_t it = 0; it < n_tiles; ++it) {
    const int buf = (int)(it & 1);
    // this wavefront's direct loads for tile `it` have landed; after the
    // barrier every wavefront's have, and the previous tile is consumed.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (it + 1 < n_tiles) issue(it + 1, buf ^ 1);

    const char* kt = k_lds[buf];
    const char* vt = v_lds[buf];
    // ---- S^T = K Q^T: [key half ct][query tile nt]
    f32x16_t s[2][2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[ct][nt][r] = 0.f;
      const int key = ct * 32 + n;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int c = 2 * ks + hf;
        const u32x4_t av =
            *reinterpret_cast<const u32x4_t*>(kt + key * (CPR * 16) + ((c ^ SH::swz_k(key)) * 16));
        const bf16x8_t aop = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          s[ct][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, qb[nt][ks], s[ct][nt], 0, 0, 0);
      }
    }

    // ---- mask (unless every row sees every key), online softmax in log2 units
    if (!s_full[buf]) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = ct * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          const int64_t kp = kpos_lds[buf][key];
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            if (!visible(kp, tq[nt], w.ret, a.S, a.W)) s[ct][nt][r] = -INFINITY;
        }
    }
    uint32_t pb[2][2][2][4];  // [nt][ct][k-step][dword]: P^T as bf16 pairs
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mx = -INFINITY;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[ct][nt][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32)) * a.scale_log2;
      const float m_new = fmaxf(m_run[nt], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[nt] - m_use);
      m_run[nt] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(fmaf(s[ct][nt][r], a.scale_log2, -m_use));
          const float p1 = fast_exp2(fmaf(s[ct][nt][r + 1], a.scale_log2, -m_use));
          psum += p0 + p1;
          pb[nt][ct][r >> 3][(r & 7) >> 1] = pack_bf16(p0, p1);
        }
      l_run[nt] = l_run[nt] * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][nt][r] *= alpha;
    }

    // ---- O^T += V^T P^T; V^T operands by transpose reads of the V tile:
    // lane (group g = lane/16, i = lane%16) reads row kb + i/4 at columns
    // dt*32 + 16*(g%2) + 4*(i%4); lane receives V[kb + 0..3][its d].
    const int g16 = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bf16x8_t bop[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const u32x4_t bw = {pb[nt][ct][st][0], pb[nt][ct][st][1], pb[nt][ct][st][2], pb[nt][ct][st][3]};
          bop[nt] = __builtin_bit_cast(bf16x8_t, bw);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          i16x4_t half[2];
#pragma unroll
          for (int rr = 0; rr < 2; ++rr) {
            const int row = ct * 32 + 16 * st + 8 * rr + 4 * hf + (i16 >> 2);
            const int col = dt * 32 + 16 * (g16 & 1) + 4 * (i16 & 3);
            const int c = col >> 3;
            const char* p = vt + row * (CPR * 16) + ((c ^ SH::swz_v(row)) * 16) + (col & 7) * 2;
            half[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p));
          }
          const u32x2_t h0 = __builtin_bit_cast(u32x2_t, half[0]);
          const u32x2_t h1 = __builtin_bit_cast(u32x2_t, half[1]);
          const u32x4_t aw = {h0[0], h0[1], h1[0], h1[1]};
          const bf16x8_t aop = __builtin_bit_cast(bf16x8_t, aw);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            o[dt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop[nt], o[dt][nt], 0, 0, 0);
        }
      }
  }

  // ---- normalise and store: lane holds d = dt*32 + 8*(r/4) + 4*hf + r%4 of query 32*nt + n
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float l_tot = l_run[nt] + __shfl_xor(l_run[nt], 32);
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
  const float *kc, *vc;
  const int32_t* posc = nullptr;
  int64_t cache_rows;
  if (ret) {
    const size_t off = ((size_t)b * a.n_ret + ci) * a.cap_ret * D;
    kc = reinterpret_cast<const float*>(a.lp.k_ret) + off;
    vc = reinterpret_cast<const float*>(a.lp.v_ret) + off;
    cache_rows = a.P;
  } else {
    const size_t hrow = ((size_t)b * a.n_str + ci) * a.cap_str;
    kc = reinterpret_cast<const float*>(a.lp.k_str) + hrow * D;
    vc = reinterpret_cast<const float*>(a.lp.v_str) + hrow * D;
    posc = a.lp.pos + hrow;
    cache_rows = a.held_str;
  }
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
        const float* kr = (from_cache ? kc : kn) + (size_t)row * D;
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
    const int nk = (int)min<int64_t>(64, n_keys - k0);
    for (int j = 0; j < nk; ++j) {
      const float pj = __shfl(p, j);
      if (pj == 0.f) continue;
      const int64_t kj = k0 + j;
      const bool from_cache = kj < cache_rows;
      const int64_t row = from_cache ? kj : kj - cache_rows;
      const float* vr = (from_cache ? vc : vn) + (size_t)row * D;
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
    const int hpi = g >= kPfWaves ? kPfWaves : g;  // query heads per work item
    *heads_per_item = hpi;
    *rows_per_item = kPfRowsPerWave * (kPfWaves / hpi);
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
