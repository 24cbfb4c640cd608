// Chunked prefill over a per-KV-head mixed KV cache, for gfx950 (CDNA4).
//
// A chunk of C tokens at absolute positions P .. P+C-1 attends over the keys
// the cache holds plus the chunk itself.  Retrieval heads use the causal mask
// (key j visible to the row at t iff j <= t); streaming heads use the
// sink + local-window mask (j <= t and (j < S or j >= t - W + 1)), with cached
// keys read from the sink and ring slots and their stored positions.  The
// chunk is committed to the cache by the append kernel afterwards.
//
// bf16: a dense contraction, tiled on MFMA (v_mfma_f32_32x32x16_bf16).  One
// workgroup = 4 wavefronts x 32 query rows of one query head; key tiles of 64.
// Each wavefront computes S^T = K Q^T (keys on the MFMA M axis, queries on N),
// so that a query's scores stay within one lane pair and the softmax needs one
// cross-lane exchange; P^T then feeds O^T = V^T P^T straight from registers,
// with V^T staged in LDS under a key permutation that matches the MFMA
// accumulator layout.  Streaming heads visit only the key tiles their mask can
// reach (sink tiles plus the local band), retrieval heads the causal prefix.
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

constexpr int kPrefillThreads = 256;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerTile = kRowsPerWave * (kPrefillThreads / 64);  // 128 query rows per workgroup
constexpr int kBN = 64;                                             // keys per tile

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) { return bf16_rne(lo) | (bf16_rne(hi) << 16); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Key tile sources.
enum : int { SRC_CACHE_LINEAR = 0, SRC_CACHE_SLOTS = 1, SRC_CHUNK = 2 };

struct WorkItem {
  int b, kvh, h, cidx, qt;
  bool ret;
};

__device__ __forceinline__ WorkItem decode_item(const PrefillArgs& a, int g) {
  WorkItem w;
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
  const int qt_rev = rem % a.q_tiles;
  rem /= a.q_tiles;
  const int hq = rem % g;
  rem /= g;
  w.cidx = rem % n_kind;
  w.b = rem / n_kind;
  w.qt = a.q_tiles - 1 - qt_rev;  // longest rows first
  w.kvh = w.ret ? a.map.orig_ret[w.cidx] : a.map.orig_str[w.cidx];
  w.h = w.kvh * g + hq;
  return w;
}

// Tile ranges (in units of kBN keys) a workgroup visits, per source.
struct TileRanges {
  int64_t cache_tiles;       // tiles over the cache part
  int64_t chunk_lo0, chunk_hi0, chunk_lo1, chunk_hi1;  // up to two ranges of chunk tiles
  int64_t cache_lo, cache_hi;
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

__device__ __forceinline__ bool visible(int64_t kp, int64_t t, bool ret, int S, int W) {
  return kp >= 0 && kp <= t && (ret || kp < S || kp >= t - W + 1);
}

// Swap bits 2 and 3 of a key index: the V^T column that makes the MFMA
// accumulator layout of P^T line up with the A-operand layout of V^T.
__device__ __forceinline__ int vt_col(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

template <int D>
__global__ __launch_bounds__(kPrefillThreads) void prefill_bf16_kernel(PrefillArgs a, int g) {
  constexpr int KROW = D * 2 + 16;  // bytes per K row in LDS (16-byte pad)
  constexpr int VTS = kBN + 8;      // bf16 elements per V^T row in LDS
  constexpr int KSTEPS = D / 16;    // MFMA k-steps over d for S^T
  constexpr int DT = D / 32;        // 32-row tiles of O^T over d
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int CHUNKS = kBN * CPR; // chunks per K (or V) tile
  constexpr int PER_THREAD = CHUNKS / kPrefillThreads;
  static_assert(CHUNKS % kPrefillThreads == 0, "tile must split evenly");

  __shared__ __attribute__((aligned(16))) char k_lds[kBN * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * VTS];
  __shared__ int64_t kpos_lds[kBN];

  const WorkItem w = decode_item(a, g);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hf = lane >> 5;
  const int64_t i0 = (int64_t)w.qt * kRowsPerTile;
  const int64_t i1 = min<int64_t>(i0 + kRowsPerTile, a.C);
  const int64_t qrow = i0 + wave * kRowsPerWave + n;
  const bool qvalid = qrow < a.C;
  const int64_t t = a.P + qrow;
  const size_t rowb = (size_t)D * 2;

  // Q^T operands: lane holds 8 consecutive d of its query row per k-step.
  bf16x8_t qb[KSTEPS];
  {
    const char* qp = static_cast<const char*>(a.q) + (((size_t)w.b * a.n_q + w.h) * a.C + (qvalid ? qrow : 0)) * rowb;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4_t v = qvalid ? *reinterpret_cast<const u32x4_t*>(qp + (ks * 16 + hf * 8) * 2) : u32x4_t{0, 0, 0, 0};
      qb[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // Key sources for this head.
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

  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Iterate: cache tiles, then up to two chunk ranges.
  const int64_t n_cache = tr.cache_hi - tr.cache_lo;
  const int64_t n_c0 = tr.chunk_hi0 - tr.chunk_lo0;
  const int64_t n_c1 = tr.chunk_hi1 - tr.chunk_lo1;
  const int64_t n_tiles = n_cache + n_c0 + n_c1;

  for (int64_t it = 0; it < n_tiles; ++it) {
    int src;
    int64_t tile;
    if (it < n_cache) {
      src = w.ret ? SRC_CACHE_LINEAR : SRC_CACHE_SLOTS;
      tile = tr.cache_lo + it;
    } else if (it < n_cache + n_c0) {
      src = SRC_CHUNK;
      tile = tr.chunk_lo0 + (it - n_cache);
    } else {
      src = SRC_CHUNK;
      tile = tr.chunk_lo1 + (it - n_cache - n_c0);
    }
    const int64_t base = tile * kBN;
    const int64_t limit = (src == SRC_CHUNK) ? a.C : cache_rows;
    const char* kt = (src == SRC_CHUNK) ? kn : kc;
    const char* vt = (src == SRC_CHUNK) ? vn : vc;

    __syncthreads();  // previous tile fully consumed
    // ---- stage K (row-major, padded) and V^T (permuted columns) in LDS
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int ci = j * kPrefillThreads + tid;
      const int r = ci / CPR, c = ci % CPR;
      const int64_t row = base + r;
      u32x4_t kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (row < limit) {
        kv = *reinterpret_cast<const u32x4_t*>(kt + (size_t)row * rowb + c * 16);
        vv = *reinterpret_cast<const u32x4_t*>(vt + (size_t)row * rowb + c * 16);
      }
      *reinterpret_cast<u32x4_t*>(k_lds + r * KROW + c * 16) = kv;
      const int col = vt_col(r);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vt_lds[(c * 8 + 2 * e) * VTS + col] = (uint16_t)(vv[e] & 0xffffu);
        vt_lds[(c * 8 + 2 * e + 1) * VTS + col] = (uint16_t)(vv[e] >> 16);
      }
    }
    if (tid < kBN) {
      const int64_t row = base + tid;
      int64_t kp = INT64_MIN;  // invalid slot: never visible
      if (row < limit) {
        if (src == SRC_CACHE_LINEAR) kp = row;
        else if (src == SRC_CACHE_SLOTS) kp = posc[row];
        else kp = a.P + row;
      }
      kpos_lds[tid] = kp;
    }
    __syncthreads();

    // ---- S^T = K Q^T for the two 32-key halves of the tile
    f32x16_t s[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[ct][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const u32x4_t av = *reinterpret_cast<const u32x4_t*>(k_lds + (ct * 32 + n) * KROW + ks * 32 + hf * 16);
        s[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av), qb[ks], s[ct], 0, 0, 0);
      }
    }

    // ---- mask, online softmax (log2 domain); lane pair (n, n+32) shares a query
    float mx = -INFINITY;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = ct * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        const bool vis = visible(kpos_lds[key], t, w.ret, a.S, a.W);
        const float v = vis ? s[ct][r] * a.scale_log2 : -INFINITY;
        s[ct][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
    uint32_t pb[2][2][4];  // [ct][k-step][dword]: P^T as bf16 pairs
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(s[ct][r] - m_use);
        const float p1 = fast_exp2(s[ct][r + 1] - m_use);
        psum += p0 + p1;
        pb[ct][r >> 3][(r & 7) >> 1] = pack_bf16(p0, p1);
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;

    // ---- O^T += V^T P^T
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u32x4_t bw = {pb[ct][st][0], pb[ct][st][1], pb[ct][st][2], pb[ct][st][3]};
        const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, bw);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const u32x4_t av =
              *reinterpret_cast<const u32x4_t*>(vt_lds + (dt * 32 + n) * VTS + ct * 32 + st * 16 + hf * 8);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av), bop, o[dt], 0, 0, 0);
        }
      }
  }

  // ---- normalise and store: lane holds d = dt*32 + 8*(r/4) + 4*hf + r%4 of its query
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!qvalid) return;
  const float inv = 1.f / l_tot;
  uint16_t* op = static_cast<uint16_t*>(a.out) + (((size_t)w.b * a.n_q + w.h) * a.C + qrow) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = dt * 32 + 8 * r4 + 4 * hf;
      uint2 v;
      v.x = pack_bf16(o[dt][4 * r4 + 0] * inv, o[dt][4 * r4 + 1] * inv);
      v.y = pack_bf16(o[dt][4 * r4 + 2] * inv, o[dt][4 * r4 + 3] * inv);
      *reinterpret_cast<uint2*>(op + d0) = v;
    }
}

// fp32 path: one wavefront per (batch, query head, chunk row); lanes own keys
// for the scores and d-chunks for the weighted sum.
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

int prefill_rows_per_tile(int dtype, int d) {
  (void)d;
  return dtype == 1 ? kRowsPerTile : 1;
}

hipError_t launch_prefill(const PrefillArgs& a, int dtype, int d, int g, hipStream_t s) {
  if (dtype == 1) {
    const int blocks = a.items_ret + a.B * a.n_str * g * a.q_tiles;
    if (blocks == 0) return hipSuccess;
    if (d == 128) prefill_bf16_kernel<128><<<blocks, kPrefillThreads, 0, s>>>(a, g);
    else if (d == 64) prefill_bf16_kernel<64><<<blocks, kPrefillThreads, 0, s>>>(a, g);
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
