// HIP kernels for gfx950 (CDNA4): cache fill, append and split-K decode over a
// per-KV-head mixed KV cache (DuoAttention: retrieval heads hold every token,
// streaming heads hold S sinks + a W-slot ring).
//
// Decode is bound by HBM bandwidth (g = n_q / n_kv flops per byte of K/V), so
// it runs on the vector ALUs, not on MFMA.  The rows held by every (batch, KV
// head) -- all T rows of a retrieval head, the min(T, S+W) sink and ring slots
// of a streaming head -- form one flattened row space cut into equal work
// items, one per compute unit, so long retrieval heads and short streaming
// heads are balanced by bytes.  Within an item each wavefront streams tiles of
// rows with coalesced 16-byte loads, two tiles in flight, scores them with
// packed bf16 dot products against the GQA query group held in registers,
// keeps online softmax statistics per lane, and accumulates P.V with bf16 dot
// products.  Partial (max, sum, acc) results of items that share a head are
// merged in-kernel by the last-arriving item of each group, then of the head.
#include "duo_internal.h"

#include <hip/hip_runtime.h>

namespace duo {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Orders LDS traffic between lanes of one wavefront.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint4 ld16(const char* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(char* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// ------------------------------------------------------------------ fill

__global__ void fill_zero_kernel(uint4* p, size_t n16, unsigned char* tail, size_t ntail) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t j = i; j < n16; j += stride) p[j] = make_uint4(0, 0, 0, 0);
  if (i < ntail) tail[i] = 0;
}

// ------------------------------------------------------------------ append
// One thread per 16-byte chunk of an input row.  Position p = p0 + i goes to
// row p of a retrieval head; for a streaming head to slot p while p < S, else
// to ring slot S + (p - S) mod W, but only if the token is among the last W of
// the batch (p >= keep_from); earlier ones would be evicted by later tokens of
// the same call, and skipping them keeps every slot written at most once.

__global__ void append_kernel(AppendArgs a) {
  const int cpr = a.row_bytes / 16;
  const int64_t total = (int64_t)a.B * a.n_kv * a.n_new * cpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int c = (int)(idx % cpr);
    int64_t rest = idx / cpr;
    const int64_t i = rest % a.n_new;
    rest /= a.n_new;
    const int kvh = (int)(rest % a.n_kv);
    const int b = (int)(rest / a.n_kv);
    const int64_t p = a.p0 + i;
    const size_t src = (size_t)idx * 16;
    char *kd, *vd;
    if (a.map.kind[kvh]) {
      const int r = a.map.cidx[kvh];
      const size_t off = (((size_t)b * a.n_ret + r) * a.cap_ret + p) * a.row_bytes + (size_t)c * 16;
      kd = a.lp.k_ret + off;
      vd = a.lp.v_ret + off;
    } else {
      int64_t slot;
      if (p < a.S) {
        slot = p;
      } else if (p >= a.keep_from) {
        slot = a.S + (p - a.S) % a.W;
      } else {
        continue;
      }
      const int s = a.map.cidx[kvh];
      const size_t hrow = ((size_t)b * a.n_str + s) * a.cap_str + slot;
      const size_t off = hrow * a.row_bytes + (size_t)c * 16;
      kd = a.lp.k_str + off;
      vd = a.lp.v_str + off;
      if (c == 0) a.lp.pos[hrow] = (int32_t)p;
    }
    st16(kd, ld16(a.k + src));
    st16(vd, ld16(a.v + src));
  }
}

// ------------------------------------------------------------------ decode
//
// Lane layout: 8 lanes share a K/V row.  Lane l has row group rg = l / 8 and
// slice s = l % 8; it holds the 16-byte chunks s, s+8, ... of its rows, so one
// wavefront load instruction reads 8 rows x 128 contiguous bytes.  The g query
// vectors of the KV head live in the same slice layout in registers for the
// whole work item.  Scores: packed bf16 dot products over the lane's slice,
// then an all-reduce over the 8 lanes of the row with DPP adds.  Softmax
// statistics are kept per lane (each lane group sees its own rows); P.V uses
// bf16 dot products over pairs of rows.  Row groups and wavefronts are merged
// once at the end of a work item.

// Tuning knobs (compile time): query heads per wavefront, prefetch depth in
// tiles, and wavefronts per SIMD the kernel is built for.
#ifndef DUO_DECODE_HW_MAX
#define DUO_DECODE_HW_MAX 4
#endif
#ifndef DUO_DECODE_STAGES
#define DUO_DECODE_STAGES 1
#endif
#ifndef DUO_DECODE_WAVES_PER_EU
#define DUO_DECODE_WAVES_PER_EU 2
#endif

template <bool BF16, int D, int G>
struct DecodeCfg {
  static constexpr int ES = BF16 ? 2 : 4;        // element bytes
  static constexpr int ROWB = D * ES;            // bytes per row
  static constexpr int CPR = ROWB / 16;          // 16-byte chunks per row
  static constexpr int CPL = CPR / 8;            // chunks per lane
  static constexpr int EPC = 16 / ES;            // elements per chunk
  static constexpr int HW = G < DUO_DECODE_HW_MAX ? G : DUO_DECODE_HW_MAX;  // query heads per wavefront
  static constexpr int HSPLIT = G / HW;          // wavefronts sharing one tile stream
  static constexpr int NW = kDecodeThreads / 64;
  static constexpr int NSTREAM = NW / HSPLIT;    // independent tile streams per workgroup
  static constexpr int RPL_RAW = 8 / CPL;
  static constexpr int RPL = RPL_RAW < 2 ? 2 : RPL_RAW;  // rows per lane per tile (2*RPL*CPL loads)
  static constexpr int STAGES = DUO_DECODE_STAGES;       // tiles in the prefetch ring
  static constexpr int TR = 8 * RPL;             // rows per wavefront tile
  static constexpr int NACC = CPL * EPC;         // output elements per lane per head
  static_assert(CPR % 8 == 0, "rows must span a multiple of 8 chunks");
  static_assert(RPL % 2 == 0, "rows are paired for the weighted sum");
  static_assert(G % HW == 0 && NW % HSPLIT == 0, "head split must tile the workgroup");
  static_assert(STAGES >= 1 && STAGES <= 4, "prefetch ring of 1..4 tiles");
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// all-reduce over the 8 lanes of a row: xor 1, xor 2, then mirror within 8
__device__ __forceinline__ float row8_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  return x;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  bf2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Partial records pass between workgroups (possibly on different XCDs, each
// with its own L2) as agent-scope relaxed atomic stores and loads.  These are
// write-through / coherent accesses (the `sc1` cache policy), so no L2
// write-back or invalidate is needed.  A writer waits until its stores are
// acknowledged (vmcnt(0)) before taking its merge ticket; the merging
// workgroup reads the records only after the last ticket, with coherent loads.
// This replaces agent-scope release/acquire fences, whose full-L2
// write-back/invalidate per workgroup costs far more than the merge itself.
__device__ __forceinline__ void rec_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float rec_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Elements of the g x d output a thread of the workgroup owns in the merge
// steps: consecutive ones, all in the same head.
template <int D, int G>
struct MergeShape {
  static constexpr int OPT = (G * D) >= kDecodeThreads ? (G * D) / kDecodeThreads : 1;
  static_assert(D % OPT == 0, "a thread's elements must stay in one head");
};

// Merge `n` partial records (acc[G][D], m[G], l[G]; m in log2 units) into
// either the final output or one record at `dst_rec`.  Records are taken in
// batches of kSplitGroup; every load of a batch is issued before any is used,
// so a batch costs one memory round trip (a merge is normally one batch).
template <bool BF16, int D, int G>
__device__ void merge_records(const float* src, int n, float* dst_rec, void* out, size_t out_off) {
  constexpr int REC = G * (D + 2);
  constexpr int NB = kSplitGroup;
  constexpr int OPT = MergeShape<D, G>::OPT;
  const int e0 = threadIdx.x * OPT;
  if (e0 >= G * D) return;
  const int h = e0 / D;
  float M = -INFINITY, L = 0.f, A[OPT];
#pragma unroll
  for (int o = 0; o < OPT; ++o) A[o] = 0.f;
  for (int i0 = 0; i0 < n; i0 += NB) {
    float mv[NB], lv[NB], av[NB][OPT];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int i = min(i0 + j, n - 1);  // in range; entries past n are weighted out below
      const float* r = src + (size_t)i * REC;
      mv[j] = rec_load(r + G * D + h);
      lv[j] = rec_load(r + G * D + G + h);
#pragma unroll
      for (int o = 0; o < OPT; ++o) av[j][o] = rec_load(r + e0 + o);
    }
    float Mb = M;
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (i0 + j < n) Mb = fmaxf(Mb, mv[j]);
    const float f = (M == -INFINITY) ? 0.f : fast_exp2(M - Mb);
    L *= f;
#pragma unroll
    for (int o = 0; o < OPT; ++o) A[o] *= f;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (i0 + j < n) {
        const float w = (mv[j] == -INFINITY) ? 0.f : fast_exp2(mv[j] - Mb);
        L += lv[j] * w;
#pragma unroll
        for (int o = 0; o < OPT; ++o) A[o] += av[j][o] * w;
      }
    }
    M = Mb;
  }
  if (dst_rec) {
#pragma unroll
    for (int o = 0; o < OPT; ++o) rec_store(dst_rec + e0 + o, A[o]);
    if (e0 % D == 0) {
      rec_store(dst_rec + G * D + h, M);
      rec_store(dst_rec + G * D + G + h, L);
    }
  } else {
    const float inv = 1.f / L;
#pragma unroll
    for (int o = 0; o < OPT; ++o) {
      if (BF16) {
        reinterpret_cast<uint16_t*>(out)[out_off + e0 + o] = (uint16_t)f32_to_bf16_bits(A[o] * inv);
      } else {
        reinterpret_cast<float*>(out)[out_off + e0 + o] = A[o] * inv;
      }
    }
  }
}

template <bool BF16, int D, int G>
struct DecodeTile {
  using C = DecodeCfg<BF16, D, G>;
  uint4 k[C::RPL][C::CPL];
  uint4 v[C::RPL][C::CPL];
};

// Rows tb + rg + 8*j, chunks s + 8*cc.  Rows at or past `last` are clamped to
// `last` (a held row), so the load is always issued and always in bounds;
// process_tile masks those rows out.  Keeping the loads unconditional lets
// the compiler count outstanding loads exactly across the prefetch ring.
// Offsets within one head fit 32 bits (T_cap * row bytes < 2^32 is checked
// by the host), so the loads use a uniform base plus a 32-bit lane offset.
template <bool BF16, int D, int G>
__device__ __forceinline__ void load_tile(DecodeTile<BF16, D, G>& t, const char* kb, const char* vb, int64_t tb,
                                          int64_t last, int rg, int s) {
  using C = DecodeCfg<BF16, D, G>;
#pragma unroll
  for (int j = 0; j < C::RPL; ++j) {
    const uint32_t row = (uint32_t)min(tb + rg + 8 * j, last);
#pragma unroll
    for (int cc = 0; cc < C::CPL; ++cc) {
      const uint32_t o = row * (uint32_t)C::ROWB + (uint32_t)(s + 8 * cc) * 16u;
      t.k[j][cc] = ld16(kb + o);
      t.v[j][cc] = ld16(vb + o);
    }
  }
  // Keep the requests where they are issued: the scheduler would otherwise
  // sink them next to their use and shorten the prefetch distance.
  __builtin_amdgcn_sched_barrier(0);
}

// Per-lane softmax state.  m is a reference maximum (log2 units); l and acc
// are kept relative to it.  The reference is raised only when a score
// exceeds it by more than kRescaleSlack, so exp2(score - m) <= 2^slack and the
// rescale of acc and l is rare after the first tiles.
constexpr float kRescaleSlack = 8.f;

template <bool BF16, int D, int G>
struct DecodeState {
  using C = DecodeCfg<BF16, D, G>;
  float m[C::HW], l[C::HW];
  float acc[C::HW][C::NACC];
};

template <bool BF16, int D, int G>
__device__ __forceinline__ void process_tile(DecodeState<BF16, D, G>& st, const DecodeTile<BF16, D, G>& t,
                                             const uint4 (&q)[DecodeCfg<BF16, D, G>::HW][DecodeCfg<BF16, D, G>::CPL],
                                             int64_t nv, int rg, float scale_log2) {
  using C = DecodeCfg<BF16, D, G>;
  constexpr int HW = C::HW;
  float sc[C::RPL][HW];
  // ---- partial scores over the lane's slice, then the 8-lane all-reduce
#pragma unroll
  for (int j = 0; j < C::RPL; ++j)
#pragma unroll
    for (int h = 0; h < HW; ++h) {
      float a = 0.f;
#pragma unroll
      for (int cc = 0; cc < C::CPL; ++cc) {
        if constexpr (BF16) {
          a = dot2_bf16(q[h][cc].x, t.k[j][cc].x, a);
          a = dot2_bf16(q[h][cc].y, t.k[j][cc].y, a);
          a = dot2_bf16(q[h][cc].z, t.k[j][cc].z, a);
          a = dot2_bf16(q[h][cc].w, t.k[j][cc].w, a);
        } else {
          a = fmaf(__uint_as_float(q[h][cc].x), __uint_as_float(t.k[j][cc].x), a);
          a = fmaf(__uint_as_float(q[h][cc].y), __uint_as_float(t.k[j][cc].y), a);
          a = fmaf(__uint_as_float(q[h][cc].z), __uint_as_float(t.k[j][cc].z), a);
          a = fmaf(__uint_as_float(q[h][cc].w), __uint_as_float(t.k[j][cc].w), a);
        }
      }
      sc[j][h] = row8_sum(a);
    }
  // ---- rows past the end (only in a segment's last tile) score -inf
  if (nv < C::TR) {
#pragma unroll
    for (int j = 0; j < C::RPL; ++j) {
      const bool ok = rg + 8 * j < nv;
#pragma unroll
      for (int h = 0; h < HW; ++h) sc[j][h] = ok ? sc[j][h] : -INFINITY;
    }
  }
  // ---- online softmax in log2 units (scale > 0, so max commutes with it)
  float p[C::RPL][HW];
  float mt[HW];
  bool need = false;
#pragma unroll
  for (int h = 0; h < HW; ++h) {
    float x = sc[0][h];
#pragma unroll
    for (int j = 1; j < C::RPL; ++j) x = fmaxf(x, sc[j][h]);
    mt[h] = x * scale_log2;
    need |= mt[h] > st.m[h] + kRescaleSlack;
  }
  if (__builtin_amdgcn_read_exec() & __ballot(need)) {  // any lane: raise the reference
#pragma unroll
    for (int h = 0; h < HW; ++h) {
      const float mn = fmaxf(st.m[h], mt[h]);
      const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(st.m[h] - mn);
      st.m[h] = mn;
      st.l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < C::NACC; ++e) st.acc[h][e] *= alpha;
    }
  }
#pragma unroll
  for (int h = 0; h < HW; ++h) {
    const float mu = (st.m[h] == -INFINITY) ? 0.f : st.m[h];
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < C::RPL; ++j) {
      p[j][h] = fast_exp2(fmaf(sc[j][h], scale_log2, -mu));
      ps += p[j][h];
    }
    st.l[h] += ps;
  }
  // ---- weighted sum of V rows
  if constexpr (BF16) {
#pragma unroll
    for (int jp = 0; jp < C::RPL; jp += 2) {
      uint32_t P[HW];
#pragma unroll
      for (int h = 0; h < HW; ++h) P[h] = pack_bf16x2(p[jp][h], p[jp + 1][h]);
#pragma unroll
      for (int cc = 0; cc < C::CPL; ++cc) {
        const uint32_t a4[4] = {t.v[jp][cc].x, t.v[jp][cc].y, t.v[jp][cc].z, t.v[jp][cc].w};
        const uint32_t b4[4] = {t.v[jp + 1][cc].x, t.v[jp + 1][cc].y, t.v[jp + 1][cc].z, t.v[jp + 1][cc].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = __builtin_amdgcn_perm(b4[i], a4[i], 0x05040100u);  // (row jp, row jp+1) at d = 2i
          const uint32_t hi = __builtin_amdgcn_perm(b4[i], a4[i], 0x07060302u);  // at d = 2i+1
#pragma unroll
          for (int h = 0; h < HW; ++h) {
            st.acc[h][cc * 8 + 2 * i] = dot2_bf16(P[h], lo, st.acc[h][cc * 8 + 2 * i]);
            st.acc[h][cc * 8 + 2 * i + 1] = dot2_bf16(P[h], hi, st.acc[h][cc * 8 + 2 * i + 1]);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < C::RPL; ++j)
#pragma unroll
      for (int cc = 0; cc < C::CPL; ++cc) {
        const float v4[4] = {__uint_as_float(t.v[j][cc].x), __uint_as_float(t.v[j][cc].y),
                             __uint_as_float(t.v[j][cc].z), __uint_as_float(t.v[j][cc].w)};
#pragma unroll
        for (int h = 0; h < HW; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) st.acc[h][cc * 4 + e] = fmaf(p[j][h], v4[e], st.acc[h][cc * 4 + e]);
      }
  }
}

// The flattened row space: retrieval heads (b, r) first, each `rows_ret`
// rows, then streaming heads (b, s), each `rows_str` rows.  Work item i covers
// rows [i*chunk, (i+1)*chunk) of it, which may span several heads; each
// (item, head) overlap is one segment with its own partial result.
template <bool BF16, int D, int G>
__global__ __launch_bounds__(kDecodeThreads)
__attribute__((amdgpu_waves_per_eu(DUO_DECODE_WAVES_PER_EU, DUO_DECODE_WAVES_PER_EU)))
void decode_kernel(DecodeArgs a) {
  using C = DecodeCfg<BF16, D, G>;
  constexpr int REC = G * (D + 2);
  constexpr int HW = C::HW, NS = C::NSTREAM;

  __shared__ float w_acc[NS][G * D];
  __shared__ float w_m[NS][G], w_l[NS][G];
  __shared__ int s_ticket;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hg = wave % C::HSPLIT;       // which HW query heads of the group this wavefront scores
  const int stream = wave / C::HSPLIT;   // which tile stream it walks
  const int rg = lane >> 3, s = lane & 7;
  const int64_t blk = blockIdx.x;
  const int64_t b0 = blk * a.chunk;
  const int64_t b1 = b0 + a.chunk < a.total_rows ? b0 + a.chunk : a.total_rows;
  const int64_t r_ret = (int64_t)a.B * a.n_ret * a.rows_ret;  // rows of all retrieval heads

  for (int64_t pos = b0; pos < b1;) {
    // ---- which head, and which of its rows
    int64_t hh, h0, hrows;
    const char *kbase, *vbase;
    int b, kvh;
    if (pos < r_ret) {
      hh = pos / a.rows_ret;
      h0 = hh * a.rows_ret;
      hrows = a.rows_ret;
      b = (int)(hh / a.n_ret);
      const int r = (int)(hh % a.n_ret);
      kvh = a.map.orig_ret[r];
      const size_t off = ((size_t)b * a.n_ret + r) * a.cap_ret * C::ROWB;
      kbase = a.lp.k_ret + off;
      vbase = a.lp.v_ret + off;
    } else {
      const int64_t x = (pos - r_ret) / a.rows_str;
      hh = (int64_t)a.B * a.n_ret + x;
      h0 = r_ret + x * a.rows_str;
      hrows = a.rows_str;
      b = (int)(x / a.n_str);
      const int sidx = (int)(x % a.n_str);
      kvh = a.map.orig_str[sidx];
      const size_t off = ((size_t)b * a.n_str + sidx) * a.cap_str * C::ROWB;
      kbase = a.lp.k_str + off;
      vbase = a.lp.v_str + off;
    }
    const int64_t seg_end = b1 < h0 + hrows ? b1 : h0 + hrows;
    const int64_t r0 = pos - h0, r1 = seg_end - h0;   // rows of this head in this segment
    pos = seg_end;
    const int fh = b * a.n_kv + kvh;
    const size_t q_off = ((size_t)b * a.n_q + (size_t)kvh * G) * D;

    // ---- this wavefront's HW queries, in the lane's slice layout
    uint4 q[HW][C::CPL];
    {
      const char* qb = static_cast<const char*>(a.q) + (q_off + (size_t)hg * HW * D) * C::ES;
#pragma unroll
      for (int h = 0; h < HW; ++h)
#pragma unroll
        for (int cc = 0; cc < C::CPL; ++cc) q[h][cc] = ld16(qb + (size_t)h * C::ROWB + (s + 8 * cc) * 16);
    }

    DecodeState<BF16, D, G> st;
#pragma unroll
    for (int h = 0; h < HW; ++h) {
      st.m[h] = -INFINITY;
      st.l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < C::NACC; ++e) st.acc[h][e] = 0.f;
    }

    // ---- tiles r0 + (stream + NS*i) * TR through a ring of STAGES register
    // tiles: tile i+STAGES-1 is requested before tile i is processed.
    const int64_t step = (int64_t)NS * C::TR;
    const int64_t t0 = r0 + (int64_t)stream * C::TR;
    const int64_t ntiles = t0 < r1 ? (r1 - t0 + step - 1) / step : 0;
    const int64_t last = r1 - 1;
    DecodeTile<BF16, D, G> T[C::STAGES];
    if (ntiles > 0) {
#pragma unroll
      for (int k = 0; k + 1 < C::STAGES; ++k) load_tile<BF16, D, G>(T[k], kbase, vbase, t0 + k * step, last, rg, s);
      for (int64_t i = 0; i < ntiles; i += C::STAGES) {
#pragma unroll
        for (int k = 0; k < C::STAGES; ++k) {
          if (i + k < ntiles) {
            const int64_t ti = t0 + (i + k) * step;
            load_tile<BF16, D, G>(T[(k + C::STAGES - 1) % C::STAGES], kbase, vbase, ti + (C::STAGES - 1) * step, last,
                                  rg, s);
            process_tile<BF16, D, G>(st, T[k], q, r1 - ti, rg, a.scale_log2);
          }
        }
      }
    }

    // ---- merge the 8 row groups of the wavefront (lanes xor 8, 16, 32)
#pragma unroll
    for (int h = 0; h < HW; ++h) {
      float M = st.m[h];
      M = fmaxf(M, __shfl_xor(M, 8));
      M = fmaxf(M, __shfl_xor(M, 16));
      M = fmaxf(M, __shfl_xor(M, 32));
      const float f = (M == -INFINITY) ? 0.f : fast_exp2(st.m[h] - M);
      float L = st.l[h] * f;
      L += __shfl_xor(L, 8);
      L += __shfl_xor(L, 16);
      L += __shfl_xor(L, 32);
#pragma unroll
      for (int e = 0; e < C::NACC; ++e) {
        float x = st.acc[h][e] * f;
        x += __shfl_xor(x, 8);
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        st.acc[h][e] = x;
      }
      st.m[h] = M;
      st.l[h] = L;
    }
    if (lane < 8) {
#pragma unroll
      for (int h = 0; h < HW; ++h)
#pragma unroll
        for (int cc = 0; cc < C::CPL; ++cc)
#pragma unroll
          for (int e = 0; e < C::EPC; ++e)
            w_acc[stream][(hg * HW + h) * D + (cc * 8 + s) * C::EPC + e] = st.acc[h][cc * C::EPC + e];
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < HW; ++h) {
        w_m[stream][hg * HW + h] = st.m[h];
        w_l[stream][hg * HW + h] = st.l[h];
      }
    }
    __syncthreads();

    // ---- merge the tile streams; segment result
    const int64_t first_blk = h0 / a.chunk;
    const int n_seg = (int)((h0 + hrows - 1) / a.chunk - first_blk + 1);
    const int seg = (int)(blk - first_blk);
    float* rec = a.ws1 + ((size_t)first_blk + (size_t)hh + seg) * REC;
    {
      constexpr int OPT = MergeShape<D, G>::OPT;
      const int e0 = threadIdx.x * OPT;
      if (e0 < G * D) {
        const int h = e0 / D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NS; ++w) M = fmaxf(M, w_m[w][h]);
        float L = 0.f, A[OPT];
#pragma unroll
        for (int o = 0; o < OPT; ++o) A[o] = 0.f;
#pragma unroll
        for (int w = 0; w < NS; ++w) {
          const float f = (w_m[w][h] == -INFINITY) ? 0.f : fast_exp2(w_m[w][h] - M);
          L += w_l[w][h] * f;
#pragma unroll
          for (int o = 0; o < OPT; ++o) A[o] += w_acc[w][e0 + o] * f;
        }
        if (n_seg == 1) {
          const float inv = 1.f / L;
#pragma unroll
          for (int o = 0; o < OPT; ++o) {
            if (BF16) {
              reinterpret_cast<uint16_t*>(a.out)[q_off + e0 + o] = (uint16_t)f32_to_bf16_bits(A[o] * inv);
            } else {
              reinterpret_cast<float*>(a.out)[q_off + e0 + o] = A[o] * inv;
            }
          }
        } else {
#pragma unroll
          for (int o = 0; o < OPT; ++o) rec_store(rec + e0 + o, A[o]);
          if (e0 % D == 0) {
            rec_store(rec + G * D + h, M);
            rec_store(rec + G * D + G + h, L);
          }
        }
      }
    }
    wait_stores_done();
    __syncthreads();  // LDS is reused by the next segment; records are written
    if (n_seg == 1) continue;

    // ---- first-level merge: the last segment of each group of kSplitGroup
    const int grp = seg / kSplitGroup;
    const int g0 = grp * kSplitGroup;
    const int gsz = min(kSplitGroup, n_seg - g0);
    const int ngrp = (n_seg + kSplitGroup - 1) / kSplitGroup;
    if (threadIdx.x == 0)
      s_ticket = __hip_atomic_fetch_add(&a.lp.cnt1[fh * kMaxGroups + grp], 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const bool last_in_group = (s_ticket == gsz - 1);
    __syncthreads();  // s_ticket is reused below
    if (!last_in_group) continue;
    if (threadIdx.x == 0)
      __hip_atomic_store(&a.lp.cnt1[fh * kMaxGroups + grp], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float* grp_src = a.ws1 + ((size_t)first_blk + (size_t)hh + g0) * REC;
    if (ngrp == 1) {
      merge_records<BF16, D, G>(grp_src, gsz, nullptr, a.out, q_off);
      continue;
    }
    float* grp_dst = a.ws2 + ((size_t)fh * kMaxGroups + grp) * REC;
    merge_records<BF16, D, G>(grp_src, gsz, grp_dst, nullptr, 0);

    // ---- second-level merge: the last group of the head
    wait_stores_done();
    __syncthreads();
    if (threadIdx.x == 0)
      s_ticket = __hip_atomic_fetch_add(&a.lp.cnt2[fh], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const bool last_group = (s_ticket == ngrp - 1);
    __syncthreads();
    if (!last_group) continue;
    if (threadIdx.x == 0) __hip_atomic_store(&a.lp.cnt2[fh], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    merge_records<BF16, D, G>(a.ws2 + (size_t)fh * kMaxGroups * REC, ngrp, nullptr, a.out, q_off);
    __syncthreads();
  }
}

template <bool BF16, int D>
hipError_t launch_decode_d(const DecodeArgs& a, int g, int blocks, hipStream_t s) {
  switch (g) {
    case 1: decode_kernel<BF16, D, 1><<<blocks, kDecodeThreads, 0, s>>>(a); break;
    case 2: decode_kernel<BF16, D, 2><<<blocks, kDecodeThreads, 0, s>>>(a); break;
    case 4: decode_kernel<BF16, D, 4><<<blocks, kDecodeThreads, 0, s>>>(a); break;
    case 8: decode_kernel<BF16, D, 8><<<blocks, kDecodeThreads, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16, ntail = bytes % 16;
  const int threads = 256;
  size_t want = (n16 + threads - 1) / threads;
  const int grid = (int)std::max<size_t>(1, std::min<size_t>(want, 4096));
  fill_zero_kernel<<<grid, threads, 0, s>>>(reinterpret_cast<uint4*>(p), n16,
                                           reinterpret_cast<unsigned char*>(p) + n16 * 16, ntail);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, int dtype, int d, hipStream_t s) {
  (void)dtype;
  (void)d;
  const int64_t total = (int64_t)a.B * a.n_kv * a.n_new * (a.row_bytes / 16);
  const int threads = 256;
  const int64_t want = (total + threads - 1) / threads;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(want, 65536));
  append_kernel<<<grid, threads, 0, s>>>(a);
  return hipGetLastError();
}

int decode_blocks_per_cu() { return DUO_DECODE_WAVES_PER_EU; }

hipError_t launch_decode(const DecodeArgs& a, int dtype, int d, int g, int blocks, hipStream_t s) {
  if (dtype == 1) {
    if (d == 128) return launch_decode_d<true, 128>(a, g, blocks, s);
    if (d == 64) return launch_decode_d<true, 64>(a, g, blocks, s);
  } else {
    if (d == 128) return launch_decode_d<false, 128>(a, g, blocks, s);
    if (d == 64) return launch_decode_d<false, 64>(a, g, blocks, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace duo
