// HIP kernels for gfx950 (CDNA4): cache fill, append and split-K decode over a
// per-KV-head mixed KV cache (DuoAttention: retrieval heads hold every token,
// streaming heads hold S sinks + a W-slot ring).
//
// Decode is bound by HBM bandwidth (g = n_q / n_kv flops per byte of K/V).
// The rows held by every (batch, KV head) -- all T rows of a retrieval head,
// the min(T, S+W) sink and ring slots of a streaming head -- are cut into work
// items of one common length, at most one per compute unit, so long retrieval
// heads and short streaming heads are balanced by bytes; an item is a
// contiguous row range of one head.  Within an item, K and V rows reach LDS by
// direct buffer->LDS loads into a ring of four 32 KB units (two or three in
// flight); at d = 128 the wavefronts score them and form P.V on the matrix
// cores (the GQA query group as one operand), elsewhere with packed bf16 dot
// products on the vector ALUs, keeping online softmax statistics.  Partial
// (max, sum, acc) results of items that share a head are merged by a second
// kernel (combine_kernel).  Retrieval rows may live in pages (a per-row page
// table); a paged head's items then start at round boundaries so that every
// round lies in one page.
#include "duo_dma.h"
#include "duo_internal.h"
#include "duo_rope.h"
#include "duo_rows.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstddef>
#include <mutex>
#include <type_traits>

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

__device__ __forceinline__ int64_t max64d(int64_t x, int64_t y) { return x > y ? x : y; }

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

__global__ void fill_kernel(uint4* p, size_t n16, unsigned char* tail, size_t ntail, uint32_t word) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t j = i; j < n16; j += stride) p[j] = make_uint4(word, word, word, word);
  if (i < ntail) tail[i] = (unsigned char)word;
}

// Token counts after an append that read them: row b advances by n if it had
// room (the append then stored its tokens), else the cache's status bit is set.
__global__ void advance_kernel(AdvanceArgs a) {
  const int b = threadIdx.x;
  if (b >= a.B) return;
  const int32_t cnt = a.lp.len[b];
  if (room_for(a.lp, b, cnt, a.n)) a.lp.len[b] = (int32_t)(cnt + a.n);
  else *a.lp.status = 1;
}

// ------------------------------------------------------------------ page tables and row copies

__global__ void table_update_kernel(TableUpdateArgs a) {
  const int i = threadIdx.x;
  if (i < a.n) a.table[a.index[i]] = a.page[i];
}

// Grid-stride over the 4-byte words of every segment (a few rows per call:
// a forked row's partial page and streaming slots).
__global__ void copy_kernel(CopyArgs a) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t t0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int i = 0; i < a.n; ++i) {
    const CopySegment& g = a.seg[i];
    const int64_t words = g.bytes / 4, total = words * g.count;
    for (int64_t t = t0; t < total; t += stride) {
      const int64_t j = t / words, w = t % words;
      reinterpret_cast<uint32_t*>(g.dst + j * g.dst_stride)[w] =
          reinterpret_cast<const uint32_t*>(g.src + j * g.src_stride)[w];
    }
  }
}

// ------------------------------------------------------------------ append
// One thread per 16-byte chunk of an input row.  Token i of batch row b is at
// position p = p0[b] + i; it goes to row p of a retrieval head; for a
// streaming head to slot p while p < S, else to ring slot S + (p - S) mod W,
// but only if the token is among the last W of the call's tokens for its row
// (p >= max(S, p0[b] + n_new - W)); earlier ones would be evicted by later
// tokens of the same call, and skipping them keeps every slot written at most
// once.

// Rotate the pairs of chunk x (dimensions c * E .. c * E + E - 1, E = 16 /
// element size) and chunk y (the same dimensions + d/2) at position p: a
// key about to be stored, so in double, rounded once to the dtype.
__device__ __forceinline__ void rope_chunks(uint4& x, uint4& y, const Rope& r, int d, int64_t p, int c, int dtype) {
  uint32_t xw[4] = {x.x, x.y, x.z, x.w}, yw[4] = {y.x, y.y, y.z, y.w};
  if (dtype == 1) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      double c0, s0, c1, s1;
      rope_cs(r, p, c * 8 + 2 * w, c0, s0);
      rope_cs(r, p, c * 8 + 2 * w + 1, c1, s1);
      const double x0 = bf_lo(xw[w]), x1 = bf_hi(xw[w]), y0 = bf_lo(yw[w]), y1 = bf_hi(yw[w]);
      xw[w] = bf16_bits_from_double(x0 * c0 - y0 * s0) | (bf16_bits_from_double(x1 * c1 - y1 * s1) << 16);
      yw[w] = bf16_bits_from_double(y0 * c0 + x0 * s0) | (bf16_bits_from_double(y1 * c1 + x1 * s1) << 16);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      double cs, sn;
      rope_cs(r, p, c * 4 + w, cs, sn);
      const double xv = __uint_as_float(xw[w]), yv = __uint_as_float(yw[w]);
      xw[w] = __float_as_uint((float)(xv * cs - yv * sn));
      yw[w] = __float_as_uint((float)(yv * cs + xv * sn));
    }
  }
  x = make_uint4(xw[0], xw[1], xw[2], xw[3]);
  y = make_uint4(yw[0], yw[1], yw[2], yw[3]);
}

// ROPE: keys rotated at their positions (a.rope.on).  The two cases are
// separate kernels: the rotation's double-precision angle code would
// otherwise hold the plain copy at a quarter of the occupancy, with spills.
template <bool ROPE>
__global__ void append_kernel(AppendArgs a) {
  const int cpr = a.row_bytes / 16;
  // work per row: its 16-byte chunks, or with rotary positions its chunk
  // pairs (c, c + cpr/2), which hold the rotation's dimension pairs
  const int units = ROPE ? cpr / 2 : cpr;
  const int64_t total = (int64_t)a.B * a.n_kv * a.n_new * units;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int c = (int)(idx % units);
    const int64_t rest = idx / units;  // input row (b, kvh, i)
    const int64_t i = rest % a.n_new;
    const int kvh = (int)((rest / a.n_new) % a.n_kv);
    const int b = (int)(rest / a.n_new / a.n_kv);
    int64_t p0 = a.p0[b];
    if (a.p0_from_device) {
      p0 = a.lp.len[b];
      if (!room_for(a.lp, b, p0, a.n_new)) {  // nothing of this row is stored
        if (i == 0 && kvh == 0 && c == 0) *a.lp.status = 1;
        continue;
      }
    } else if (idx < a.B) {
      a.lp.len[idx] = (int32_t)(a.p0[idx] + a.n_new);  // nothing in this launch reads the counts
    }
    const int64_t p = p0 + i;
    const int64_t keep_from = max64d((int64_t)a.S, p0 + a.n_new - a.W);
    const size_t src = (size_t)rest * a.row_bytes;
    char *kd, *vd;
    if (a.map.kind[kvh]) {
      const int r = a.map.cidx[kvh];
      const size_t off = (size_t)ret_row(a.lp, a.n_ret, a.cap_ret, b, r, p) * a.row_bytes;
      kd = a.lp.k_ret + off;
      vd = a.lp.v_ret + off;
    } else {
      int64_t slot;
      if (p < a.S) {
        slot = p;
      } else if (p >= keep_from) {
        slot = a.S + (p - a.S) % a.W;
      } else {
        continue;
      }
      const int s = a.map.cidx[kvh];
      const size_t hrow = ((size_t)b * a.n_str + s) * a.cap_str + slot;
      const size_t off = hrow * a.row_bytes;
      kd = a.lp.k_str + off;
      vd = a.lp.v_str + off;
      if (c == 0) a.lp.pos[hrow] = (int32_t)p;
    }
    if constexpr (!ROPE) {
      st16(kd + c * 16, ld16(a.k + src + c * 16));
      st16(vd + c * 16, ld16(a.v + src + c * 16));
    } else {
      const int c2 = c + cpr / 2;
      uint4 x = ld16(a.k + src + c * 16), y = ld16(a.k + src + c2 * 16);
      rope_chunks(x, y, a.rope, a.d, p, c, a.dtype);
      st16(kd + c * 16, x);
      st16(kd + c2 * 16, y);
      st16(vd + c * 16, ld16(a.v + src + c * 16));
      st16(vd + c2 * 16, ld16(a.v + src + c2 * 16));
    }
  }
}

// Prefill with rotary positions: chunk row i of batch row b at position
// p0[b] + i, one thread per (row, dimension pair); queries and keys.
__global__ void rope_kernel(RopeArgs a) {
  const int half = a.d / 2;
  const int64_t q_pairs = (int64_t)a.B * a.n_q * a.C * half;
  const int64_t total = q_pairs + (int64_t)a.B * a.n_kv * a.C * half;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total; t += stride) {
    const bool isq = t < q_pairs;
    const int64_t u = isq ? t : t - q_pairs;
    const int i = (int)(u % half);
    const int64_t row = u / half;  // (b, head, chunk row)
    const int64_t ci = row % a.C;
    const int b = (int)(row / a.C / (isq ? a.n_q : a.n_kv));
    double cs, sn;  // keys are stored from these copies: rotated in double, rounded once
    rope_cs(a.rope, a.p0[b] + ci, i, cs, sn);
    const size_t e0 = (size_t)row * a.d + i, e1 = e0 + half;
    if (a.dtype == 1) {
      const uint16_t* in = static_cast<const uint16_t*>(isq ? a.q : a.k);
      uint16_t* out = static_cast<uint16_t*>(isq ? a.q_out : a.k_out);
      const double x = __uint_as_float((uint32_t)in[e0] << 16), y = __uint_as_float((uint32_t)in[e1] << 16);
      out[e0] = (uint16_t)bf16_bits_from_double(x * cs - y * sn);
      out[e1] = (uint16_t)bf16_bits_from_double(y * cs + x * sn);
    } else {
      const float* in = static_cast<const float*>(isq ? a.q : a.k);
      float* out = static_cast<float*>(isq ? a.q_out : a.k_out);
      const double x = in[e0], y = in[e1];
      out[e0] = (float)(x * cs - y * sn);
      out[e1] = (float)(y * cs + x * sn);
    }
  }
}

// ------------------------------------------------------------------ decode
//
// One workgroup of 8 wavefronts per compute unit walks the contiguous rows of
// one work item (part of one head).  K and V rows reach LDS through direct
// buffer->LDS loads into a ring of four 32 KB units (the K rows, then the V
// rows, of one round of tiles); DEPTH units are in flight while one is
// consumed, so the prefetch depth costs no registers.  A round is SLOTS tiles
// of TR rows; each wavefront reads its slot's tile from LDS, so no row is
// fetched twice.  At the end the wavefronts' softmax states are merged into one
// partial (max, sum, acc) per query head: an item that is a whole head writes
// the output, otherwise its partial goes to the workspace and the combine
// kernel merges the partials of the head.
//
// Vector-ALU lane layout within a tile (d = 64 and fp32 rows; the matrix-core
// layouts are described at mf_scores): 8 lanes share a row.  Lane l has row group
// rg = l / 8 and slice s = l % 8; it holds the 16-byte chunks s, s+8, ... of
// rows rg, rg+8, ...  Rows are XOR-swizzled in LDS (odd rows swap the two
// halves of every 256 bytes) so the 8-row reads are free of bank conflicts.
// Scores: packed bf16 dot products over the lane's slice, then an all-reduce
// over the 8 lanes of the row with DPP adds.  P.V: bf16 dot products over
// pairs of rows.

constexpr int kDecWaves = kDecodeThreads / 64;              // 8
constexpr int kUnitBytes = 32768;                           // K (or V) rows of one round
constexpr int kRingUnits = 4;                               // 128 KB of LDS
constexpr int kUnitPieces = kUnitBytes / 1024;              // wavefront-wide 16-byte loads per unit
constexpr int kPiecesPerWave = kUnitPieces / kDecWaves;     // 4
static_assert(kUnitPieces % kDecWaves == 0, "unit pieces split evenly over the wavefronts");

// KT: 0 = fp32 everywhere, 1 = bf16 everywhere, 2 = bf16 queries, inputs and
// outputs with FP8 (E4M3) K/V rows in the cache plus one fp32 scale per row,
// 3 = the same with INT4 rows (two codes per byte) plus one fp32 scale per row.
template <int KT, int D, int G>
struct DecodeCfg {
  static constexpr bool BF16 = KT != 0;          // queries, inputs, outputs in bf16
  static constexpr bool KV8 = KT == 2;           // K/V rows stored as FP8 codes + row scales
  static constexpr bool KV4 = KT == 3;           // K/V rows stored as INT4 codes + row scales
  static constexpr bool LOWBIT = KV8 || KV4;     // rows carry an fp32 scale each
  static constexpr int ES = BF16 ? 2 : 4;        // query / input / output element bytes
  static constexpr int IROWB = D * ES;           // bytes per query or input row
  static constexpr int KES = KV8 ? 1 : ES;       // stored K/V element bytes (INT4: half a byte)
  static constexpr int ROWB = KV4 ? D / 2 : D * KES;  // bytes per stored K/V row
  static constexpr int CPR = ROWB / 16;          // 16-byte chunks per stored row
  // Weighted sum: the 8 lanes of a row each take CPL pieces of the V row;
  // INT4 rows (64 bytes) give each lane one 8-byte piece of 16 codes.
  static constexpr int CPL = KV4 ? 1 : CPR / 8;  // V pieces per lane
  static constexpr int EPC = KV4 ? 32 : 16 / KES;  // elements per 16-byte chunk
  static constexpr int EPV = KV4 ? 16 : EPC;     // elements per V piece
  // bf16, FP8 and INT4 rows, d = 128: scores and weighted sums on the matrix
  // cores (see mf_scores, mf8_scores, mf4_scores), each wavefront taking all
  // the group's query heads over its own rows of a round (16 bf16, 32 FP8 or
  // 64 INT4 rows)
  static constexpr bool MF = KT >= 1 && D == 128;
  // query heads per wavefront: the whole group on the matrix cores (up to 16,
  // one column each of the 16-column tile); otherwise 4, 2 or 1, whichever
  // divides the group (the four-lane score layout needs a divisor of 4)
  static constexpr int HW = MF ? G : (G % 4 == 0 ? 4 : G % 2 == 0 ? 2 : 1);
  static constexpr int HSPLIT = G / HW;          // wavefronts per slot
  static constexpr int SLOTS_W = kDecWaves / HSPLIT;
  static constexpr int SLOTS_B = kUnitBytes / (16 * ROWB);  // keeps TR >= 16
  static constexpr int SLOTS = SLOTS_W < SLOTS_B ? SLOTS_W : SLOTS_B;
  static constexpr int TR = kUnitBytes / (SLOTS * ROWB);    // rows per tile
  static constexpr int RPL = TR / 8;             // rows per lane
  static constexpr int SLOT_BYTES = TR * ROWB;
  static constexpr int ROUND_ROWS = SLOTS * TR;
  static constexpr int NACC = CPL * EPV;         // output elements per lane per head
  static constexpr int REC = (G * (D + 2) + 3) / 4 * 4;  // floats per partial record (16-byte multiple)
  // Ring units in flight ahead of the one being consumed: FP8 and INT4 rows
  // (256 and 512 rows a unit) measured faster with two, bf16 and fp32 rows
  // with three.
  static constexpr int DEPTH = LOWBIT ? 2 : 3;
  static_assert(KV4 ? (CPR == 4 && D == 128) : CPR % 8 == 0, "rows must span a multiple of 8 chunks");
  static_assert(RPL >= 2 && RPL % 2 == 0, "rows are paired for the weighted sum");
  static_assert(SLOT_BYTES % 1024 == 0, "a load piece stays within one tile");
  static_assert(G % HW == 0, "head split must tile the group");
  static_assert(MF ? G <= 16 : HSPLIT <= kDecWaves, "a slot's head split fits the workgroup");
  static_assert(!LOWBIT || MF, "FP8 and INT4 rows are decoded on the matrix cores, at d = 128");
};

// Chunk slot of chunk c of row r in LDS.
template <int CPR>
__device__ __forceinline__ int dec_swz(int r) { return CPR >= 16 ? 8 * (r & 1) : 0; }

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

// Combine each lane's value with those of lanes l ^ 8, l ^ 16 and l ^ 32 (the
// 8 row groups holding the same slice), on the vector ALU: DPP row_ror:8 is
// l ^ 8 within a row of 16 lanes, and the lane-swap instructions exchange
// rows (16 lanes) and halves (32 lanes) between two registers, so the sum
// (or max) of the two results is the value combined with its partner lane.
__device__ __forceinline__ float swap16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float rowgroups_sum(float x) {
  x += dpp<0x128>(x);  // row_ror:8
  return swap32_sum(swap16_sum(x));
}
__device__ __forceinline__ float rowgroups_max(float x) {
  x = fmaxf(x, dpp<0x128>(x));
  return swap32_max(swap16_max(x));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  bf2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ------------------------------------------------------------------ FP8 rows
// A row stored as FP8 (E4M3) holds code_i = E4M3(x_i / s) with s = max|x| / 448
// (both quotients correctly rounded fp32 divisions, the conversion rounding to
// nearest even); a row of zeros has s = 0 and codes 0.  Rows are quantized by
// groups of 16 lanes (one DPP row), 8 bf16 values per lane.

// E4M3 codes of four quotients x / s.  |x / s| <= 448 up to the rounding of
// the two divisions; the clamp maps that overshoot of the row maximum to 448,
// where rounding to nearest puts it as well.
__device__ __forceinline__ uint32_t fp8x4(float y0, float y1, float y2, float y3) {
  auto c = [](float y) { return fminf(fmaxf(y, -448.f), 448.f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c(y0), c(y1), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c(y2), c(y3), w, true);
  return (uint32_t)w;
}

// The 8 codes of this lane's bf16 values x (one 16-byte piece of a row whose
// 16 pieces sit in the 16 lanes of a DPP row), and the row's scale.
__device__ __forceinline__ uint2 quant_row16(uint4 x, float& scale) {
  const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf_lo(w4[i]);
    f[2 * i + 1] = bf_hi(w4[i]);
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
  m = fmaxf(m, dpp<0xB1>(m));   // quad_perm [1,0,3,2]
  m = fmaxf(m, dpp<0x4E>(m));   // quad_perm [2,3,0,1]
  m = fmaxf(m, dpp<0x141>(m));  // row_half_mirror
  m = fmaxf(m, dpp<0x140>(m));  // row_mirror
  scale = m / 448.f;
  if (!(scale > 0.f)) return make_uint2(0u, 0u);
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = f[i] / scale;
  return make_uint2(fp8x4(y[0], y[1], y[2], y[3]), fp8x4(y[4], y[5], y[6], y[7]));
}

// INT4 rows: s = max|x| / 7 (a correctly rounded fp32 division) and c =
// x / s (the same) rounded to the nearest integer, ties to even, kept in
// -7 .. 7; the code c + 8 goes to a nibble, element 2k of the lane's 8 in the
// low nibble of byte k.  A row of zeros has s = 0 and codes 8.  The row's 16
// pieces sit in the 16 lanes of a DPP row, as for quant_row16.
__device__ __forceinline__ uint32_t quant_row16_int4(uint4 x, float& scale) {
  const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf_lo(w4[i]);
    f[2 * i + 1] = bf_hi(w4[i]);
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
  m = fmaxf(m, dpp<0xB1>(m));   // quad_perm [1,0,3,2]
  m = fmaxf(m, dpp<0x4E>(m));   // quad_perm [2,3,0,1]
  m = fmaxf(m, dpp<0x141>(m));  // row_half_mirror
  m = fmaxf(m, dpp<0x140>(m));  // row_mirror
  scale = m / 7.f;
  if (!(scale > 0.f)) return 0x88888888u;
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float c = fminf(fmaxf(rintf(f[i] / scale), -7.f), 7.f);
    w |= (uint32_t)((int)c + 8) << (4 * i);
  }
  return w;
}

// Append to an FP8 or INT4 cache: one group of 16 lanes per (batch row, KV
// head, token, K or V) row, each lane taking 8 consecutive bf16 values.  Slot
// rules as append_kernel.
// Rotary positions in decode: rows [0, nq) of the staging area (the group's
// queries, row_bytes apart) and, if with_k, the new token's K row at k_row,
// rotated in place; one thread per (row, dimension pair).  Every row turns by
// the same angles: (cs, sn) are those of pair lane % (d/2), which is the pair
// of every thread's share (d/2 divides 64).  Queries turn in float; the K
// row, which the step stores, in double (rounded once, as the append does).
template <int ES>
__device__ __forceinline__ void rope_stage(char* stage, int nq, char* k_row, bool with_k, int row_bytes, int d,
                                           double dcs, double dsn) {
  const int half = d / 2;
  const int n = (nq + (with_k ? 1 : 0)) * half;
  const float cs = (float)dcs, sn = (float)dsn;
  for (int t = threadIdx.x; t < n; t += kDecodeThreads) {
    const int row = t / half, i = t % half;
    if (row == nq) {  // the new key
      if constexpr (ES == 2) {
        uint16_t* e = reinterpret_cast<uint16_t*>(k_row);
        const double x = __uint_as_float((uint32_t)e[i] << 16), y = __uint_as_float((uint32_t)e[i + half] << 16);
        e[i] = (uint16_t)bf16_bits_from_double(x * dcs - y * dsn);
        e[i + half] = (uint16_t)bf16_bits_from_double(y * dcs + x * dsn);
      } else {
        float* e = reinterpret_cast<float*>(k_row);
        const double x = e[i], y = e[i + half];
        e[i] = (float)(x * dcs - y * dsn);
        e[i + half] = (float)(y * dcs + x * dsn);
      }
      continue;
    }
    char* base = stage + row * row_bytes;
    if constexpr (ES == 2) {
      uint16_t* e = reinterpret_cast<uint16_t*>(base);
      const float x = __uint_as_float((uint32_t)e[i] << 16), y = __uint_as_float((uint32_t)e[i + half] << 16);
      e[i] = (uint16_t)f32_to_bf16_bits(x * cs - y * sn);
      e[i + half] = (uint16_t)f32_to_bf16_bits(y * cs + x * sn);
    } else {
      float* e = reinterpret_cast<float*>(base);
      const float x = e[i], y = e[i + half];
      e[i] = x * cs - y * sn;
      e[i + half] = y * cs + x * sn;
    }
  }
}

// A bf16 row of d = 128 held by the 16 lanes of a DPP row, lane j holding
// dimensions 8j .. 8j+7, rotated at position p (in double, rounded once to
// bf16, as every stored key): the other half of lane j's pairs sits in lane
// j ^ 8, read with a row rotation by 8 lanes.
__device__ __forceinline__ uint4 rope_row16(uint4 x, const Rope& r, int64_t p, int j) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t o[4];
  const bool first = j < 8;  // this lane holds x_i (else x_(i + d/2))
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t q = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w[k], 0x128, 0xF, 0xF, false);  // row_ror:8
    double cs0, sn0, cs1, sn1;
    rope_cs(r, p, 8 * (j & 7) + 2 * k, cs0, sn0);
    rope_cs(r, p, 8 * (j & 7) + 2 * k + 1, cs1, sn1);
    const double a0 = bf_lo(w[k]), a1 = bf_hi(w[k]), b0 = bf_lo(q), b1 = bf_hi(q);
    const double v0 = first ? a0 * cs0 - b0 * sn0 : a0 * cs0 + b0 * sn0;
    const double v1 = first ? a1 * cs1 - b1 * sn1 : a1 * cs1 + b1 * sn1;
    o[k] = bf16_bits_from_double(v0) | (bf16_bits_from_double(v1) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// ROPE as for append_kernel: the rotation is a kernel of its own.
template <bool INT4, bool ROPE>
__global__ void append_lowbit_kernel(AppendArgs a) {
  const int64_t rows = (int64_t)a.B * a.n_kv * a.n_new * 2;
  const int64_t row = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
  const int j = threadIdx.x & 15;
  if (row >= rows) return;  // whole groups of 16 leave together
  const int tensor = (int)(row & 1);  // 0 = K, 1 = V
  int64_t rest = row >> 1;
  const int64_t i = rest % a.n_new;
  rest /= a.n_new;
  const int kvh = (int)(rest % a.n_kv);
  const int b = (int)(rest / a.n_kv);
  int64_t p0 = a.p0[b];
  if (a.p0_from_device) {
    p0 = a.lp.len[b];
    if (!room_for(a.lp, b, p0, a.n_new)) {  // nothing of this row is stored (the whole group leaves)
      if (i == 0 && kvh == 0 && tensor == 0 && j == 0) *a.lp.status = 1;
      return;
    }
  } else {
    // nothing in this launch reads the counts; the first B threads set them
    // (they all hold a row: there are 2 B n_kv n_new rows of 16 threads)
    const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gt < a.B) a.lp.len[gt] = (int32_t)(a.p0[gt] + a.n_new);
  }
  const int64_t p = p0 + i;
  const int64_t keep_from = max64d((int64_t)a.S, p0 + a.n_new - a.W);
  const size_t src = (((size_t)b * a.n_kv + kvh) * a.n_new + i) * a.in_row_bytes + (size_t)j * 16;
  float sc;
  uint4 x = ld16((tensor ? a.v : a.k) + src);
  if (ROPE && tensor == 0) x = rope_row16(x, a.rope, p, j);  // the whole group takes this branch
  uint2 codes = make_uint2(0u, 0u);
  uint32_t codes4 = 0u;
  if constexpr (INT4) codes4 = quant_row16_int4(x, sc);
  else codes = quant_row16(x, sc);
  char* dst;
  float* sdst;
  if (a.map.kind[kvh]) {
    const size_t hrow = (size_t)ret_row(a.lp, a.n_ret, a.cap_ret, b, a.map.cidx[kvh], p);
    dst = (tensor ? a.lp.v_ret : a.lp.k_ret) + hrow * a.row_bytes;
    sdst = (tensor ? a.lp.vsc_ret : a.lp.ksc_ret) + hrow;
  } else {
    int64_t slot;
    if (p < a.S) slot = p;
    else if (p >= keep_from) slot = a.S + (p - a.S) % a.W;
    else return;
    const size_t hrow = ((size_t)b * a.n_str + a.map.cidx[kvh]) * a.cap_str + slot;
    dst = (tensor ? a.lp.v_str : a.lp.k_str) + hrow * a.row_bytes;
    sdst = (tensor ? a.lp.vsc_str : a.lp.ksc_str) + hrow;
    if (tensor == 0 && j == 0) a.lp.pos[hrow] = (int32_t)p;
  }
  if constexpr (INT4) *reinterpret_cast<uint32_t*>(dst + j * 4) = codes4;
  else *reinterpret_cast<uint2*>(dst + j * 8) = codes;
  if (j == 0) *sdst = sc;
}

// FP8 or INT4 rows -> bf16 rows (code value times the row scale, rounded to
// nearest even), 8 values per thread.
__global__ void dequant_kernel(DequantArgs a) {
  const int pieces = a.d / 8;
  const int64_t n_ret = a.heads_ret * a.rows_ret, n_str = a.heads_str * a.rows_str;
  const int64_t total = (n_ret + n_str) * 2 * pieces;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int pc = (int)(idx % pieces);
    const int64_t rest = idx / pieces;
    const int tensor = (int)(rest & 1);
    int64_t rr = rest >> 1;
    const uint8_t* codes;
    const float* sc;
    uint16_t* dst;
    if (rr < n_ret) {
      const int64_t h = rr / a.rows_ret, r = rr % a.rows_ret;
      const int64_t srow = ret_row(a.src, a.n_ret, a.cap_ret_src, h / a.n_ret, (int)(h % a.n_ret), r);
      const int64_t drow = h * a.cap_ret_dst + r;
      codes = reinterpret_cast<const uint8_t*>(tensor ? a.src.v_ret : a.src.k_ret) + srow * (a.int4 ? a.d / 2 : a.d);
      sc = (tensor ? a.src.vsc_ret : a.src.ksc_ret) + srow;
      dst = reinterpret_cast<uint16_t*>(tensor ? a.dst.v_ret : a.dst.k_ret) + drow * a.d;
    } else {
      rr -= n_ret;
      const int64_t h = rr / a.rows_str, r = rr % a.rows_str;
      const int64_t row = h * a.cap_str + r;
      codes = reinterpret_cast<const uint8_t*>(tensor ? a.src.v_str : a.src.k_str) + row * (a.int4 ? a.d / 2 : a.d);
      sc = (tensor ? a.src.vsc_str : a.src.ksc_str) + row;
      dst = reinterpret_cast<uint16_t*>(tensor ? a.dst.v_str : a.dst.k_str) + row * a.d;
    }
    const float s = *sc;
    uint32_t o[4];
    if (a.int4) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + pc * 4);  // 8 nibbles
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float c0 = (float)((int)((w >> (8 * k)) & 15u) - 8), c1 = (float)((int)((w >> (8 * k + 4)) & 15u) - 8);
        o[k] = f32_to_bf16_bits(c0 * s) | (f32_to_bf16_bits(c1 * s) << 16);
      }
    } else {
      const uint2 c8 = *reinterpret_cast<const uint2*>(codes + pc * 8);
      const uint32_t cw[2] = {c8.x, c8.y};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[k], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[k], true);
        o[2 * k] = f32_to_bf16_bits(lo[0] * s) | (f32_to_bf16_bits(lo[1] * s) << 16);
        o[2 * k + 1] = f32_to_bf16_bits(hi[0] * s) | (f32_to_bf16_bits(hi[1] * s) << 16);
      }
    }
    *reinterpret_cast<uint4*>(dst + pc * 8) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that waits only for this wavefront's LDS operations:
// direct buffer->LDS loads stay in flight across it (their completion is
// waited for explicitly with wait_vmcnt before the barrier that publishes
// them).  __syncthreads would wait for every outstanding vector-memory load,
// draining the prefetch ring at each step.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A work item is a contiguous row range of one head.  Heads are numbered
// retrieval first ((b, r) -> b * n_ret + r), then streaming; the retrieval
// heads of batch row b are cut into rows[b].nb_ret items each and its
// streaming heads into rows[b].nb_str; items follow the same order.
struct DecodeItem {
  int64_t hh;       // head number
  int64_t r0, r1;   // rows of the head
  int64_t cnt;      // the batch row's token count when the kernel runs (before a fused append), -1 if not read
  int part, nparts;
  int b, kvh;
  int row;          // batch row (index into DecodeArgs::rows)
  // A shared item (share group rows b .. b + qrows - 1, their shared rows of
  // retrieval head hh - b * n_ret): its queries are the group's qrows * g
  // queries; it is never the last item of a head.  single: the item is its
  // head's only partial result (it writes the output).
  int qrows;
  bool shared, single;
  int sh_rec, sh_stride;  // a shared item: its record for row i of the group is sh_rec + i * sh_stride
  char* kbase;
  char* vbase;
  float* ksc;       // FP8 rows: per-row scales of the head (else null)
  float* vsc;
  // Paged retrieval head: the batch row's page table (else null); kbase,
  // vbase, ksc and vsc then point at the head's rows in page 0.
  const int32_t* ptab;
  int shift;
  int64_t pstride;  // rows from one page of the head to the next

  // Row of position `row` of the head, counted from kbase / ksc (uniform
  // `row`: the table read adds no vector-memory load to the counts the
  // ring's waits rely on).
  __device__ __forceinline__ int64_t at(int64_t row) const { return ptab ? paged_row(ptab, shift, pstride, row) : row; }
};

// Entry i (wavefront-uniform) of an int8 table in the kernel arguments: the
// dword that holds it comes by a scalar load and the byte is extracted (gfx9
// has no scalar byte load, and a vector byte load would have to be waited for
// before the item's first loads are issued).
static_assert(offsetof(DecodeArgs, map) % 4 == 0 && offsetof(HeadMap, orig_ret) % 4 == 0 &&
                  offsetof(HeadMap, orig_str) % 4 == 0 && kMaxKV % 4 == 0,
              "head-map tables are read as aligned dwords");
__device__ __forceinline__ int arg_byte(const int8_t* table, int i) {
  const uint32_t word = *reinterpret_cast<const uint32_t*>(table + (i & ~3));
  return (int)(int8_t)(word >> (8 * (i & 3)));
}

template <int ROWB, int RR, bool SH>
__device__ __forceinline__ DecodeItem decode_item(const DecodeArgs& a, int blk) {
  // Index arithmetic in 32 bits (item and row counts fit), the head index
  // made wavefront-uniform so the head-map lookups are scalar loads: this
  // runs before the first loads of the item are issued.
  DecodeItem w;
  w.ptab = nullptr;
  w.shift = 0;
  w.pstride = 0;
  w.qrows = 1;
  w.shared = false;
  int rows, base = 0;  // the item's rows are positions base .. rows - 1 of its head, cut in nparts
  if (SH && blk >= a.items_sh) {
    int k = 0;
    while (k + 1 < a.n_share && blk >= a.share[k + 1].first) ++k;  // share group of the item (uniform)
    const DecodeShare& S = a.share[k];
    const int rel = blk - S.first;
    const int r = __builtin_amdgcn_readfirstlane(rel / S.nb);
    const int b = S.b0;
    w.part = rel - r * S.nb;
    w.nparts = S.nb;
    rows = S.rows;
    w.row = b;
    w.b = b;
    w.hh = (int64_t)b * a.n_ret + r;
    w.kvh = arg_byte(a.map.orig_ret, r);
    w.qrows = S.R;
    w.shared = true;
    w.single = false;
    w.sh_rec = S.rec + r * S.nb + w.part;
    w.sh_stride = a.n_ret * S.nb;
    // the group's shared pages, as row b's table names them
    w.ptab = a.lp.table + (size_t)b * a.lp.max_pages;
    w.shift = a.lp.page_shift;
    w.pstride = (int64_t)a.n_ret << a.lp.page_shift;
    const size_t srow = (size_t)r << a.lp.page_shift;
    w.kbase = a.lp.k_ret + srow * ROWB;
    w.vbase = a.lp.v_ret + srow * ROWB;
    w.ksc = a.lp.ksc_ret ? a.lp.ksc_ret + srow : nullptr;
    w.vsc = a.lp.vsc_ret ? a.lp.vsc_ret + srow : nullptr;
  } else if (blk < a.items_ret) {
    int b = 0;
    while (b + 1 < a.B && blk >= a.rows[b + 1].first_ret) ++b;  // batch row of the item (uniform)
    const DecodeRow& R = a.rows[b];
    const int rel = blk - R.first_ret;
    const int r = __builtin_amdgcn_readfirstlane(rel / R.nb_ret);
    w.part = rel - r * R.nb_ret;
    w.nparts = R.nb_ret;
    rows = R.rows_ret;
    if constexpr (SH) base = a.rsh[b].sh_rows;  // rows shared items read for this row
    w.single = w.nparts == 1 && base == 0;
    w.row = b;
    w.b = b;
    w.hh = (int64_t)b * a.n_ret + r;
    w.kvh = arg_byte(a.map.orig_ret, r);
    // first row of the head: row 0 of its contiguous rows, or its part of page 0
    size_t srow = ((size_t)b * a.n_ret + r) * a.cap_ret;
    if (a.lp.table) {
      w.ptab = a.lp.table + (size_t)b * a.lp.max_pages;
      w.shift = a.lp.page_shift;
      w.pstride = (int64_t)a.n_ret << a.lp.page_shift;
      srow = (size_t)r << a.lp.page_shift;
    }
    w.kbase = a.lp.k_ret + srow * ROWB;
    w.vbase = a.lp.v_ret + srow * ROWB;
    w.ksc = a.lp.ksc_ret ? a.lp.ksc_ret + srow : nullptr;
    w.vsc = a.lp.vsc_ret ? a.lp.vsc_ret + srow : nullptr;
  } else {
    int b = 0;
    while (b + 1 < a.B && blk >= a.rows[b + 1].first_str) ++b;
    const DecodeRow& R = a.rows[b];
    const int rel = blk - R.first_str;
    const int si = __builtin_amdgcn_readfirstlane(rel / R.nb_str);
    w.part = rel - si * R.nb_str;
    w.nparts = R.nb_str;
    rows = R.rows_str;
    w.single = w.nparts == 1;
    w.row = b;
    w.b = b;
    w.hh = (int64_t)a.B * a.n_ret + (int64_t)b * a.n_str + si;
    w.kvh = arg_byte(a.map.orig_str, si);
    const size_t off = ((size_t)b * a.n_str + si) * a.cap_str * ROWB;
    w.kbase = a.lp.k_str + off;
    w.vbase = a.lp.v_str + off;
    const size_t srow = ((size_t)b * a.n_str + si) * a.cap_str;
    w.ksc = a.lp.ksc_str ? a.lp.ksc_str + srow : nullptr;
    w.vsc = a.lp.vsc_str ? a.lp.vsc_str + srow : nullptr;
  }
  // The items of a head split the rows held at planning.  The last one ends
  // at the rows held when the kernel runs (end_last_item: a replayed step
  // may find more); until then it ends where the plan did.
  int per = __builtin_amdgcn_readfirstlane((rows - base + w.nparts - 1) / w.nparts);
  if (w.ptab) per = (per + RR - 1) / RR * RR;  // paged: every round of rows lies in one page (base is whole pages)
  w.r0 = (int64_t)base + (int64_t)w.part * per;
  w.r1 = w.r0 + per < rows ? w.r0 + per : rows;
  if (w.r0 > rows) w.r0 = rows;
  w.cnt = -1;
  return w;
}

// The batch row's token count when the kernel runs, read through the scalar
// cache (the decode kernel never writes the counts), so the read adds nothing
// to the vector-memory counts the ring's waits rely on.
__device__ __forceinline__ int64_t row_count(const DecodeArgs& a, int b) {
  return *(const __attribute__((address_space(4))) int32_t*)(a.lp.len + b);
}

// rope_stage for a shared item's queries: rows [0, nrows * nq) of the
// staging area, query row q of batch row b0 + q / nq turned at that batch
// row's position (its count, less one unless the call appends).
template <int ES>
__device__ __forceinline__ void rope_stage_rows(const DecodeArgs& a, int b0, char* stage, int nq, int nrows,
                                                int row_bytes, int d) {
  const int half = d / 2;
  const int n = nrows * nq * half;
  for (int t = threadIdx.x; t < n; t += kDecodeThreads) {
    const int row = t / half, i = t % half;
    // rows 64 t' / d .. of 512 threads: the batch row is uniform in each
    // wavefront (nq >= 4, d = 128), so its count comes by a scalar load
    const int set = __builtin_amdgcn_readfirstlane(row / nq);
    double dc, ds;
    rope_cs(a.rope, row_count(a, b0 + set) - (a.new_k ? 0 : 1), i, dc, ds);
    const float c = (float)dc, s = (float)ds;
    char* base = stage + row * row_bytes;
    if constexpr (ES == 2) {
      uint16_t* e = reinterpret_cast<uint16_t*>(base);
      const float x = __uint_as_float((uint32_t)e[i] << 16), y = __uint_as_float((uint32_t)e[i + half] << 16);
      e[i] = (uint16_t)f32_to_bf16_bits(x * c - y * s);
      e[i + half] = (uint16_t)f32_to_bf16_bits(y * c + x * s);
    } else {
      float* e = reinterpret_cast<float*>(base);
      const float x = e[i], y = e[i + half];
      e[i] = x * c - y * s;
      e[i + half] = y * c + x * s;
    }
  }
}


// The last item of a head ends at the rows its batch row holds now.
__device__ __forceinline__ void end_last_item(const DecodeArgs& a, DecodeItem& w) {
  const int64_t now = w.hh < (int64_t)a.B * a.n_ret ? w.cnt : (w.cnt < a.cap_str ? w.cnt : a.cap_str);
  w.r1 = now;
  if (w.r0 > now) w.r0 = now;
}

// Per-lane softmax state.  m is a reference maximum (log2 units); l and acc
// are kept relative to it.  The reference is raised only when a score
// exceeds it by more than kRescaleSlack, so exp2(score - m) <= 2^slack and the
// rescale of acc and l is rare after the first tiles.
constexpr float kRescaleSlack = 8.f;

template <int KT, int D, int G>
struct DecodeState {
  using C = DecodeCfg<KT, D, G>;
  float m[C::HW], l[C::HW];
  float acc[C::HW][C::NACC];
};

// Scores of the lane's rows against its HW queries, online-softmax update,
// and the probabilities p[j][h] for the weighted sum.  `kt` is the tile in
// LDS, `nv` its valid rows.
template <int KT, int D, int G>
__device__ __forceinline__ void tile_scores(DecodeState<KT, D, G>& st, float (&p)[DecodeCfg<KT, D, G>::RPL][DecodeCfg<KT, D, G>::HW],
                                            const char* kt, const uint4 (&q)[DecodeCfg<KT, D, G>::HW][DecodeCfg<KT, D, G>::CPL],
                                            int nv, int excl, int rg, int s, float scale_log2) {
  using C = DecodeCfg<KT, D, G>;
  [[maybe_unused]] constexpr bool BF16 = C::BF16;
  constexpr int HW = C::HW;
  float sc[C::RPL][HW];
#pragma unroll
  for (int j = 0; j < C::RPL; ++j) {
    const int row = rg + 8 * j;
    uint4 k[C::CPL];
#pragma unroll
    for (int cc = 0; cc < C::CPL; ++cc)
      k[cc] = *reinterpret_cast<const uint4*>(kt + row * C::ROWB + (((s + 8 * cc) ^ dec_swz<C::CPR>(row)) * 16));
    // the HW dot products advance together (independent chains for the ALU)
    float acc[HW];
#pragma unroll
    for (int h = 0; h < HW; ++h) acc[h] = 0.f;
#pragma unroll
    for (int cc = 0; cc < C::CPL; ++cc) {
      const uint32_t kw[4] = {k[cc].x, k[cc].y, k[cc].z, k[cc].w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < HW; ++h) {
          const uint32_t qw[4] = {q[h][cc].x, q[h][cc].y, q[h][cc].z, q[h][cc].w};
          if constexpr (BF16) acc[h] = dot2_bf16(qw[i], kw[i], acc[h]);
          else acc[h] = fmaf(__uint_as_float(qw[i]), __uint_as_float(kw[i]), acc[h]);
        }
    }
#pragma unroll
    for (int h = 0; h < HW; ++h) sc[j][h] = row8_sum(acc[h]);
  }
  // rows past the item's end (only in its last tiles), and a row whose token
  // is being evicted (excl, tile-relative; -1 if none), score -inf
  if (nv < C::TR || excl >= 0) {
#pragma unroll
    for (int j = 0; j < C::RPL; ++j) {
      const bool ok = rg + 8 * j < nv && rg + 8 * j != excl;
#pragma unroll
      for (int h = 0; h < HW; ++h) sc[j][h] = ok ? sc[j][h] : -INFINITY;
    }
  }
  // online softmax in log2 units (scale > 0, so max commutes with it)
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
  if (__builtin_amdgcn_ballot_w64(need) != 0) {  // some lane raises its reference
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
}

// acc += sum over the lane's rows of p[j][h] * V[row]; `vt` is the V tile in LDS.
template <int KT, int D, int G>
__device__ __forceinline__ void tile_pv(DecodeState<KT, D, G>& st, const float (&p)[DecodeCfg<KT, D, G>::RPL][DecodeCfg<KT, D, G>::HW],
                                        const char* vt, int rg, int s) {
  using C = DecodeCfg<KT, D, G>;
  [[maybe_unused]] constexpr bool BF16 = C::BF16;
  constexpr int HW = C::HW;
  if constexpr (BF16) {
#pragma unroll
    for (int jp = 0; jp < C::RPL; jp += 2) {
      const int row0 = rg + 8 * jp, row1 = row0 + 8;  // same parity: same swizzle
      uint32_t P[HW];
#pragma unroll
      for (int h = 0; h < HW; ++h) P[h] = pack_bf16x2(p[jp][h], p[jp + 1][h]);
#pragma unroll
      for (int cc = 0; cc < C::CPL; ++cc) {
        const int off = ((s + 8 * cc) ^ dec_swz<C::CPR>(row0)) * 16;
        const uint4 va = *reinterpret_cast<const uint4*>(vt + row0 * C::ROWB + off);
        const uint4 vb = *reinterpret_cast<const uint4*>(vt + row1 * C::ROWB + off);
        const uint32_t a4[4] = {va.x, va.y, va.z, va.w};
        const uint32_t b4[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t lo = __builtin_amdgcn_perm(b4[i], a4[i], 0x05040100u);  // (row0, row1) at d = 2i
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
    for (int j = 0; j < C::RPL; ++j) {
      const int row = rg + 8 * j;
#pragma unroll
      for (int cc = 0; cc < C::CPL; ++cc) {
        const uint4 vv = *reinterpret_cast<const uint4*>(vt + row * C::ROWB + (((s + 8 * cc) ^ dec_swz<C::CPR>(row)) * 16));
        const float v4[4] = {__uint_as_float(vv.x), __uint_as_float(vv.y), __uint_as_float(vv.z), __uint_as_float(vv.w)};
#pragma unroll
        for (int h = 0; h < HW; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) st.acc[h][cc * 4 + e] = fmaf(p[j][h], v4[e], st.acc[h][cc * 4 + e]);
      }
    }
  }
}

// ---- four-lane score layout (bf16, four query heads per wavefront)
//
// In bf16 the scores are computed with 4 lanes per row instead of 8: lane l
// has row group r16 = l / 4 (rows r16, r16 + 16, ... of the tile) and slice
// s4 = l % 4 (16-byte chunks s4, s4 + 4, ... of the row).  After a 4-lane
// all-reduce each lane keeps only the scores of query head s4 % HW, so with
// four heads per wavefront the lanes of a row do not repeat each other's
// exponentials (with fewer heads, lanes s4 and s4 + HW hold the same head).
// The softmax state of (row group rg, head h) -- the rows rg + 8 j that lane
// (rg, s) of the weighted sum accumulates -- is kept by the lanes
// (r16 = rg, s4) and (r16 = rg + 8, s4) with s4 % HW = h, 32 lanes apart,
// which share one reference max.  The probabilities reach the weighted-sum layout through
// a small per-wavefront LDS buffer, already as the bf16 pairs (rows
// rg + 16 q and rg + 16 q + 8) the weighted sum's dot products take; the
// rescale factors of a raised reference go the same way.
template <int KT, int D, int G>
struct Score4 {
  using C = DecodeCfg<KT, D, G>;
  static constexpr bool ON = C::BF16 && !C::MF;
  static constexpr int HW = C::HW;
  static constexpr int CPL4 = C::CPR / 4;   // chunks per lane
  static constexpr int RPL4 = C::TR / 16;   // rows per lane
  static constexpr int NQ = C::RPL / 2;     // row pairs per weighted-sum lane
  static constexpr int PBUF = 8 * NQ * HW;  // probability pairs per wavefront (dwords)
  static_assert(!ON || 4 % HW == 0, "heads per wavefront divide the 4 lanes of a row");
};

// Two bf16 values (exact) from the FP8 codes in bytes 0, 1 (hi = false) or
// 2, 3 (hi = true) of w.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI));
}

// K-tile chunk swizzle of the 4-lane layout: the 4 rows a group of 16 lanes
// reads fall into 4 distinct quarters of the 256-byte bank space.
template <int CPR>
__device__ __forceinline__ int dec_swz_k4(int r) { return CPR >= 16 ? 4 * (r & 3) : CPR >= 8 ? 4 * ((r >> 1) & 1) : 0; }

// INT4 codes to bf16 pairs.  A nibble n read as the low mantissa bits of
// 0x4300 (the bf16 value 128) gives the bf16 value 128 + n = c + 136 exactly
// (c = n - 8 is the level), so dot products over these pairs exceed the ones
// over the levels by 136 times the other factor's sum, which the callers
// subtract.  lo / hi hold the low / high nibbles of four code bytes, one per
// byte; pair t takes byte t of lo (low half) and of hi (high half), i.e. the
// elements 2t and 2t + 1 of the four bytes.
template <int T>
__device__ __forceinline__ uint32_t int4_pair(uint32_t lo, uint32_t hi) {
  constexpr uint32_t sel = (uint32_t)T | (0x0Cu << 8) | ((4u + T) << 16) | (0x0Cu << 24);  // 0x0C: zero byte
  return __builtin_amdgcn_perm(hi, lo, sel) | 0x43004300u;
}
constexpr float kInt4Bias = 136.f;  // (128 + n) - (n - 8)

// all-reduce over the 4 lanes of a row
__device__ __forceinline__ float row4_sum(float x) {
  x += dpp<0xB1>(x);  // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);  // quad_perm [2,3,0,1]
  return x;
}

__device__ __forceinline__ uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// Scores of the lane's rows against query head s4, the online-softmax update
// of the lane's (m, l), and the probabilities written to `pbuf` (this
// wavefront's pairs, dword (rg, q, h) = rows rg + 16 q and rg + 16 q + 8).
// Rescale factors go to `abuf` [rg][h]; the result says whether any lane of
// the wavefront raised its reference (then every (rg, h) factor is written).
template <int KT, int D, int G>
__device__ __forceinline__ bool tile_scores4(float& m, float& l, uint16_t* pbuf, float* abuf, const char* kt,
                                             const uint4 (&q)[Score4<KT, D, G>::HW]
                                                             [Score4<KT, D, G>::CPL4],
                                             int nv, int excl, int r16, int s4, float scale_log2) {
  using C = DecodeCfg<KT, D, G>;
  static_assert(C::BF16 && !C::LOWBIT, "the four-lane layout serves bf16 rows (low-bit rows take the matrix cores)");
  using S4 = Score4<KT, D, G>;
  constexpr int HW = S4::HW;
  const int hown = s4 % HW;  // the head whose state this lane keeps
  float sc[S4::RPL4];
#pragma unroll
  for (int j = 0; j < S4::RPL4; ++j) {
    const int row = r16 + 16 * j;
    uint4 k[S4::CPL4];
#pragma unroll
    for (int cc = 0; cc < S4::CPL4; ++cc)
      k[cc] = *reinterpret_cast<const uint4*>(kt + row * C::ROWB + (((s4 + 4 * cc) ^ dec_swz_k4<C::CPR>(row)) * 16));
    float acc[HW];
#pragma unroll
    for (int h = 0; h < HW; ++h) acc[h] = 0.f;
#pragma unroll
    for (int cc = 0; cc < S4::CPL4; ++cc) {
      const uint32_t kw[4] = {k[cc].x, k[cc].y, k[cc].z, k[cc].w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < HW; ++h) {
          const uint32_t qw[4] = {q[h][cc].x, q[h][cc].y, q[h][cc].z, q[h][cc].w};
          acc[h] = dot2_bf16(qw[i], kw[i], acc[h]);
        }
    }
#pragma unroll
    for (int h = 0; h < HW; ++h) acc[h] = row4_sum(acc[h]);
    float own = acc[0];
#pragma unroll
    for (int h = 1; h < HW; ++h) own = hown == h ? acc[h] : own;
    sc[j] = (row < nv && row != excl) ? own : -INFINITY;
  }
  // reference max of (rg, s4), shared with the partner lane 32 away
  float x = sc[0];
#pragma unroll
  for (int j = 1; j < S4::RPL4; ++j) x = fmaxf(x, sc[j]);
  x = fmaxf(x, __shfl_xor(x, 32));
  const float mt = x * scale_log2;  // scale > 0, so max commutes with it
  const bool any = __builtin_amdgcn_ballot_w64(mt > m + kRescaleSlack) != 0;
  if (any) {
    const float mn = fmaxf(m, mt);
    const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m - mn);
    m = mn;
    l *= alpha;
    if (r16 < 8 && s4 < HW) abuf[r16 * HW + s4] = alpha;
  }
  const float mu = (m == -INFINITY) ? 0.f : m;
  const int rg = r16 & 7, half = r16 >> 3;
#pragma unroll
  for (int j = 0; j < S4::RPL4; ++j) {
    const float pj = fast_exp2(fmaf(sc[j], scale_log2, -mu));
    const uint16_t pb = bf16_bits(pj);
    // The sum takes the weight the weighted sum really applies to the row,
    // the rounded probability, so the weights of the result sum to one: an
    // unrounded sum would leave a relative error of up to 2^-9 in every
    // output element.
    l += __uint_as_float((uint32_t)pb << 16);
    if (s4 < HW) pbuf[((rg * S4::NQ + j) * HW + s4) * 2 + half] = pb;
  }
  return any;
}

// acc += sum over the lane's rows of p * V[row], with the probability pairs
// and rescale factors from tile_scores4.
template <int KT, int D, int G>
__device__ __forceinline__ void tile_pv4(DecodeState<KT, D, G>& st, const uint16_t* pbuf, const float* abuf,
                                         bool rescale, const char* vt, int rg, int s) {
  using C = DecodeCfg<KT, D, G>;
  static_assert(C::BF16 && !C::LOWBIT, "the four-lane layout serves bf16 rows");
  using S4 = Score4<KT, D, G>;
  constexpr int HW = S4::HW;
  if (rescale) {
#pragma unroll
    for (int h = 0; h < HW; ++h) {
      const float al = abuf[rg * HW + h];
#pragma unroll
      for (int e = 0; e < C::NACC; ++e) st.acc[h][e] *= al;
    }
  }
#pragma unroll
  for (int qq = 0; qq < S4::NQ; ++qq) {
    const int row0 = rg + 16 * qq, row1 = row0 + 8;  // same parity: same swizzle
    uint32_t P[HW];
    const uint32_t* pq = reinterpret_cast<const uint32_t*>(pbuf) + (rg * S4::NQ + qq) * HW;
#pragma unroll
    for (int h = 0; h < HW; ++h) P[h] = pq[h];
#pragma unroll
    for (int cc = 0; cc < C::CPL; ++cc) {
      const int off = ((s + 8 * cc) ^ dec_swz<C::CPR>(row0)) * 16;
      const uint4 va = *reinterpret_cast<const uint4*>(vt + row0 * C::ROWB + off);
      const uint4 vb = *reinterpret_cast<const uint4*>(vt + row1 * C::ROWB + off);
      const uint32_t a4[4] = {va.x, va.y, va.z, va.w};
      const uint32_t b4[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = __builtin_amdgcn_perm(b4[i], a4[i], 0x05040100u);  // (row0, row1) at d = 2i
        const uint32_t hi = __builtin_amdgcn_perm(b4[i], a4[i], 0x07060302u);  // at d = 2i+1
#pragma unroll
        for (int h = 0; h < HW; ++h) {
          st.acc[h][cc * 8 + 2 * i] = dot2_bf16(P[h], lo, st.acc[h][cc * 8 + 2 * i]);
          st.acc[h][cc * 8 + 2 * i + 1] = dot2_bf16(P[h], hi, st.acc[h][cc * 8 + 2 * i + 1]);
        }
      }
    }
  }
}

// ---- matrix-core tiles (bf16 rows, d = 128)
//
// A wavefront scores its 16 rows of a round against the group's g <= 8
// queries as S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (keys on M, queries
// on N; the queries fill g of the 16 columns, the others are zero), and
// accumulates O^T += V^T P^T with v_mfma_f32_16x16x16_bf16 (d on M).  Lane
// l = 16 g + j holds query j: its scores of rows 4 g .. 4 g + 3, the bf16
// probabilities of those rows (the B operand of the weighted sum as they
// are), and the output elements d = 16 t + 4 g .. + 3 of each 16-row d tile
// t.  The K operand (key j's 8 elements 32 k + 8 g ..) is a 16-byte read;
// the V^T operand (d = 16 t + j of rows 4 g .. 4 g + 3) a transpose read.
// Rows are stored in the round with the chunk swizzles of the prefill tiles
// (K: chunk c at c ^ (r & 15); V: c ^ 4 (r & 3)), so both reads are free of
// bank conflicts.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8v_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int mf_swz_k(int r) { return r & 15; }
__device__ __forceinline__ int mf_swz_v(int r) { return 4 * (r & 3); }

struct MfState {
  f32x4_t o[8];    // O^T tiles: d = 16 t + 4 g + e of query j
  float m, l;      // running max (log2 units; the same in the four lanes of a query) and the lane's partial sum
  // the current tile's probabilities as bf16 pairs: rows 4 g .. 4 g + 3
  // (FP8 rows: then rows 16 + 4 g .. + 3; INT4 rows: 16 q + 4 g .. + 3 for
  // q = 0 .. 3; low-bit rows each times its V scale)
  uint32_t p[8];
  float w;         // INT4 rows: the lane's sum of the weights it applied (the levels' bias, see mf4_pv)
};

__device__ __forceinline__ void mf_init(MfState& st) {
#pragma unroll
  for (int t = 0; t < 8; ++t) st.o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) st.p[i] = 0u;
  st.w = 0.f;
}

// Scores of the tile's rows (nv valid; row excl, tile-relative, masked; -1
// for none), the lazy online-softmax update and the probabilities.
__device__ __forceinline__ void mf_scores(MfState& st, const char* kt, const bf16x8v_t (&qm)[4], int nv, int excl,
                                          int lane, float scale_log2) {
  const int j = lane & 15, g = lane >> 4;
  f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = 4 * k + g;
    const u32x4_t av = *reinterpret_cast<const u32x4_t*>(kt + j * 256 + ((c ^ mf_swz_k(j)) * 16));
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v_t, av), qm[k], sc, 0, 0, 0);
  }
  if (nv < 16 || excl >= 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * g + e;
      if (r >= nv || r == excl) sc[e] = -INFINITY;
    }
  }
  // the query's max over the tile: the lane's four rows, then the four lanes g
  const float mx = swap32_max(swap16_max(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])))) * scale_log2;
  if (__builtin_amdgcn_ballot_w64(mx > st.m + kRescaleSlack) != 0) {  // some query raises its reference
    const float mn = fmaxf(st.m, mx);
    const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(st.m - mn);
    st.m = mn;
    st.l *= alpha;
#pragma unroll
    for (int t = 0; t < 8; ++t) st.o[t] *= alpha;
  }
  const float mu = (st.m == -INFINITY) ? 0.f : st.m;
  const float p0 = fast_exp2(fmaf(sc[0], scale_log2, -mu)), p1 = fast_exp2(fmaf(sc[1], scale_log2, -mu));
  const float p2 = fast_exp2(fmaf(sc[2], scale_log2, -mu)), p3 = fast_exp2(fmaf(sc[3], scale_log2, -mu));
  st.p[0] = pack_bf16x2(p0, p1);
  st.p[1] = pack_bf16x2(p2, p3);
  // the row sums add the bf16-rounded probabilities, the values P V uses
  constexpr uint32_t kOnes = 0x3f803f80u;
  st.l = dot2_bf16(st.p[1], kOnes, dot2_bf16(st.p[0], kOnes, st.l));
}

// O^T += V^T P^T over the tile's rows (rows past nv carry probability 0).
__device__ __forceinline__ void mf_pv(MfState& st, const char* vt, int lane) {
  const int i16 = lane & 15, g = lane >> 4;
  const i16x4_t pb = __builtin_bit_cast(i16x4_t, u32x2_t{st.p[0], st.p[1]});
  const int row = 4 * g + (i16 >> 2);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int col = 16 * t + 4 * (i16 & 3);
    const char* ptr = vt + row * 256 + (((col >> 3) ^ mf_swz_v(row)) * 16) + (col & 7) * 2;
    const i16x4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(ptr));
    st.o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, st.o[t], 0, 0, 0);
  }
}

// ---- matrix-core tiles over FP8 rows (d = 128, 128-byte rows)
//
// A wavefront takes 32 rows of a round, two groups of 16 for the scores.
// The K operand is key j's 8 codes 32 k + 8 g .. (an 8-byte read), turned
// into bf16 exactly (every E4M3 value is a bf16 value); the scores are then
// scaled by their rows' K scales.  The weighted sum contracts over all 32
// rows at once with v_mfma_f32_16x16x32_bf16: lane 16 g + j's eight
// contraction slots are its own rows 4 g .. 4 g + 3 and 16 + 4 g .. + 3,
// whose probabilities (times the rows' V scales, in bf16) it already holds;
// the V^T operand comes from a transpose read of bytes (ds_read_b64_tr_b8:
// lane i of a 16-lane group receives byte column i of the eight rows the
// group's lanes 2 e and 2 e + 1 address), each lane addressing the row of
// its group's slot e >> 1.  The denominator adds the same rounded values
// divided back by the V scales.  Chunk swizzles: K chunk c of row r at
// c ^ ((r >> 1) & 7); V at c ^ ((r >> 1) & 7) ^ 4 ((r >> 4) & 1); both reads
// are then free of bank conflicts.
__device__ __forceinline__ int mf8_swz_k(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int mf8_swz_v(int r) { return ((r >> 1) & 7) ^ (4 * ((r >> 4) & 1)); }

// eight FP8 codes (two words) as an exact bf16 operand
__device__ __forceinline__ bf16x8v_t fp8x8_bf16(uint32_t w0, uint32_t w1) {
  const u32x4_t v = {fp8x2_bf16<false>(w0), fp8x2_bf16<true>(w0), fp8x2_bf16<false>(w1), fp8x2_bf16<true>(w1)};
  return __builtin_bit_cast(bf16x8v_t, v);
}

__device__ __forceinline__ void mf8_scores(MfState& st, const char* kt, const bf16x8v_t (&qm)[4], const float* ks,
                                           const float* vs, int nv, int excl, int lane, float scale_log2) {
  const int j = lane & 15, g = lane >> 4;
  f32x4_t sc[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    sc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int row = 16 * q + j;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = 2 * k + (g >> 1);
      const u32x2_t w = *reinterpret_cast<const u32x2_t*>(kt + row * 128 + ((c ^ mf8_swz_k(row)) * 16) + 8 * (g & 1));
      sc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_bf16(w[0], w[1]), qm[k], sc[q], 0, 0, 0);
    }
  }
  float vsc[2][4];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const float4 k4 = *reinterpret_cast<const float4*>(ks + 16 * q + 4 * g);
    const float4 v4 = *reinterpret_cast<const float4*>(vs + 16 * q + 4 * g);
    sc[q][0] *= k4.x;
    sc[q][1] *= k4.y;
    sc[q][2] *= k4.z;
    sc[q][3] *= k4.w;
    vsc[q][0] = v4.x;
    vsc[q][1] = v4.y;
    vsc[q][2] = v4.z;
    vsc[q][3] = v4.w;
  }
  if (nv < 32 || excl >= 0) {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * q + 4 * g + e;
        if (r >= nv || r == excl) sc[q][e] = -INFINITY;
      }
  }
  const float m8 = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                         fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
  const float mx = swap32_max(swap16_max(m8)) * scale_log2;
  if (__builtin_amdgcn_ballot_w64(mx > st.m + kRescaleSlack) != 0) {
    const float mn = fmaxf(st.m, mx);
    const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(st.m - mn);
    st.m = mn;
    st.l *= alpha;
#pragma unroll
    for (int t = 0; t < 8; ++t) st.o[t] *= alpha;
  }
  const float mu = (st.m == -INFINITY) ? 0.f : st.m;
  float l = st.l;
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const float p0 = fast_exp2(fmaf(sc[q][e], scale_log2, -mu));
      const float p1 = fast_exp2(fmaf(sc[q][e + 1], scale_log2, -mu));
      const uint32_t pp = pack_bf16x2(p0 * vsc[q][e], p1 * vsc[q][e + 1]);
      st.p[2 * q + e / 2] = pp;
      // the weight the weighted sum applies, divided back by the V scale (a
      // row of zeros, scale 0, adds its probability itself)
      l += vsc[q][e] > 0.f ? bf_lo(pp) * __builtin_amdgcn_rcpf(vsc[q][e]) : p0;
      l += vsc[q][e + 1] > 0.f ? bf_hi(pp) * __builtin_amdgcn_rcpf(vsc[q][e + 1]) : p1;
    }
  st.l = l;
}

__device__ __forceinline__ void mf8_pv(MfState& st, const char* vt, int lane) {
  const int i16 = lane & 15, g = lane >> 4;
  const bf16x8v_t pb = __builtin_bit_cast(bf16x8v_t, u32x4_t{st.p[0], st.p[1], st.p[2], st.p[3]});
  const int e = i16 >> 1;                                    // the group's slot this lane addresses
  const int row = e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4);  // that slot's row
  const int half = i16 & 1;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const char* ptr = vt + row * 128 + ((t ^ mf8_swz_v(row)) * 16) + 8 * half;
    const u32x2_t v = __builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)(ptr)));
    st.o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_bf16(v[0], v[1]), pb, st.o[t], 0, 0, 0);
  }
}

// ---- matrix-core tiles over INT4 rows (d = 128, 64-byte rows)
//
// A wavefront takes 64 rows of a round, four groups of 16 for the scores.
// The K operand is key j's eight codes 32 k + 8 g .. (a 4-byte read), each
// nibble n read as the bf16 value 128 + n = c + 136 (see int4_pair); the
// scores then drop 136 times the query's element sum and take their rows'
// K scales.  The weighted sum runs two v_mfma_f32_16x16x32_bf16 per d tile:
// a 4-bit transpose read (ds_read_b64_tr_b4: lane i of a 16-lane group
// receives element i of the 16 rows its group's lanes address, one nibble
// per row) gives a lane element d = 16 t + i of the 16 rows 16 q + 4 g + b
// its group holds probabilities for, the first eight (q = 0, 1) for one
// MFMA and the last eight for the other.  The accumulators then exceed the
// weighted sums over the levels by 136 times the sum of the weights, which
// the merge subtracts.  Chunk swizzles: K chunk c of row r at c ^ ((r >> 2)
// & 3), V at c ^ ((r >> 4) & 3); both reads are free of bank conflicts.
__device__ __forceinline__ int mf4_swz_k(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int mf4_swz_v(int r) { return (r >> 4) & 3; }

// eight INT4 codes (one word, element 2k in the low nibble of byte k) as
// the bf16 operand of their values + 136
__device__ __forceinline__ bf16x8v_t int4x8_bf16(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  const u32x4_t v = {int4_pair<0>(lo, hi), int4_pair<1>(lo, hi), int4_pair<2>(lo, hi), int4_pair<3>(lo, hi)};
  return __builtin_bit_cast(bf16x8v_t, v);
}

__device__ __forceinline__ void mf4_scores(MfState& st, const char* kt, const bf16x8v_t (&qm)[4], float qbias,
                                           const float* ks, const float* vs, int nv, int excl, int lane,
                                           float scale_log2) {
  const int j = lane & 15, g = lane >> 4;
  f32x4_t sc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    sc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int row = 16 * q + j;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(kt + row * 64 + ((k ^ mf4_swz_k(row)) * 16) + 4 * g);
      sc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(int4x8_bf16(w), qm[k], sc[q], 0, 0, 0);
    }
  }
  float vsc[4][4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 k4 = *reinterpret_cast<const float4*>(ks + 16 * q + 4 * g);
    const float4 v4 = *reinterpret_cast<const float4*>(vs + 16 * q + 4 * g);
    sc[q][0] = (sc[q][0] - qbias) * k4.x;
    sc[q][1] = (sc[q][1] - qbias) * k4.y;
    sc[q][2] = (sc[q][2] - qbias) * k4.z;
    sc[q][3] = (sc[q][3] - qbias) * k4.w;
    vsc[q][0] = v4.x;
    vsc[q][1] = v4.y;
    vsc[q][2] = v4.z;
    vsc[q][3] = v4.w;
  }
  if (nv < 64 || excl >= 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * q + 4 * g + e;
        if (r >= nv || r == excl) sc[q][e] = -INFINITY;
      }
  }
  float m16 = -INFINITY;
#pragma unroll
  for (int q = 0; q < 4; ++q) m16 = fmaxf(m16, fmaxf(fmaxf(sc[q][0], sc[q][1]), fmaxf(sc[q][2], sc[q][3])));
  const float mx = swap32_max(swap16_max(m16)) * scale_log2;
  if (__builtin_amdgcn_ballot_w64(mx > st.m + kRescaleSlack) != 0) {
    const float mn = fmaxf(st.m, mx);
    const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(st.m - mn);
    st.m = mn;
    st.l *= alpha;
    st.w *= alpha;
#pragma unroll
    for (int t = 0; t < 8; ++t) st.o[t] *= alpha;
  }
  const float mu = (st.m == -INFINITY) ? 0.f : st.m;
  float l = st.l, wsum = st.w;
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const float p0 = fast_exp2(fmaf(sc[q][e], scale_log2, -mu));
      const float p1 = fast_exp2(fmaf(sc[q][e + 1], scale_log2, -mu));
      const uint32_t pp = pack_bf16x2(p0 * vsc[q][e], p1 * vsc[q][e + 1]);
      st.p[2 * q + e / 2] = pp;
      wsum += bf_lo(pp) + bf_hi(pp);
      l += vsc[q][e] > 0.f ? bf_lo(pp) * __builtin_amdgcn_rcpf(vsc[q][e]) : p0;
      l += vsc[q][e + 1] > 0.f ? bf_hi(pp) * __builtin_amdgcn_rcpf(vsc[q][e + 1]) : p1;
    }
  st.l = l;
  st.w = wsum;
}

__device__ __forceinline__ void mf4_pv(MfState& st, const char* vt, int lane) {
  const int i16 = lane & 15, g = lane >> 4;
  const bf16x8v_t pa = __builtin_bit_cast(bf16x8v_t, u32x4_t{st.p[0], st.p[1], st.p[2], st.p[3]});
  const bf16x8v_t pb = __builtin_bit_cast(bf16x8v_t, u32x4_t{st.p[4], st.p[5], st.p[6], st.p[7]});
  const int row = 16 * (i16 >> 2) + 4 * g + (i16 & 3);  // the row this lane addresses: slot i16 of its group
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const char* ptr = vt + row * 64 + (((t >> 1) ^ mf4_swz_v(row)) * 16) + 8 * (t & 1);
    const u32x2_t v = __builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_ds_read_tr4_b64_v2i32((__attribute__((address_space(3))) i32x2_t*)(ptr)));
    st.o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(int4x8_bf16(v[0]), pa, st.o[t], 0, 0, 0);
    st.o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(int4x8_bf16(v[1]), pb, st.o[t], 0, 0, 0);
  }
}

template <int X>
using UnitTag = std::integral_constant<int, X>;

// SH: the plan has share groups (the kernel then also runs shared items);
// only the matrix-core instantiations with g = 4 or 8 take them.
template <int KT, int D, int G, bool SH>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(DecodeArgs a) {
  using C = DecodeCfg<KT, D, G>;
  [[maybe_unused]] constexpr bool BF16 = C::BF16;
  constexpr int HW = C::HW, SLOTS = C::SLOTS, TR = C::TR;

  // The four ring units are separate arrays so that the compiler can tell a
  // unit being read from the units the direct loads are filling (it would
  // otherwise wait for every load in flight before each LDS read).
  __shared__ __attribute__((aligned(1024))) char ring0[kUnitBytes];
  __shared__ __attribute__((aligned(1024))) char ring1[kUnitBytes];
  __shared__ __attribute__((aligned(1024))) char ring2[kUnitBytes];
  __shared__ __attribute__((aligned(1024))) char ring3[kUnitBytes];
  // merge state: max and sum of every (slot, row group, query head) partial,
  // its weight in the merged result, and the merged max and sum per head
  __shared__ __attribute__((aligned(16))) float w_m[G][SLOTS * 8], w_l[G][SLOTS * 8], w_w[G][SLOTS * 8],
      w_lw[G][SLOTS * 8];
  __shared__ float w_mt[G];
  // the group's queries (a shared item: the queries of its share group's
  // rows, up to 16) and the new token's K and V rows, loaded by direct loads
  constexpr bool SHARE = SH && C::MF && (G == 4 || G == 8);  // shared items (bf16 queries, d = 128)
  constexpr int QGROUP = (G * C::IROWB + 1023) / 1024 * 1024;  // one row's query group, whole pieces
  constexpr int QSTAGE = SHARE ? 16 * C::IROWB : QGROUP;
  static_assert(!SHARE || (G * C::IROWB) % 1024 == 0, "a row's queries are whole staging pieces");
  constexpr int NSTAGE = (C::IROWB + 1023) / 1024 * 1024;
  static_assert(QSTAGE / 1024 + 2 <= kDecWaves, "one staging piece per wavefront");
  __shared__ __attribute__((aligned(1024))) char stage[QSTAGE + 2 * NSTAGE];
  using S4 = Score4<KT, D, G>;
  constexpr bool SC4 = S4::ON;
  constexpr bool MF = C::MF;
  // four-lane score layout: per-wavefront probability pairs and rescale factors
  __shared__ __attribute__((aligned(16))) uint16_t pbuf_all[SC4 ? kDecWaves : 1][SC4 ? 2 * S4::PBUF : 8];
  __shared__ __attribute__((aligned(16))) float abuf_all[SC4 ? kDecWaves : 1][32];
  // FP8 / INT4 rows: the K scales, then the V scales, of the rows of a round;
  // one buffer per K unit of the ring (units 0 and 2), loaded with that unit
  constexpr bool KV8 = C::KV8, KV4 = C::KV4, LOWBIT = C::LOWBIT;
  __shared__ __attribute__((aligned(16))) float sbuf[LOWBIT ? 2 : 1][LOWBIT ? 2 * C::ROUND_ROWS : 4];
  [[maybe_unused]] const uint32_t sbuf_lds = lds_addr(&sbuf[0][0]);  // its LDS byte address
  // a round's scales: SPW wavefront loads of 64 rows per wavefront (waves 0-3
  // the K scales, 4-7 the V scales); FP8 rounds hold 256 rows, INT4 rounds 512
  constexpr int SPW = LOWBIT ? C::ROUND_ROWS / 256 : 0;
  static_assert(!LOWBIT || C::ROUND_ROWS % 256 == 0, "a round's scales are whole wavefront loads");
  // Vector-memory loads per unit and wavefront: the ring pieces, plus SPW
  // scale loads with each K unit of low-bit rows.  When unit u has landed,
  // the DEPTH - 1 units after it may be in flight: WAITN loads after a K
  // unit, WAITV after a V unit.
  constexpr int DEPTH = C::DEPTH;
  static_assert(DEPTH == 2 || DEPTH == 3, "ring depth");
  constexpr int WAITN = DEPTH == 3 ? 2 * kPiecesPerWave + SPW : kPiecesPerWave;
  constexpr int WAITV = DEPTH == 3 ? 2 * kPiecesPerWave + SPW : kPiecesPerWave + SPW;
  char* const rings[kRingUnits] = {ring0, ring1, ring2, ring3};  // indexed by constants only
  // their LDS byte addresses (constants), where the direct loads write
  const uint32_t ring_lds[kRingUnits] = {lds_addr(ring0), lds_addr(ring1), lds_addr(ring2), lds_addr(ring3)};
  auto ring_at = [&](int i) -> char* { return i == 0 ? ring0 : i == 1 ? ring1 : i == 2 ? ring2 : ring3; };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = wave / C::HSPLIT;   // tile of the round this wavefront reads
  const int hg = wave % C::HSPLIT;     // which HW query heads of the group it scores
  const bool active = slot < SLOTS;
  const int rg = lane >> 3, s = lane & 7;
  DecodeItem w = decode_item<C::ROWB, C::ROUND_ROWS, SHARE>(a, blockIdx.x);
  // The row's token count: needed before the first loads by the last item of
  // a head (where it ends, where a fused append's token goes) and by the items
  // of a streaming head under a fused append (the slot the new token evicts);
  // other items wait for it only if rotary positions need the query's position.
  const bool last_item = w.part == w.nparts - 1 && !w.shared;
  if (last_item || (a.new_k != nullptr && w.hh >= (int64_t)a.B * a.n_ret)) {
    w.cnt = row_count(a, w.b);
    if (last_item) end_last_item(a, w);
  }
  // The item's rows in 32-bit wavefront-uniform values (the host keeps T_cap
  // at least 4,096 under 2^31, so a round past the item's end still fits),
  // so the per-unit row arithmetic is a few scalar instructions.
  const int32_t r0 = __builtin_amdgcn_readfirstlane((int)w.r0), r1 = __builtin_amdgcn_readfirstlane((int)w.r1);
  const int32_t nrounds = ((r1 - r0 + TR - 1) / TR + SLOTS - 1) / SLOTS;
  const size_t q_off = ((size_t)w.b * a.n_q + (size_t)w.kvh * G) * D;  // first query of the group

  // fused append: the last item of every head adds the new token at position
  // w.cnt; the step stores it only if the row has room (else it is attended
  // from the staging area alone and the cache's status bit is set)
  const bool add_new = a.new_k != nullptr && last_item;
  const bool ret_head = w.hh < (int64_t)a.B * a.n_ret;
  const int64_t cap_str = a.cap_str;
  // streaming slot masked in the held rows (its token is evicted by the new one)
  const int32_t excl_row =
      (a.new_k != nullptr && !ret_head && w.cnt >= cap_str) ? (int32_t)(a.S + (w.cnt - a.S) % a.W) : -1;
  // per-lane byte offset, within a round of rows, of this wavefront's load
  // pieces: piece n of a unit covers LDS bytes [n*1024, n*1024+1024), lane i
  // byte n*1024 + 16 i, i.e. row (n*1024 + 16 i) / ROWB of the round at a
  // chunk slot that is the row's swizzle applied to the global chunk
  // (K units use the four-lane score layout's swizzle when it is on)
  uint32_t poff_k[kPiecesPerWave], poff_v[kPiecesPerWave];
#pragma unroll
  for (int j = 0; j < kPiecesPerWave; ++j) {
    const int off = (wave + kDecWaves * j) * 1024 + lane * 16;
    const int r = off / C::ROWB;  // row of the round; a slot's tile starts at a multiple of 4 rows
    const int c = (off % C::ROWB) / 16;
    const int ck = c ^ (MF ? (KV4 ? mf4_swz_k(r % TR) : KV8 ? mf8_swz_k(r % TR) : mf_swz_k(r % TR))
                          : SC4 ? dec_swz_k4<C::CPR>(r % TR) : dec_swz<C::CPR>(r % TR));
    const int cv = c ^ (MF ? (KV4 ? mf4_swz_v(r % TR) : KV8 ? mf8_swz_v(r % TR) : mf_swz_v(r % TR))
                          : dec_swz<C::CPR>(r % TR));
    poff_k[j] = (uint32_t)(r * C::ROWB + ck * 16);
    poff_v[j] = (uint32_t)(r * C::ROWB + cv * 16);
  }
  static_assert(TR % 4 == 0, "tiles start at a multiple of 4 rows");

  // Issue unit `uu` (round uu / 2; K rows if uu is even, else V rows) into
  // `dst`: the round's rows are contiguous, so one buffer resource covers
  // them, sized to the rows the item still has.  Past the item's end every
  // piece is out of range (it reads nothing and writes zeros to LDS) but is
  // still issued, so each wavefront has the same number of loads per unit,
  // and every byte of a unit is written before it is read.
  auto issue = [&](int32_t uu, uint32_t dst) {  // dst: the ring unit's LDS byte address
    const int32_t row0 = r0 + (uu >> 1) * C::ROUND_ROWS;
    const int32_t left = r1 - row0;
    const int rows = left <= 0 ? 0 : (left > C::ROUND_ROWS ? C::ROUND_ROWS : left);
    const int64_t roff = rows > 0 ? w.at(row0) : 0;
    const char* src = ((uu & 1) ? w.vbase : w.kbase) + (size_t)roff * C::ROWB;
    const i32x4_t rs = dma_rsrc(src, rows * C::ROWB);
#pragma unroll
    for (int j = 0; j < kPiecesPerWave; ++j)
      dma_lds16_at(rs, dst + (uint32_t)((wave + kDecWaves * j) * 1024), (uu & 1) ? poff_v[j] : poff_k[j], 0u);
    if constexpr (LOWBIT) {
      if ((uu & 1) == 0) {  // wavefronts 0-3: K scales, 4-7: V scales, SPW x 64 rows each
        const int tensor = wave >> 2, part = wave & 3;
        const float* ssrc = (tensor ? w.vsc : w.ksc) + roff;
        const i32x4_t srs = dma_rsrc(reinterpret_cast<const char*>(ssrc), rows * 4);
#pragma unroll
        for (int j = 0; j < SPW; ++j)
          dma_lds4_at(srs,
                      sbuf_lds + (uint32_t)((((uu >> 1) & 1) * 2 * C::ROUND_ROWS + tensor * C::ROUND_ROWS +
                                             (part * SPW + j) * 64) * 4),
                      (uint32_t)(((part * SPW + j) * 64 + lane) * 4));
      }
    }
  };
  // The first unit, then the group's queries and the new token's K and V rows
  // into the staging area (one load piece per wavefront for the first
  // wavefronts), then the next DEPTH - 1 units.  Unit 0's wait below covers
  // the staging loads, which were issued before those units.
  issue(0, ring_lds[0]);
  {
    constexpr int PPR = QGROUP / 1024;  // query pieces per batch row
    const int nqp = w.qrows * PPR;      // query pieces of this item
    if (wave < nqp) {
      const int qi = wave / PPR;        // row of the share group (0 for other items)
      const char* qsrc = static_cast<const char*>(a.q) + (q_off + (size_t)qi * a.n_q * D) * C::ES;
      dma_lds16(dma_rsrc(qsrc, G * C::IROWB), stage + wave * 1024, (uint32_t)((wave % PPR) * 1024 + lane * 16));
    } else if (add_new && wave < nqp + 2) {
      const char* nsrc = (wave == nqp ? a.new_k : a.new_v) + ((size_t)w.b * a.n_kv + w.kvh) * C::IROWB;
      dma_lds16(dma_rsrc(nsrc, C::IROWB), stage + QSTAGE + (wave - nqp) * NSTAGE, (uint32_t)(lane * 16));
    }
  }
  issue(1, ring_lds[1]);
  if constexpr (DEPTH == 3) issue(2, ring_lds[2]);
  // rotary positions: this lane's angle (pair lane % (D/2)) at the query's
  // position, computed while the loads are in flight
  // (a shared item's rows each have their own position: it takes their
  // angles in its rotation pass below)
  double rcs = 1.0, rsn = 0.0;
  if (a.rope.on && !(SHARE && w.shared)) {
    const int64_t cnt = w.cnt >= 0 ? w.cnt : row_count(a, w.b);
    rope_cs(a.rope, cnt - (a.new_k ? 0 : 1), lane % (D / 2), rcs, rsn);
  }
  wait_vmcnt<WAITN>();  // unit 0 and the staging loads have landed
  lds_barrier();
  if (a.rope.on) {
    // the queries (and the new token's K row) turned at the query's position
    if (SHARE && w.shared) rope_stage_rows<C::ES>(a, w.b, stage, G, w.qrows, C::IROWB, D);
    else rope_stage<C::ES>(stage, G, stage + QSTAGE, add_new, C::IROWB, D, rcs, rsn);
    lds_barrier();
  }
  // this wavefront's HW queries, in the lane's slice layout (of the four-lane
  // score layout when it is on)
  constexpr int QCPL = SC4 ? S4::CPL4 : C::CPL;
  const int r16 = lane >> 2, s4 = lane & 3;
  uint4 q[HW][QCPL];
#pragma unroll
  for (int h = 0; h < HW; ++h)
#pragma unroll
    for (int c2 = 0; c2 < QCPL; ++c2)
      q[h][c2] = *reinterpret_cast<const uint4*>(
          stage + (size_t)(hg * HW + h) * C::IROWB +
          (SC4 ? (s4 + 4 * c2) : (s + 8 * c2)) * 16);
  uint16_t* const pbuf = pbuf_all[SC4 ? wave : 0];
  float* const abuf = abuf_all[SC4 ? wave : 0];
  float m4 = -INFINITY, l4 = 0.f;  // four-lane layout: softmax state of (r16 % 8, head s4)
  bool resc = false;               // four-lane layout: the K unit raised a reference

  DecodeState<KT, D, G> st;
#pragma unroll
  for (int h = 0; h < HW; ++h) {
    st.m[h] = -INFINITY;
    st.l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < C::NACC; ++e) st.acc[h][e] = 0.f;
  }
  float p[C::RPL][HW];
  // matrix-core tiles: the queries as the B operand (lane 16 g + j: query j,
  // elements 32 k + 8 g .. + 7 of k-step k; columns 8 .. 15 zero) and the state
  bf16x8v_t qm[4];
  MfState mst;
  float mqbias = 0.f;  // INT4 rows: 136 times the lane's query's element sum
  if constexpr (MF) {
    const int j = lane & 15, g = lane >> 4;
    float qs = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const u32x4_t v = j < w.qrows * G ? *reinterpret_cast<const u32x4_t*>(stage + (size_t)j * C::IROWB + (32 * k + 8 * g) * 2)
                              : u32x4_t{0u, 0u, 0u, 0u};
      qm[k] = __builtin_bit_cast(bf16x8v_t, v);
      if constexpr (KV4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) qs += bf_lo(v[i]) + bf_hi(v[i]);
      }
    }
    if constexpr (KV4) mqbias = swap32_sum(swap16_sum(qs)) * kInt4Bias;
    mf_init(mst);
  }

  // Unit u of the stream, held in ring unit X = u % 4 (K rows when X is even).
  auto unit = [&](auto tag, int32_t u) {
    constexpr int X = decltype(tag)::value;
    constexpr bool V_PART = (X & 1) != 0;
    wait_vmcnt<V_PART ? WAITV : WAITN>();  // unit u has landed; the next DEPTH - 1 may be in flight
    lds_barrier();                          // ... for every wavefront; unit u-1 is consumed
    issue(u + DEPTH, ring_lds[(X + DEPTH) % kRingUnits]);
    const int32_t row0 = r0 + ((u >> 1) * SLOTS + slot) * TR;
    const int32_t left = r1 - row0;
    const int nv = active ? (int)(left < 0 ? 0 : (left > TR ? TR : left)) : 0;
    const char* tile = rings[X] + slot * C::SLOT_BYTES;
    if (V_PART) {
      if constexpr (MF && KV4) {
        if (nv > 0) mf4_pv(mst, tile, lane);
      } else if constexpr (MF && KV8) {
        if (nv > 0) mf8_pv(mst, tile, lane);
      } else if constexpr (MF) {
        if (nv > 0) mf_pv(mst, tile, lane);
      } else if constexpr (SC4) {
        if (nv > 0) tile_pv4<KT, D, G>(st, pbuf, abuf, resc, tile, rg, s);
      } else {
        if (nv > 0) tile_pv<KT, D, G>(st, p, tile, rg, s);
      }
    } else {
      const int32_t ex = excl_row - row0;
      const int exr = (ex >= 0 && ex < TR) ? (int)ex : -1;
      if constexpr (MF && LOWBIT) {
        const float* ks = &sbuf[(u >> 1) & 1][slot * TR];
        if constexpr (KV4) {
          if (nv > 0) mf4_scores(mst, tile, qm, mqbias, ks, ks + C::ROUND_ROWS, nv, exr, lane, a.scale_log2);
        } else {
          if (nv > 0) mf8_scores(mst, tile, qm, ks, ks + C::ROUND_ROWS, nv, exr, lane, a.scale_log2);
        }
      } else if constexpr (MF) {
        if (nv > 0) mf_scores(mst, tile, qm, nv, exr, lane, a.scale_log2);
      } else if constexpr (SC4) {
        resc = false;
        if (nv > 0) resc = tile_scores4<KT, D, G>(m4, l4, pbuf, abuf, tile, q, nv, exr, r16, s4, a.scale_log2);
      } else {
        if (nv > 0) tile_scores<KT, D, G>(st, p, tile, q, nv, exr, rg, s, a.scale_log2);
      }
    }
  };
  const int32_t n_units = 2 * nrounds;
  for (int32_t u = 0; u < n_units; u += 4) {  // n_units is even
    unit(UnitTag<0>{}, u);
    unit(UnitTag<1>{}, u + 1);
    if (u + 2 >= n_units) break;
    unit(UnitTag<2>{}, u + 2);
    unit(UnitTag<3>{}, u + 3);
  }

  // the loads issued past the last unit (out of range, nothing read) land
  // before the workgroup can leave
  wait_vmcnt<0>();

  // ---- fused append: score the new token as a one-row tile (K in row 0 of
  // ring0, V in row 0 of ring1; the other rows are masked), then store it
  uint4 nkv = make_uint4(0, 0, 0, 0);
  uint2 ncodes = make_uint2(0u, 0u);  // FP8 rows: the new token's codes (lanes 0-31 of wavefront 0)
  uint32_t ncodes4 = 0u;              // INT4 rows: the same
  float nscale = 0.f;
  if (add_new) {
    lds_barrier();  // every wavefront is done with the ring
    if constexpr (KV8) {
      // quantize the new K (lanes 0-15) and V (lanes 16-31) rows as the
      // append would, and place them in row 0 of ring0 / ring1
      if (wave == 0 && lane < 32) {
        const int t = lane >> 4, j = lane & 15;
        ncodes = quant_row16(*reinterpret_cast<const uint4*>(stage + QSTAGE + t * NSTAGE + j * 16), nscale);
        *reinterpret_cast<uint2*>((t ? ring1 : ring0) + j * 8) = ncodes;  // row 0: no swizzle
        if (j == 0) sbuf[0][t * C::ROUND_ROWS] = nscale;
      }
    } else if constexpr (KV4) {
      if (wave == 0 && lane < 32) {
        const int t = lane >> 4, j = lane & 15;
        ncodes4 = quant_row16_int4(*reinterpret_cast<const uint4*>(stage + QSTAGE + t * NSTAGE + j * 16), nscale);
        *reinterpret_cast<uint32_t*>((t ? ring1 : ring0) + j * 4) = ncodes4;  // row 0
        if (j == 0) sbuf[0][t * C::ROUND_ROWS] = nscale;
      }
    } else {
      if (wave == 0 && lane < 2 * C::CPR) {
        nkv = *reinterpret_cast<const uint4*>(stage + QSTAGE + (lane < C::CPR ? 0 : NSTAGE) + (lane % C::CPR) * 16);
        *reinterpret_cast<uint4*>((lane < C::CPR ? ring0 : ring1) + (lane % C::CPR) * 16) = nkv;  // row 0: no swizzle
      }
    }
    lds_barrier();
    if (slot == 0) {
      if constexpr (MF && KV4) {
        mf4_scores(mst, ring0, qm, mqbias, &sbuf[0][0], &sbuf[0][C::ROUND_ROWS], 1, -1, lane, a.scale_log2);
        mf4_pv(mst, ring1, lane);
      } else if constexpr (MF && KV8) {
        mf8_scores(mst, ring0, qm, &sbuf[0][0], &sbuf[0][C::ROUND_ROWS], 1, -1, lane, a.scale_log2);
        mf8_pv(mst, ring1, lane);
      } else if constexpr (MF) {
        mf_scores(mst, ring0, qm, 1, -1, lane, a.scale_log2);
        mf_pv(mst, ring1, lane);
      } else if constexpr (SC4) {
        const bool r1 = tile_scores4<KT, D, G>(m4, l4, pbuf, abuf, ring0, q, 1, -1, r16, s4, a.scale_log2);
        tile_pv4<KT, D, G>(st, pbuf, abuf, r1, ring1, rg, s);
      } else {
        tile_scores<KT, D, G>(st, p, ring0, q, 1, -1, rg, s, a.scale_log2);
        tile_pv<KT, D, G>(st, p, ring1, rg, s);
      }
    }
    const int64_t slot_str = w.cnt < a.S ? w.cnt : a.S + (w.cnt - a.S) % a.W;
    if (room_for(a.lp, w.b, w.cnt, 1)) {
      const int64_t row = ret_head ? w.at(w.cnt) : slot_str;
      if constexpr (KV8) {
        if (wave == 0 && lane < 32) {
          const int t = lane >> 4, j = lane & 15;
          *reinterpret_cast<uint2*>((t ? w.vbase : w.kbase) + (size_t)row * C::ROWB + j * 8) = ncodes;
          if (j == 0) (t ? w.vsc : w.ksc)[row] = nscale;
        }
      } else if constexpr (KV4) {
        if (wave == 0 && lane < 32) {
          const int t = lane >> 4, j = lane & 15;
          *reinterpret_cast<uint32_t*>((t ? w.vbase : w.kbase) + (size_t)row * C::ROWB + j * 4) = ncodes4;
          if (j == 0) (t ? w.vsc : w.ksc)[row] = nscale;
        }
      } else {
        if (wave == 0 && lane < 2 * C::CPR) {
          char* dst = (lane < C::CPR ? w.kbase : w.vbase) + (size_t)row * C::ROWB + (lane % C::CPR) * 16;
          *reinterpret_cast<uint4*>(dst) = nkv;
        }
      }
      if (wave == 0 && lane == 0 && !ret_head) {
        const int64_t si = w.hh - (int64_t)a.B * a.n_ret;  // b * n_str + streaming index
        a.lp.pos[si * a.cap_str + slot_str] = (int32_t)w.cnt;
      }
    } else if (wave == 0 && lane == 0) {
      *a.lp.status = 1;
    }
  }

  if constexpr (MF) {
    // ---- merge the eight wavefronts' states through LDS (the ring is free):
    // query column j's accumulators X[wave][j][d], WPR wavefront blocks to a
    // ring unit (units 0-2), the (max, sum) pairs in ring unit 3.  A column
    // takes D + 16 floats: the 64-byte pad puts the columns a lane group
    // stores at once (16 t + 4 g of columns j) on different banks; at D
    // floats apart they all met on the same banks, eight-way.
    lds_barrier();  // every wavefront is done with the ring
    constexpr int NCOL = (SHARE || G > 8) ? 16 : G;  // columns per wavefront block of X
    constexpr int MS = SHARE ? 16 : G;               // columns per wavefront block of the (max, sum) pairs
    constexpr int CS = D + 16;                       // floats per column of X
    constexpr int XB = NCOL * CS * 4;                // bytes per wavefront block
    constexpr int WPR = kUnitBytes / XB;             // wavefront blocks per ring unit
    static_assert(WPR >= 1 && (kDecWaves + WPR - 1) / WPR <= 3, "X fits ring units 0-2");
    float* const xml = reinterpret_cast<float*>(ring3);
    // element e of column col of wavefront v (v wavefront-uniform, so the
    // ring unit is a scalar choice; a compile-time one in the merge loop)
    auto xat = [&](int v, int col, int e) -> float* {
      return reinterpret_cast<float*>(ring_at(v / WPR) + (v % WPR) * XB + (col * CS + e) * 4);
    };
    const int j = lane & 15, g = lane >> 4;
    const int ncol = SHARE ? w.qrows * G : G;  // query columns in use
    const float lsum = swap32_sum(swap16_sum(mst.l));  // the query's sum over its four lanes
    if constexpr (KV4) {  // the accumulators held the levels + 136: drop 136 times the weights' sum
      const float wb = swap32_sum(swap16_sum(mst.w)) * kInt4Bias;
#pragma unroll
      for (int t = 0; t < 8; ++t) mst.o[t] -= wb;
    }
    if (j < ncol) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
        *reinterpret_cast<float4*>(xat(wave, j, 16 * t + 4 * g)) =
            make_float4(mst.o[t][0], mst.o[t][1], mst.o[t][2], mst.o[t][3]);
      if (g == 0) {
        xml[wave * MS + j] = mst.m;
        xml[kDecWaves * MS + wave * MS + j] = lsum;
      }
    }
    lds_barrier();
    // four consecutive output elements per thread: query column h = e4 / D
    // (a shared item: row h / G of its group, query head h % G); every LDS
    // read of the thread is issued before the arithmetic that needs it
    for (int e4 = threadIdx.x * 4; e4 < ncol * D; e4 += kDecodeThreads * 4) {
      const int h = e4 / D, d = e4 % D;
      float mv[kDecWaves], lv[kDecWaves];
      float4 xv[kDecWaves];
#pragma unroll
      for (int v = 0; v < kDecWaves; ++v) {
        mv[v] = xml[v * MS + h];
        lv[v] = xml[kDecWaves * MS + v * MS + h];
        xv[v] = *reinterpret_cast<const float4*>(xat(v, h, d));
      }
      float M = -INFINITY;
#pragma unroll
      for (int v = 0; v < kDecWaves; ++v) M = fmaxf(M, mv[v]);
      float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
      float L = 0.f;
#pragma unroll
      for (int v = 0; v < kDecWaves; ++v) {
        const float wt = (mv[v] == -INFINITY) ? 0.f : fast_exp2(mv[v] - M);
        L = fmaf(lv[v], wt, L);
        A.x = fmaf(xv[v].x, wt, A.x);
        A.y = fmaf(xv[v].y, wt, A.y);
        A.z = fmaf(xv[v].z, wt, A.z);
        A.w = fmaf(xv[v].w, wt, A.w);
      }
      if (w.single) {
        const float inv = 1.f / L;
        uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + q_off + e4;
        o[0] = (uint16_t)f32_to_bf16_bits(A.x * inv);
        o[1] = (uint16_t)f32_to_bf16_bits(A.y * inv);
        o[2] = (uint16_t)f32_to_bf16_bits(A.z * inv);
        o[3] = (uint16_t)f32_to_bf16_bits(A.w * inv);
      } else {
        const int qi = h / G, hq = h % G;
        const size_t slot = w.shared ? (size_t)w.sh_rec + (size_t)qi * w.sh_stride : (size_t)blockIdx.x;
        float* rec = a.ws1 + slot * C::REC;
        *reinterpret_cast<float4*>(rec + hq * D + d) = A;
        if (d == 0) {
          rec[G * D + hq] = M;
          rec[G * D + G + hq] = L;
        }
      }
    }
  } else {
    // ---- merge the partials of the SLOTS x 8 row groups through LDS.  The ring
    // is free now; it holds every lane's accumulators as X[slot][rg][h][d]
    // (SLOTS * 8 * G * D floats <= 128 KB), split over the four ring arrays.
    constexpr int XB = kUnitBytes;  // bytes per ring array
    static_assert(SLOTS * 8 * G * D * 4 <= kRingUnits * XB, "partials fit the ring");
    lds_barrier();  // every wavefront is done with the ring
    if (active) {
  #pragma unroll
      for (int h = 0; h < HW; ++h) {
        const int hG = hg * HW + h;
  #pragma unroll
        for (int c2 = 0; c2 < C::CPL; ++c2) {
          const int off = ((((slot * 8 + rg) * G + hG) * D) + (c2 * 8 + s) * C::EPV) * 4;
          float* dst = reinterpret_cast<float*>(ring_at(off / XB) + off % XB);
  #pragma unroll
          for (int e = 0; e < C::EPV; e += 4)
            *reinterpret_cast<float4*>(dst + e) =
                make_float4(st.acc[h][c2 * C::EPV + e], st.acc[h][c2 * C::EPV + e + 1], st.acc[h][c2 * C::EPV + e + 2],
                            st.acc[h][c2 * C::EPV + e + 3]);
        }
        if constexpr (!SC4) {
          if (s == 0) {
            w_m[hG][slot * 8 + rg] = st.m[h];
            w_l[hG][slot * 8 + rg] = st.l[h];
          }
        }
      }
      if constexpr (SC4) {  // (rg, h) state: lanes (r16 = rg, s4) and (rg + 8, s4), s4 % HW = h
        const float l_pair = l4 + __shfl_xor(l4, 32);
        if (r16 < 8 && s4 < HW) {
          w_m[hg * HW + s4][slot * 8 + r16] = m4;
          w_l[hg * HW + s4][slot * 8 + r16] = l_pair;
        }
      }
    }
    __syncthreads();
    constexpr int NP = SLOTS * 8;  // partials per query head
    static_assert(NP * G <= kDecodeThreads && NP % 4 == 0, "one thread per (partial, head)");
    if (threadIdx.x < NP * G) {  // weight of partial i of head h in the merged result
      const int h = threadIdx.x / NP, i = threadIdx.x % NP;
      float M = -INFINITY;
  #pragma unroll
      for (int j = 0; j < NP; j += 4) {
        const float4 m4 = *reinterpret_cast<const float4*>(&w_m[h][j]);
        M = fmaxf(fmaxf(M, fmaxf(m4.x, m4.y)), fmaxf(m4.z, m4.w));
      }
      const float wt = (w_m[h][i] == -INFINITY) ? 0.f : fast_exp2(w_m[h][i] - M);
      w_w[h][i] = wt;
      w_lw[h][i] = w_l[h][i] * wt;
      if (i == 0) w_mt[h] = M;
    }
    __syncthreads();
    // four consecutive output elements per thread
    float* rec = a.ws1 + (size_t)blockIdx.x * C::REC;
    for (int e4 = threadIdx.x * 4; e4 < G * D; e4 += kDecodeThreads * 4) {
      const int h = e4 / D, d = e4 % D;
      float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
      float L = 0.f;
  #pragma unroll
      for (int i0 = 0; i0 < NP; i0 += 4) {
        const float4 wt4 = *reinterpret_cast<const float4*>(&w_w[h][i0]);
        const float4 lw4 = *reinterpret_cast<const float4*>(&w_lw[h][i0]);
        L += (lw4.x + lw4.y) + (lw4.z + lw4.w);
        const float wv[4] = {wt4.x, wt4.y, wt4.z, wt4.w};
  #pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int off = (((i0 + k) * G + h) * D + d) * 4;
          const float4 x = *reinterpret_cast<const float4*>(ring_at(off / XB) + off % XB);
          A.x = fmaf(x.x, wv[k], A.x);
          A.y = fmaf(x.y, wv[k], A.y);
          A.z = fmaf(x.z, wv[k], A.z);
          A.w = fmaf(x.w, wv[k], A.w);
        }
      }
      if (w.single) {
        const float inv = 1.f / L;
        if (BF16) {
          uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + q_off + e4;
          o[0] = (uint16_t)f32_to_bf16_bits(A.x * inv);
          o[1] = (uint16_t)f32_to_bf16_bits(A.y * inv);
          o[2] = (uint16_t)f32_to_bf16_bits(A.z * inv);
          o[3] = (uint16_t)f32_to_bf16_bits(A.w * inv);
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + q_off + e4) =
              make_float4(A.x * inv, A.y * inv, A.z * inv, A.w * inv);
        }
      } else {
        *reinterpret_cast<float4*>(rec + e4) = A;
        if (d == 0) {
          rec[G * D + h] = w_mt[h];
          rec[G * D + G + h] = L;
        }
      }
    }
  }
}

// Merges the partial records of every head that spans several work items.
// Workgroup = (flat head, query head, 32 output elements); its 512 threads are
// 16 record groups x 32 elements, each thread folding every 16th record.
constexpr int kCombineElems = 32;
constexpr int kCombineGroups = kDecodeThreads / kCombineElems;  // 16

template <int KT, int D, int G, bool SH>
__global__ __launch_bounds__(kDecodeThreads) void combine_kernel(DecodeArgs a) {
  using C = DecodeCfg<KT, D, G>;
  [[maybe_unused]] constexpr bool BF16 = C::BF16;
  constexpr int DC = D / kCombineElems;
  __shared__ float c_m[kCombineGroups][kCombineElems], c_l[kCombineGroups][kCombineElems],
      c_a[kCombineGroups][kCombineElems];
  const int64_t n_heads = (int64_t)a.B * (a.n_ret + a.n_str);
  if ((int64_t)blockIdx.x >= n_heads * G * DC) {
    // the launch's extra last workgroup (fused appends only): the step is
    // done, so every row advances by its new token if it had room (the
    // decode kernel, which read the counts, has finished).  A workgroup of
    // its own, so that its two dependent loads do not delay a merge.
    if (threadIdx.x < a.B) {
      const int b = threadIdx.x;
      const int32_t cnt = a.lp.len[b];
      if (room_for(a.lp, b, cnt, 1)) a.lp.len[b] = cnt + 1;
    }
    return;
  }
  const int64_t hh = blockIdx.x / (G * DC);
  const int h = (int)((blockIdx.x / DC) % G);
  const int dcn = (int)(blockIdx.x % DC);
  const int64_t n_ret_heads = (int64_t)a.B * a.n_ret;
  int64_t first;
  int n_seg, b, kvh;
  int n_all;                       // the head's records: its own items', then its shared items'
  const float* rec_sh = nullptr;   // the first shared item's record for this row and head
  if (hh < n_ret_heads) {
    b = (int)(hh / a.n_ret);
    const int r = (int)(hh % a.n_ret);
    first = a.rows[b].first_ret + (int64_t)r * a.rows[b].nb_ret;
    n_seg = a.rows[b].nb_ret;
    kvh = arg_byte(a.map.orig_ret, r);
    n_all = n_seg;
    if (SH && a.rsh[b].sh_rows > 0) {
      rec_sh = a.ws1 + ((size_t)a.rsh[b].sh_rec + (size_t)r * a.rsh[b].sh_nb) * C::REC;
      n_all += a.rsh[b].sh_nb;
    }
  } else {
    const int64_t x = hh - n_ret_heads;
    b = (int)(x / a.n_str);
    const int si = (int)(x % a.n_str);
    first = a.rows[b].first_str + (int64_t)si * a.rows[b].nb_str;
    n_seg = a.rows[b].nb_str;
    kvh = arg_byte(a.map.orig_str, si);
    n_all = n_seg;
  }
  if (n_all == 1) return;  // written by the decode kernel
  const float* rec0 = a.ws1 + (size_t)first * C::REC;
  auto rec_at = [&](int i) { return i < n_seg ? rec0 + (size_t)i * C::REC : rec_sh + (size_t)(i - n_seg) * C::REC; };
  const int el = threadIdx.x % kCombineElems, grp = threadIdx.x / kCombineElems;
  const int e = h * D + dcn * kCombineElems + el;
  float M = -INFINITY, L = 0.f, A = 0.f;
  constexpr int NB = 8;  // records per batch, loads issued together
  for (int i0 = grp; i0 < n_all; i0 += NB * kCombineGroups) {
    float mv[NB], lv[NB], av[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int i = i0 + j * kCombineGroups;
      const float* r = rec_at(i < n_all ? i : i0);
      mv[j] = i < n_all ? r[G * D + h] : -INFINITY;
      lv[j] = r[G * D + G + h];
      av[j] = r[e];
    }
    float Mb = M;
#pragma unroll
    for (int j = 0; j < NB; ++j) Mb = fmaxf(Mb, mv[j]);
    const float f = (M == -INFINITY) ? 0.f : fast_exp2(M - Mb);
    L *= f;
    A *= f;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float w = (mv[j] == -INFINITY) ? 0.f : fast_exp2(mv[j] - Mb);
      L += lv[j] * w;
      A += av[j] * w;
    }
    M = Mb;
  }
  c_m[grp][el] = M;
  c_l[grp][el] = L;
  c_a[grp][el] = A;
  __syncthreads();
  if (grp != 0) return;
  // every group's (max, sum, accumulator) read before the arithmetic
  float gm[kCombineGroups], gl[kCombineGroups], ga[kCombineGroups];
#pragma unroll
  for (int k = 0; k < kCombineGroups; ++k) {
    gm[k] = c_m[k][el];
    gl[k] = c_l[k][el];
    ga[k] = c_a[k][el];
  }
  float Mt = -INFINITY;
#pragma unroll
  for (int k = 0; k < kCombineGroups; ++k) Mt = fmaxf(Mt, gm[k]);
  float Lt = 0.f, At = 0.f;
#pragma unroll
  for (int k = 0; k < kCombineGroups; ++k) {
    const float w = (gm[k] == -INFINITY) ? 0.f : fast_exp2(gm[k] - Mt);
    Lt += gl[k] * w;
    At += ga[k] * w;
  }
  const size_t o = ((size_t)b * a.n_q + (size_t)kvh * G) * D + e;
  if (BF16) reinterpret_cast<uint16_t*>(a.out)[o] = (uint16_t)f32_to_bf16_bits(At / Lt);
  else reinterpret_cast<float*>(a.out)[o] = At / Lt;
}

template <int KT, int D, int G, bool SH>
hipError_t launch_decode_sh(const DecodeArgs& a, int blocks, hipStream_t s) {
  decode_kernel<KT, D, G, SH><<<blocks, kDecodeThreads, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!a.multi) {  // every head finished in one item; a fused append's counts still advance
    if (a.new_k == nullptr) return hipSuccess;
    AdvanceArgs v{};
    v.lp = a.lp;
    v.B = a.B;
    v.n = 1;
    return launch_advance(v, s);
  }
  const int64_t heads = (int64_t)a.B * (a.n_ret + a.n_str);
  const int64_t extra = a.new_k != nullptr ? 1 : 0;  // the workgroup that advances a fused append's counts
  combine_kernel<KT, D, G, SH><<<(unsigned)(heads * G * (D / kCombineElems) + extra), kDecodeThreads, 0, s>>>(a);
  return hipGetLastError();
}

template <int KT, int D, int G>
hipError_t launch_decode_g(const DecodeArgs& a, int blocks, hipStream_t s) {
  // plans with share groups exist only at d = 128, bf16 queries, g = 4 or 8
  if constexpr (DecodeCfg<KT, D, G>::MF && (G == 4 || G == 8)) {
    if (a.n_share > 0) return launch_decode_sh<KT, D, G, true>(a, blocks, s);
  }
  return launch_decode_sh<KT, D, G, false>(a, blocks, s);
}

// Group sizes built: 1 .. 16 on the matrix cores (bf16, FP8 and INT4 rows
// at d = 128), 1 .. 8 on the vector ALU (fp32 rows, d = 64).
template <int KT, int D>
constexpr int max_group() { return DecodeCfg<KT, D, 1>::MF ? 16 : 8; }

template <int KT, int D, int G = 1>
hipError_t launch_decode_d(const DecodeArgs& a, int g, int blocks, hipStream_t s) {
  if constexpr (G > max_group<KT, D>()) {
    return hipErrorInvalidValue;
  } else {
    if (g == G) return launch_decode_g<KT, D, G>(a, blocks, s);
    return launch_decode_d<KT, D, G + 1>(a, g, blocks, s);
  }
}

template <int KT, int D, int G = 1>
int64_t round_rows_d(int g) {
  if constexpr (G > max_group<KT, D>()) {
    return 0;
  } else {
    if (g == G) return DecodeCfg<KT, D, G>::ROUND_ROWS;
    return round_rows_d<KT, D, G + 1>(g);
  }
}

}  // namespace

// Partial records of duo_decode_append_noalloc.  In host code `scratch` only
// names the variable; its device address comes from hipGetSymbolAddress, once
// per device (each device holds its own copy), and only that address is
// passed to kernels.
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_table_update(const TableUpdateArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  table_update_kernel<<<1, kMaxTableUpdates, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_rope(const RopeArgs& a, hipStream_t s) {
  const int64_t pairs = (int64_t)a.B * (a.n_q + a.n_kv) * a.C * (a.d / 2);
  if (pairs == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((pairs + 255) / 256, 8192);
  rope_kernel<<<(unsigned)blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_copy(const CopyArgs& a, hipStream_t s) {
  int64_t words = 0;
  for (int i = 0; i < a.n; ++i) words += a.seg[i].bytes / 4 * a.seg[i].count;
  if (words == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((words + 255) / 256, 2048);
  copy_kernel<<<(unsigned)blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

namespace {
hipError_t launch_fill(void* p, size_t bytes, uint32_t word, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16, ntail = bytes % 16;
  const int threads = 256;
  size_t want = (n16 + threads - 1) / threads;
  const int grid = (int)std::max<size_t>(1, std::min<size_t>(want, 4096));
  fill_kernel<<<grid, threads, 0, s>>>(reinterpret_cast<uint4*>(p), n16,
                                       reinterpret_cast<unsigned char*>(p) + n16 * 16, ntail, word);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) { return launch_fill(p, bytes, 0u, s); }
hipError_t launch_fill_ones(void* p, size_t bytes, hipStream_t s) { return launch_fill(p, bytes, 0xffffffffu, s); }

hipError_t launch_advance(const AdvanceArgs& a, hipStream_t s) {
  advance_kernel<<<1, kMaxRows, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, int dtype, int d, int kvfmt, hipStream_t s) {
  (void)dtype;
  (void)d;
  if (kvfmt != 0) {
    const int64_t threads = (int64_t)a.B * a.n_kv * a.n_new * 2 * 16;
    const int64_t grid = (threads + 255) / 256;
    if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
    if (kvfmt == 2) {
      if (a.rope.on) append_lowbit_kernel<true, true><<<(unsigned)grid, 256, 0, s>>>(a);
      else append_lowbit_kernel<true, false><<<(unsigned)grid, 256, 0, s>>>(a);
    } else {
      if (a.rope.on) append_lowbit_kernel<false, true><<<(unsigned)grid, 256, 0, s>>>(a);
      else append_lowbit_kernel<false, false><<<(unsigned)grid, 256, 0, s>>>(a);
    }
    return hipGetLastError();
  }
  const int64_t total = (int64_t)a.B * a.n_kv * a.n_new * (a.row_bytes / 16);
  const int threads = 256;
  const int64_t want = (total + threads - 1) / threads;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(want, 65536));
  if (a.rope.on) append_kernel<true><<<grid, threads, 0, s>>>(a);
  else append_kernel<false><<<grid, threads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_dequant(const DequantArgs& a, hipStream_t s) {
  const int64_t total = (a.heads_ret * a.rows_ret + a.heads_str * a.rows_str) * 2 * (a.d / 8);
  if (total == 0) return hipSuccess;
  const int64_t want = (total + 255) / 256;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(want, 65536));
  dequant_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

int64_t decode_round_rows(int dtype, int d, int g, int kvfmt) {
  if (kvfmt == 2) return round_rows_d<3, 128>(g);
  if (kvfmt == 1) return round_rows_d<2, 128>(g);
  if (dtype == 1) return d == 128 ? round_rows_d<1, 128>(g) : round_rows_d<1, 64>(g);
  return d == 128 ? round_rows_d<0, 128>(g) : round_rows_d<0, 64>(g);
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int d, int g, int kvfmt, int blocks, hipStream_t s) {
  if (kvfmt != 0) {
    if (dtype != 1 || d != 128) return hipErrorInvalidValue;
    return kvfmt == 2 ? launch_decode_d<3, 128>(a, g, blocks, s) : launch_decode_d<2, 128>(a, g, blocks, s);
  }
  if (dtype == 1) {
    if (d == 128) return launch_decode_d<1, 128>(a, g, blocks, s);
    if (d == 64) return launch_decode_d<1, 64>(a, g, blocks, s);
  } else {
    if (d == 128) return launch_decode_d<0, 128>(a, g, blocks, s);
    if (d == 64) return launch_decode_d<0, 64>(a, g, blocks, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace duo
