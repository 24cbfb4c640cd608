// HIP kernels for gfx950 (CDNA4): cache fill, append and split-K decode over a
// per-KV-head mixed KV cache (DuoAttention: retrieval heads hold every token,
// streaming heads hold S sinks + a W-slot ring).
//
// Decode is bound by HBM bandwidth (g = n_q / n_kv flops per byte of K/V), so
// it runs on the vector ALUs, not on MFMA.  The rows held by every (batch, KV
// head) -- all T rows of a retrieval head, the min(T, S+W) sink and ring slots
// of a streaming head -- form one flattened row space cut into equal work
// items, one per compute unit, so long retrieval heads and short streaming
// heads are balanced by bytes.  Within an item, K and V rows reach LDS by
// direct buffer->LDS loads into a ring of four 32 KB units (three in flight);
// the wavefronts score them with packed bf16 dot products against the GQA
// query group held in registers, keep online softmax statistics per lane, and
// accumulate P.V with bf16 dot products.  Partial (max, sum, acc) results of
// items that share a head are merged by a second kernel (combine_kernel).
// Retrieval rows may live in pages (a per-row page table); a paged head's
// items then start at round boundaries so that every round lies in one page.
#include "duo_internal.h"
#include "duo_rope.h"
#include "duo_rows.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
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

__global__ void fill_zero_kernel(uint4* p, size_t n16, unsigned char* tail, size_t ntail) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t j = i; j < n16; j += stride) p[j] = make_uint4(0, 0, 0, 0);
  if (i < ntail) tail[i] = 0;
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
      rope_cs(r, d, p, c * 8 + 2 * w, c0, s0);
      rope_cs(r, d, p, c * 8 + 2 * w + 1, c1, s1);
      const double x0 = bf_lo(xw[w]), x1 = bf_hi(xw[w]), y0 = bf_lo(yw[w]), y1 = bf_hi(yw[w]);
      xw[w] = bf16_bits_from_double(x0 * c0 - y0 * s0) | (bf16_bits_from_double(x1 * c1 - y1 * s1) << 16);
      yw[w] = bf16_bits_from_double(y0 * c0 + x0 * s0) | (bf16_bits_from_double(y1 * c1 + x1 * s1) << 16);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      double cs, sn;
      rope_cs(r, d, p, c * 4 + w, cs, sn);
      const double xv = __uint_as_float(xw[w]), yv = __uint_as_float(yw[w]);
      xw[w] = __float_as_uint((float)(xv * cs - yv * sn));
      yw[w] = __float_as_uint((float)(yv * cs + xv * sn));
    }
  }
  x = make_uint4(xw[0], xw[1], xw[2], xw[3]);
  y = make_uint4(yw[0], yw[1], yw[2], yw[3]);
}

__global__ void append_kernel(AppendArgs a) {
  const int cpr = a.row_bytes / 16;
  // work per row: its 16-byte chunks, or with rotary positions its chunk
  // pairs (c, c + cpr/2), which hold the rotation's dimension pairs
  const int units = a.rope.on ? cpr / 2 : cpr;
  const int64_t total = (int64_t)a.B * a.n_kv * a.n_new * units;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total; idx += stride) {
    const int c = (int)(idx % units);
    const int64_t rest = idx / units;  // input row (b, kvh, i)
    const int64_t i = rest % a.n_new;
    const int kvh = (int)((rest / a.n_new) % a.n_kv);
    const int b = (int)(rest / a.n_new / a.n_kv);
    const int64_t p = a.p0[b] + i;
    const int64_t keep_from = max64d((int64_t)a.S, (int64_t)a.p0[b] + a.n_new - a.W);
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
    if (!a.rope.on) {
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
    rope_cs(a.rope, a.d, a.p0[b] + ci, i, cs, sn);
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

// One wavefront-wide direct buffer->LDS load of 16 bytes per lane: lane i
// writes LDS bytes [lds + 16 i, lds + 16 i + 16) from byte offset voff of the
// buffer resource; offsets out of the resource's range read as zero.
//
// Written as inline assembly on purpose: the load has no register result
// (its data goes to LDS), and the compiler, not knowing that it writes LDS,
// adds no wait of its own before later LDS reads.  Every read of a unit is
// ordered after its loads by an explicit vmcnt wait and a barrier (see
// wait_vmcnt / lds_barrier), which keeps three units in flight; the compiler's
// own analysis would wait for all of them.  The "memory" clobber stops the
// compiler from assuming LDS contents across the load.  M0 (the LDS base of
// the load) is saved and restored.
typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4_t dec_rsrc(const char* base, int nbytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return i32x4_t{(int)__builtin_amdgcn_readfirstlane((uint32_t)b),
                 (int)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xffffu),  // stride 0
                 __builtin_amdgcn_readfirstlane(nbytes), 0x00020000};                 // raw buffer
}

__device__ __forceinline__ void dec_dma(i32x4_t rsrc, char* lds, uint32_t voff) {
  const uint32_t m0v =
      __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(__attribute__((address_space(3))) char*)lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0v), "v"(voff), "s"(rsrc)
      : "memory");
}

// The same with 4 bytes per lane: lane i writes LDS bytes [lds + 4 i, lds + 4 i + 4).
__device__ __forceinline__ void dec_dma4(i32x4_t rsrc, char* lds, uint32_t voff) {
  const uint32_t m0v =
      __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(__attribute__((address_space(3))) char*)lds);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0v), "v"(voff), "s"(rsrc)
      : "memory");
}

// ------------------------------------------------------------------ decode
//
// One workgroup of 8 wavefronts per compute unit walks a contiguous range of
// the flattened row space.  K and V rows reach LDS through direct buffer->LDS
// loads into a ring of four 32 KB units (the K rows, then the V rows, of one
// round of tiles); three units are in flight while one is consumed, so the
// prefetch depth costs no registers.  A round is SLOTS tiles of TR rows; the
// wavefronts of a slot split the g query heads (HW heads each) and read the
// slot's tile from LDS, so no row is fetched twice.  Rounds never straddle two
// heads: a range that covers parts of several heads is a sequence of
// segments, and at the end of each segment the wavefronts' softmax states are
// merged into one partial (max, sum, acc) per query head.  A segment that is a
// whole head writes the output; otherwise its partial goes to the workspace
// and the combine kernel merges the partials of the head.
//
// Lane layout within a tile: 8 lanes share a row.  Lane l has row group
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
// outputs with FP8 (E4M3) K/V rows in the cache plus one fp32 scale per row.
template <int KT, int D, int G>
struct DecodeCfg {
  static constexpr bool BF16 = KT != 0;          // queries, inputs, outputs in bf16
  static constexpr bool KV8 = KT == 2;           // K/V rows stored as FP8 codes + row scales
  static constexpr int ES = BF16 ? 2 : 4;        // query / input / output element bytes
  static constexpr int IROWB = D * ES;           // bytes per query or input row
  static constexpr int KES = KV8 ? 1 : ES;       // stored K/V element bytes
  static constexpr int ROWB = D * KES;           // bytes per stored K/V row
  static constexpr int CPR = ROWB / 16;          // 16-byte chunks per stored row
  static constexpr int CPL = CPR / 8;            // chunks per lane
  static constexpr int EPC = 16 / KES;           // elements per chunk
  static constexpr int HW = G < 4 ? G : 4;       // query heads per wavefront
  static constexpr int HSPLIT = G / HW;          // wavefronts per slot
  static constexpr int SLOTS_W = kDecWaves / HSPLIT;
  static constexpr int SLOTS_B = kUnitBytes / (16 * ROWB);  // keeps TR >= 16
  static constexpr int SLOTS = SLOTS_W < SLOTS_B ? SLOTS_W : SLOTS_B;
  static constexpr int TR = kUnitBytes / (SLOTS * ROWB);    // rows per tile
  static constexpr int RPL = TR / 8;             // rows per lane
  static constexpr int SLOT_BYTES = TR * ROWB;
  static constexpr int ROUND_ROWS = SLOTS * TR;
  static constexpr int NACC = CPL * EPC;         // output elements per lane per head
  static constexpr int REC = (G * (D + 2) + 3) / 4 * 4;  // floats per partial record (16-byte multiple)
  static_assert(CPR % 8 == 0, "rows must span a multiple of 8 chunks");
  static_assert(RPL >= 2 && RPL % 2 == 0, "rows are paired for the weighted sum");
  static_assert(SLOT_BYTES % 1024 == 0, "a load piece stays within one tile");
  static_assert(G % HW == 0, "head split must tile the group");
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

// Append to an FP8 cache: one group of 16 lanes per (batch row, KV head,
// token, K or V) row, each lane taking 8 consecutive bf16 values.  Slot rules
// as append_kernel.
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
    rope_cs(r, 128, p, 8 * (j & 7) + 2 * k, cs0, sn0);
    rope_cs(r, 128, p, 8 * (j & 7) + 2 * k + 1, cs1, sn1);
    const double a0 = bf_lo(w[k]), a1 = bf_hi(w[k]), b0 = bf_lo(q), b1 = bf_hi(q);
    const double v0 = first ? a0 * cs0 - b0 * sn0 : a0 * cs0 + b0 * sn0;
    const double v1 = first ? a1 * cs1 - b1 * sn1 : a1 * cs1 + b1 * sn1;
    o[k] = bf16_bits_from_double(v0) | (bf16_bits_from_double(v1) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

__global__ void append_fp8_kernel(AppendArgs a) {
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
  const int64_t p = a.p0[b] + i;
  const int64_t keep_from = max64d((int64_t)a.S, (int64_t)a.p0[b] + a.n_new - a.W);
  const size_t src = (((size_t)b * a.n_kv + kvh) * a.n_new + i) * a.in_row_bytes + (size_t)j * 16;
  float sc;
  uint4 x = ld16((tensor ? a.v : a.k) + src);
  if (a.rope.on && tensor == 0) x = rope_row16(x, a.rope, p, j);  // the whole group takes this branch
  const uint2 codes = quant_row16(x, sc);
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
  *reinterpret_cast<uint2*>(dst + j * 8) = codes;
  if (j == 0) *sdst = sc;
}

// FP8 rows -> bf16 rows (code value times the row scale, rounded to nearest
// even), 8 values per thread.
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
      codes = reinterpret_cast<const uint8_t*>(tensor ? a.src.v_ret : a.src.k_ret) + srow * a.d;
      sc = (tensor ? a.src.vsc_ret : a.src.ksc_ret) + srow;
      dst = reinterpret_cast<uint16_t*>(tensor ? a.dst.v_ret : a.dst.k_ret) + drow * a.d;
    } else {
      rr -= n_ret;
      const int64_t h = rr / a.rows_str, r = rr % a.rows_str;
      const int64_t row = h * a.cap_str + r;
      codes = reinterpret_cast<const uint8_t*>(tensor ? a.src.v_str : a.src.k_str) + row * a.d;
      sc = (tensor ? a.src.vsc_str : a.src.ksc_str) + row;
      dst = reinterpret_cast<uint16_t*>(tensor ? a.dst.v_str : a.dst.k_str) + row * a.d;
    }
    const uint2 c8 = *reinterpret_cast<const uint2*>(codes + pc * 8);
    const float s = *sc;
    const uint32_t cw[2] = {c8.x, c8.y};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[k], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[k], true);
      o[2 * k] = f32_to_bf16_bits(lo[0] * s) | (f32_to_bf16_bits(lo[1] * s) << 16);
      o[2 * k + 1] = f32_to_bf16_bits(hi[0] * s) | (f32_to_bf16_bits(hi[1] * s) << 16);
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
  int part, nparts;
  int b, kvh;
  int row;          // batch row (index into DecodeArgs::rows)
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

template <int ROWB, int RR>
__device__ __forceinline__ DecodeItem decode_item(const DecodeArgs& a, int64_t blk) {
  DecodeItem w;
  w.ptab = nullptr;
  w.shift = 0;
  w.pstride = 0;
  int64_t rows;
  if (blk < a.items_ret) {
    int b = 0;
    while (b + 1 < a.B && blk >= a.rows[b + 1].first_ret) ++b;  // batch row of the item (uniform)
    const DecodeRow& R = a.rows[b];
    const int64_t rel = blk - R.first_ret;
    const int r = (int)(rel / R.nb_ret);
    w.part = (int)(rel % R.nb_ret);
    w.nparts = R.nb_ret;
    rows = R.rows_ret;
    w.row = b;
    w.b = b;
    w.hh = (int64_t)b * a.n_ret + r;
    w.kvh = a.map.orig_ret[r];
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
    const int64_t rel = blk - R.first_str;
    const int si = (int)(rel / R.nb_str);
    w.part = (int)(rel % R.nb_str);
    w.nparts = R.nb_str;
    rows = R.rows_str;
    w.row = b;
    w.b = b;
    w.hh = (int64_t)a.B * a.n_ret + (int64_t)b * a.n_str + si;
    w.kvh = a.map.orig_str[si];
    const size_t off = ((size_t)b * a.n_str + si) * a.cap_str * ROWB;
    w.kbase = a.lp.k_str + off;
    w.vbase = a.lp.v_str + off;
    const size_t srow = ((size_t)b * a.n_str + si) * a.cap_str;
    w.ksc = a.lp.ksc_str ? a.lp.ksc_str + srow : nullptr;
    w.vsc = a.lp.vsc_str ? a.lp.vsc_str + srow : nullptr;
  }
  int64_t per = (rows + w.nparts - 1) / w.nparts;
  if (w.ptab) per = (per + RR - 1) / RR * RR;  // paged: every round of rows lies in one page
  w.r0 = w.part * per;
  w.r1 = w.r0 + per < rows ? w.r0 + per : rows;
  if (w.r0 > rows) w.r0 = rows;
  return w;
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
  static constexpr bool ON = C::BF16;
  static constexpr int HW = C::HW;
  static constexpr int CPL4 = C::CPR / 4;   // chunks per lane
  static constexpr int RPL4 = C::TR / 16;   // rows per lane
  static constexpr int NQ = C::RPL / 2;     // row pairs per weighted-sum lane
  static constexpr int PBUF = 8 * NQ * HW;  // probability pairs per wavefront (dwords)
  static constexpr int QPC = C::EPC >= 8 ? C::EPC / 8 : 1;  // 16-byte query pieces per stored chunk (FP8 rows: 2)
  static_assert(4 % HW == 0, "heads per wavefront divide the 4 lanes of a row");
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
__device__ __forceinline__ int dec_swz_k4(int r) { return CPR >= 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

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
                                                             [Score4<KT, D, G>::CPL4 * Score4<KT, D, G>::QPC],
                                             const float* ksc, const float* vsc, int nv, int excl, int r16, int s4,
                                             float scale_log2) {
  using C = DecodeCfg<KT, D, G>;
  [[maybe_unused]] constexpr bool BF16 = C::BF16;
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
      if constexpr (C::KV8) {
        // 16 codes -> 8 bf16 pairs (exact), dotted with the query's values
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t kb[2] = {fp8x2_bf16<false>(kw[i]), fp8x2_bf16<true>(kw[i])};
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int h = 0; h < HW; ++h) {
              const uint4 qv = q[h][2 * cc + i / 2];
              const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
              acc[h] = dot2_bf16(qw[(2 * i + t) % 4], kb[t], acc[h]);
            }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int h = 0; h < HW; ++h) {
            const uint32_t qw[4] = {q[h][cc].x, q[h][cc].y, q[h][cc].z, q[h][cc].w};
            acc[h] = dot2_bf16(qw[i], kw[i], acc[h]);
          }
      }
    }
#pragma unroll
    for (int h = 0; h < HW; ++h) acc[h] = row4_sum(acc[h]);
    float own = acc[0];
#pragma unroll
    for (int h = 1; h < HW; ++h) own = hown == h ? acc[h] : own;
    if constexpr (C::KV8) own *= ksc[row];  // the K row's scale
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
    l += pj;
    // FP8 rows: the V row's scale joins the probability the weighted sum uses
    const float pw = C::KV8 ? pj * vsc[r16 + 16 * j] : pj;
    if (s4 < HW) pbuf[((rg * S4::NQ + j) * HW + s4) * 2 + half] = bf16_bits(pw);
  }
  return any;
}

// acc += sum over the lane's rows of p * V[row], with the probability pairs
// and rescale factors from tile_scores4.
template <int KT, int D, int G>
__device__ __forceinline__ void tile_pv4(DecodeState<KT, D, G>& st, const uint16_t* pbuf, const float* abuf,
                                         bool rescale, const char* vt, int rg, int s) {
  using C = DecodeCfg<KT, D, G>;
  [[maybe_unused]] constexpr bool BF16 = C::BF16;
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
        if constexpr (C::KV8) {
          // codes of d = 4i .. 4i+3 of the two rows, interleaved by row, then
          // converted to the (row0, row1) bf16 pairs the dot products take
          const uint32_t x0 = __builtin_amdgcn_perm(b4[i], a4[i], 0x05010400u);  // d = 4i, 4i+1
          const uint32_t x1 = __builtin_amdgcn_perm(b4[i], a4[i], 0x07030602u);  // d = 4i+2, 4i+3
          const uint32_t pr[4] = {fp8x2_bf16<false>(x0), fp8x2_bf16<true>(x0), fp8x2_bf16<false>(x1),
                                  fp8x2_bf16<true>(x1)};
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int h = 0; h < HW; ++h)
              st.acc[h][cc * 16 + 4 * i + t] = dot2_bf16(P[h], pr[t], st.acc[h][cc * 16 + 4 * i + t]);
        } else {
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
}

template <int X>
using UnitTag = std::integral_constant<int, X>;

template <int KT, int D, int G>
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
  // the group's queries and the new token's K and V rows, loaded by direct loads
  constexpr int QSTAGE = (G * C::IROWB + 1023) / 1024 * 1024;
  constexpr int NSTAGE = (C::IROWB + 1023) / 1024 * 1024;
  static_assert(QSTAGE / 1024 + 2 <= kDecWaves, "one staging piece per wavefront");
  __shared__ __attribute__((aligned(1024))) char stage[QSTAGE + 2 * NSTAGE];
  using S4 = Score4<KT, D, G>;
  constexpr bool SC4 = S4::ON;
  // four-lane score layout: per-wavefront probability pairs and rescale factors
  __shared__ __attribute__((aligned(16))) uint16_t pbuf_all[SC4 ? kDecWaves : 1][SC4 ? 2 * S4::PBUF : 8];
  __shared__ __attribute__((aligned(16))) float abuf_all[SC4 ? kDecWaves : 1][32];
  // FP8 rows: the K scales, then the V scales, of the rows of a round; one
  // buffer per K unit of the ring (units 0 and 2), loaded with that unit
  constexpr bool KV8 = C::KV8;
  __shared__ __attribute__((aligned(16))) float sbuf[KV8 ? 2 : 1][KV8 ? 2 * C::ROUND_ROWS : 4];
  static_assert(!KV8 || C::ROUND_ROWS == 4 * 64, "a round's scales are 4 wavefront loads per tensor");
  // vector-memory loads per unit and wavefront: the ring pieces, plus one
  // scale load with each K unit of FP8 rows; units u+1 and u+2 hold WAITN
  constexpr int WAITN = 2 * kPiecesPerWave + (KV8 ? 1 : 0);
  char* const rings[kRingUnits] = {ring0, ring1, ring2, ring3};  // indexed by constants only
  auto ring_at = [&](int i) -> char* { return i == 0 ? ring0 : i == 1 ? ring1 : i == 2 ? ring2 : ring3; };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = wave / C::HSPLIT;   // tile of the round this wavefront reads
  const int hg = wave % C::HSPLIT;     // which HW query heads of the group it scores
  const bool active = slot < SLOTS;
  const int rg = lane >> 3, s = lane & 7;
  const DecodeItem w = decode_item<C::ROWB, C::ROUND_ROWS>(a, blockIdx.x);
  const int64_t nrounds = ((w.r1 - w.r0 + TR - 1) / TR + SLOTS - 1) / SLOTS;
  const size_t q_off = ((size_t)w.b * a.n_q + (size_t)w.kvh * G) * D;  // first query of the group

  // fused append: the last item of every head adds the new token
  const bool add_new = a.new_k != nullptr && w.part == w.nparts - 1;
  const bool ret_head = w.hh < (int64_t)a.B * a.n_ret;
  // streaming slot masked in the held rows (its token is evicted by the new one)
  const int64_t excl_row = (a.new_k != nullptr && !ret_head) ? a.rows[w.row].excl_str : -1;
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
    const int ck = c ^ (SC4 ? dec_swz_k4<C::CPR>(r % TR) : dec_swz<C::CPR>(r % TR));
    poff_k[j] = (uint32_t)(r * C::ROWB + ck * 16);
    poff_v[j] = (uint32_t)(r * C::ROWB + (c ^ dec_swz<C::CPR>(r % TR)) * 16);
  }
  static_assert(TR % 4 == 0, "tiles start at a multiple of 4 rows");

  // Issue unit `uu` (round uu / 2; K rows if uu is even, else V rows) into
  // `dst`: the round's rows are contiguous, so one buffer resource covers
  // them, sized to the rows the item still has.  Past the item's end every
  // piece is out of range (it reads nothing and writes zeros to LDS) but is
  // still issued, so each wavefront has the same number of loads per unit,
  // and every byte of a unit is written before it is read.
  auto issue = [&](int64_t uu, char* dst) {
    const int64_t row0 = w.r0 + (uu >> 1) * (int64_t)C::ROUND_ROWS;
    const int64_t left = w.r1 - row0;
    const int rows = (int)(left <= 0 ? 0 : (left > C::ROUND_ROWS ? C::ROUND_ROWS : left));
    const int64_t roff = rows > 0 ? w.at(row0) : 0;
    const char* src = ((uu & 1) ? w.vbase : w.kbase) + (size_t)roff * C::ROWB;
    const i32x4_t rs = dec_rsrc(src, rows * C::ROWB);
#pragma unroll
    for (int j = 0; j < kPiecesPerWave; ++j)
      dec_dma(rs, dst + (wave + kDecWaves * j) * 1024, (uu & 1) ? poff_v[j] : poff_k[j]);
    if constexpr (KV8) {
      if ((uu & 1) == 0) {  // wavefronts 0-3: K scales, 4-7: V scales, 64 rows each
        const int tensor = wave >> 2, part = wave & 3;
        const float* ssrc = (tensor ? w.vsc : w.ksc) + roff;
        dec_dma4(dec_rsrc(reinterpret_cast<const char*>(ssrc), rows * 4),
                 reinterpret_cast<char*>(&sbuf[(uu >> 1) & 1][tensor * C::ROUND_ROWS + part * 64]),
                 (uint32_t)((part * 64 + lane) * 4));
      }
    }
  };
  // The first unit, then the group's queries and the new token's K and V rows
  // into the staging area (one load piece per wavefront for the first
  // wavefronts), then two more units.  Unit 0's wait below covers the staging
  // loads, which were issued before units 1 and 2.
  issue(0, ring0);
  {
    constexpr int NQP = QSTAGE / 1024;  // query pieces
    if (wave < NQP) {
      const char* qsrc = static_cast<const char*>(a.q) + q_off * C::ES;
      dec_dma(dec_rsrc(qsrc, G * C::IROWB), stage + wave * 1024, (uint32_t)(wave * 1024 + lane * 16));
    } else if (add_new && wave < NQP + 2) {
      const char* nsrc = (wave == NQP ? a.new_k : a.new_v) + ((size_t)w.b * a.n_kv + w.kvh) * C::IROWB;
      dec_dma(dec_rsrc(nsrc, C::IROWB), stage + QSTAGE + (wave - NQP) * NSTAGE, (uint32_t)(lane * 16));
    }
  }
  issue(1, ring1);
  issue(2, ring2);
  // rotary positions: this lane's angle (pair lane % (D/2)) at the query's
  // position, computed while the loads are in flight
  double rcs = 1.0, rsn = 0.0;
  if (a.rope.on) rope_cs(a.rope, D, a.rows[w.row].new_pos - (a.new_k ? 0 : 1), lane % (D / 2), rcs, rsn);
  wait_vmcnt<WAITN>();  // unit 0 and the staging loads have landed
  lds_barrier();
  if (a.rope.on) {
    // the queries (and the new token's K row) turned at the query's position
    rope_stage<C::ES>(stage, G, stage + QSTAGE, add_new, C::IROWB, D, rcs, rsn);
    lds_barrier();
  }
  // this wavefront's HW queries, in the lane's slice layout (of the four-lane
  // score layout when it is on)
  constexpr int QCPL = SC4 ? S4::CPL4 * S4::QPC : C::CPL;
  const int r16 = lane >> 2, s4 = lane & 3;
  uint4 q[HW][QCPL];
#pragma unroll
  for (int h = 0; h < HW; ++h)
#pragma unroll
    for (int c2 = 0; c2 < QCPL; ++c2)
      q[h][c2] = *reinterpret_cast<const uint4*>(
          stage + (size_t)(hg * HW + h) * C::IROWB +
          (SC4 ? ((s4 + 4 * (c2 / S4::QPC)) * S4::QPC + c2 % S4::QPC) : (s + 8 * c2)) * 16);
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

  // Unit u of the stream, held in ring unit X = u % 4 (K rows when X is even).
  auto unit = [&](auto tag, int64_t u) {
    constexpr int X = decltype(tag)::value;
    constexpr bool V_PART = (X & 1) != 0;
    wait_vmcnt<WAITN>();  // unit u has landed; u+1, u+2 may be in flight
    lds_barrier();                     // ... for every wavefront; unit u-1 is consumed
    issue(u + 3, rings[(X + 3) % kRingUnits]);
    const int64_t row0 = w.r0 + ((u >> 1) * SLOTS + slot) * (int64_t)TR;
    const int64_t left = w.r1 - row0;
    const int nv = active ? (int)(left < 0 ? 0 : (left > TR ? TR : left)) : 0;
    const char* tile = rings[X] + slot * C::SLOT_BYTES;
    if (V_PART) {
      if constexpr (SC4) {
        if (nv > 0) tile_pv4<KT, D, G>(st, pbuf, abuf, resc, tile, rg, s);
      } else {
        if (nv > 0) tile_pv<KT, D, G>(st, p, tile, rg, s);
      }
    } else {
      const int64_t ex = excl_row - row0;
      const int exr = (ex >= 0 && ex < TR) ? (int)ex : -1;
      if constexpr (SC4) {
        resc = false;
        const float* ks = &sbuf[KV8 ? (u >> 1) & 1 : 0][KV8 ? slot * TR : 0];
        const float* vs = ks + (KV8 ? C::ROUND_ROWS : 0);
        if (nv > 0) resc = tile_scores4<KT, D, G>(m4, l4, pbuf, abuf, tile, q, ks, vs, nv, exr, r16, s4, a.scale_log2);
      } else {
        if (nv > 0) tile_scores<KT, D, G>(st, p, tile, q, nv, exr, rg, s, a.scale_log2);
      }
    }
  };
  const int64_t n_units = 2 * nrounds;
  for (int64_t u = 0; u < n_units; u += 4) {  // n_units is even
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
    } else {
      if (wave == 0 && lane < 2 * C::CPR) {
        nkv = *reinterpret_cast<const uint4*>(stage + QSTAGE + (lane < C::CPR ? 0 : NSTAGE) + (lane % C::CPR) * 16);
        *reinterpret_cast<uint4*>((lane < C::CPR ? ring0 : ring1) + (lane % C::CPR) * 16) = nkv;  // row 0: no swizzle
      }
    }
    lds_barrier();
    if (slot == 0) {
      if constexpr (SC4) {
        const bool r1 = tile_scores4<KT, D, G>(m4, l4, pbuf, abuf, ring0, q, &sbuf[0][0], &sbuf[0][KV8 ? C::ROUND_ROWS : 0],
                                               1, -1, r16, s4, a.scale_log2);
        tile_pv4<KT, D, G>(st, pbuf, abuf, r1, ring1, rg, s);
      } else {
        tile_scores<KT, D, G>(st, p, ring0, q, 1, -1, rg, s, a.scale_log2);
        tile_pv<KT, D, G>(st, p, ring1, rg, s);
      }
    }
    const int64_t row = ret_head ? w.at(a.rows[w.row].new_pos) : a.rows[w.row].new_slot_str;
    if constexpr (KV8) {
      if (wave == 0 && lane < 32) {
        const int t = lane >> 4, j = lane & 15;
        *reinterpret_cast<uint2*>((t ? w.vbase : w.kbase) + (size_t)row * C::ROWB + j * 8) = ncodes;
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
      a.lp.pos[si * a.cap_str + a.rows[w.row].new_slot_str] = a.rows[w.row].new_pos;
    }
  }

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
        const int off = ((((slot * 8 + rg) * G + hG) * D) + (c2 * 8 + s) * C::EPC) * 4;
        float* dst = reinterpret_cast<float*>(ring_at(off / XB) + off % XB);
#pragma unroll
        for (int e = 0; e < C::EPC; e += 4)
          *reinterpret_cast<float4*>(dst + e) =
              make_float4(st.acc[h][c2 * C::EPC + e], st.acc[h][c2 * C::EPC + e + 1], st.acc[h][c2 * C::EPC + e + 2],
                          st.acc[h][c2 * C::EPC + e + 3]);
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
    if (w.nparts == 1) {
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

// Merges the partial records of every head that spans several work items.
// Workgroup = (flat head, query head, 32 output elements); its 512 threads are
// 16 record groups x 32 elements, each thread folding every 16th record.
constexpr int kCombineElems = 32;
constexpr int kCombineGroups = kDecodeThreads / kCombineElems;  // 16

template <int KT, int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void combine_kernel(DecodeArgs a) {
  using C = DecodeCfg<KT, D, G>;
  [[maybe_unused]] constexpr bool BF16 = C::BF16;
  constexpr int DC = D / kCombineElems;
  __shared__ float c_m[kCombineGroups][kCombineElems], c_l[kCombineGroups][kCombineElems],
      c_a[kCombineGroups][kCombineElems];
  const int64_t hh = blockIdx.x / (G * DC);
  const int h = (int)((blockIdx.x / DC) % G);
  const int dcn = (int)(blockIdx.x % DC);
  const int64_t n_ret_heads = (int64_t)a.B * a.n_ret;
  int64_t first;
  int n_seg, b, kvh;
  if (hh < n_ret_heads) {
    b = (int)(hh / a.n_ret);
    const int r = (int)(hh % a.n_ret);
    first = a.rows[b].first_ret + (int64_t)r * a.rows[b].nb_ret;
    n_seg = a.rows[b].nb_ret;
    kvh = a.map.orig_ret[r];
  } else {
    const int64_t x = hh - n_ret_heads;
    b = (int)(x / a.n_str);
    const int si = (int)(x % a.n_str);
    first = a.rows[b].first_str + (int64_t)si * a.rows[b].nb_str;
    n_seg = a.rows[b].nb_str;
    kvh = a.map.orig_str[si];
  }
  if (n_seg == 1) return;  // written by the decode kernel
  const float* rec0 = a.ws1 + (size_t)first * C::REC;
  const int el = threadIdx.x % kCombineElems, grp = threadIdx.x / kCombineElems;
  const int e = h * D + dcn * kCombineElems + el;
  float M = -INFINITY, L = 0.f, A = 0.f;
  constexpr int NB = 8;  // records per batch, loads issued together
  for (int i0 = grp; i0 < n_seg; i0 += NB * kCombineGroups) {
    float mv[NB], lv[NB], av[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int i = i0 + j * kCombineGroups;
      const float* r = rec0 + (size_t)(i < n_seg ? i : i0) * C::REC;
      mv[j] = i < n_seg ? r[G * D + h] : -INFINITY;
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
  float Mt = -INFINITY;
#pragma unroll
  for (int k = 0; k < kCombineGroups; ++k) Mt = fmaxf(Mt, c_m[k][el]);
  float Lt = 0.f, At = 0.f;
#pragma unroll
  for (int k = 0; k < kCombineGroups; ++k) {
    const float w = (c_m[k][el] == -INFINITY) ? 0.f : fast_exp2(c_m[k][el] - Mt);
    Lt += c_l[k][el] * w;
    At += c_a[k][el] * w;
  }
  const size_t o = ((size_t)b * a.n_q + (size_t)kvh * G) * D + e;
  if (BF16) reinterpret_cast<uint16_t*>(a.out)[o] = (uint16_t)f32_to_bf16_bits(At / Lt);
  else reinterpret_cast<float*>(a.out)[o] = At / Lt;
}

template <int KT, int D, int G>
hipError_t launch_decode_g(const DecodeArgs& a, int blocks, hipStream_t s) {
  decode_kernel<KT, D, G><<<blocks, kDecodeThreads, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!a.multi) return hipSuccess;  // every head finished in one item
  const int64_t heads = (int64_t)a.B * (a.n_ret + a.n_str);
  combine_kernel<KT, D, G><<<(unsigned)(heads * G * (D / kCombineElems)), kDecodeThreads, 0, s>>>(a);
  return hipGetLastError();
}

template <int KT, int D>
hipError_t launch_decode_d(const DecodeArgs& a, int g, int blocks, hipStream_t s) {
  switch (g) {
    case 1: return launch_decode_g<KT, D, 1>(a, blocks, s);
    case 2: return launch_decode_g<KT, D, 2>(a, blocks, s);
    case 4: return launch_decode_g<KT, D, 4>(a, blocks, s);
    case 8: return launch_decode_g<KT, D, 8>(a, blocks, s);
    default: return hipErrorInvalidValue;
  }
}

template <int KT, int D>
int64_t round_rows_d(int g) {
  switch (g) {
    case 1: return DecodeCfg<KT, D, 1>::ROUND_ROWS;
    case 2: return DecodeCfg<KT, D, 2>::ROUND_ROWS;
    case 4: return DecodeCfg<KT, D, 4>::ROUND_ROWS;
    case 8: return DecodeCfg<KT, D, 8>::ROUND_ROWS;
    default: return 0;
  }
}

}  // namespace

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

hipError_t launch_append(const AppendArgs& a, int dtype, int d, bool fp8, hipStream_t s) {
  (void)dtype;
  (void)d;
  if (fp8) {
    const int64_t threads = (int64_t)a.B * a.n_kv * a.n_new * 2 * 16;
    const int64_t grid = (threads + 255) / 256;
    if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
    append_fp8_kernel<<<(unsigned)grid, 256, 0, s>>>(a);
    return hipGetLastError();
  }
  const int64_t total = (int64_t)a.B * a.n_kv * a.n_new * (a.row_bytes / 16);
  const int threads = 256;
  const int64_t want = (total + threads - 1) / threads;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(want, 65536));
  append_kernel<<<grid, threads, 0, s>>>(a);
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

int64_t decode_round_rows(int dtype, int d, int g, bool fp8) {
  if (fp8) return round_rows_d<2, 128>(g);
  if (dtype == 1) return d == 128 ? round_rows_d<1, 128>(g) : round_rows_d<1, 64>(g);
  return d == 128 ? round_rows_d<0, 128>(g) : round_rows_d<0, 64>(g);
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int d, int g, bool fp8, int blocks, hipStream_t s) {
  if (fp8) {
    if (dtype == 1 && d == 128) return launch_decode_d<2, 128>(a, g, blocks, s);
    return hipErrorInvalidValue;
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
