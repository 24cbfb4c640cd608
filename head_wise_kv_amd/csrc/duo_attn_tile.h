// MFMA attention tile pieces shared by the bf16 prefill and the gated forward
// kernels (gfx950, v_mfma_f32_32x32x16_bf16).  One wavefront owns 32 query
// rows (one 32-row MFMA N tile; the pieces take kPfNT tiles) and consumes
// 64-key tiles of K and V that sit in LDS, XOR-swizzled in 16-byte chunks;
// scores are computed as S^T = K Q^T so a lane holds one query's scores, the
// online softmax runs in log2 units with a lazy rescale, and O^T = V^T P^T is
// accumulated in fp32 registers.
//
// 32 rows per wavefront keeps a wavefront under 256 registers, so two of them
// share each SIMD: one's MFMA work then overlaps the other's softmax and
// LDS waits.  (64 rows halve the LDS operand reads per MFMA but need about
// 330 registers, one wavefront per SIMD, and every latency of that single
// wavefront stays exposed.)
//
// Only included by the HIP sources of this library; everything is internal.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "duo_dma.h"

namespace duo {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr int kPfRowWaves = 4;                    // wavefronts per key half (one row block each)
constexpr int kPfHalves = 2;                      // key halves: even / odd key tiles
constexpr int kPfThreads = 64 * kPfRowWaves * kPfHalves;
constexpr int kPfRowsPerWave = 32;                // query rows per wavefront
constexpr int kPfNT = kPfRowsPerWave / 32;        // 32-row MFMA N tiles per wavefront
constexpr int kBN = 64;                           // keys per tile

// A value the same in every lane, moved to a scalar register (so that the
// compiler treats what is computed from it as wavefront-uniform).
__device__ __forceinline__ int32_t uniform32(int64_t x) { return (int32_t)__builtin_amdgcn_readfirstlane((int)x); }

// Integer min / max by plain comparison (kept off any floating-point path).
__device__ __forceinline__ int64_t min64(int64_t x, int64_t y) { return x < y ? x : y; }
__device__ __forceinline__ int64_t max64(int64_t x, int64_t y) { return x > y ? x : y; }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  bf2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maxima of scores with IEEE maximum (a NaN would propagate; scores are
// finite or -inf).  Unlike fmaxf it needs no quieting of its inputs, so it
// lowers to bare v_maximum3_f32 on MFMA results.
__device__ __forceinline__ float max2(float x, float y) { return __builtin_elementwise_maximum(x, y); }
__device__ __forceinline__ float max3(float x, float y, float z) { return max2(max2(x, y), z); }

// Max and sum over the lane pair (i, i ^ 32).  One v_permlane32_swap exchanges
// the two 32-lane halves on the vector ALU (no LDS round trip): result r[0]
// holds the lower half's values in both halves and r[1] the upper half's, so
// both lanes of a pair combine the same two values in the same order.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
constexpr bf16x2_t kOnesBf16x2 = {(__bf16)1.0f, (__bf16)1.0f};

// Visibility of a key as an interval of query rows: the key is seen by the
// rows i with lo <= i <= lo + span, tested with one unsigned compare,
// (unsigned)(i - lo) <= span.  A key no row sees gets lo = -1, span = 0 (no
// row i >= 0 passes).  Rows and positions stay below 2^31, so every
// difference fits in 32 bits.
struct KeySpan {
  int32_t lo;
  uint32_t span;
};
__device__ __forceinline__ bool sees(int32_t i, int32_t lo, uint32_t span) { return (uint32_t)(i - lo) <= span; }

// Skip the O rescale until the running max has grown by more than this many
// log2 units; probabilities then stay below 2^kRescaleSlack, well inside bf16
// and fp32 range.
constexpr float kRescaleSlack = 8.f;

template <int D>
struct PfShape {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int TILE_BYTES = kBN * D * 2;    // one K (or V) tile
  static constexpr int DMA_PER_TILE = TILE_BYTES / 1024;  // 1 KB per wavefront-wide direct load
  static constexpr int KSTEPS = D / 16;             // MFMA k-steps over d for S^T
  static constexpr int DT = D / 32;                 // 32-row tiles of O^T over d
  static_assert(DMA_PER_TILE % kPfRowWaves == 0, "tile loads split over the wavefronts");
  // K rows: chunk c of key r sits at chunk slot c ^ swz_k(r) (A-operand reads
  // of 16 consecutive keys at one chunk hit 16 distinct bank groups).
  __host__ __device__ static constexpr int swz_k(int r) { return CPR == 16 ? (r & 15) : ((r >> 1) & 7); }
  // V rows: chunk c of key r at c ^ swz_v(r) (a transpose read of 4 rows x
  // 4 chunks by 32 lanes hits 16 distinct bank groups).
  __host__ __device__ static constexpr int swz_v(int r) { return CPR == 16 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

// Direct global->LDS copies of a 64-row tile (K or V) through a buffer
// resource.  The tile is 1 KB pieces; piece n covers LDS bytes
// [n*1024, n*1024+1024), lane i writing 16 bytes at n*1024 + i*16, i.e. row
// (n*64 + i) / CPR at chunk slot (n*64 + i) % CPR; the global chunk it fetches
// is that slot XOR the row's swizzle.  The byte offset of that chunk within the
// tile depends only on (n, lane), so it is computed once per kernel; each tile
// only rebuilds the scalar resource (base = first row, size = rows present).
// Rows past the end are out of range for the resource and read as zero.
template <int D, bool IS_V>
__host__ __device__ constexpr uint32_t dma_offset(int n, int lane) {
  using SH = PfShape<D>;
  const int piece = n * 64 + lane;
  const int r = piece / SH::CPR;
  const int c = (piece % SH::CPR) ^ (IS_V ? SH::swz_v(r) : SH::swz_k(r));
  return (uint32_t)(r * (D * 2) + c * 16);
}

// The property TileLoads relies on: a wavefront's piece wave + kPfRowWaves j
// is its piece `wave` moved by j * kPfRowWaves KB (checked at compile time
// for every wavefront, piece and lane).
template <int D, bool IS_V>
constexpr bool pieces_are_strided() {
  for (int wave = 0; wave < kPfRowWaves; ++wave)
    for (int j = 0; j < PfShape<D>::DMA_PER_TILE / kPfRowWaves; ++j)
      for (int lane = 0; lane < 64; ++lane)
        if (dma_offset<D, IS_V>(wave + kPfRowWaves * j, lane) !=
            dma_offset<D, IS_V>(wave, lane) + (uint32_t)(kPfRowWaves * j * 1024))
          return false;
  return true;
}
static_assert(pieces_are_strided<128, false>() && pieces_are_strided<128, true>(), "d = 128 pieces");
static_assert(pieces_are_strided<64, false>() && pieces_are_strided<64, true>(), "d = 64 pieces");

// This wavefront's direct loads of one K/V tile (its pieces wave,
// wave + kPfRowWaves, ... of each tensor), issued in four parts: the K
// pieces in two, then the V pieces in two.  The kernels spread the parts of
// the next tile over the four regions of the current tile's work, so that no
// wavefront stalls on a burst of load issues right after a barrier (all
// eight wavefronts would issue their loads at once).  The loads are not
// waited for here: the kernel waits for them (vmcnt) and publishes them with
// a barrier before any wavefront reads the tile.
template <int D>
struct TileLoads {
  static constexpr int N = PfShape<D>::DMA_PER_TILE / kPfRowWaves;  // pieces per tensor and wavefront
  static_assert(N % 2 == 0, "two parts per tensor");
  // Buffer resources over the tile's K and V rows.  Without a tile to load
  // they cover no bytes: every piece is then out of range, reads as zero and
  // touches no memory (it fills a buffer nobody reads), and the loads need
  // no branch.
  i32x4_t rk, rv;
  uint32_t kdst, vdst;   // LDS byte addresses of this wavefront's first K / V piece
  uint32_t koff, voff;   // the lane's offsets (dma_offset) within its first K / V piece

  // The wavefront's pieces n = wave + kPfRowWaves j lie kPfRowWaves KB apart
  // both in LDS and in the tile's rows (the swizzle only permutes chunks
  // within a row, and rows wave + kPfRowWaves j share it), so piece j is piece
  // 0 moved by j * kPfRowWaves KB on both sides.
  __device__ __forceinline__ void operator()(int part) const {
    const bool v = part >= 2;
    const int j0 = (part & 1) * (N / 2);
#pragma unroll
    for (int j = j0; j < j0 + N / 2; ++j)
      dma_lds16_at(v ? rv : rk, (v ? vdst : kdst) + kPfRowWaves * j * 1024, v ? voff : koff,
                   kPfRowWaves * j * 1024);
  }
  __device__ __forceinline__ void all() const {
#pragma unroll
    for (int part = 0; part < 4; ++part) (*this)(part);
  }
};

// A pf_tile `next` that issues nothing (the loads were issued before the tile).
struct NoLoads {
  __device__ __forceinline__ void operator()(int) const {}
};

// ---- per-tile pieces of the MFMA path (one wavefront, 64 query rows = two
// 32-row N tiles nt, one 64-key tile = two 32-key halves ct)

// S^T = K Q^T for the keys ct*32 .. ct*32+31 of the tile: s[nt] register r of
// lane (n, hf) is the score of key ct*32 + 8*(r/4) + 4*hf + r%4 and query
// 32*nt + n.
template <int D>
__device__ __forceinline__ void pf_scores(f32x16_t (&s)[kPfNT], const bf16x8_t (&qb)[kPfNT][D / 16], const char* kt, int ct,
                                          int lane) {
  using SH = PfShape<D>;
  const int key = ct * 32 + (lane & 31);
  const int hf = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < SH::KSTEPS; ++ks) {
    const int c = 2 * ks + hf;
    const u32x4_t av = *reinterpret_cast<const u32x4_t*>(kt + key * (SH::CPR * 16) + ((c ^ SH::swz_k(key)) * 16));
    const bf16x8_t aop = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
    for (int nt = 0; nt < kPfNT; ++nt)
      s[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, qb[nt][ks], ks == 0 ? f32x16_t{} : s[nt], 0, 0, 0);
  }
}

// Scores of keys a row does not see (half ct of the tile) become -inf.
__device__ __forceinline__ void pf_mask(f32x16_t (&s)[kPfNT], const int32_t* klo, const uint32_t* kspan,
                                        const int32_t (&iq)[kPfNT], int ct, int lane) {
  const int hf = lane >> 5;
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const int key0 = ct * 32 + 8 * r4 + 4 * hf;  // keys key0 .. key0+3 in registers 4*r4 .. 4*r4+3
    const int4 lo4 = *reinterpret_cast<const int4*>(klo + key0);
    const uint4 sp4 = *reinterpret_cast<const uint4*>(kspan + key0);
    const int32_t lo[4] = {lo4.x, lo4.y, lo4.z, lo4.w};
    const uint32_t sp[4] = {sp4.x, sp4.y, sp4.z, sp4.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int nt = 0; nt < kPfNT; ++nt)
        if (!sees(iq[nt], lo[j], sp[j])) s[nt][4 * r4 + j] = -INFINITY;
  }
}

// Online softmax of one half: updates the running max m (lazily: a row's
// max moves only when it has grown past the slack), the running sum l, and
// returns P^T as bf16 pairs pb[nt][k-step st][dword] plus the factor
// alpha[nt] the accumulators must be scaled by; the result says whether any
// lane's alpha differs from 1.
__device__ __forceinline__ bool pf_softmax(const f32x16_t (&s)[kPfNT], float (&m_run)[kPfNT], float (&l_run)[kPfNT],
                                           uint32_t (&pb)[kPfNT][2][4], float (&alpha)[kPfNT], float scale_log2) {
  bool grow = false;
#pragma unroll
  for (int nt = 0; nt < kPfNT; ++nt) {
    const f32x16_t& x = s[nt];
    const float v = max2(max3(max3(x[0], x[1], x[2]), max3(x[3], x[4], x[5]), max3(x[6], x[7], x[8])),
                         max3(max3(x[9], x[10], x[11]), max3(x[12], x[13], x[14]), x[15]));
    const float mx = pair_max(v) * scale_log2;
    const bool g = mx > m_run[nt] + kRescaleSlack;
    grow |= g;
    const float m_new = g ? mx : m_run[nt];  // mx > m_run here
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    alpha[nt] = fast_exp2(m_run[nt] - m_use);
    m_run[nt] = m_new;
    // the row sum adds the bf16-rounded probabilities, the same values the
    // P V product uses
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = fast_exp2(fmaf(x[r], scale_log2, -m_use));
      const float p1 = fast_exp2(fmaf(x[r + 1], scale_log2, -m_use));
      const uint32_t pp = pack_bf16(p0, p1);
      pb[nt][r >> 3][(r & 7) >> 1] = pp;
      psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pp), kOnesBf16x2, psum, false);
    }
    l_run[nt] = l_run[nt] * alpha[nt] + psum;
  }
  return __builtin_amdgcn_ballot_w64(grow) != 0;
}

// Keeps the probabilities computed where they are written in the source: an
// empty asm statement that reads them (it emits no instruction), so the
// compiler cannot sink their computation past the branch that follows.
__device__ __forceinline__ void pf_pin(const uint32_t (&pb)[kPfNT][2][4], const float (&l_run)[kPfNT]) {
#pragma unroll
  for (int nt = 0; nt < kPfNT; ++nt)
    asm volatile("" ::"v"(l_run[nt]), "v"(pb[nt][0][0]), "v"(pb[nt][0][1]), "v"(pb[nt][0][2]), "v"(pb[nt][0][3]),
                 "v"(pb[nt][1][0]), "v"(pb[nt][1][1]), "v"(pb[nt][1][2]), "v"(pb[nt][1][3]));
}

template <int DT>
__device__ __forceinline__ void pf_rescale(f32x16_t (&o)[DT][kPfNT], const float (&alpha)[kPfNT]) {
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int nt = 0; nt < kPfNT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][nt][r] *= alpha[nt];
}

// O^T += V^T P^T for the keys of half ct.  V^T operands come from transpose
// reads of the row-major V tile: lane (g16 = lane/16, i16 = lane%16) reads
// row kb + i16/4 at columns dt*32 + 16*(g16%2) + 4*(i16%4) and receives
// V[kb + 0..3][its d].
template <int D>
__device__ __forceinline__ void pf_pv(f32x16_t (&o)[D / 32][kPfNT], const uint32_t (&pb)[kPfNT][2][4], const char* vt,
                                      int ct, int lane) {
  using SH = PfShape<D>;
  const int hf = lane >> 5, g16 = lane >> 4, i16 = lane & 15;
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    bf16x8_t bop[kPfNT];
#pragma unroll
    for (int nt = 0; nt < kPfNT; ++nt) {
      const u32x4_t bw = {pb[nt][st][0], pb[nt][st][1], pb[nt][st][2], pb[nt][st][3]};
      bop[nt] = __builtin_bit_cast(bf16x8_t, bw);
    }
#pragma unroll
    for (int dt = 0; dt < SH::DT; ++dt) {
      i16x4_t half[2];
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int row = ct * 32 + 16 * st + 8 * rr + 4 * hf + (i16 >> 2);
        const int col = dt * 32 + 16 * (g16 & 1) + 4 * (i16 & 3);
        const int c = col >> 3;
        const char* p = vt + row * (SH::CPR * 16) + ((c ^ SH::swz_v(row)) * 16) + (col & 7) * 2;
        half[rr] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(p));
      }
      const u32x2_t h0 = __builtin_bit_cast(u32x2_t, half[0]);
      const u32x2_t h1 = __builtin_bit_cast(u32x2_t, half[1]);
      const u32x4_t aw = {h0[0], h0[1], h1[0], h1[1]};
      const bf16x8_t aop = __builtin_bit_cast(bf16x8_t, aw);
#pragma unroll
      for (int nt = 0; nt < kPfNT; ++nt)
        o[dt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop[nt], o[dt][nt], 0, 0, 0);
    }
  }
}

// One 64-key tile, ordered over its halves so that the MFMA work of one half
// is independent of the softmax next to it:
//   S(0) | mask(0) | S(1) + softmax(0) | rescale(0), mask(1) | P V(0) + softmax(1) | rescale(1) | P V(1)
// The masks and rescales are wavefront-uniform branches between the regions;
// the compiler orders the instructions within a region.  `next` issues part
// k of the next tile's loads at the start of the k-th main region.
template <int D, class Next>
__device__ __forceinline__ void pf_tile(f32x16_t (&o)[D / 32][kPfNT], float (&m_run)[kPfNT], float (&l_run)[kPfNT],
                                        const bf16x8_t (&qb)[kPfNT][D / 16], const char* kt, const char* vt,
                                        bool masked, const int32_t* klo, const uint32_t* kspan,
                                        const int32_t (&iq)[kPfNT], float scale_log2, int lane, const Next& next) {
  constexpr int DT = D / 32;
  f32x16_t s0[kPfNT], s1[kPfNT];
  uint32_t p0[kPfNT][2][4], p1[kPfNT][2][4];
  float a0[kPfNT], a1[kPfNT];

  next(0);
  pf_scores<D>(s0, qb, kt, 0, lane);
  // the first and last regions are MFMA runs with nothing to overlap: their
  // LDS operand reads are issued ahead of the MFMAs (eight K reads; the V
  // transpose reads of each k-step's four MFMAs), not one or two ahead
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // LDS reads
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);  // MFMA
  __builtin_amdgcn_sched_barrier(0);
  if (masked) pf_mask(s0, klo, kspan, iq, 0, lane);
  __builtin_amdgcn_sched_barrier(0);
  next(1);
  pf_scores<D>(s1, qb, kt, 1, lane);
  const bool g0 = pf_softmax(s0, m_run, l_run, p0, a0, scale_log2);
  __builtin_amdgcn_sched_barrier(0);
  pf_pin(p0, l_run);
  if (g0) pf_rescale<DT>(o, a0);
  if (masked) pf_mask(s1, klo, kspan, iq, 1, lane);
  __builtin_amdgcn_sched_barrier(0);
  next(2);
  pf_pv<D>(o, p0, vt, 0, lane);
  const bool g1 = pf_softmax(s1, m_run, l_run, p1, a1, scale_log2);
  __builtin_amdgcn_sched_barrier(0);
  pf_pin(p1, l_run);
  if (g1) pf_rescale<DT>(o, a1);
  __builtin_amdgcn_sched_barrier(0);
  next(3);
  pf_pv<D>(o, p1, vt, 1, lane);
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

}  // namespace
}  // namespace duo
