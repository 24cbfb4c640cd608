// Head-gated forward over one whole sequence, for gfx950 (CDNA4): for every
// query head, alpha * (causal attention) + (1 - alpha) * (sink + window
// attention), both over the same Q, K, V.
//
// This is the forward pass that head identification trains its gates through
// ("DuoAttention: Dual Retrieval & Streaming Heads Guide", section 3,
// item 2): a continuous gate per head mixes full and streaming attention.
// One gate per KV head, shared by the g query heads that read it.
//
// For the row at position t the sink + window keys (j < S or t - W < j <= t)
// and the remaining causal keys (S <= j <= t - W) split the causal key set in
// two.  A work item therefore makes one pass over its causal keys in two
// phases.  Phase 1 visits the tiles that hold sink or window keys, with that
// mask; its softmax state (running max, running sum, O accumulators) is then
// exactly the streaming attention's, and is saved.  Phase 2 continues the same
// online softmax over the tiles of the remaining keys, with the complementary
// mask, and ends in the full attention's state.  So every score and every
// P V product is computed once; only the one to three tiles the window's lower
// edge crosses are visited in both phases (with complementary masks).  The
// output mixes the two normalised results.
//
// bf16: the MFMA tile pipeline of the prefill (eight wavefronts: four 32-row
// blocks x two key halves that take the even and the odd tiles of each phase,
// direct buffer->LDS loads, double buffered), with the saved phase-1 state
// held in registers through phase 2; the halves merge both states through LDS
// at the end.
// fp32: a plain vector-ALU path (one wavefront per query row) kept for
// completeness of the dtype surface; it is not tuned.
#include "duo_attn_tile.h"
#include "duo_internal.h"

#include <hip/hip_runtime.h>

namespace duo {
namespace {

// Rows that see key j (row = position), per phase.  Phase 1 (sink + window):
// rows j .. j + W - 1, or every row from j on for a sink key (j < S).
// Phase 2 (the rest of the causal keys): every row from j + W on, none for a
// sink key.  Keys past the end of the sequence are seen by no row.
__device__ __forceinline__ KeySpan span_window(int64_t j, int64_t N, int S, int W) {
  KeySpan k;
  if (j >= N) {
    k.lo = -1;
    k.span = 0;
  } else {
    k.lo = (int32_t)j;
    k.span = (j < S) ? (uint32_t)0x7fffffff - (uint32_t)k.lo : (uint32_t)(W - 1);
  }
  return k;
}
__device__ __forceinline__ KeySpan span_rest(int64_t j, int64_t N, int S, int W) {
  KeySpan k;
  if (j >= N || j < S) {
    k.lo = -1;
    k.span = 0;
  } else {
    k.lo = (int32_t)(j + W);
    k.span = (uint32_t)0x7fffffff - (uint32_t)k.lo;
  }
  return k;
}

// Key tiles (units of kBN keys) of the rows [i0, i1): phase 1 in up to two
// ranges (sink tiles, then the band the windows reach), phase 2 in one.
struct GatedTiles {
  int64_t w_lo0, w_hi0, w_lo1, w_hi1;
  int64_t r_lo, r_hi;
};

__device__ __forceinline__ GatedTiles gated_tiles(int64_t i0, int64_t i1, int S, int W) {
  GatedTiles t;
  const int64_t hi = (i1 + kBN - 1) / kBN;                     // causal: keys j <= i1 - 1
  const int64_t sink_tiles = (min64(S, i1) + kBN - 1) / kBN;   // keys j < S
  const int64_t band_lo = max64(0, i0 - W + 1) / kBN;          // keys j >= i0 - W + 1
  if (band_lo <= sink_tiles) {
    t.w_lo0 = 0;
    t.w_hi0 = hi;
    t.w_lo1 = t.w_hi1 = 0;
  } else {
    t.w_lo0 = 0;
    t.w_hi0 = sink_tiles;
    t.w_lo1 = band_lo;
    t.w_hi1 = hi;
  }
  const int64_t j_last = i1 - 1 - W;  // last key outside the window of the item's last row
  if (j_last >= S) {
    t.r_lo = S / kBN;
    t.r_hi = j_last / kBN + 1;
  } else {
    t.r_lo = t.r_hi = 0;
  }
  return t;
}

// Folds the other key half's softmax state (x: its O registers, one float per
// lane and register, 64 apart; ml: its m at [nt*64], l at [(kPfNT+nt)*64])
// into this half's.
template <int DT>
__device__ __forceinline__ void merge_half(f32x16_t (&o)[DT][kPfNT], float (&m)[kPfNT], float (&l)[kPfNT],
                                           const float* x, const float* ml) {
#pragma unroll
  for (int nt = 0; nt < kPfNT; ++nt) {
    const float m2 = ml[nt * 64], l2 = ml[(kPfNT + nt) * 64];
    const float m_new = fmaxf(m[nt], m2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float a1 = fast_exp2(m[nt] - m_use), a2 = fast_exp2(m2 - m_use);
    m[nt] = m_new;
    l[nt] = l[nt] * a1 + l2 * a2;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][nt][r] = o[dt][nt][r] * a1 + x[((dt * kPfNT + nt) * 16 + r) * 64] * a2;
  }
}

template <int DT>
__device__ __forceinline__ void spill_half(const f32x16_t (&o)[DT][kPfNT], const float (&m)[kPfNT],
                                           const float (&l)[kPfNT], float* x, float* ml) {
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int nt = 0; nt < kPfNT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[((dt * kPfNT + nt) * 16 + r) * 64] = o[dt][nt][r];
#pragma unroll
  for (int nt = 0; nt < kPfNT; ++nt) {
    ml[nt * 64] = m[nt];
    ml[(kPfNT + nt) * 64] = l[nt];
  }
}

// Work item = (query tile, batch row, head group, KV head); query tiles with
// the most keys come first, and the KV head varies fastest, so that the items
// of one KV head land on the same XCD (workgroups are dealt to the XCDs in
// turn) and share its K and V in that XCD's L2.
template <int D>
__global__ __launch_bounds__(kPfThreads) void gated_mfma_kernel(GatedArgs a, int g, int hpi) {
  using SH = PfShape<D>;
  constexpr int KSTEPS = SH::KSTEPS, DT = SH::DT;

  // [key half][buffer]
  __shared__ __attribute__((aligned(1024))) char k_lds[kPfHalves][2][SH::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds[kPfHalves][2][SH::TILE_BYTES];
  __shared__ int32_t klo_lds[kPfHalves][2][kBN];
  __shared__ uint32_t kspan_lds[kPfHalves][2][kBN];
  __shared__ int s_full[kPfHalves][2];
  __shared__ float ml_lds[2][kPfRowWaves][2 * kPfNT * 64];  // [state][row wavefront]: m and l of the odd half

  const int ngrp = g / hpi;
  const int per_level = a.B * a.n_kv * ngrp;
  const int level = (int)blockIdx.x / per_level;
  int rem = (int)blockIdx.x % per_level;
  const int kvh = rem % a.n_kv;
  rem /= a.n_kv;
  const int hg = rem % ngrp;
  const int b = rem / ngrp;
  const int qt = a.q_tiles - 1 - level;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = wave / kPfRowWaves;   // key half
  const int sub = wave % kPfRowWaves;  // row wavefront within the half
  const int n = lane & 31, hf = lane >> 5;
  const int h = kvh * g + hg * hpi + (sub % hpi);
  const int rows_item = kPfRowsPerWave * (kPfRowWaves / hpi);
  const int64_t i0 = (int64_t)qt * rows_item;
  const int64_t i1 = min64(i0 + rows_item, a.N);
  const int64_t wr0 = i0 + (int64_t)(sub / hpi) * kPfRowsPerWave;
  const size_t rowb = (size_t)D * 2;

  // Q^T operands: lane holds 8 consecutive d of query row (wr0 + 32*nt + n) per k-step.
  bf16x8_t qb[kPfNT][KSTEPS];
  int32_t iq[kPfNT];
  bool qvalid[kPfNT];
#pragma unroll
  for (int nt = 0; nt < kPfNT; ++nt) {
    const int64_t qrow = wr0 + 32 * nt + n;
    qvalid[nt] = qrow < a.N;
    iq[nt] = (int32_t)qrow;
    const char* qp = static_cast<const char*>(a.q) + (((size_t)b * a.n_q + h) * a.N + (qvalid[nt] ? qrow : 0)) * rowb;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4_t v = qvalid[nt] ? *reinterpret_cast<const u32x4_t*>(qp + (ks * 16 + hf * 8) * 2) : u32x4_t{0, 0, 0, 0};
      qb[nt][ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  const size_t head_off = ((size_t)b * a.n_kv + kvh) * a.N * rowb;
  const char* kn = static_cast<const char*>(a.k) + head_off;
  const char* vn = static_cast<const char*>(a.v) + head_off;

  // Tile numbers and rows in 32-bit wavefront-uniform values (N + W fits
  // int32, checked on the host), so the per-step arithmetic is a few scalar
  // instructions.
  const GatedTiles tt = gated_tiles(i0, i1, a.S, a.W);
  const int32_t n_w0 = uniform32(tt.w_hi0 - tt.w_lo0);
  const int32_t n_w = n_w0 + uniform32(tt.w_hi1 - tt.w_lo1);
  const int32_t n_r = uniform32(tt.r_hi - tt.r_lo);
  const int32_t steps_w = (n_w + 1) / 2;  // the halves take tiles 2s and 2s+1 of a phase at step s
  const int32_t n_steps = steps_w + (n_r + 1) / 2;
  const int32_t w_lo0 = uniform32(tt.w_lo0), w_lo1 = uniform32(tt.w_lo1), r_lo = uniform32(tt.r_lo);
  const int32_t n_rows = uniform32(a.N), r0 = uniform32(i0), r1 = uniform32(i1);
  const int32_t S = a.S, W = a.W;

  // per-lane byte offsets of this wavefront's first K / V piece within a tile
  const uint32_t koff = dma_offset<D, false>(sub, lane);
  const uint32_t voff = dma_offset<D, true>(sub, lane);
  // Rows past the end read as zero; clear both buffers once so no stale bit
  // pattern (which could be a NaN) ever meets a zero probability.
  {
    const u32x4_t z = {0, 0, 0, 0};
    for (int off = tid * 16; off < kPfHalves * 2 * SH::TILE_BYTES; off += kPfThreads * 16) {
      *reinterpret_cast<u32x4_t*>(&k_lds[0][0][0] + off) = z;
      *reinterpret_cast<u32x4_t*>(&v_lds[0][0][0] + off) = z;
    }
    __syncthreads();
  }

  // Step -> this half's key tile (or -1 when the half has none at that step)
  // and its phase.
  auto tile_at = [&](int32_t step, bool& rest) -> int32_t {
    if (step < steps_w) {
      rest = false;
      const int32_t i = 2 * step + kh;
      if (i >= n_w) return -1;
      return i < n_w0 ? w_lo0 + i : w_lo1 + (i - n_w0);
    }
    rest = true;
    const int32_t i = 2 * (step - steps_w) + kh;
    return i < n_r ? r_lo + i : -1;
  };
  // Whether every row of the item sees every key of a tile in its phase,
  // decided from scalars: then the tile needs no mask and no per-key
  // bookkeeping.  Phase 2 keys j >= S are seen by the rows from j + W on;
  // phase 1 keys by the rows j .. j + W - 1 (every row from j on for a sink).
  auto tile_full = [&](int32_t tile, bool rest) -> bool {
    const int32_t base = tile * kBN;  // < N: a tile starts at a row that exists
    if (base > n_rows - kBN) return false;
    const int32_t last = base + kBN - 1;
    if (rest) return base >= S && last <= r0 - W;
    return last <= r0 && (last < S || base >= r1 - W);
  };
  // Prepare a tile (-1: none) for buffer `buf` of this half: for a tile that
  // does not pass tile_full, the keys' visible-row intervals and the no-mask
  // flag by the half's first wavefront; and the direct loads of its K/V
  // pieces (split over the half's wavefronts), which the caller issues.
  auto prepare = [&](int32_t tile, bool rest, int buf) -> TileLoads<D> {
    TileLoads<D> ld;
    ld.kdst = lds_addr(k_lds[kh][buf] + sub * 1024);
    ld.vdst = lds_addr(v_lds[kh][buf] + sub * 1024);
    ld.koff = koff;
    ld.voff = voff;
    if (!(tile >= 0)) {
      ld.rk = ld.rv = dma_rsrc(kn, 0);
      return ld;
    }
    const int32_t base = tile * kBN;
    const int nbytes = min(n_rows - base, kBN) * (int)rowb;
    if (sub == 0 && !tile_full(tile, rest)) {
      const int64_t j = base + lane;
      const KeySpan ks = rest ? span_rest(j, a.N, a.S, a.W) : span_window(j, a.N, a.S, a.W);
      klo_lds[kh][buf][lane] = ks.lo;
      kspan_lds[kh][buf][lane] = ks.span;
      const bool all = sees((int32_t)i0, ks.lo, ks.span) && sees((int32_t)(i1 - 1), ks.lo, ks.span);
      const uint64_t bal = __builtin_amdgcn_ballot_w64(all);
      if (lane == 0) s_full[kh][buf] = (bal == ~0ull) ? 1 : 0;
    }
    ld.rk = dma_rsrc(kn + (size_t)base * rowb, nbytes);
    ld.rv = dma_rsrc(vn + (size_t)base * rowb, nbytes);
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
  // the state after phase 1 (sink + window keys only)
  f32x16_t o_w[DT][kPfNT];
  float m_w[kPfNT], l_w[kPfNT];

  {
    bool rest;
    const int32_t t0 = tile_at(0, rest);
    prepare(t0, rest, 0).all();
  }
  for (int32_t step = 0; step < n_steps; ++step) {
    if (step == steps_w) {  // phase 1 done (wavefront-uniform)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int nt = 0; nt < kPfNT; ++nt) o_w[dt][nt] = o[dt][nt];
#pragma unroll
      for (int nt = 0; nt < kPfNT; ++nt) {
        m_w[nt] = m_run[nt];
        l_w[nt] = l_run[nt];
      }
    }
    const int buf = (int)(step & 1);
    // this wavefront's direct loads for the current tile have landed; after
    // the barrier every wavefront's have, and the previous tile is consumed.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // the next tile's loads, issued before the current tile's work (spread
    // over it as the prefill does, they would push this kernel, which also
    // holds the saved phase-1 state, past 256 registers)
    bool rest_n = false;
    const int32_t tn = step + 1 < n_steps ? tile_at(step + 1, rest_n) : -1;
    prepare(tn, rest_n, buf ^ 1).all();
    bool rest;
    const int32_t tc = tile_at(step, rest);
    if (tc < 0) continue;  // wavefront-uniform: no tile for this half at this step
    const bool masked = !tile_full(tc, rest) && s_full[kh][buf] == 0;
    pf_tile<D>(o, m_run, l_run, qb, k_lds[kh][buf], v_lds[kh][buf], masked, klo_lds[kh][buf],
               kspan_lds[kh][buf], iq, a.scale_log2, lane, NoLoads{});
  }
  if (n_steps == steps_w) {  // no phase-2 tile at all
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int nt = 0; nt < kPfNT; ++nt) o_w[dt][nt] = o[dt][nt];
#pragma unroll
    for (int nt = 0; nt < kPfNT; ++nt) {
      m_w[nt] = m_run[nt];
      l_w[nt] = l_run[nt];
    }
  }

  // ---- merge the odd half's two states into the even half's through LDS
  // (the tile buffers are free now): per lane, registers in order (dt, nt, r).
  constexpr int NREG = DT * kPfNT * 16;
  static_assert(kPfRowWaves * NREG * 64 * 4 <= kPfHalves * 2 * SH::TILE_BYTES, "one state fits a K or V buffer");
  float* x_full = reinterpret_cast<float*>(&k_lds[0][0][0]) + sub * NREG * 64 + lane;
  float* x_win = reinterpret_cast<float*>(&v_lds[0][0][0]) + sub * NREG * 64 + lane;
  float* ml_full = &ml_lds[0][sub][lane];
  float* ml_win = &ml_lds[1][sub][lane];
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (kh == 1) {
    spill_half<DT>(o, m_run, l_run, x_full, ml_full);
    spill_half<DT>(o_w, m_w, l_w, x_win, ml_win);
  }
  __syncthreads();
  if (kh == 1) return;
  merge_half<DT>(o, m_run, l_run, x_full, ml_full);
  merge_half<DT>(o_w, m_w, l_w, x_win, ml_win);

  // ---- mix and store: lane holds d = dt*32 + 8*(r/4) + 4*hf + r%4 of query 32*nt + n
  const float alpha = a.alpha[kvh];
#pragma unroll
  for (int nt = 0; nt < kPfNT; ++nt) {
    const float l_full = pair_sum(l_run[nt]);
    const float l_win = pair_sum(l_w[nt]);
    if (!qvalid[nt]) continue;
    const float cf = alpha / l_full, cw = (1.f - alpha) / l_win;
    const int64_t qrow = wr0 + 32 * nt + n;
    uint16_t* op = static_cast<uint16_t*>(a.out) + (((size_t)b * a.n_q + h) * a.N + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = dt * 32 + 8 * r4 + 4 * hf;
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = o[dt][nt][4 * r4 + j] * cf + o_w[dt][nt][4 * r4 + j] * cw;
        uint2 v;
        v.x = pack_bf16(y[0], y[1]);
        v.y = pack_bf16(y[2], y[3]);
        *reinterpret_cast<uint2*>(op + d0) = v;
      }
  }
}

// ------------------------------------------------------------------ fp32 path
// One wavefront per (batch, query head, row t); lanes own keys for the scores
// and d-chunks for the weighted sums; two online softmaxes (all causal keys,
// and the sink + window keys) share the scores.
template <int D>
__global__ __launch_bounds__(256) void gated_f32_kernel(GatedArgs a, int g) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t total = (int64_t)a.B * a.n_q * a.N;
  if (gw >= total) return;
  const int64_t t = gw % a.N;
  const int h = (int)((gw / a.N) % a.n_q);
  const int b = (int)(gw / ((int64_t)a.N * a.n_q));
  const int kvh = h / g;
  const float* q = static_cast<const float*>(a.q) + (((size_t)b * a.n_q + h) * a.N + t) * D;
  const size_t head_off = ((size_t)b * a.n_kv + kvh) * a.N * D;
  const float* kb = static_cast<const float*>(a.k) + head_off;
  const float* vb = static_cast<const float*>(a.v) + head_off;
  constexpr int EPL = D / 64;
  float acc_f[EPL], acc_w[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc_f[e] = acc_w[e] = 0.f;
  float m_f = -INFINITY, l_f = 0.f, m_w = -INFINITY, l_w = 0.f;
  for (int64_t k0 = 0; k0 <= t; k0 += 64) {
    const int64_t j = k0 + lane;
    float s_f = -INFINITY, s_w = -INFINITY;
    if (j <= t) {
      const float* kr = kb + (size_t)j * D;
      float s = 0.f;
      for (int d = 0; d < D; ++d) s = fmaf(q[d], kr[d], s);
      s_f = s * a.scale_log2;
      if (j < a.S || j >= t - a.W + 1) s_w = s_f;
    }
    float mx_f = s_f, mx_w = s_w;
    for (int o2 = 32; o2 > 0; o2 >>= 1) {
      mx_f = fmaxf(mx_f, __shfl_xor(mx_f, o2));
      mx_w = fmaxf(mx_w, __shfl_xor(mx_w, o2));
    }
    const float mn_f = fmaxf(m_f, mx_f), mn_w = fmaxf(m_w, mx_w);
    const float mu_f = (mn_f == -INFINITY) ? 0.f : mn_f;
    const float mu_w = (mn_w == -INFINITY) ? 0.f : mn_w;
    const float al_f = fast_exp2(m_f - mu_f), al_w = fast_exp2(m_w - mu_w);
    m_f = mn_f;
    m_w = mn_w;
    const float p_f = fast_exp2(s_f - mu_f), p_w = fast_exp2(s_w - mu_w);
    l_f = l_f * al_f + p_f;
    l_w = l_w * al_w + p_w;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      acc_f[e] *= al_f;
      acc_w[e] *= al_w;
    }
    const int nk = (int)min64(64, t + 1 - k0);
    for (int jj = 0; jj < nk; ++jj) {
      const float pf = __shfl(p_f, jj), pw = __shfl(p_w, jj);
      if (pf == 0.f && pw == 0.f) continue;
      const float* vr = vb + (size_t)(k0 + jj) * D;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float x = vr[lane + 64 * e];
        acc_f[e] = fmaf(pf, x, acc_f[e]);
        acc_w[e] = fmaf(pw, x, acc_w[e]);
      }
    }
  }
  for (int o2 = 32; o2 > 0; o2 >>= 1) {
    l_f += __shfl_xor(l_f, o2);
    l_w += __shfl_xor(l_w, o2);
  }
  const float alpha = a.alpha[kvh];
  const float cf = alpha / l_f, cw = (1.f - alpha) / l_w;
  float* op = static_cast<float*>(a.out) + (((size_t)b * a.n_q + h) * a.N + t) * D;
#pragma unroll
  for (int e = 0; e < EPL; ++e) op[lane + 64 * e] = acc_f[e] * cf + acc_w[e] * cw;
}

}  // namespace

// Query heads per work item: the largest of 4, 2, 1 that divides g (each
// K / V tile then serves that many heads' rows).
int gated_heads_per_item(int dtype, int g) {
  if (dtype != 1) return 1;
  static_assert(kPfRowWaves == 4, "head packing assumes four row wavefronts");
  return (g % 4 == 0) ? 4 : (g % 2 == 0) ? 2 : 1;
}

int gated_rows_per_item(int dtype, int g) {
  if (dtype != 1) return 1;
  return kPfRowsPerWave * (kPfRowWaves / gated_heads_per_item(dtype, g));
}

hipError_t launch_gated(const GatedArgs& a, int dtype, int d, int g, hipStream_t s) {
  if (dtype == 1) {
    const int hpi = gated_heads_per_item(dtype, g);
    const int64_t blocks = (int64_t)a.B * a.n_kv * (g / hpi) * a.q_tiles;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    if (d == 128) gated_mfma_kernel<128><<<(unsigned)blocks, kPfThreads, 0, s>>>(a, g, hpi);
    else if (d == 64) gated_mfma_kernel<64><<<(unsigned)blocks, kPfThreads, 0, s>>>(a, g, hpi);
    else return hipErrorInvalidValue;
  } else {
    const int64_t blocks = ((int64_t)a.B * a.n_q * a.N + 3) / 4;
    if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
    if (d == 128) gated_f32_kernel<128><<<(unsigned)blocks, 256, 0, s>>>(a, g);
    else if (d == 64) gated_f32_kernel<64><<<(unsigned)blocks, 256, 0, s>>>(a, g);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace duo
