// HIP kernels for gfx950 (CDNA4): cache fill, append and split-K decode over a
// per-KV-head mixed KV cache (DuoAttention: retrieval heads hold every token,
// streaming heads hold S sinks + a W-slot ring).
//
// Decode is bound by HBM bandwidth (g = n_q / n_kv flops per byte of K/V), so
// it runs on the vector ALUs, not on MFMA: K rows are staged through LDS with
// coalesced 16-byte loads, each lane then scores one key row against the g
// queries of its KV head with packed bf16 dot products, the softmax statistics
// are merged with wavefront reductions, and V rows are read with 16-byte loads
// in a d-major lane layout for the weighted sum.  Work items are uniform
// ranges of rows across both head kinds; their partial (max, sum, acc) results
// are merged in-kernel by the last-arriving work item of each group and then
// of each head.
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

template <bool BF16, int D>
struct DecodeShape {
  static constexpr int ES = BF16 ? 2 : 4;          // element bytes
  static constexpr int ROWB = D * ES;              // bytes per K/V row
  static constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
  static constexpr int EPC = 16 / ES;              // elements per chunk
  static constexpr int RPI = 64 / CPR;             // rows per wavefront load (d-major layout)
  // LDS swizzle: lane t reads chunk c of its own row t at (c ^ swz(t)); chosen
  // so that 16 consecutive lanes touch 16 distinct 16-byte bank groups.
  static constexpr int SWZ_DIV = CPR >= 16 ? 1 : 16 / CPR;
  static constexpr int SWZ_MOD = CPR >= 16 ? 16 : CPR;
  __device__ static __forceinline__ int swz(int r) { return (r / SWZ_DIV) % SWZ_MOD; }
};

// Merge `n` partial records (acc[G][D], m[G], l[G]; m in log2 units) into
// either the final output or one record at `dst_rec`.
template <bool BF16, int D, int G>
__device__ void merge_records(const float* src, int n, float* dst_rec, void* out, size_t out_off) {
  constexpr int REC = G * (D + 2);
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int h = idx / D, d = idx % D;
    float M = -INFINITY;
    for (int i = 0; i < n; ++i) M = fmaxf(M, src[(size_t)i * REC + G * D + h]);
    float L = 0.f, A = 0.f;
    for (int i = 0; i < n; ++i) {
      const float* r = src + (size_t)i * REC;
      const float w = fast_exp2(r[G * D + h] - M);
      L += r[G * D + G + h] * w;
      A += r[h * D + d] * w;
    }
    if (dst_rec) {
      dst_rec[h * D + d] = A;
      if (d == 0) {
        dst_rec[G * D + h] = M;
        dst_rec[G * D + G + h] = L;
      }
    } else {
      const float o = A / L;
      if (BF16) {
        reinterpret_cast<uint16_t*>(out)[out_off + idx] = (uint16_t)f32_to_bf16_bits(o);
      } else {
        reinterpret_cast<float*>(out)[out_off + idx] = o;
      }
    }
  }
}

template <bool BF16, int D, int G>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(DecodeArgs a) {
  using SH = DecodeShape<BF16, D>;
  constexpr int CPR = SH::CPR, EPC = SH::EPC, RPI = SH::RPI, ROWB = SH::ROWB;
  constexpr int REC = G * (D + 2);
  constexpr int NW = kDecodeThreads / 64;

  // K tiles during the row loop; afterwards the same LDS holds each
  // wavefront's accumulator for the work-item merge.
  static_assert(NW * 64 * CPR * 16 >= NW * G * D * 4, "merge buffer must fit in the K tiles");
  __shared__ uint4 k_tile[NW][64 * CPR];
  __shared__ float p_tile[NW][64 * G];
  __shared__ float w_m[NW][G], w_l[NW][G];
  __shared__ int s_ticket;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int bid = blockIdx.x;

  // ---- which head and which rows this work item covers
  int b, kvh, sp, split;
  int64_t rows;
  const char *kbase, *vbase;
  if (bid < a.blocks_ret) {
    const int hid = bid / a.split_ret;
    sp = bid % a.split_ret;
    split = a.split_ret;
    b = hid / a.n_ret;
    const int r = hid % a.n_ret;
    kvh = a.map.orig_ret[r];
    const size_t off = ((size_t)b * a.n_ret + r) * a.cap_ret * ROWB;
    kbase = a.lp.k_ret + off;
    vbase = a.lp.v_ret + off;
    rows = a.rows_ret;
  } else {
    const int x = bid - a.blocks_ret;
    const int hid = x / a.split_str;
    sp = x % a.split_str;
    split = a.split_str;
    b = hid / a.n_str;
    const int s = hid % a.n_str;
    kvh = a.map.orig_str[s];
    const size_t off = ((size_t)b * a.n_str + s) * a.cap_str * ROWB;
    kbase = a.lp.k_str + off;
    vbase = a.lp.v_str + off;
    rows = a.rows_str;
  }
  const int64_t r0 = (int64_t)sp * a.chunk;
  const int64_t r1 = min(r0 + a.chunk, rows);
  const int fh = b * a.n_kv + kvh;                         // flat head id for merge state
  const size_t q_off = ((size_t)b * a.n_q + (size_t)kvh * G) * D;  // first of the G query heads

  float m[G], l[G], acc[G][EPC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[h][e] = 0.f;
  }

  for (int64_t tb = r0 + (int64_t)wave * 64; tb < r1; tb += (int64_t)NW * 64) {
    const int nt = (int)min<int64_t>(64, r1 - tb);
    const char* kt = kbase + tb * ROWB;
    const char* vt = vbase + tb * ROWB;

    // K tile (row-major, swizzled chunks) and V tile (d-major lanes) in flight together.
    uint4 kreg[CPR], vreg[CPR];
#pragma unroll
    for (int j = 0; j < CPR; ++j) {
      const int ci = j * 64 + lane;
      const int r = ci / CPR;
      const int c = (ci % CPR) ^ SH::swz(r);
      kreg[j] = r < nt ? ld16(kt + r * ROWB + c * 16) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < CPR; ++j) {
      const int r = j * RPI + lane / CPR;
      vreg[j] = r < nt ? ld16(vt + r * ROWB + (lane % CPR) * 16) : make_uint4(0, 0, 0, 0);
    }
    wave_sync();
#pragma unroll
    for (int j = 0; j < CPR; ++j) k_tile[wave][j * 64 + lane] = kreg[j];
    wave_sync();

    // ---- scores: lane owns key row `lane`
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = 0.f;
#pragma unroll
    for (int c = 0; c < CPR; ++c) {
      const uint4 kc = k_tile[wave][lane * CPR + (c ^ SH::swz(lane))];
      if constexpr (BF16) {
        const uint32_t* q32 = reinterpret_cast<const uint32_t*>(a.q) + q_off / 2;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const uint32_t* qh = q32 + h * (D / 2) + c * 4;
          s[h] = dot2_bf16(qh[0], kc.x, s[h]);
          s[h] = dot2_bf16(qh[1], kc.y, s[h]);
          s[h] = dot2_bf16(qh[2], kc.z, s[h]);
          s[h] = dot2_bf16(qh[3], kc.w, s[h]);
        }
      } else {
        const float* qf = reinterpret_cast<const float*>(a.q) + q_off;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float* qh = qf + h * D + c * 4;
          s[h] = fmaf(qh[0], __uint_as_float(kc.x), s[h]);
          s[h] = fmaf(qh[1], __uint_as_float(kc.y), s[h]);
          s[h] = fmaf(qh[2], __uint_as_float(kc.z), s[h]);
          s[h] = fmaf(qh[3], __uint_as_float(kc.w), s[h]);
        }
      }
    }

    // ---- online softmax (log2 domain)
    float alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float sv = lane < nt ? s[h] * a.scale_log2 : -INFINITY;
      const float mn = fmaxf(m[h], wave_max(sv));
      alpha[h] = fast_exp2(m[h] - mn);
      const float p = fast_exp2(sv - mn);
      l[h] = l[h] * alpha[h] + p;
      m[h] = mn;
      p_tile[wave][lane * G + h] = p;
    }
    wave_sync();

    // ---- weighted sum of V: lane owns chunk (lane % CPR) of rows j*RPI + lane/CPR
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[h][e] *= alpha[h];
#pragma unroll
    for (int j = 0; j < CPR; ++j) {
      const int r = j * RPI + lane / CPR;
      float v[EPC];
      if constexpr (BF16) {
        v[0] = bf_lo(vreg[j].x); v[1] = bf_hi(vreg[j].x);
        v[2] = bf_lo(vreg[j].y); v[3] = bf_hi(vreg[j].y);
        v[4] = bf_lo(vreg[j].z); v[5] = bf_hi(vreg[j].z);
        v[6] = bf_lo(vreg[j].w); v[7] = bf_hi(vreg[j].w);
      } else {
        v[0] = __uint_as_float(vreg[j].x); v[1] = __uint_as_float(vreg[j].y);
        v[2] = __uint_as_float(vreg[j].z); v[3] = __uint_as_float(vreg[j].w);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = p_tile[wave][r * G + h];
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][e] = fmaf(p, v[e], acc[h][e]);
      }
    }
  }

  // ---- wavefront result: sum the RPI row groups of each d-chunk, then the row sums
#pragma unroll
  for (int o = CPR; o < 64; o <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[h][e] += __shfl_xor(acc[h][e], o);
#pragma unroll
  for (int h = 0; h < G; ++h) l[h] = wave_sum(l[h]);
  __syncthreads();  // every wavefront is done with its K tile
  float (*w_acc)[G * D] = reinterpret_cast<float (*)[G * D]>(&k_tile[0][0]);
  if (lane < CPR) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPC; ++e) w_acc[wave][h * D + lane * EPC + e] = acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      w_m[wave][h] = m[h];
      w_l[wave][h] = l[h];
    }
  }
  __syncthreads();

  // ---- work-item result from the NW wavefronts (a wavefront without rows has m = -inf)
  const size_t out_off = q_off;
  float* rec = a.ws1 + (size_t)bid * REC;
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int h = idx / D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, w_m[w][h]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(w_m[w][h] - M);
      L += w_l[w][h] * f;
      A += w_acc[w][idx] * f;
    }
    if (split == 1) {
      const float o = A / L;
      if (BF16) {
        reinterpret_cast<uint16_t*>(a.out)[out_off + idx] = (uint16_t)f32_to_bf16_bits(o);
      } else {
        reinterpret_cast<float*>(a.out)[out_off + idx] = o;
      }
    } else {
      rec[idx] = A;
      if ((idx % D) == 0) {
        rec[G * D + h] = M;
        rec[G * D + G + h] = L;
      }
    }
  }
  if (split == 1) return;

  // ---- first-level merge: the last work item of each group of kSplitGroup
  const int grp = sp / kSplitGroup;
  const int g0 = grp * kSplitGroup;
  const int gsz = min(kSplitGroup, split - g0);
  const int ngrp = (split + kSplitGroup - 1) / kSplitGroup;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_ticket = atomicAdd(&a.lp.cnt1[fh * kMaxGroups + grp], 1);
  __syncthreads();
  if (s_ticket != gsz - 1) return;
  __threadfence();
  if (threadIdx.x == 0) a.lp.cnt1[fh * kMaxGroups + grp] = 0;
  const float* grp_src = a.ws1 + (size_t)(bid - sp + g0) * REC;
  if (ngrp == 1) {
    merge_records<BF16, D, G>(grp_src, gsz, nullptr, a.out, out_off);
    return;
  }
  float* grp_dst = a.ws2 + ((size_t)fh * kMaxGroups + grp) * REC;
  merge_records<BF16, D, G>(grp_src, gsz, grp_dst, nullptr, 0);

  // ---- second-level merge: the last group of the head
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_ticket = atomicAdd(&a.lp.cnt2[fh], 1);
  __syncthreads();
  if (s_ticket != ngrp - 1) return;
  __threadfence();
  if (threadIdx.x == 0) a.lp.cnt2[fh] = 0;
  merge_records<BF16, D, G>(a.ws2 + (size_t)fh * kMaxGroups * REC, ngrp, nullptr, a.out, out_off);
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
