// Direct buffer->LDS loads for the HIP kernels (gfx950), shared by the decode,
// prefill and gated kernels.
//
// A wavefront-wide direct load reads one 16-byte (or 4-byte) piece per lane
// from a buffer resource and writes it straight into LDS: lane i writes LDS
// bytes [lds + 16 i, lds + 16 i + 16) from byte offset voff of the resource;
// offsets out of the resource's range read as zero.
//
// Written as inline assembly on purpose: the load has no register result
// (its data goes to LDS), and the compiler, not knowing that it writes LDS,
// adds no wait of its own before later LDS reads.  (Through the builtin, the
// compiler treats every LDS read after the load as a possible reader of its
// data and waits for the load first, so a tile prefetched for the next step
// is waited for before the current tile is read.)  Each kernel therefore
// orders every read of a tile after its loads itself, by an explicit vmcnt
// wait and a workgroup barrier.  The "memory" clobber stops the compiler from
// assuming LDS contents across the load.  M0 (the LDS base of the load) is
// saved and restored.
//
// The compiler's own vmcnt waits for ordinary loads stay correct: it counts
// fewer loads in flight than there are (it does not see these), so its waits
// are stricter than needed, never weaker.
//
// Only included by the HIP sources of this library; everything is internal.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace duo {
namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Raw (untyped) buffer resource over [base, base + nbytes), stride 0.
__device__ __forceinline__ i32x4_t dma_rsrc(const char* base, int nbytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return i32x4_t{(int)__builtin_amdgcn_readfirstlane((uint32_t)b),
                 (int)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xffffu),  // stride 0
                 __builtin_amdgcn_readfirstlane(nbytes), 0x00020000};                 // raw buffer
}

// LDS byte address of a pointer into LDS (a workgroup-uniform value).
__device__ __forceinline__ uint32_t lds_addr(const void* lds) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(size_t)(const __attribute__((address_space(3))) char*)(const char*)lds);
}

// The load with its LDS destination given as an LDS byte address, reading
// from byte offset voff + soff of the resource (soff the same in every lane).
__device__ __forceinline__ void dma_lds16_at(i32x4_t rsrc, uint32_t m0v, uint32_t voff, uint32_t soff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0v), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}

__device__ __forceinline__ void dma_lds16(i32x4_t rsrc, char* lds, uint32_t voff) {
  dma_lds16_at(rsrc, lds_addr(lds), voff, 0);
}

// The same with 4 bytes per lane: lane i writes LDS bytes [m0v + 4 i, m0v + 4 i + 4),
// m0v an LDS byte address.
__device__ __forceinline__ void dma_lds4_at(i32x4_t rsrc, uint32_t m0v, uint32_t voff) {
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

__device__ __forceinline__ void dma_lds4(i32x4_t rsrc, char* lds, uint32_t voff) {
  dma_lds4_at(rsrc, lds_addr(lds), voff);
}

}  // namespace
}  // namespace duo
