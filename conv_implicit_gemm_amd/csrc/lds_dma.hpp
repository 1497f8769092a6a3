// lds_dma.hpp -- gfx950 operand staging by DMA into LDS, and transposed LDS
// reads that turn a staged tile into MFMA fragments.
//
// buffer_load_dwordx4 ... lds moves 16 bytes per lane from global memory
// straight into LDS: lane l's bytes land at (M0 + 16*l), so one wave
// instruction fills 1 KB of LDS with no VGPR holding the data while it is in
// flight.  A kernel can therefore keep several stages of operands in flight
// per block (bytes in flight is what an HBM-bound kernel is short of).  The
// order of the 16-byte pieces inside that 1 KB is free: each lane chooses
// which global piece it fetches, which is how the tiles below are swizzled.
//
// The loads are issued from inline assembly on purpose: for the builtin, the
// compiler cannot tell ring slots apart and waits for every outstanding DMA
// before each LDS read, which serialises the ring.  Here the kernel counts
// its own DMA instructions and waits with an explicit vmcnt before the
// barrier that publishes a stage (wait_dma_barrier).  Kernels that use these
// helpers issue no other vector-memory load between a DMA and its wait (a
// load issued before the DMAs only makes the wait more conservative:
// vmcnt counts in issue order).
//
// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane i's
// element t (t = 0..3) is element (i % 4) of the 8 bytes that lane
// 4*t + i/4 addresses.  If lane j of a group addresses row r0 + j/4, columns
// c0 + 4*(j%4) .. +3 of a row-major 16-bit tile, lane i receives column
// c0 + i at rows r0 .. r0+3: a 4x16 transpose, i.e. four consecutive k of
// one MFMA row when rows are k.  Two such reads give the eight k of a
// 32x32x16 bf16 fragment from a tile stored k-major (pixel-contiguous rows
// of an NCHW image), with no repacking in registers.
#pragma once

#include "engine.hpp"

namespace ox {

#define OX_LDS __attribute__((address_space(3)))

typedef short i16x4_t __attribute__((ext_vector_type(4)));

// Raw-buffer descriptor words: base address, range in bytes (a load whose
// offset is at or past the range returns zeros), 32-bit raw access.
__device__ __forceinline__ u32x4_t buffer_words(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  return u32x4_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// An offset past every tensor a kernel reads: with the tensor below 2^30
// bytes, adding chunk steps to it never wraps below the range.
constexpr uint32_t kDmaOutside = 0x80000000u;

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const OX_LDS char*)p;
}

// 16 bytes per lane: global [rsrc + voff] -> LDS [lds + 16*lane].  lds must
// be the same in every lane of the wave.
// (M0 is bound as an input operand, so the compiler writes it and knows it
// is in use; the nop keeps one wait state between that write and the DMA.)
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, u32x4_t rsrc) {
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rsrc), "{m0}"(lds)
      : "memory");
}

// 4 bytes per lane: global [rsrc + voff] -> LDS [lds + 4*lane] (packed:
// one wave instruction fills 256 contiguous bytes).  The 2-byte form does not
// pack (each lane still fills a dword), so no narrower form is offered.
__device__ __forceinline__ void dma4(uint32_t lds, uint32_t voff, u32x4_t rsrc) {
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dword %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rsrc), "{m0}"(lds)
      : "memory");
}

// Wait until at most N of this wave's vector-memory instructions are
// outstanding and all its LDS reads have returned, then the workgroup
// barrier: every wave's DMA of the stage is then in LDS and no wave still
// reads the slot the next DMA reuses.
template <int N>
__device__ __forceinline__ void wait_dma_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations have
// completed; outstanding DMA and global stores are not waited for.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

// The same with N chosen at run time among 0, D, 2D, .. (R+1 cases).
template <int D, int R>
__device__ __forceinline__ void wait_dma_barrier_rt(int n) {
  if constexpr (R == 0) {
    wait_dma_barrier<0>();
  } else {
    if (n >= R) wait_dma_barrier<D * R>();
    else wait_dma_barrier_rt<D, R - 1>(n);
  }
}

// Transposed 16-bit read (see above): 4 values as two dwords.
__device__ __forceinline__ u32x2_t lds_read_tr16(uint32_t addr) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((OX_LDS i16x4_t*)(uintptr_t)addr);
  return __builtin_bit_cast(u32x2_t, v);
}

__device__ __forceinline__ u32x4_t lds_read_b128(uint32_t addr) {
  return *(const OX_LDS u32x4_t*)(uintptr_t)addr;
}

}  // namespace ox
