// Device helpers shared by the LDS-streaming kernels (gfx950): the LDS-DMA
// copy, explicit memory-counter waits and the decode work-record read.
#pragma once

#include "kernels.h"
#include "stage_layout.h"

namespace mla {
namespace ddev {

// One wave-wide 16-byte-per-lane copy global -> LDS.  The LDS destination is
// M0 + 16 * lane (a 1 KB block per instruction).  Issued from inline asm so the
// compiler neither reorders it nor adds its own (conservative) waits; the
// kernels wait with explicit s_waitcnt vmcnt.  An SALU write of M0 needs one
// wait state before an LDS-DMA load.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_addr)
               : "memory", "m0");
}

// The same copy with the non-temporal hint, for cache rows a launch reads
// exactly once (no other workgroup of the part streams them): streamed lines
// do not displace reused data in L2, and on gfx950 this copy then reaches
// ~7.1 TB/s from HBM against ~6 TB/s without the hint (measured, 1 GiB
// streamed by one workgroup per compute unit).
__device__ __forceinline__ void dma16_nt(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(g), "s"(lds_addr)
               : "memory", "m0");
}

template <bool NT>
__device__ __forceinline__ void dma16h(const void* g, uint32_t lds_addr) {
  if constexpr (NT) dma16_nt(g, lds_addr);
  else dma16(g, lds_addr);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

typedef const __attribute__((address_space(4))) DecodeWork* ConstWorkPtr;

// Field by field: a constant-address-space object cannot bind to the implicit
// copy constructor.  Read through the constant address space, the records stay
// on scalar loads.
__device__ __forceinline__ DecodeWork load_work(ConstWorkPtr p) {
  DecodeWork w;
  w.row = p->row;
  w.n = p->n;
  w.b = p->b;
  w.pidx = p->pidx;
  w.next = p->next;
  w.nseg = p->nseg;
  w.pstart = p->pstart;
  return w;
}

// Cache row of position r of a work record's segment (r counted from the
// segment's first position; a tile start, so a tile never crosses a page:
// segments start on multiples of 32 positions and pages hold 2^k >= 32 rows).
// The page list is read through the constant address space (scalar loads).
__device__ __forceinline__ int64_t seg_row(const DecodeMeta& mt, int64_t wrow, int r) {
  if (mt.page_shift == 0) return wrow + r;
  typedef const __attribute__((address_space(4))) int32_t* ConstI32Ptr;
  const int32_t pg = (int32_t)(wrow >> 32);
  const int32_t t = (int32_t)(wrow & 0x7fffffff) + r;
  const int32_t page = reinterpret_cast<ConstI32Ptr>((uintptr_t)mt.pages)[pg + (t >> mt.page_shift)];
  return ((int64_t)page << mt.page_shift) + (t & ((1 << mt.page_shift) - 1));
}

// Rows of a work record's segment that token j (of q_len) sees: all of them,
// except on the sequence's last segment, where the tokens after j are not
// visible to it.
__device__ __forceinline__ int token_rows(const DecodeWork& w, int q_len, int j) {
  return w.pidx == w.pstart + w.nseg - 1 ? w.n - (q_len - 1 - j) : w.n;
}

}  // namespace ddev
}  // namespace mla
