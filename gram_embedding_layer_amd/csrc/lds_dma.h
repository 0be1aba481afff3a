// The global-to-LDS load the projection's A and W loaders and the stand-alone LDS gather
// share: 16 bytes per lane straight from global memory into LDS, no register round trip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ngram {

typedef __attribute__((address_space(3))) char lds_char;

// LDS byte address of a __shared__ object (the m0 operand of the load below).
__device__ __forceinline__ uint32_t lds_address(const char* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const lds_char*)p));
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane
// (global_load_lds_dwordx4). Written as asm so that its completion is waited for only by
// explicit vmcnt waits (the compiler would otherwise drain every load in flight before each
// LDS read); it has no register result. The LDS address is an input operand bound to m0
// ("{m0}"), so the compiler itself writes m0 before the instruction and knows that m0 holds
// this value: nothing of its own can be lost. The s_nop covers the one wait state an LDS DMA
// needs after an m0 write. Lanes outside EXEC load nothing.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\t"
               "global_load_lds_dwordx4 %0, off"
               :: "v"(gptr), "{m0}"(lds_addr) : "memory");
}

}  // namespace ngram
