// Global -> LDS copy helpers shared by the phase-1 and backward kernels.
#pragma once

#include "gdn_common.h"

#define GDN_LDS __attribute__((address_space(3)))
#define GDN_GLB __attribute__((address_space(1)))

namespace gdn {

// Global -> LDS copies, issued as inline asm: lane i's bytes land at
// lds + 16 i (dma16) or lds + 4 i (dma4). The instruction has no result
// register. The compiler does not track these copies (when it does, it cannot
// tell the ring slots apart and waits for every copy in flight before any LDS
// read), so every wait for them is explicit; its own vmcnt waits can only
// over-wait because of them.
// M0 is a reserved register: clobbering it in asm is only sound because no
// other instruction of the kernels that use these helpers reads M0 (checked in
// their ISA: the only M0 writes are the ones below).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(GDN_LDS void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(m0), "v"(g)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, void* lds, bool active) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(GDN_LDS void*)lds);
  if (active)
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(m0), "v"(g)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace gdn
