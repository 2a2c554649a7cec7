// Loads that write LDS straight from memory (no register) on gfx950, for the expert kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace eff {

// LDS byte address of a shared array (uniform)
template <typename T>
__device__ inline uint32_t lds_address(T* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)((__attribute__((address_space(3))) T*)p));
}

// 16 bytes per lane from src (the lane's own address) straight into LDS at lds + 16 * lane (lds
// uniform), without a register: global_load_lds_dwordx4.  The compiler does not see this write, so the
// caller waits for it with vm_wait before anything reads the bytes.  It sets M0, which no other code
// in these kernels uses (M0 is on the clobber list).
__device__ inline void lds_copy16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(lds), "v"(src) : "memory", "m0");
}

// waits until at most N vector memory operations of this wave are outstanding.  Loads complete in the
// order they were issued, so once N is the number of loads issued after a given LDS copy, that copy
// is complete (stores issued meanwhile only make the wait stricter).
template <int N>
__device__ inline void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

}  // namespace eff
