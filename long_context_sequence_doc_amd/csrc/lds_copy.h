// Direct global -> LDS copies for the gfx950 attention kernels, and the wait
// that publishes them.
//
// The copies are written as inline assembly rather than with the compiler's
// builtin. The builtin makes the compiler put a wait for every copy in flight
// before each transposing LDS read (ds_read_b64_tr_b16), because it cannot
// tell the LDS slots a copy writes from the ones a read takes; in the kernels'
// double-buffered loops that stalls a tile's products on the copies of the
// next tile. The assembly form writes no register, so nothing the compiler
// allocates can be overwritten by a copy in flight. The kernels copy into a
// stage only when no wave reads it, and wait for their copies themselves
// (wait_copies) before the barrier that hands the stage to the other waves.
// The statement declares no memory effect: its order against the LDS reads
// comes from those barriers (a stage is copied into only after the barrier
// that ends every read of it, and read only after the barrier that follows
// the wait), so keep every copy and every read of one stage on opposite
// sides of a barrier.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace sap {

typedef __attribute__((address_space(3))) unsigned char lds_u8;

// One copy: 16 bytes per lane from src into the LDS bytes
// [b + 16 lane, b + 16 lane + 16), b = the LDS address of lds + off, where lds
// is a kernel's LDS array and off a wave-uniform byte offset (it goes to M0).
__device__ inline void copy_to_lds(const void *src, const unsigned char *lds, int off) {
  const unsigned base = static_cast<unsigned>(reinterpret_cast<uintptr_t>((const lds_u8 *)lds)) + unsigned(off);
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(__builtin_amdgcn_readfirstlane(base)));
}

// Waits until this wave's copies (and every other vector memory access it
// issued) have completed: s_waitcnt vmcnt(0), with the expcnt and lgkmcnt
// fields at their no-wait maxima (gfx9 encoding). Written with the builtin so
// that the compiler's own wait tracking sees it.
__device__ inline void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace sap
