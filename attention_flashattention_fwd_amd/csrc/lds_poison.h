// lds_poison.h -- the LDS-poisoned debug build of the library.
//
// The kernels order their LDS traffic by hand: explicit vmcnt waits for the
// loads that go from global memory straight into LDS, and barriers between a
// buffer's last reader and its refill.  A missing wait or barrier shows only
// as a timing race, and a launch that follows an identical one finds the
// previous launch's data still in LDS, which hides a read that comes too
// early.  Built with -DTESSERA_LDS_POISON (the library's build script makes
// it as a second library beside the production one):
//   * every kernel first fills its whole static LDS with 0xFFFFFFFF, a NaN as
//     bf16 and as fp32, and
//   * every global->LDS load first writes the same pattern over the 16 bytes
//     per lane that it is about to fill, and waits for that write,
// so a read that comes before its data has landed, or after a refill has
// been issued, reads NaN, and the NaN reaches the outputs through the
// products.  A correct kernel never reads the pattern, so the debug build's
// outputs equal the production build's bit for bit.  Without the macro
// both helpers are empty.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifdef TESSERA_LDS_POISON
constexpr uint32_t kLdsPoison = 0xFFFFFFFFu;

// All of the workgroup's static LDS, then a barrier.  Called by every thread
// of the workgroup before its first LDS access (the kernels use no dynamic
// LDS, so static LDS is all there is, from address 0).
__device__ __forceinline__ void lds_poison_all() {
    const uint32_t bytes = __builtin_amdgcn_groupstaticsize();
    for (uint32_t b = threadIdx.x * 4; b + 4 <= bytes; b += blockDim.x * 4)
        asm volatile("ds_write_b32 %0, %1" : : "v"(b), "v"(kLdsPoison) : "memory");
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
    __syncthreads();
}

// The 16 bytes a global->LDS dwordx4 load of this lane writes at LDS byte
// address lds + 16 * lane; the wait makes the pattern land before the load
// is issued (LDS writes of the load itself arrive later).
__device__ __forceinline__ void lds_poison_lane16(uint32_t lds) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const u32x4 pat = {kLdsPoison, kLdsPoison, kLdsPoison, kLdsPoison};
    asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                 :
                 : "v"(lds + 16 * lane), "v"(pat)
                 : "memory");
}
#else
__device__ __forceinline__ void lds_poison_all() {}
__device__ __forceinline__ void lds_poison_lane16(uint32_t) {}
#endif
