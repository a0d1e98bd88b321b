// launch.h -- the kernel launch of every entry point in this library.
//
// hipLaunchKernel returns the status of the launch it makes, so a failure is
// reported by the call that caused it: an error left behind by an earlier HIP
// call of the caller is neither blamed on this launch nor consumed by it.
#pragma once

#include <hip/hip_runtime.h>

#include <tuple>

// Maps a launch result to a library status (TESSERA_OK or
// TESSERA_ERR_LAUNCH) and, on failure, keeps the HIP error text for
// tessera_attn_last_error() on the calling thread.  Defined in
// tessera_attn.hip.
__attribute__((visibility("hidden"))) int tessera_launch_result(hipError_t e);

// Checks the arguments of a forward entry point (pointers, sizes, causal,
// scale, alignment, aliasing of out and lse with the inputs; `elem` is the
// element size in bytes) and returns TESSERA_OK or the status to return.
// Defined in tessera_attn.hip.
__attribute__((visibility("hidden"))) int
tessera_validate_fwd(const void *q, const void *k, const void *v, const void *out, const void *lse,
                     int B, int Hq, int Hkv, int Tq, int Tk, int D, int causal, float scale,
                     size_t elem);

// Launches `kernel` on `stream` with no dynamic LDS.  Each argument is
// converted to the kernel's parameter type and held here until
// hipLaunchKernel has copied it.
template <typename... P, typename... A>
__attribute__((visibility("hidden"))) inline int
tessera_launch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream, A... args) {
    static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
    std::tuple<P...> held{static_cast<P>(args)...};
    return std::apply(
        [&](auto &...x) {
            void *argv[] = {(void *)&x...};
            return tessera_launch_result(
                hipLaunchKernel((const void *)kernel, grid, block, argv, 0, stream));
        },
        held);
}
