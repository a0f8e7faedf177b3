// Tag of a kernel launch, for words that workgroups of one launch publish to
// each other: a word that carries the current launch's tag was written by this
// launch, one left by an earlier launch carries another tag, so such words
// never need to be reset between launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// The launch's dispatch id (a user SGPR the command processor sets for every
// dispatch), through the LLVM intrinsic that reads it.
extern "C" __device__ uint64_t nvfp4_llvm_dispatch_id() __asm("llvm.amdgcn.dispatch.id");

namespace nvfp4 {

// The dispatch id mixed with the queue address (dispatch ids count per queue);
// never 0, the value of a word nothing has written.
__device__ __forceinline__ uint64_t launch_tag() {
    const uint64_t q = (uint64_t)(uintptr_t)__builtin_amdgcn_queue_ptr();
    const uint64_t h = ((nvfp4_llvm_dispatch_id() + 1) * 0x9E3779B97F4A7C15ull) ^ (q * 0xC2B2AE3D27D4EB4Full);
    return h | 1u;
}

}  // namespace nvfp4
