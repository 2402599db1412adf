// Register-ring software pipeline, one lane's view.
//
// The Pallas software-pipelining guide, section 4, overlaps the copy of step
// i+1 with the compute of step i (double buffering; section 4.1 packages it
// as double_buffered_pipeline) and generalises to more buffers.  In a GPU
// lane the buffers are registers.  ring_pipeline<S> keeps the loads of the
// next S steps in flight, consumes the steps in ascending order and refills
// a slot right after consuming it:
//   copy_start  = load(i, slot), issued S steps before step i is consumed;
//   copy_wait   = the compiler's s_waitcnt before the first use of the slot;
//   compute     = compute(i, slot);
//   release     = the slot is reloaded for step i+S right after compute.
// Steps are consumed strictly in order 0, 1, ..., steps-1, so a compute that
// accumulates (the guide's section 7.2 reduction) sees the same order as the
// plain loop.  The ring is indexed only with compile-time slot numbers (the
// loop is unrolled by S), so it lives in VGPRs.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pgemm {

template <int S, class Slot, class Load, class Compute>
__device__ __forceinline__ void ring_pipeline(int64_t steps, Load&& load, Compute&& compute) {
    static_assert(S >= 1, "at least one buffer");
    Slot ring[S];
#pragma unroll
    for (int s = 0; s < S; ++s)  // prologue: copy_start of steps 0 .. S-1
        if (s < steps) load((int64_t)s, ring[s]);
    int64_t i = 0;
    for (; i + S <= steps; i += S) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            compute(i + s, ring[s]);
            if (i + s + S < steps) load(i + s + S, ring[s]);
        }
    }
#pragma unroll
    for (int s = 0; s < S; ++s)  // epilogue: the last steps, already loaded
        if (i + s < steps) compute(i + s, ring[s]);
}

}  // namespace pgemm
