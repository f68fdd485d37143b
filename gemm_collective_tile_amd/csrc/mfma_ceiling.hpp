// The dense fp16 MFMA rate of the chip with no memory traffic (a measuring
// kernel, apart from the fused ops). See mfma_ceiling.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iris {

// Runs the measuring kernel on `grid` workgroups of 256 threads, `iters`
// loop trips each, on stream `s` (after one short warm-up launch) and waits
// for it. *ms: the timed launch's duration; *cycles, *ticks: the shader-clock
// and constant-rate counter intervals summed over its workgroups.
hipError_t mfma_ceiling_run(bool random_operands, int iters, int grid, hipStream_t s, float* ms, double* cycles,
                            double* ticks);

// FLOP of one workgroup's loop trip: 4 waves x 8 MFMAs of 32x32x16.
constexpr double kCeilingFlopPerTrip = 4.0 * 8.0 * 2.0 * 32 * 32 * 16;

}  // namespace iris
