// Measurement aids of the library (not on the decode path): the matrix-core
// throughput probe.  The read-ceiling probe is declared with the cache
// kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace pkv {

// workgroups x 4 wavefronts, each running `iterations` rounds of eight
// independent v_mfma_f32_16x16x32_bf16 chains (16,384 FLOPs per
// instruction) on register operands; sink (device, 4 bytes) is written only
// if the accumulators sum to a fixed key.
hipError_t launch_mfma_peak(float* sink, int workgroups, int iterations, hipStream_t stream);

}  // namespace pkv
