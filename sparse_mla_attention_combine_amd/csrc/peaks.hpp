// Throughput probes (measurement only, not steps of the method): `workgroups` x 256
// threads; sink holds workgroups * 256 values.  launch_peak_mfma sets *flops to the
// launch's dense FLOPs.
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace dsv4 {

hipError_t launch_peak_mfma(int shape, int workgroups, int iters, float* sink, double* flops,
                            hipStream_t stream);
hipError_t launch_peak_stream(const void* src, void* dst, size_t bytes, uint32_t* sink,
                              int workgroups, hipStream_t stream);

}  // namespace dsv4
