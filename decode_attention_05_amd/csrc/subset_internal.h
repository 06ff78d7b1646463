// Internal declarations of the structured subset selection.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowram {

// |A| for n body rows under the policy (sinks, stride, recent window)
__host__ __device__ int64_t subset_count(int64_t n, int n_sink, int n_recent, int stride);
hipError_t launch_subset(const int32_t *n_body, int N, int B, int n_sink, int n_recent, int stride,
                         int32_t *off, int32_t *idx, hipStream_t st);

}  // namespace lowram
