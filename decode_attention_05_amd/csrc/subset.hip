// The structured subset of attended body rows: sinks, a stride through the
// middle and a recent window, as CSR.  Every count and index has a closed
// form, so one workgroup per sequence writes its list directly; the offsets
// sum the closed-form counts of the sequences before it.
#include "subset_internal.h"

namespace lowram {

// |A| for n body rows (see lowram_subset.h); the middle is [s, w)
__host__ __device__ int64_t subset_count(int64_t n, int n_sink, int n_recent, int stride) {
  const int64_t s = n < n_sink ? n : n_sink;
  const int64_t w = (n - n_recent > s) ? n - n_recent : s;
  const int64_t mid = (stride > 0 && w > s) ? (w - s + stride - 1) / stride : 0;
  return s + mid + (n - w);
}

namespace {

__global__ void __launch_bounds__(256) subset_kernel(const int32_t *n_body, int N, int B, int n_sink,
                                                     int n_recent, int stride, int32_t *off, int32_t *idx) {
  const int b = blockIdx.x;
  __shared__ int64_t s_base;
  if (threadIdx.x == 0) {
    int64_t base = 0;
    for (int q = 0; q < b; ++q) base += subset_count(max(min(n_body[q], N), 0), n_sink, n_recent, stride);
    s_base = base;
    off[b] = (int32_t)base;
    if (b == B - 1) off[B] = (int32_t)(base + subset_count(max(min(n_body[b], N), 0), n_sink, n_recent, stride));
  }
  __syncthreads();
  const int64_t n = max(min(n_body[b], N), 0);   // lengths outside [0, N] are clamped
  const int64_t s = n < n_sink ? n : n_sink;
  const int64_t w = (n - n_recent > s) ? n - n_recent : s;
  const int64_t mid = (stride > 0 && w > s) ? (w - s + stride - 1) / stride : 0;
  const int64_t cnt = s + mid + (n - w);
  int32_t *out = idx + s_base;
  for (int64_t k = threadIdx.x; k < cnt; k += blockDim.x) {
    int64_t t;
    if (k < s) t = k;
    else if (k < s + mid) t = s + (k - s) * stride;
    else t = w + (k - s - mid);
    out[k] = (int32_t)t;
  }
}

}  // namespace

hipError_t launch_subset(const int32_t *n_body, int N, int B, int n_sink, int n_recent, int stride,
                         int32_t *off, int32_t *idx, hipStream_t st) {
  hipLaunchKernelGGL(subset_kernel, dim3(B), dim3(256), 0, st, n_body, N, B, n_sink, n_recent, stride, off, idx);
  return hipGetLastError();
}

}  // namespace lowram
