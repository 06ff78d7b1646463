// Split combine and epilogue of decode attention.
//
// Each split of the attended rows leaves a record (M, L, acc1, acc_h[d],
// acc_v[d]) for one (sequence, query head): M is the split's largest score,
// L = sum exp(s - M), acc1 = sum exp(s - M) over body rows, acc_h the same
// weighted sum of the predictor's hidden activations, and acc_v the weighted
// sum of everything already in value space (residuals, tail values, or whole
// values when the kernel does not hoist W2).  The records are merged by
// log-sum-exp and the output is
//   out = (W2 acc_h + b2 acc1 + acc_v) / L,   lse = M + ln L,
// where moving W2 out of the row sum is exact algebra:
//   sum_t p_t (W2 h_t + b2) = W2 (sum_t p_t h_t) + b2 sum_t p_t.
// (Flash-decoding style split of softmax attention; the value predictor is
// the per-head MLP of "Value cache amortisation in plain language",
// "LowRAM Paper: Amortised Values and Low-Rank Keys for KV Compression".)
#include "lowram_internal.h"

namespace lowram {
namespace {

template <typename DT>
__global__ void __launch_bounds__(128) combine_kernel(DecodeArgs a, int hoisted) {
  const Dims s = a.s;
  const int d = s.d, j = threadIdx.x;
  const int b = blockIdx.x / s.Hq, qh = blockIdx.x % s.Hq, h = qh / s.grp;
  const int ps = part_stride(d);
  const float *rec = a.partials + ((int64_t)b * s.Hq + qh) * a.n_splits * ps;
  __shared__ float sh_h[128];

  float Mx = -INFINITY;
  for (int sp = 0; sp < a.n_splits; ++sp) Mx = fmaxf(Mx, rec[sp * ps]);
  DT *out = reinterpret_cast<DT *>(a.out);
  const int64_t o = ((int64_t)b * s.Hq + qh) * d + j;
  if (Mx == -INFINITY) {                    // nothing attended
    stf(out, o, 0.f);
    if (a.lse && j == 0) a.lse[(int64_t)b * s.Hq + qh] = -INFINITY;
    return;
  }
  float L = 0.f, a1 = 0.f, ah = 0.f, av = 0.f;
  for (int sp = 0; sp < a.n_splits; ++sp) {
    const float *r = rec + sp * ps;
    const float w = __expf(r[0] - Mx);
    L += w * r[1];
    a1 += w * r[2];
    ah += w * r[4 + j];
    av += w * r[4 + d + j];
  }
  float v = av;
  if (hoisted) {
    sh_h[j] = ah;
    __syncthreads();
    const int pb = s.pred_shared ? 0 : b;
    const int64_t wo = ((int64_t)pb * s.G + a.layer) * s.H + h;
    const DT *W2 = reinterpret_cast<const DT *>(a.c.w2) + wo * d * d;
    const DT *B2 = reinterpret_cast<const DT *>(a.c.b2) + wo * d;
    float t = 0.f;
    for (int u = 0; u < d; ++u) t += ldf(W2, (int64_t)j * d + u) * sh_h[u];
    v += t + ldf(B2, j) * a1;
  }
  stf(out, o, v / L);
  if (a.lse && j == 0) a.lse[(int64_t)b * s.Hq + qh] = Mx + logf(L);
}

}  // namespace

hipError_t launch_combine(const DecodeArgs &a, bool hoisted, hipStream_t st) {
  dim3 grid(a.s.B * a.s.Hq), block(a.s.d);
  if (a.s.dtype == LOWRAM_F32)
    hipLaunchKernelGGL((combine_kernel<float>), grid, block, 0, st, a, (int)hoisted);
  else
    hipLaunchKernelGGL((combine_kernel<bf16_t>), grid, block, 0, st, a, (int)hoisted);
  return hipGetLastError();
}

}  // namespace lowram
