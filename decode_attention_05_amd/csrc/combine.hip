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

constexpr int kMaxSplits = 4096;

template <typename DT>
__global__ void __launch_bounds__(128) combine_kernel(DecodeArgs a, int hoisted) {
  const Dims s = a.s;
  const int d = s.d, j = threadIdx.x;
  const int b = blockIdx.x / s.Hq, qh = blockIdx.x % s.Hq, h = qh / s.grp;
  const int ps = part_stride(d);
  const int ns = a.n_splits;
  const float *rec = a.partials + ((int64_t)b * s.Hq + qh) * ns * ps;
  __shared__ float sh_h[128];
  __shared__ float sw[kMaxSplits];
  __shared__ float sLs[kMaxSplits], s1s[kMaxSplits];
  __shared__ float sM, sL, s1;
  // Every load is issued before the first reduction: the record heads
  // (M, L, acc1) of all splits into registers/LDS, this thread's element of
  // the first kPre records, and its row of W2.
  constexpr int kPre = 16;
  float xh[kPre], xv[kPre];
  const bool el = j < d;
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const bool ok = el && u < ns;
    xh[u] = ok ? rec[(int64_t)u * ps + 4 + j] : 0.f;
    xv[u] = ok ? rec[(int64_t)u * ps + 4 + d + j] : 0.f;
  }
  const int pb = s.pred_shared ? 0 : b;
  const int64_t wo = ((int64_t)pb * s.G + a.layer) * s.H + h;
  const DT *W2 = reinterpret_cast<const DT *>(a.c.w2) + wo * d * d;
  const DT *B2 = reinterpret_cast<const DT *>(a.c.b2) + wo * d;
  uint4 wv[16];
  if (hoisted && sizeof(DT) == 2 && el) {
    const uint4 *w2r = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(W2) + (int64_t)j * d);
#pragma unroll
    for (int uc = 0; uc < 16; ++uc) wv[uc] = (8 * uc < d) ? w2r[uc] : uint4{0u, 0u, 0u, 0u};
  }
  float bias = (hoisted && el) ? ldf(B2, j) : 0.f;
  // record heads (M, L, acc1) of all splits, one 16-byte load each
  for (int sp = j; sp < ns; sp += blockDim.x) {
    const float4 hd = *reinterpret_cast<const float4 *>(rec + (int64_t)sp * ps);
    sw[sp] = hd.x;
    sLs[sp] = hd.y;
    s1s[sp] = hd.z;
  }
  __syncthreads();
  if (j < 64) {
    float mx = -INFINITY;
    for (int sp = j; sp < ns; sp += 64) mx = fmaxf(mx, sw[sp]);
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float L = 0.f, a1 = 0.f;
    if (mx != -INFINITY)
      for (int sp = j; sp < ns; sp += 64) {
        const float w = __expf(sw[sp] - mx);
        L += w * sLs[sp];
        a1 += w * s1s[sp];
      }
    for (int o = 32; o > 0; o >>= 1) { L += __shfl_xor(L, o, 64); a1 += __shfl_xor(a1, o, 64); }
    if (j == 0) { sM = mx; sL = L; s1 = a1; }
  }
  __syncthreads();
  const float Mx = sM;
  for (int sp = j; sp < ns; sp += blockDim.x) sw[sp] = (Mx == -INFINITY) ? 0.f : __expf(sw[sp] - Mx);
  __syncthreads();
  DT *out = reinterpret_cast<DT *>(a.out);
  const int64_t o = ((int64_t)b * s.Hq + qh) * d + j;
  if (Mx == -INFINITY) {                    // nothing attended
    if (el) stf(out, o, 0.f);
    if (a.lse && j == 0) a.lse[(int64_t)b * s.Hq + qh] = -INFINITY;
    return;
  }
  float ah = 0.f, av = 0.f;
  if (el) {
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      if (u < ns) {
        ah += sw[u] * xh[u];
        av += sw[u] * xv[u];
      }
    }
    // remaining records, 8 in flight per batch
    int sp = kPre;
    for (; sp + 8 <= ns; sp += 8) {
      float yh[8], yv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        yh[u] = rec[(int64_t)(sp + u) * ps + 4 + j];
        yv[u] = rec[(int64_t)(sp + u) * ps + 4 + d + j];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        ah += sw[sp + u] * yh[u];
        av += sw[sp + u] * yv[u];
      }
    }
    for (; sp < ns; ++sp) {
      ah += sw[sp] * rec[(int64_t)sp * ps + 4 + j];
      av += sw[sp] * rec[(int64_t)sp * ps + 4 + d + j];
    }
  }
  float v = av;
  if (hoisted) {
    if (el) sh_h[j] = ah;
    __syncthreads();
    if (el) {
      float t = 0.f;
      if (sizeof(DT) == 2) {
#pragma unroll
        for (int uc = 0; uc < 16; ++uc) {
          if (8 * uc >= d) break;
          const uint32_t ww[4] = {wv[uc].x, wv[uc].y, wv[uc].z, wv[uc].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            t += __uint_as_float(ww[e] << 16) * sh_h[8 * uc + 2 * e];
            t += __uint_as_float(ww[e] & 0xffff0000u) * sh_h[8 * uc + 2 * e + 1];
          }
        }
      } else {
        for (int u = 0; u < d; ++u) t += ldf(W2, (int64_t)j * d + u) * sh_h[u];
      }
      v += t + bias * s1;
    }
  }
  if (el) stf(out, o, v / sL);
  if (a.lse && j == 0) a.lse[(int64_t)b * s.Hq + qh] = Mx + logf(sL);
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
