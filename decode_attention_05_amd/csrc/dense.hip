// Softmax decode attention of one query token over exact bf16 K/V rows.
//
// Two uses: the uncompressed comparator over a whole cache [B, T, Hkv, d]
// (the cache LowRAM compresses: "The bottleneck LowRAM targets", "LowRAM
// Paper: Amortised Values and Low-Rank Keys for KV Compression"), and the
// exact tail of newly decoded tokens of one layer, which LowRAM keeps
// uncompressed ("Asymmetric key compression with xKV", same page).
//
// HBM-bound: every key and value byte is read once.  Grid (KV head, split,
// sequence), four waves per workgroup, 32-row tiles per wave (16 for the
// 64-row tail splits):
//   scores  S^T = K Q^T with 16x16x32 bf16 MFMAs; key rows load straight
//           into the A-operand layout (16 bytes per lane per k-step);
//   values  requested with the keys in one burst per tile (16-byte pieces,
//           four rows per load instruction) and weighted by the row
//           probabilities staged in LDS.
// Waves keep their own online-softmax state and merge through LDS; splits
// merge in the combine kernel.
#include "dense_body.h"
#include "lowram_internal.h"

namespace lowram {
namespace {

using dense_detail::kWaves;
using dense_detail::kMaxGrp;
using dense_detail::bf16x8;
using dense_detail::f32x4;
using dense_detail::as_bf16x8;

// grid (KV head, split, sequence): the heads of one row range are adjacent
// workgroup ids, so the whole [Hkv, d] rows of a range stream together
template <int TT>
__global__ void __launch_bounds__(64 * kWaves) dense128_kernel(DenseArgs a) {
  __shared__ dense_detail::DenseLds<TT, kWaves> sh;
  dense_detail::dense128_body<TT, kWaves>(a, blockIdx.y, blockIdx.x, blockIdx.z, sh);
}

// D = 64: one row per lane on VALU (head_dim 64 is served by the plain path)
__global__ void __launch_bounds__(64 * kWaves) dense64_kernel(DenseArgs a) {
  constexpr int D = 64;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = a.grp;
  __shared__ float qs[kMaxGrp][D];
  __shared__ float pw[kWaves][kMaxGrp][64];
  __shared__ float wm[kWaves][kMaxGrp], wl[kWaves][kMaxGrp];
  __shared__ float wacc[kWaves][kMaxGrp][D];
  const uint16_t *q = reinterpret_cast<const uint16_t *>(a.q);
  for (int i = tid; i < kMaxGrp * D; i += blockDim.x)
    qs[i / D][i % D] = (i / D < grp) ? bf16_to_f32(q[((int64_t)b * a.Hq + h * grp + i / D) * D + i % D]) * 0.125f : 0.f;
  __syncthreads();
  const int n = min(a.ctx_len[b], a.T);
  const int r0 = split * a.split_rows, r1 = min(n, r0 + a.split_rows);
  const uint16_t *K = reinterpret_cast<const uint16_t *>(a.k);
  const uint16_t *V = reinterpret_cast<const uint16_t *>(a.v);
  const int64_t rs = (int64_t)a.H * D;
  const int64_t base = (int64_t)b * a.kv_b_stride + a.kv_off + (int64_t)h * D;
  float M[kMaxGrp], Lp[kMaxGrp], acc[kMaxGrp];
  for (int q2 = 0; q2 < kMaxGrp; ++q2) { M[q2] = -INFINITY; Lp[q2] = 0.f; acc[q2] = 0.f; }
  for (int t0 = r0 + wave * 64; t0 < r1; t0 += 64 * kWaves) {
    const int t = t0 + lane;
    const bool ok = t < r1;
    const uint16_t *kp = K + base + (int64_t)(ok ? t : t0) * rs;
    float sc[kMaxGrp];
    for (int q2 = 0; q2 < kMaxGrp; ++q2) sc[q2] = 0.f;
    for (int j = 0; j < D; ++j) {
      const float kj = bf16_to_f32(kp[j]);
      for (int q2 = 0; q2 < grp; ++q2) sc[q2] += qs[q2][j] * kj;
    }
    for (int q2 = 0; q2 < grp; ++q2) {
      float mx = ok ? sc[q2] : -INFINITY;
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      const float mn = fmaxf(M[q2], mx);
      const float cr = __expf(M[q2] - mn);
      const float pg = ok ? __expf(sc[q2] - mn) : 0.f;
      Lp[q2] = Lp[q2] * cr + pg;
      acc[q2] *= cr;
      M[q2] = mn;
      pw[wave][q2][lane] = pg;
    }
    const int cnt = min(64, r1 - t0);
    for (int i = 0; i < cnt; ++i) {
      const float v = bf16_to_f32(V[base + (int64_t)(t0 + i) * rs + lane]);
      for (int q2 = 0; q2 < grp; ++q2) acc[q2] += pw[wave][q2][i] * v;
    }
  }
  for (int q2 = 0; q2 < grp; ++q2) {
    float l = Lp[q2];
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
    if (lane == 0) { wm[wave][q2] = M[q2]; wl[wave][q2] = l; }
    wacc[wave][q2][lane] = acc[q2];
  }
  __syncthreads();
  const int ps = part_stride(D);
  for (int i = tid; i < grp * D; i += blockDim.x) {
    const int q2 = i / D, j = i % D;
    float mx = -INFINITY;
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, wm[w][q2]);
    float Ls = 0.f, as = 0.f;
    if (mx != -INFINITY)
      for (int w = 0; w < kWaves; ++w) {
        const float cw = __expf(wm[w][q2] - mx);
        Ls += cw * wl[w][q2];
        as += cw * wacc[w][q2][j];
      }
    float *rec = a.partials + (((int64_t)b * a.Hq + h * grp + q2) * a.n_splits + a.split_base + split) * ps;
    if (j == 0) { rec[0] = mx; rec[1] = Ls; rec[2] = 0.f; rec[3] = 0.f; }
    rec[4 + j] = 0.f;
    rec[4 + D + j] = as;
  }
}

}  // namespace

hipError_t launch_dense_splits(const DenseArgs &a, int n_grid_splits, hipStream_t st) {
  dim3 block(64 * kWaves);
  if (a.d == 128) {
    dim3 grid(a.H, n_grid_splits, a.B);
    if (a.split_rows <= 64) hipLaunchKernelGGL(dense128_kernel<1>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(dense128_kernel<2>, grid, block, 0, st, a);
  } else {
    hipLaunchKernelGGL(dense64_kernel, dim3(n_grid_splits, a.H, a.B), block, 0, st, a);
  }
  return hipGetLastError();
}

DenseArgs tail_args(const DecodeArgs &d, int split_index, int split_rows) {
  const Dims &s = d.s;
  DenseArgs a{};
  a.B = s.B; a.Hq = s.Hq; a.H = s.H; a.d = s.d; a.T = s.Te; a.grp = s.grp;
  a.q = d.q; a.k = d.c.tail_k; a.v = d.c.tail_v; a.ctx_len = d.c.tail_len;
  a.partials = d.partials; a.n_splits = d.n_splits; a.split_rows = split_rows;
  a.kv_b_stride = (int64_t)s.G * s.Te * s.H * s.d;
  a.kv_off = (int64_t)d.layer * s.Te * s.H * s.d;
  a.split_base = split_index;
  return a;
}

hipError_t launch_tail(const DecodeArgs &d, int split_index, int split_rows, int n_tail_splits,
                       hipStream_t st) {
  return launch_dense_splits(tail_args(d, split_index, split_rows), n_tail_splits, st);
}

hipError_t launch_dense(const DenseArgs &a, hipStream_t st) {
  hipError_t e = launch_dense_splits(a, a.n_splits, st);
  if (e != hipSuccess) return e;
  DecodeArgs c{};
  c.s.B = a.B; c.s.Hq = a.Hq; c.s.H = a.H; c.s.d = a.d; c.s.grp = a.grp;
  c.s.dtype = LOWRAM_BF16;
  c.out = a.out; c.lse = a.lse; c.partials = a.partials; c.n_splits = a.n_splits;
  return launch_combine(c, false, st);
}

}  // namespace lowram
