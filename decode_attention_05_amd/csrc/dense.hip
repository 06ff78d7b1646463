// Softmax decode attention of one query token over exact bf16 K/V rows.
//
// Two uses: the uncompressed comparator over a whole cache [B, T, Hkv, d]
// (the cache LowRAM compresses: "The bottleneck LowRAM targets", "LowRAM
// Paper: Amortised Values and Low-Rank Keys for KV Compression"), and the
// exact tail of newly decoded tokens of one layer, which LowRAM keeps
// uncompressed ("Asymmetric key compression with xKV", same page).
//
// HBM-bound: every key and value byte is read once.  Grid (split, KV head,
// sequence), four waves per workgroup, 64-row tiles per wave:
//   scores  S^T = K Q^T with 16x16x32 bf16 MFMAs; key rows load straight
//           into the A-operand layout (16 bytes per lane per k-step);
//   values  two head-dim elements per lane; rows are read 16 at a time
//           (independent loads in flight) and weighted by the row
//           probabilities staged in LDS.
// Waves keep their own online-softmax state and merge through LDS; splits
// merge in the combine kernel.
#include "lowram_internal.h"

namespace lowram {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxGrp = 8;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// D = 128 with MFMA scores; lane = (c = lane % 16, g = lane / 16); each wave
// takes 16 * TT rows at a time
template <int TT>
__global__ void __launch_bounds__(64 * kWaves) dense128_kernel(DenseArgs a) {
  constexpr int D = 128;
  constexpr int WR = 16 * TT;                       // rows per wave tile
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int grp = a.grp;
  __shared__ float pw[kWaves][kMaxGrp][64];
  __shared__ float wm[kWaves][kMaxGrp], wl[kWaves][kMaxGrp];
  __shared__ float wacc[kWaves][kMaxGrp][D];

  // Q^T as the B operand: lane (c = query head, g) holds q[c][32 ks + 8 g .. + 8]
  const uint16_t *q = reinterpret_cast<const uint16_t *>(a.q) + ((int64_t)b * a.Hq + h * grp) * D;
  bf16x8 qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qf[ks] = as_bf16x8(c < grp ? *reinterpret_cast<const uint4 *>(q + c * D + 32 * ks + 8 * g) : uint4{0u, 0u, 0u, 0u});
  const float scale = 0.08838834764831845f;       // 1 / sqrt(128)

  const int n = min(a.ctx_len[b], a.T);
  const int r0 = split * a.split_rows, r1 = min(n, r0 + a.split_rows);
  const uint16_t *K = reinterpret_cast<const uint16_t *>(a.k);
  const uint16_t *V = reinterpret_cast<const uint16_t *>(a.v);
  const int64_t rs = (int64_t)a.H * D;              // row stride (elements)
  const int64_t base = (int64_t)b * a.kv_b_stride + a.kv_off + (int64_t)h * D;

  float M = -INFINITY, Lp = 0.f;                    // lane (c = qh, g)
  float acc[kMaxGrp][2];                            // lane = head-dim pair 2 lane, 2 lane + 1
#pragma unroll
  for (int q2 = 0; q2 < kMaxGrp; ++q2) acc[q2][0] = acc[q2][1] = 0.f;
  for (int t0 = r0 + wave * WR; t0 < r1; t0 += WR * kWaves) {
    const int cnt = min(WR, r1 - t0);
    // ---- scores S^T[t, qh] = K Q^T: A = key rows straight from memory
    f32x4 sacc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int row = t0 + min(16 * tt + c, cnt - 1);
      const uint16_t *kp = K + base + (int64_t)row * rs + 8 * g;
      uint4 kf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[ks] = *reinterpret_cast<const uint4 *>(kp + 32 * ks);
      sacc[tt] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[ks]), qf[ks], sacc[tt], 0, 0, 0);
    }
    // ---- online softmax on lanes (c = qh, g): rows 16 tt + 4 g + i
    float sv[4 * TT];
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4 * TT; ++e) {
      const int tl = 16 * (e >> 2) + 4 * g + (e & 3);
      sv[e] = tl < cnt ? sacc[e >> 2][e & 3] * scale : -INFINITY;
      mt = fmaxf(mt, sv[e]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float mn = fmaxf(M, mt);                  // finite: the tile has >= 1 row
    const float cr = __expf(M - mn);
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 4 * TT; ++e) {
      const float pe = __expf(sv[e] - mn);
      ps += pe;
      if (c < grp) pw[wave][c][16 * (e >> 2) + 4 * g + (e & 3)] = pe;
    }
    Lp = Lp * cr + ps;
    M = mn;
    // ---- values: rescale, then 16 rows of loads in flight at a time
#pragma unroll
    for (int q2 = 0; q2 < kMaxGrp; ++q2) {
      if (q2 >= grp) break;
      const float crq = __shfl(cr, q2, 64);
      acc[q2][0] *= crq;
      acc[q2][1] *= crq;
    }
    for (int i0 = 0; i0 < cnt; i0 += 16) {
      uint32_t vv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = t0 + min(i0 + i, cnt - 1);
        vv[i] = *reinterpret_cast<const uint32_t *>(V + base + (int64_t)row * rs + 2 * lane);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i0 + i >= cnt) break;
        const float v0 = __uint_as_float(vv[i] << 16), v1 = __uint_as_float(vv[i] & 0xffff0000u);
#pragma unroll
        for (int q2 = 0; q2 < kMaxGrp; ++q2) {
          if (q2 >= grp) break;
          const float pi = pw[wave][q2][i0 + i];
          acc[q2][0] += pi * v0;
          acc[q2][1] += pi * v1;
        }
      }
    }
  }
  Lp += __shfl_xor(Lp, 16, 64);
  Lp += __shfl_xor(Lp, 32, 64);
  if (g == 0 && c < grp) { wm[wave][c] = M; wl[wave][c] = Lp; }
#pragma unroll
  for (int q2 = 0; q2 < kMaxGrp; ++q2) {
    if (q2 >= grp) break;
    wacc[wave][q2][2 * lane] = acc[q2][0];
    wacc[wave][q2][2 * lane + 1] = acc[q2][1];
  }
  __syncthreads();
  // merge the waves and write the split record (value-space accumulator only)
  const int ps = part_stride(D);
  for (int i = tid; i < grp * D; i += blockDim.x) {
    const int q2 = i / D, j = i % D;
    float mx = -INFINITY;
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, wm[w][q2]);
    float Ls = 0.f, as = 0.f;
    if (mx != -INFINITY) {
      for (int w = 0; w < kWaves; ++w) {
        const float cw = __expf(wm[w][q2] - mx);
        Ls += cw * wl[w][q2];
        as += cw * wacc[w][q2][j];
      }
    }
    float *rec = a.partials + (((int64_t)b * a.Hq + h * grp + q2) * a.n_splits + a.split_base + split) * ps;
    if (j == 0) { rec[0] = mx; rec[1] = Ls; rec[2] = 0.f; rec[3] = 0.f; }
    rec[4 + j] = 0.f;
    rec[4 + D + j] = as;
  }
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
  dim3 grid(n_grid_splits, a.H, a.B), block(64 * kWaves);
  if (a.d == 128 && a.split_rows <= 64) hipLaunchKernelGGL(dense128_kernel<1>, grid, block, 0, st, a);
  else if (a.d == 128) hipLaunchKernelGGL(dense128_kernel<4>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(dense64_kernel, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_tail(const DecodeArgs &d, int split_index, int split_rows, int n_tail_splits,
                       hipStream_t st) {
  const Dims &s = d.s;
  DenseArgs a{};
  a.B = s.B; a.Hq = s.Hq; a.H = s.H; a.d = s.d; a.T = s.Te; a.grp = s.grp;
  a.q = d.q; a.k = d.c.tail_k; a.v = d.c.tail_v; a.ctx_len = d.c.tail_len;
  a.partials = d.partials; a.n_splits = d.n_splits; a.split_rows = split_rows;
  a.kv_b_stride = (int64_t)s.G * s.Te * s.H * s.d;
  a.kv_off = (int64_t)d.layer * s.Te * s.H * s.d;
  a.split_base = split_index;
  return launch_dense_splits(a, n_tail_splits, st);
}

hipError_t launch_dense(const DenseArgs &a, hipStream_t st) {
  hipError_t e = mark_kernel_start(st);
  if (e != hipSuccess) return e;
  e = launch_dense_splits(a, a.n_splits, st);
  if (e != hipSuccess) return e;
  if ((e = mark_kernel_end(st)) != hipSuccess) return e;
  DecodeArgs c{};
  c.s.B = a.B; c.s.Hq = a.Hq; c.s.H = a.H; c.s.d = a.d; c.s.grp = a.grp;
  c.s.dtype = LOWRAM_BF16;
  c.out = a.out; c.lse = a.lse; c.partials = a.partials; c.n_splits = a.n_splits;
  return launch_combine(c, false, st);
}

}  // namespace lowram
