// Uncompressed comparator: decode attention of one query token over an exact
// bf16 KV cache [B, T, Hkv, d] — the cache that LowRAM compresses ("The
// bottleneck LowRAM targets", "LowRAM Paper: Amortised Values and Low-Rank
// Keys for KV Compression").  HBM-bound: every key and value byte is read
// once.
//
// Grid (split, KV head, sequence), four waves per workgroup.  A wave takes
// 64 rows at a time with one row per lane for the scores (each lane reads its
// row's 256 contiguous key bytes), then switches to two head-dim elements
// per lane for the value sum (each value row is one coalesced 256-byte
// read), broadcasting every row's probability with a lane read.  Waves keep
// their own online-softmax state and merge through LDS at the end; splits
// merge in the combine kernel.
#include "lowram_internal.h"

namespace lowram {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxGrp = 8;

template <int D>
__global__ void __launch_bounds__(64 * kWaves) dense_kernel(DenseArgs a) {
  constexpr int EPL = D / 64;                 // value elements per lane
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = a.grp;
  __shared__ float qs[kMaxGrp][D];
  __shared__ float wm[kWaves][kMaxGrp], wl[kWaves][kMaxGrp];
  __shared__ float wacc[kWaves][kMaxGrp][D];

  const uint16_t *q = reinterpret_cast<const uint16_t *>(a.q);
  const float scale = rsqrtf(static_cast<float>(D));
  for (int i = tid; i < grp * D; i += blockDim.x)
    qs[i / D][i % D] = bf16_to_f32(q[((int64_t)b * a.Hq + h * grp + i / D) * D + i % D]) * scale;
  __syncthreads();

  const int n = min(a.ctx_len[b], a.T);
  const int r0 = split * a.split_rows, r1 = min(n, r0 + a.split_rows);
  const uint16_t *K = reinterpret_cast<const uint16_t *>(a.k);
  const uint16_t *V = reinterpret_cast<const uint16_t *>(a.v);
  const int64_t rs = (int64_t)a.H * D;              // row stride (elements)
  const int64_t base = (int64_t)b * a.kv_b_stride + a.kv_off + (int64_t)h * D;

  float M[kMaxGrp], L[kMaxGrp], acc[kMaxGrp][EPL];
  for (int g = 0; g < kMaxGrp; ++g) {
    M[g] = -INFINITY; L[g] = 0.f;
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }
  for (int t0 = r0 + wave * 64; t0 < r1; t0 += 64 * kWaves) {
    const int t = t0 + lane;
    const bool ok = t < r1;
    float sc[kMaxGrp];
    for (int g = 0; g < kMaxGrp; ++g) sc[g] = 0.f;
    if (ok) {
      const uint4 *kr = reinterpret_cast<const uint4 *>(K + base + t * rs);
#pragma unroll 4
      for (int c = 0; c < D / 8; ++c) {
        const uint4 w = kr[c];
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __uint_as_float(u[e] << 16), hi = __uint_as_float(u[e] & 0xffff0000u);
          for (int g = 0; g < grp; ++g) sc[g] += qs[g][c * 8 + 2 * e] * lo + qs[g][c * 8 + 2 * e + 1] * hi;
        }
      }
    }
    float p[kMaxGrp];
    for (int g = 0; g < grp; ++g) {
      float mx = ok ? sc[g] : -INFINITY;
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
      const float mn = fmaxf(M[g], mx);
      const float c = __expf(M[g] - mn);
      p[g] = ok ? __expf(sc[g] - mn) : 0.f;
      L[g] = L[g] * c + p[g];                        // per-lane partial sum
      for (int e = 0; e < EPL; ++e) acc[g][e] *= c;
      M[g] = mn;
    }
    const int cnt = min(64, r1 - t0);
    for (int i = 0; i < cnt; ++i) {
      const int64_t vo = base + (int64_t)(t0 + i) * rs + lane * EPL;
      float vv[EPL];
      if (EPL == 2) {
        const uint32_t w = *reinterpret_cast<const uint32_t *>(V + vo);
        vv[0] = __uint_as_float(w << 16);
        vv[EPL - 1] = __uint_as_float(w & 0xffff0000u);
      } else {
        vv[0] = bf16_to_f32(V[vo]);
      }
      for (int g = 0; g < grp; ++g) {
        const float pi = __shfl(p[g], i, 64);
        for (int e = 0; e < EPL; ++e) acc[g][e] += pi * vv[e];
      }
    }
  }
  for (int g = 0; g < grp; ++g) {
    float l = L[g];
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
    if (lane == 0) { wm[wave][g] = M[g]; wl[wave][g] = l; }
    for (int e = 0; e < EPL; ++e) wacc[wave][g][lane * EPL + e] = acc[g][e];
  }
  __syncthreads();
  // merge the waves and write the split record (value-space accumulator only)
  const int ps = part_stride(D);
  for (int i = tid; i < grp * D; i += blockDim.x) {
    const int g = i / D, j = i % D;
    float mx = -INFINITY;
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, wm[w][g]);
    float Ls = 0.f, as = 0.f;
    if (mx != -INFINITY) {
      for (int w = 0; w < kWaves; ++w) {
        const float c = __expf(wm[w][g] - mx);
        Ls += c * wl[w][g];
        as += c * wacc[w][g][j];
      }
    }
    float *rec = a.partials + (((int64_t)b * a.Hq + h * grp + g) * a.n_splits + a.split_base + split) * ps;
    if (j == 0) { rec[0] = mx; rec[1] = Ls; rec[2] = 0.f; rec[3] = 0.f; }
    rec[4 + j] = 0.f;
    rec[4 + D + j] = as;
  }
}

}  // namespace

hipError_t launch_dense_splits(const DenseArgs &a, int n_grid_splits, hipStream_t st) {
  dim3 grid(n_grid_splits, a.H, a.B), block(64 * kWaves);
  if (a.d == 128) hipLaunchKernelGGL((dense_kernel<128>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((dense_kernel<64>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_tail(const DecodeArgs &d, int split_index, hipStream_t st) {
  const Dims &s = d.s;
  DenseArgs a{};
  a.B = s.B; a.Hq = s.Hq; a.H = s.H; a.d = s.d; a.T = s.Te; a.grp = s.grp;
  a.q = d.q; a.k = d.c.tail_k; a.v = d.c.tail_v; a.ctx_len = d.c.tail_len;
  a.partials = d.partials; a.n_splits = d.n_splits; a.split_rows = s.Te;
  a.kv_b_stride = (int64_t)s.G * s.Te * s.H * s.d;
  a.kv_off = (int64_t)d.layer * s.Te * s.H * s.d;
  a.split_base = split_index;
  return launch_dense_splits(a, 1, st);
}

hipError_t launch_dense(const DenseArgs &a, hipStream_t st) {
  dim3 grid(a.n_splits, a.H, a.B), block(64 * kWaves);
  if (a.d == 128) hipLaunchKernelGGL((dense_kernel<128>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((dense_kernel<64>), grid, block, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  DecodeArgs c{};
  c.s.B = a.B; c.s.Hq = a.Hq; c.s.H = a.H; c.s.d = a.d; c.s.grp = a.grp;
  c.s.dtype = LOWRAM_BF16;
  c.out = a.out; c.lse = a.lse; c.partials = a.partials; c.n_splits = a.n_splits;
  return launch_combine(c, false, st);
}

}  // namespace lowram
