// Body of the head_dim-128 softmax decode attention over exact bf16 K/V
// rows, used by the comparator and tail kernels (dense.hip) and by the
// decode body kernel, whose last workgroups take the exact tail rows
// (decode_mfma.hip).  One workgroup of NW waves handles rows
// [split * split_rows, ...) of KV head h of sequence b and writes one split
// record; its LDS comes from the caller.
#ifndef LOWRAM_DENSE_BODY_H
#define LOWRAM_DENSE_BODY_H
#include "lowram_internal.h"

namespace lowram {
namespace dense_detail {

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
// takes 16 * TT rows at a time.  Every key and value byte of a wave tile is
// requested in one burst at the top of the tile (keys straight into the
// MFMA A layout, values as 16-byte pieces: lane (rg = lane / 16, cq =
// lane % 16) holds head dims 8 cq .. 8 cq + 7 of rows 4 i + rg), so one wait
// covers the tile and the loads of all resident waves overlap.
// LDS of one workgroup: per-wave row probabilities, softmax states and
// value accumulators
template <int TT, int NW>
struct DenseLds {
  __attribute__((aligned(16))) float pw[NW][16 * TT][kMaxGrp];   // probabilities [row][query head]
  float wm[NW][kMaxGrp], wl[NW][kMaxGrp];
  float wacc[NW][kMaxGrp][128];
};

template <int TT, int NW>
__device__ __forceinline__ void dense128_body(const DenseArgs &a, int split, int h, int b, DenseLds<TT, NW> &sh) {
  constexpr int D = 128;
  constexpr int WR = 16 * TT;                       // rows per wave tile
  constexpr int NV = WR / 4;                        // value pieces per lane
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int grp = a.grp;
  auto &pw = sh.pw;
  auto &wm = sh.wm;
  auto &wl = sh.wl;
  auto &wacc = sh.wacc;

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
  float acc[kMaxGrp][8];                            // lane (g, c): head dims 8 c .. 8 c + 7, rows 4 i + g
#pragma unroll
  for (int q2 = 0; q2 < kMaxGrp; ++q2)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[q2][e] = 0.f;
  for (int t0 = r0 + wave * WR; t0 < r1; t0 += WR * NW) {
    const int cnt = min(WR, r1 - t0);
    // ---- one burst: key fragments, then value pieces (rows past cnt re-read
    // the tile's last row and are weighted 0)
    uint4 kf[TT][4], vf[NV];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int row = t0 + min(16 * tt + c, cnt - 1);
      const uint16_t *kp = K + base + (int64_t)row * rs + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[tt][ks] = *reinterpret_cast<const uint4 *>(kp + 32 * ks);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int row = t0 + min(4 * i + g, cnt - 1);
      vf[i] = *reinterpret_cast<const uint4 *>(V + base + (int64_t)row * rs + 8 * c);
    }
    // ---- scores S^T[t, qh] = K Q^T
    f32x4 sacc[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      sacc[tt] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[tt][ks]), qf[ks], sacc[tt], 0, 0, 0);
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
      if (c < kMaxGrp) pw[wave][16 * (e >> 2) + 4 * g + (e & 3)][c] = (c < grp) ? pe : 0.f;
    }
    Lp = Lp * cr + ps;
    M = mn;
    // ---- values: rescale, then weight this lane's rows
#pragma unroll
    for (int q2 = 0; q2 < kMaxGrp; ++q2) {
      if (q2 >= grp) break;
      const float crq = __shfl(cr, q2, 64);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[q2][e] *= crq;
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float v[8];
      const uint32_t w[4] = {vf[i].x, vf[i].y, vf[i].z, vf[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float(w[k] << 16);
        v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
      }
      const int tl = 4 * i + g;
      const float4 p0 = *reinterpret_cast<const float4 *>(&pw[wave][tl][0]);
      const float4 p1 = *reinterpret_cast<const float4 *>(&pw[wave][tl][4]);
      const float pr[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
      for (int q2 = 0; q2 < kMaxGrp; ++q2) {
        if (q2 >= grp) break;
        const float pi = tl < cnt ? pr[q2] : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[q2][e] += pi * v[e];
      }
    }
  }
  Lp += __shfl_xor(Lp, 16, 64);
  Lp += __shfl_xor(Lp, 32, 64);
  if (g == 0 && c < grp) { wm[wave][c] = M; wl[wave][c] = Lp; }
  // sum the four row groups of lanes (g), then lanes g = 0 hold the wave's
  // value accumulator for head dims 8 c .. 8 c + 7
#pragma unroll
  for (int q2 = 0; q2 < kMaxGrp; ++q2) {
    if (q2 >= grp) break;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[q2][e];
      x += __shfl_xor(x, 16, 64);
      x += __shfl_xor(x, 32, 64);
      if (g == 0) wacc[wave][q2][8 * c + e] = x;
    }
  }
  __syncthreads();
  // merge the waves and write the split record (value-space accumulator only)
  const int ps = part_stride(D);
  for (int i = tid; i < grp * D; i += blockDim.x) {
    const int q2 = i / D, j = i % D;
    float mx = -INFINITY;
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, wm[w][q2]);
    float Ls = 0.f, as = 0.f;
    if (mx != -INFINITY) {
      for (int w = 0; w < NW; ++w) {
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

}  // namespace dense_detail
}  // namespace lowram
#endif  // LOWRAM_DENSE_BODY_H
