// Test-time fitting of the value predictors on the matrix cores (gfx950).
//
// LowRAM (arXiv:2611.07025), "LowRAM Paper: Amortised Values and Low-Rank
// Keys for KV Compression": "Value cache amortisation in plain language"
// (during prefill a small per-head MLP is fitted to map each token's key to
// its value) and "Step-by-step mental model for one decoding session" item 1;
// arXiv listing, Abstract (the predictors are fitted at test time).  The
// loss and the optimiser are not on the pages: the mean squared error of
// f(k^) against v over the body rows, minimised by full-batch Adam (Kingma
// and Ba, "Adam: A Method for Stochastic Optimization", 2015, Algorithm 1).
//
// Stream order of one call:
//   fit_prep_kernel    once per (64-row chunk, layer-head, sequence): the
//                      rebuilt pre-RoPE keys k^ = c basis (bf16 MFMAs for
//                      bf16 caches, fp32 FMAs otherwise), kept as
//                      bf16 pairs (x = hi + lo) row-major [row][dim] and
//                      chunk-transposed [dim][row], and the values as fp32
//                      [dim][row]; rows past n_body are zero
//   fit_adam_kernel    t = 0: fp32 master weights from the caller's, moments 0
//   for t = 1 .. steps:
//     fit_grad_kernel  per (row split, layer-head, sequence): forward and
//                      backward of the MLP over 64-row chunks; the split's
//                      gradient sums and loss sum go to the workspace
//     fit_adam_kernel  sums the splits in a fixed order, scales by
//                      1 / (rows d), one Adam step on the fp32 master weights;
//                      writes the bf16-pair copies of W1, W2 and W2^T that the
//                      next gradient pass reads and, after the last step, the
//                      caller's weights
//
// One gradient pass over a 64-row chunk (K^ rows x d; every product on
// 16x16x32 bf16 MFMAs with both operands split into bf16 pairs, hi*hi +
// hi*lo + lo*hi, fp32 accumulation):
//   Z  = K^ W1^T + b1,  A = GELU(Z)            product 1
//   F  = A W2^T + b2,   E = F - V,  G = 2 E    product 2
//   GA = G W2,          GZ = GA * GELU'(Z)     product 3
//   dW2 += G^T A,       dW1 += GZ^T K^         products 4 and 5
//   db2 += sum of G, db1 += sum of GZ over rows, loss += sum of E^2
// (G = 2 E is the gradient of the summed squared error; the 1 / (rows d) of
// the mean is applied once the splits are summed.)
// The d / 16 waves (two per SIMD at d = 128) split products 1-3 by output
// dim (16 each) and products 4-5 by gradient row (16 each).  Rows inside
// each 16-row MFMA tile follow the index order of the prefill kernels (row
// m of tile t is chunk row 32 (t / 2) +
// 8 (m / 4) + 4 (t % 2) + m % 4), so a lane's accumulators of tiles 2a and
// 2a + 1 hold 8 consecutive rows of one dim: they go to LDS as [dim][row]
// with 16-byte stores (the row-contracted operands of products 4-5) and as
// [row][dim] element by element (the dim-contracted operands of products
// 2-3).
#include <algorithm>
#include <cmath>

#include "lowram_internal.h"
#include "mfma_common.h"

namespace lowram {
namespace {

using namespace mfma;

constexpr int kT = 64;               // rows per chunk
constexpr int kGradMaxThreads = 512; // d / 16 waves: eight for d = 128, four for d = 64
constexpr int kPrepThreads = 256;
constexpr int kAdamThreads = 256;
constexpr float kInvSqrt2 = 0.70710678118654752440f;
constexpr float kInvSqrt2Pi = 0.39894228040143267794f;
constexpr float kHalfLog2E = -0.72134752044448170368f;   // -log2(e) / 2

// chunk row held by row m of MFMA tile mb (four tiles of 16 rows)
__device__ __forceinline__ int tile_tok(int mb, int m) {
  return 32 * (mb >> 1) + 8 * (m >> 2) + 4 * (mb & 1) + (m & 3);
}

// Byte offset of (row t, dim f) in one bf16 plane stored [row][dim].  The
// 16-byte chunk index is XORed with bits of the row, chosen so that the 16
// rows of one MFMA operand read (rows tile_tok(mb, 0..15)) land on 16
// different chunk positions (128-dim rows) or on distinct banks (64-dim
// rows, two rows per bank line).
template <int kD>
__device__ __forceinline__ int tf_off(int t, int f) {
  const int sw = kD == 128 ? ((((t >> 3) & 3) << 2) | (t & 3)) : ((((t >> 3) & 3) << 1) | ((t >> 1) & 1));
  return t * (2 * kD) + (((f >> 3) ^ sw) << 4) + ((f & 7) << 1);
}

// byte offset of (dim f, row t) in one bf16 plane stored [dim][row] (64 rows:
// eight 16-byte chunks per dim, XORed with bits of the dim)
__device__ __forceinline__ int ft_off(int f, int t) {
  return f * (2 * kT) + (((t >> 3) ^ ((f >> 1) & 7)) << 4) + ((t & 7) << 1);
}

__device__ __forceinline__ bf16x8 lds16(const char *p) { return as_bf16x8(*reinterpret_cast<const uint4 *>(p)); }
__device__ __forceinline__ bf16x8 gld16(const uint16_t *p) { return as_bf16x8(*reinterpret_cast<const uint4 *>(p)); }

// Buffer loads: a scalar descriptor (base and size of one workgroup's
// array) and a 32-bit byte offset per lane keep each address in one VGPR
// (64-bit pointers per lane do not fit beside the accumulators); reads past
// the size return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// bf16 pair of 8 values: hi = bf16(x), lo = bf16(x - hi), both rounded to
// nearest even by the hardware conversion
__device__ __forceinline__ void pair8(const float *x, bf16x8 *hi, bf16x8 *lo) {
  const bf16x8 h = pack8_bf16(f32x4{x[0], x[1], x[2], x[3]}, f32x4{x[4], x[5], x[6], x[7]});
  f32x4 ra, rb;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ra[e] = x[e] - static_cast<float>(h[e]);
    rb[e] = x[4 + e] - static_cast<float>(h[4 + e]);
  }
  *hi = h;
  *lo = pack8_bf16(ra, rb);
}

// The [row][dim] swizzle of tf_off for row t = 32 a + 8 g + e, split into a
// lane part (g) and a compile-time part (e): sw(t) = tf_sw_g(g) | tf_sw_e(e).
template <int kD>
__device__ __forceinline__ int tf_sw_g(int g) { return kD == 128 ? (g << 2) : (g << 1); }
template <int kD>
__device__ __forceinline__ constexpr int tf_sw_e(int e) { return kD == 128 ? (e & 3) : ((e >> 1) & 1); }

// store 8 rows (32 a + 8 g + e, e = 0..7) of dim f of both planes to a region
// stored [row][dim]
template <int kD>
__device__ __forceinline__ void store_rows_tf(char *R, int a, int g, int f, bf16x8 hi, bf16x8 lo) {
  constexpr int kPlane = 64 * kD * 2;
  const int base = (32 * a + 8 * g) * (2 * kD) + ((f & 7) << 1);
  const int cb = (f >> 3) ^ tf_sw_g<kD>(g);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int off = base + e * (2 * kD) + ((cb ^ tf_sw_e<kD>(e)) << 4);
    *reinterpret_cast<__bf16 *>(R + off) = hi[e];
    *reinterpret_cast<__bf16 *>(R + kPlane + off) = lo[e];
  }
}

// hi*hi + hi*lo + lo*hi of one 16x16x32 tile
__device__ __forceinline__ f32x4 mfma3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 acc) {
  acc = mfma_bf16(ah, bh, acc);
  acc = mfma_bf16(ah, bl, acc);
  return mfma_bf16(al, bh, acc);
}

// =====================================================================
// fit_prep_kernel: rebuilt keys and transposed values of one chunk
// =====================================================================
template <int kD, bool kF32, bool kInt4>
__global__ void __launch_bounds__(kPrepThreads) fit_prep_kernel(FitDev p) {
  constexpr int kCols = kD / 16;                 // dims per thread
  __shared__ float cs[kT][33];                   // coefficients [row][rank of the block]
  __shared__ float bs[32][kD + 4];               // basis block [rank][dim]
  const int q = blockIdx.x, lh = blockIdx.y, b = blockIdx.z;
  const int GH = p.G * p.H, l = lh / p.H, h = lh % p.H;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int n = min(max(p.n_body[b], 0), p.N);
  const int t0 = q * kT;
  const int64_t D = (int64_t)GH * kD;
  float acc[4][kCols];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kCols; ++j) acc[i][j] = 0.f;

  if constexpr (!kF32 && !kInt4) {
    // bf16 coefficients and basis are exact MFMA operands (their products
    // are exact in fp32): k^ = C B on 16x16x32 bf16 MFMAs.  Wave w takes
    // chunk rows 16 w .. 16 w + 15 and all kD dims; per block of 32 ranks
    // the basis block goes to LDS as [dim][rank] (80-byte rows: the 16 lanes
    // of one operand read hit 16 disjoint bank groups).  The result passes
    // through LDS into the thread layout of the stores below.
    constexpr int kNT = kD / 16;
    __shared__ __attribute__((aligned(16))) uint16_t bt[kD][40];
    __shared__ float ot[kT][kD + 4];
    const int wave = tid >> 6, lane = tid & 63, c = lane & 15, g = lane >> 4;
    const int trow = t0 + 16 * wave + c;
    const uint16_t *crow = static_cast<const uint16_t *>(p.coef) + ((int64_t)b * p.N + (trow < n ? trow : 0)) * p.r;
    f32x4 mac[kNT];
#pragma unroll
    for (int jt = 0; jt < kNT; ++jt) mac[jt] = f32x4{0, 0, 0, 0};
    for (int k0 = 0; k0 < p.r; k0 += 32) {
      {   // basis rank k0 + tid / 8, dims (kD / 8) (tid % 8) + [0, kD / 8) of (l, h), transposed
        constexpr int kPer = kD / 8;
        const int kr = tid >> 3, c0 = kPer * (tid & 7);
        const uint16_t *src = static_cast<const uint16_t *>(p.basis) + ((int64_t)b * p.r + k0 + kr) * D + (int64_t)lh * kD + c0;
#pragma unroll
        for (int e = 0; e < kPer; e += 8) {
          const uint4 u = *reinterpret_cast<const uint4 *>(src + e);
          const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            bt[c0 + e + 2 * x][kr] = static_cast<uint16_t>(wv[x] & 0xffffu);
            bt[c0 + e + 2 * x + 1][kr] = static_cast<uint16_t>(wv[x] >> 16);
          }
        }
      }
      __syncthreads();
      uint4 a = *reinterpret_cast<const uint4 *>(crow + k0 + 8 * g);
      if (trow >= n) a = uint4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int jt = 0; jt < kNT; ++jt)
        mac[jt] = mfma_bf16(as_bf16x8(a), as_bf16x8(*reinterpret_cast<const uint4 *>(&bt[16 * jt + c][8 * g])), mac[jt]);
      __syncthreads();
    }
    // lane (c, g) of wave w holds dims 16 jt + c of rows 16 w + 4 g + i
#pragma unroll
    for (int jt = 0; jt < kNT; ++jt)
#pragma unroll
      for (int e = 0; e < 4; ++e) ot[16 * wave + 4 * g + e][16 * jt + c] = mac[jt][e];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < kCols; ++jj) acc[i][jj] = ot[4 * ty + i][kCols * tx + jj];
  } else {
  for (int k0 = 0; k0 < p.r; k0 += 32) {
      {   // coefficients of row tid / 4, ranks k0 + 8 (tid % 4) + [0, 8)
        const int rr = tid >> 2, kk = 8 * (tid & 3), t = t0 + rr;
        float x[8];
  #pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
        if (t < n) {
          const int64_t row = (int64_t)b * p.N + t;
          if (kInt4) {
            const uint32_t w = *reinterpret_cast<const uint32_t *>(
                static_cast<const uint8_t *>(p.coef) + row * (p.r / 2) + (k0 + kk) / 2);
            const float sc = f16_to_f32(static_cast<const uint16_t *>(p.coef_scale)[row * (p.r / 32) + k0 / 32]);
  #pragma unroll
            for (int e = 0; e < 8; ++e) {
              int code = (w >> (4 * e)) & 0xF;
              code = code >= 8 ? code - 16 : code;
              x[e] = static_cast<float>(code) * sc;     // exact: 4-bit code times an fp16 scale
            }
          } else if (kF32) {
            const float4 *src = reinterpret_cast<const float4 *>(static_cast<const float *>(p.coef) + row * p.r + k0 + kk);
            const float4 u0 = src[0], u1 = src[1];
            x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w; x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
          } else {
            const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.coef) + row * p.r + k0 + kk);
            const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
  #pragma unroll
            for (int e = 0; e < 4; ++e) {
              x[2 * e] = __uint_as_float(wv[e] << 16);
              x[2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
            }
          }
        }
  #pragma unroll
        for (int e = 0; e < 8; ++e) cs[rr][kk + e] = x[e];
      }
      {   // basis rank k0 + tid / 8, dims (kD / 8) (tid % 8) + [0, kD / 8) of (l, h)
        constexpr int kPer = kD / 8;
        const int kr = tid >> 3, c0 = kPer * (tid & 7);
        const int64_t base = ((int64_t)b * p.r + k0 + kr) * D + (int64_t)lh * kD + c0;
  #pragma unroll
        for (int e = 0; e < kPer; ++e)
          bs[kr][c0 + e] = kF32 ? static_cast<const float *>(p.basis)[base + e]
                                : bf16_to_f32(static_cast<const uint16_t *>(p.basis)[base + e]);
      }
      __syncthreads();
  #pragma unroll 4
      for (int k = 0; k < 32; ++k) {
        float bv[kCols];
  #pragma unroll
        for (int j = 0; j < kCols; ++j) bv[j] = bs[k][kCols * tx + j];
  #pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = cs[4 * ty + i][k];
  #pragma unroll
          for (int j = 0; j < kCols; ++j) acc[i][j] = fmaf(a, bv[j], acc[i][j]);
        }
      }
      __syncthreads();
    }
  }

  // keys: [plane][row][dim] and, per chunk, [plane][dim][row]
  const int64_t bh = (int64_t)b * GH + lh;
  uint16_t *kh = p.kh + bh * 2 * p.NP * kD;
  uint16_t *kt = p.kt + (bh * p.NC + q) * 2 * kD * kT;
  float *vt = p.vt + (bh * p.NC + q) * kD * kT;
  uint16_t hi[4][kCols], lo[4][kCols];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kCols; ++j) {
      hi[i][j] = f32_to_bf16(acc[i][j]);
      lo[i][j] = f32_to_bf16(acc[i][j] - bf16_to_f32(hi[i][j]));
    }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = (int64_t)t0 + 4 * ty + i;
#pragma unroll
    for (int j = 0; j < kCols; ++j) {
      kh[row * kD + kCols * tx + j] = hi[i][j];
      kh[(p.NP + row) * kD + kCols * tx + j] = lo[i][j];
    }
  }
#pragma unroll
  for (int j = 0; j < kCols; ++j) {
    const int f = kCols * tx + j;
    uint2 uh, ul;
    uh.x = hi[0][j] | (uint32_t)hi[1][j] << 16; uh.y = hi[2][j] | (uint32_t)hi[3][j] << 16;
    ul.x = lo[0][j] | (uint32_t)lo[1][j] << 16; ul.y = lo[2][j] | (uint32_t)lo[3][j] << 16;
    *reinterpret_cast<uint2 *>(kt + f * kT + 4 * ty) = uh;
    *reinterpret_cast<uint2 *>(kt + (kD + f) * kT + 4 * ty) = ul;
  }
  // values: fp32 [dim][row]
  float vv[4][kCols];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * ty + i;
    const int64_t base = ((((int64_t)b * p.G + l) * p.N + t) * p.H + h) * kD + kCols * tx;
#pragma unroll
    for (int j = 0; j < kCols; ++j)
      vv[i][j] = t < n ? (kF32 ? static_cast<const float *>(p.v)[base + j]
                               : bf16_to_f32(static_cast<const uint16_t *>(p.v)[base + j]))
                       : 0.f;
  }
#pragma unroll
  for (int j = 0; j < kCols; ++j)
    *reinterpret_cast<float4 *>(vt + (kCols * tx + j) * kT + 4 * ty) = make_float4(vv[0][j], vv[1][j], vv[2][j], vv[3][j]);
}

// =====================================================================
// fit_grad_kernel: gradient sums of one row split of one (sequence, head)
// =====================================================================
template <int kD>
__global__ void __launch_bounds__(kGradMaxThreads) fit_grad_kernel(FitDev p) {
  constexpr int kWaves = kD / 16, kThreads = 64 * kWaves;
  constexpr int kF = 16, kFT = 1, kKS = kD / 32, kNT = kD / 16, kCH = kD / 8;
  constexpr int kPlane = kT * kD * 2, kRegion = 2 * kPlane;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  char *const R0 = lds, *const R1 = lds + kRegion, *const R2 = lds + 2 * kRegion, *const R3 = lds + 3 * kRegion;
  float *const red = reinterpret_cast<float *>(lds + 4 * kRegion);

  // Block order (layer-head, sequence, split), dealt to the XCDs in
  // contiguous ranges: the workgroups that run together on one XCD share a
  // few predictors, whose bf16-pair weights (6 d^2 x 2 bytes each) then stay
  // in that XCD's L2 across their chunks.
  const int GH = p.G * p.H;
  int j = blockIdx.x;
  if ((gridDim.x & 7) == 0) j = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int s = j % p.S, lh = j / (p.S * p.B), b = (j / p.S) % p.B;
  const int64_t bh = (int64_t)b * GH + lh;
  const int pidx = (p.pred_shared ? 0 : b) * GH + lh;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, c = lane & 15, g = lane >> 4;
  const int n = min(max(p.n_body[b], 0), p.N);
  const int nch = (n + kT - 1) / kT;
  const int cps = (p.NC + p.S - 1) / p.S;
  const int q0 = s * cps, q1 = min(nch, q0 + cps);

  const uint16_t *const wc = p.wc + (int64_t)pidx * 6 * kD * kD;
  const float *const mw = p.master + (int64_t)pidx * p.npar;
  float bias1[kFT], bias2[kFT];
#pragma unroll
  for (int ft = 0; ft < kFT; ++ft) {
    bias1[ft] = mw[kD * kD + kF * w + 16 * ft + c];
    bias2[ft] = mw[2 * kD * kD + kD + kF * w + 16 * ft + c];
  }

  f32x4 dw1[kFT][kNT], dw2[kFT][kNT];
#pragma unroll
  for (int i = 0; i < kFT; ++i)
#pragma unroll
    for (int j = 0; j < kNT; ++j) dw1[i][j] = dw2[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float db1[kFT], db2[kFT], loss = 0.f;
#pragma unroll
  for (int ft = 0; ft < kFT; ++ft) db1[ft] = db2[ft] = 0.f;

  // this workgroup's arrays: keys [plane][row][dim], per chunk transposed
  // keys [plane][dim][row] and values [dim][row], the predictor's weight pairs
  const __amdgpu_buffer_rsrc_t rs_kh = buf_rsrc(p.kh + bh * 2 * p.NP * kD, 2 * p.NP * kD * 2);
  const __amdgpu_buffer_rsrc_t rs_kt = buf_rsrc(p.kt + bh * p.NC * 2 * kD * kT, (int64_t)p.NC * 2 * kD * kT * 2);
  const __amdgpu_buffer_rsrc_t rs_vt = buf_rsrc(p.vt + bh * p.NC * kD * kT, (int64_t)p.NC * kD * kT * 4);
  const __amdgpu_buffer_rsrc_t rs_w = buf_rsrc(wc, 6 * kD * kD * 2);
  // byte offset of key piece i (16 bytes: 8 dims of one row) of chunk q
  auto kh_off = [&](int i, int q) {
    const int pl = i / (kT * kCH), rem = i % (kT * kCH), t = rem / kCH, ch = rem % kCH;
    return ((pl * static_cast<int>(p.NP) + q * kT + t) * kD + 8 * ch) * 2;
  };

  auto stage_keys = [&](int q) {
    constexpr int kPieces = 2 * kT * kCH;
    for (int i = tid; i < kPieces; i += kThreads) {
      const int pl = i / (kT * kCH), rem = i % (kT * kCH), t = rem / kCH, ch = rem % kCH;
      *reinterpret_cast<uint4 *>(R0 + pl * kPlane + tf_off<kD>(t, 8 * ch)) = bload16(rs_kh, kh_off(i, q), 0);
    }
  };

  if (q0 < q1) stage_keys(q0);
  __syncthreads();
  for (int q = q0; q < q1; ++q) {
    f32x4 acc[4][kFT];
    float gp[2][kFT][8];                      // GELU'(Z) of the lane's rows and dims

    // ---- product 1: Z = K^ W1^T for this wave's dims (j = kF w + 16 ft + c)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int ft = 0; ft < kFT; ++ft) acc[mb][ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      bf16x8 bh8[kFT], bl8[kFT];
#pragma unroll
      for (int ft = 0; ft < kFT; ++ft) {
        const int j = kF * w + 16 * ft + c;
        bh8[ft] = as_bf16x8(bload16(rs_w, (j * kD + 8 * g) * 2, 64 * ks));
        bl8[ft] = as_bf16x8(bload16(rs_w, (j * kD + 8 * g) * 2, 64 * ks + kD * kD * 2));
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int t = tile_tok(mb, c);
        const bf16x8 ah = lds16(R0 + tf_off<kD>(t, 32 * ks + 8 * g));
        const bf16x8 al = lds16(R0 + kPlane + tf_off<kD>(t, 32 * ks + 8 * g));
#pragma unroll
        for (int ft = 0; ft < kFT; ++ft) acc[mb][ft] = mfma3(ah, al, bh8[ft], bl8[ft], acc[mb][ft]);
      }
    }
    // A = GELU(Z + b1) to R1 as [row][dim] and R2 as [dim][row]; keep GELU'
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int ft = 0; ft < kFT; ++ft) {
        const int f = kF * w + 16 * ft + c;
        float av[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float z = (e < 4 ? acc[2 * a][ft][e] : acc[2 * a + 1][ft][e - 4]) + bias1[ft];
          const float cdf = 0.5f * (1.0f + erff(z * kInvSqrt2));
          av[e] = z * cdf;
          // GELU'(z) = Phi(z) + z phi(z), phi(z) = exp(-z^2 / 2) / sqrt(2 pi) via the hardware exp2
          gp[a][ft][e] = fmaf(z * kInvSqrt2Pi, __builtin_amdgcn_exp2f(z * z * kHalfLog2E), cdf);
        }
        bf16x8 h8, l8;
        pair8(av, &h8, &l8);
        *reinterpret_cast<bf16x8 *>(R2 + ft_off(f, 32 * a + 8 * g)) = h8;
        *reinterpret_cast<bf16x8 *>(R2 + kPlane + ft_off(f, 32 * a + 8 * g)) = l8;
        store_rows_tf<kD>(R1, a, g, f, h8, l8);
      }
    __syncthreads();

    // ---- product 2: F = A W2^T for this wave's output dims
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int ft = 0; ft < kFT; ++ft) acc[mb][ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      bf16x8 bh8[kFT], bl8[kFT];
#pragma unroll
      for (int ft = 0; ft < kFT; ++ft) {
        const int j = kF * w + 16 * ft + c;
        bh8[ft] = as_bf16x8(bload16(rs_w, (j * kD + 8 * g) * 2, 64 * ks + 2 * kD * kD * 2));
        bl8[ft] = as_bf16x8(bload16(rs_w, (j * kD + 8 * g) * 2, 64 * ks + 3 * kD * kD * 2));
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int t = tile_tok(mb, c);
        const bf16x8 ah = lds16(R1 + tf_off<kD>(t, 32 * ks + 8 * g));
        const bf16x8 al = lds16(R1 + kPlane + tf_off<kD>(t, 32 * ks + 8 * g));
#pragma unroll
        for (int ft = 0; ft < kFT; ++ft) acc[mb][ft] = mfma3(ah, al, bh8[ft], bl8[ft], acc[mb][ft]);
      }
    }
    // E = F + b2 - V on rows < n; G = 2 E to R0 as [row][dim] and R3 as [dim][row]
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int ft = 0; ft < kFT; ++ft) {
        const int f = kF * w + 16 * ft + c;
        const int vo = ((q * kD + f) * kT + 32 * a + 8 * g) * 4;
        const float4 v0 = __builtin_bit_cast(float4, bload16(rs_vt, vo, 0));
        const float4 v1 = __builtin_bit_cast(float4, bload16(rs_vt, vo, 16));
        const float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        float gv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int t = 32 * a + 8 * g + e;
          float err = (e < 4 ? acc[2 * a][ft][e] : acc[2 * a + 1][ft][e - 4]) + bias2[ft] - vv[e];
          err = (q * kT + t < n) ? err : 0.f;
          loss = fmaf(err, err, loss);
          gv[e] = 2.f * err;
          db2[ft] += gv[e];
        }
        bf16x8 h8, l8;
        pair8(gv, &h8, &l8);
        *reinterpret_cast<bf16x8 *>(R3 + ft_off(f, 32 * a + 8 * g)) = h8;
        *reinterpret_cast<bf16x8 *>(R3 + kPlane + ft_off(f, 32 * a + 8 * g)) = l8;
        store_rows_tf<kD>(R0, a, g, f, h8, l8);
      }
    __syncthreads();

    // Request this chunk's transposed keys and the next chunk's keys now;
    // they land in LDS once products 3 and 4 have released R2 and R0.
    constexpr int kPer = (2 * kT * kCH) / kThreads;   // 16-byte pieces per thread, each kind
    static_assert(kPer == 4 && kPer * kThreads == 2 * kD * (kT / 8), "four pieces of each kind per thread");
    const bool more = q + 1 < q1;
    const int qn = more ? q + 1 : q;             // a chunk in range either way; stored only when more
    // piece u of this thread: transposed keys [plane][dim][row] (8 rows a
    // piece) and keys [plane][row][dim] of the next chunk
    auto kt_load = [&](int u) { return bload16(rs_kt, 16 * (tid + u * kThreads), q * 2 * kD * kT * 2); };
    auto kh_load = [&](int u) { return bload16(rs_kh, kh_off(tid + u * kThreads, qn), 0); };
    const uint4 kt0 = kt_load(0), kt1 = kt_load(1), kt2 = kt_load(2), kt3 = kt_load(3);
    const uint4 kh0 = kh_load(0), kh1 = kh_load(1), kh2 = kh_load(2), kh3 = kh_load(3);

    // ---- product 4 over the chunk's 64 rows: dW2 += G^T A for this wave's
    // gradient rows (kF w + 16 mt + [0, 16)) against all kD columns
#pragma unroll
    for (int ts = 0; ts < 2; ++ts) {
      bf16x8 gh[kFT], gl[kFT];
#pragma unroll
      for (int mt = 0; mt < kFT; ++mt) {
        const int jr = kF * w + 16 * mt + c;
        gh[mt] = lds16(R3 + ft_off(jr, 32 * ts + 8 * g));
        gl[mt] = lds16(R3 + kPlane + ft_off(jr, 32 * ts + 8 * g));
      }
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        if (nt == kNT / 2) __builtin_amdgcn_sched_barrier(0);   // half the column tiles' operands in flight
        const int i = 16 * nt + c;
        const bf16x8 ah = lds16(R2 + ft_off(i, 32 * ts + 8 * g));
        const bf16x8 al = lds16(R2 + kPlane + ft_off(i, 32 * ts + 8 * g));
#pragma unroll
        for (int mt = 0; mt < kFT; ++mt) dw2[mt][nt] = mfma3(gh[mt], gl[mt], ah, al, dw2[mt][nt]);
      }
    }

    // ---- product 3: GA = G W2 for this wave's hidden dims (i = kF w + 16 ft + c)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int ft = 0; ft < kFT; ++ft) acc[mb][ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int ks = 0; ks < kKS; ++ks) {
      bf16x8 bh8[kFT], bl8[kFT];
#pragma unroll
      for (int ft = 0; ft < kFT; ++ft) {
        const int i = kF * w + 16 * ft + c;
        bh8[ft] = as_bf16x8(bload16(rs_w, (i * kD + 8 * g) * 2, 64 * ks + 4 * kD * kD * 2));
        bl8[ft] = as_bf16x8(bload16(rs_w, (i * kD + 8 * g) * 2, 64 * ks + 5 * kD * kD * 2));
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int t = tile_tok(mb, c);
        const bf16x8 ah = lds16(R0 + tf_off<kD>(t, 32 * ks + 8 * g));
        const bf16x8 al = lds16(R0 + kPlane + tf_off<kD>(t, 32 * ks + 8 * g));
#pragma unroll
        for (int ft = 0; ft < kFT; ++ft) acc[mb][ft] = mfma3(ah, al, bh8[ft], bl8[ft], acc[mb][ft]);
      }
    }
    // GZ = GA * GELU'(Z) to R1 as [dim][row]
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int ft = 0; ft < kFT; ++ft) {
        const int i = kF * w + 16 * ft + c;
        float gz[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          gz[e] = (e < 4 ? acc[2 * a][ft][e] : acc[2 * a + 1][ft][e - 4]) * gp[a][ft][e];
          db1[ft] += gz[e];
        }
        bf16x8 h8, l8;
        pair8(gz, &h8, &l8);
        *reinterpret_cast<bf16x8 *>(R1 + ft_off(i, 32 * a + 8 * g)) = h8;
        *reinterpret_cast<bf16x8 *>(R1 + kPlane + ft_off(i, 32 * a + 8 * g)) = l8;
      }
    __syncthreads();

    // the requested keys to LDS: transposed ones to R2 (A's [dim][row] copy,
    // last read by product 4), the next chunk's to R0 (last read by product 3)
    auto kt_store = [&](int u, uint4 x) {
      const int i = tid + u * kThreads;
      const int pl = i / (kD * (kT / 8)), rem = i % (kD * (kT / 8)), f = rem / (kT / 8), grp = rem % (kT / 8);
      *reinterpret_cast<uint4 *>(R2 + pl * kPlane + ft_off(f, 8 * grp)) = x;
    };
    auto kh_store = [&](int u, uint4 x) {
      const int i = tid + u * kThreads;
      const int pl = i / (kT * kCH), rem = i % (kT * kCH), t = rem / kCH, ch = rem % kCH;
      *reinterpret_cast<uint4 *>(R0 + pl * kPlane + tf_off<kD>(t, 8 * ch)) = x;
    };
    kt_store(0, kt0); kt_store(1, kt1); kt_store(2, kt2); kt_store(3, kt3);
    if (more) {
      kh_store(0, kh0); kh_store(1, kh1); kh_store(2, kh2); kh_store(3, kh3);
    }
    __syncthreads();

    // ---- product 5 over the chunk's 64 rows: dW1 += GZ^T K^
#pragma unroll
    for (int ts = 0; ts < 2; ++ts) {
      bf16x8 zh[kFT], zl[kFT];
#pragma unroll
      for (int mt = 0; mt < kFT; ++mt) {
        const int jr = kF * w + 16 * mt + c;
        zh[mt] = lds16(R1 + ft_off(jr, 32 * ts + 8 * g));
        zl[mt] = lds16(R1 + kPlane + ft_off(jr, 32 * ts + 8 * g));
      }
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const int i = 16 * nt + c;
        const bf16x8 kh8 = lds16(R2 + ft_off(i, 32 * ts + 8 * g));
        const bf16x8 kl8 = lds16(R2 + kPlane + ft_off(i, 32 * ts + 8 * g));
#pragma unroll
        for (int mt = 0; mt < kFT; ++mt) dw1[mt][nt] = mfma3(zh[mt], zl[mt], kh8, kl8, dw1[mt][nt]);
      }
    }
    __syncthreads();
  }

  // ---- the split's sums: dW1 | db1 | dW2 | db2 | loss
  float *const slot = p.part + (bh * p.S + s) * (int64_t)p.ps;
#pragma unroll
  for (int mt = 0; mt < kFT; ++mt)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = kF * w + 16 * mt + 4 * g + e, col = 16 * nt + c;
        slot[row * kD + col] = dw1[mt][nt][e];
        slot[kD * kD + kD + row * kD + col] = dw2[mt][nt][e];
      }
#pragma unroll
  for (int ft = 0; ft < kFT; ++ft) {
    float x1 = db1[ft], x2 = db2[ft];
    x1 += __shfl_xor(x1, 16, 64);
    x1 += __shfl_xor(x1, 32, 64);
    x2 += __shfl_xor(x2, 16, 64);
    x2 += __shfl_xor(x2, 32, 64);
    if (g == 0) {
      slot[kD * kD + kF * w + 16 * ft + c] = x1;
      slot[2 * kD * kD + kD + kF * w + 16 * ft + c] = x2;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) loss += __shfl_xor(loss, o, 64);
  if (lane == 0) red[w] = loss;
  __syncthreads();
  if (tid == 0) {
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) sum += red[i];
    slot[2 * kD * kD + 2 * kD] = sum;
  }
}

// =====================================================================
// fit_adam_kernel: t = 0 loads the caller's weights; t >= 1 one Adam step
// =====================================================================
template <int kD, bool kF32>
__global__ void __launch_bounds__(kAdamThreads) fit_adam_kernel(FitDev p, int t, float c1, float c2, int last) {
  const int pi = blockIdx.y;
  const int k = blockIdx.x * kAdamThreads + threadIdx.x;
  const int GH = p.G * p.H, pb = pi / GH, lh = pi % GH;
  const int b0 = p.pred_shared ? 0 : pb, b1 = p.pred_shared ? p.B : pb + 1;
  float ninv = 0.f;
  {
    int64_t rows = 0;
    for (int b = b0; b < b1; ++b) rows += min(max(p.n_body[b], 0), p.N);
    if (rows > 0) ninv = static_cast<float>(1.0 / (static_cast<double>(rows) * kD));
  }
  if (t >= 1 && p.loss_out && blockIdx.x == 0 && threadIdx.x == 0) {
    float sum = 0.f;
    for (int b = b0; b < b1; ++b)
      for (int s = 0; s < p.S; ++s) sum += p.part[(((int64_t)b * GH + lh) * p.S + s) * p.ps + p.npar];
    p.loss_out[(int64_t)(t - 1) * (p.Bp * GH) + pi] = sum * ninv;
  }
  if (k >= p.npar) return;
  // caller's array and element of parameter k (order W1, b1, W2, b2)
  void *arr;
  int64_t at;
  if (k < kD * kD) { arr = p.w1; at = (int64_t)pi * kD * kD + k; }
  else if (k < kD * kD + kD) { arr = p.b1; at = (int64_t)pi * kD + (k - kD * kD); }
  else if (k < 2 * kD * kD + kD) { arr = p.w2; at = (int64_t)pi * kD * kD + (k - kD * kD - kD); }
  else { arr = p.b2; at = (int64_t)pi * kD + (k - 2 * kD * kD - kD); }
  float *const mw = p.master + (int64_t)pi * p.npar;
  float *const m1 = p.mom1 + (int64_t)pi * p.npar;
  float *const m2 = p.mom2 + (int64_t)pi * p.npar;
  float wk;
  if (t == 0) {
    wk = kF32 ? static_cast<const float *>(arr)[at] : bf16_to_f32(static_cast<const uint16_t *>(arr)[at]);
    m1[k] = 0.f;
    m2[k] = 0.f;
  } else {
    float gs = 0.f;
    for (int b = b0; b < b1; ++b)
      for (int s = 0; s < p.S; ++s) gs += p.part[(((int64_t)b * GH + lh) * p.S + s) * p.ps + k];
    const float gk = gs * ninv;
    if (t == 1 && p.grad_out) p.grad_out[(int64_t)pi * p.npar + k] = gk;
    const float mk = fmaf(p.beta1, m1[k], (1.f - p.beta1) * gk);
    const float vk = fmaf(p.beta2, m2[k], (1.f - p.beta2) * gk * gk);
    m1[k] = mk;
    m2[k] = vk;
    wk = mw[k] - p.lr * (mk * c1) / (sqrtf(vk * c2) + p.eps);
  }
  mw[k] = wk;
  // bf16-pair copies read by the next gradient pass: W1, W2, W2^T
  uint16_t *const wc = p.wc + (int64_t)pi * 6 * kD * kD;
  const uint16_t hi = f32_to_bf16(wk), lo = f32_to_bf16(wk - bf16_to_f32(hi));
  if (k < kD * kD) {
    wc[k] = hi;
    wc[kD * kD + k] = lo;
  } else if (k >= kD * kD + kD && k < 2 * kD * kD + kD) {
    const int kk = k - kD * kD - kD, j = kk / kD, i = kk % kD;
    wc[2 * kD * kD + kk] = hi;
    wc[3 * kD * kD + kk] = lo;
    wc[4 * kD * kD + i * kD + j] = hi;
    wc[5 * kD * kD + i * kD + j] = lo;
  }
  if (last) {
    if (kF32) static_cast<float *>(arr)[at] = wk;
    else static_cast<uint16_t *>(arr)[at] = f32_to_bf16(wk);
  }
}

template <int kD>
hipError_t launch_fit_d(const FitArgs &a, const FitDev &p, hipStream_t st) {
  const Dims &s = a.s;
  const bool f32 = s.dtype == LOWRAM_F32, int4 = s.coef_store == LOWRAM_STORE_INT4_G32;
  const int GH = s.G * s.H;
  if (p.NC > 0) {
    const dim3 grid(p.NC, GH, s.B);
    if (f32) hipLaunchKernelGGL((fit_prep_kernel<kD, true, false>), grid, dim3(kPrepThreads), 0, st, p);
    else if (int4) hipLaunchKernelGGL((fit_prep_kernel<kD, false, true>), grid, dim3(kPrepThreads), 0, st, p);
    else hipLaunchKernelGGL((fit_prep_kernel<kD, false, false>), grid, dim3(kPrepThreads), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 agrid((p.npar + kAdamThreads - 1) / kAdamThreads, p.Bp * GH);
  auto adam = [&](int t, float c1, float c2, int last) {
    if (f32) hipLaunchKernelGGL((fit_adam_kernel<kD, true>), agrid, dim3(kAdamThreads), 0, st, p, t, c1, c2, last);
    else hipLaunchKernelGGL((fit_adam_kernel<kD, false>), agrid, dim3(kAdamThreads), 0, st, p, t, c1, c2, last);
    return hipGetLastError();
  };
  hipError_t e = adam(0, 1.f, 1.f, 0);
  if (e != hipSuccess) return e;
  const size_t lds = fit_grad_lds(s.d);
  e = hipFuncSetAttribute(reinterpret_cast<const void *>(&fit_grad_kernel<kD>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  const dim3 ggrid(p.S * GH * s.B);
  for (int t = 1; t <= a.steps; ++t) {
    hipLaunchKernelGGL((fit_grad_kernel<kD>), ggrid, dim3(64 * (kD / 16)), lds, st, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // bias corrections 1 / (1 - beta^t), in fp64
    const double c1 = 1.0 / (1.0 - std::pow(a.beta1, t)), c2 = 1.0 / (1.0 - std::pow(a.beta2, t));
    if ((e = adam(t, static_cast<float>(c1), static_cast<float>(c2), t == a.steps)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t fit_grad_lds(int d) { return (size_t)4 * 2 * kT * d * 2 + 64; }

FitLayout fit_layout(const Dims &s) {
  FitLayout L{};
  const int64_t nbh = (int64_t)s.B * s.G * s.H;
  const int64_t nph = (int64_t)(s.pred_shared ? 1 : s.B) * s.G * s.H;
  L.NC = (s.N + kT - 1) / kT;
  L.NP = (int64_t)L.NC * kT;
  L.S = std::max(1, std::min(std::max(L.NC, 1), (int)((1024 + nbh - 1) / nbh)));
  L.npar = 2 * s.d * s.d + 2 * s.d;
  L.ps = L.npar + 64;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = (off + bytes + 255) & ~(size_t)255;
    return at;
  };
  L.kh = take((size_t)nbh * 2 * L.NP * s.d * 2);
  L.kt = take((size_t)nbh * L.NC * 2 * s.d * kT * 2);
  L.vt = take((size_t)nbh * L.NC * s.d * kT * 4);
  L.master = take((size_t)nph * L.npar * 4);
  L.mom1 = take((size_t)nph * L.npar * 4);
  L.mom2 = take((size_t)nph * L.npar * 4);
  L.wc = take((size_t)nph * 6 * s.d * s.d * 2);
  L.part = take((size_t)nbh * L.S * L.ps * 4);
  L.total = off;
  return L;
}

hipError_t launch_fit(const FitArgs &a, hipStream_t st) {
  const Dims &s = a.s;
  const FitLayout L = fit_layout(s);
  char *ws = static_cast<char *>(a.workspace);
  FitDev p{};
  p.B = s.B; p.G = s.G; p.H = s.H; p.N = s.N; p.r = s.r; p.Bp = s.pred_shared ? 1 : s.B;
  p.NC = L.NC; p.S = L.S; p.npar = L.npar; p.ps = L.ps; p.pred_shared = s.pred_shared; p.NP = L.NP;
  p.coef = a.coef; p.coef_scale = a.coef_scale; p.basis = a.basis; p.v = a.v; p.n_body = a.n_body;
  p.w1 = a.w1; p.b1 = a.b1; p.w2 = a.w2; p.b2 = a.b2; p.loss_out = a.loss_out; p.grad_out = a.grad_out;
  p.kh = reinterpret_cast<uint16_t *>(ws + L.kh);
  p.kt = reinterpret_cast<uint16_t *>(ws + L.kt);
  p.vt = reinterpret_cast<float *>(ws + L.vt);
  p.master = reinterpret_cast<float *>(ws + L.master);
  p.mom1 = reinterpret_cast<float *>(ws + L.mom1);
  p.mom2 = reinterpret_cast<float *>(ws + L.mom2);
  p.wc = reinterpret_cast<uint16_t *>(ws + L.wc);
  p.part = reinterpret_cast<float *>(ws + L.part);
  p.lr = static_cast<float>(a.lr); p.beta1 = static_cast<float>(a.beta1);
  p.beta2 = static_cast<float>(a.beta2); p.eps = static_cast<float>(a.eps);
  return s.d == 128 ? launch_fit_d<128>(a, p, st) : launch_fit_d<64>(a, p, st);
}

}  // namespace lowram
