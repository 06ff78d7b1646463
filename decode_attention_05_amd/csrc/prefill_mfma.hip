// MFMA prefill kernels for bf16 inputs with head_dim 128 (gfx950).
//
// LowRAM (arXiv:2611.07025), "LowRAM Paper: Amortised Values and Low-Rank
// Keys for KV Compression": "Step-by-step mental model for one decoding
// session" item 1 (compress at prefill), "Asymmetric key compression with
// xKV" (project the pre-RoPE keys of the layer group on a shared basis) and
// "Value cache amortisation in plain language" (the per-head value predictor
// scores how well each token is regenerated); arXiv listing, Abstract
// (residuals are kept for the worst-regenerated tokens only).
//
//   project_kernel  coefficients of every body row, C = X B^T, where row t of
//                   X is the concatenation over (layer, head) of the keys
//                   with their rotation undone; stored in bf16 or int4-g32
//   project_small_kernel  the same for calls with few rows per sequence
//   score_kernel    per (sequence, layer, head): keys rebuilt from the
//                   stored coefficients, predictor f = W2 GELU(W1 k + b1) + b2,
//                   squared error |v - f|^2 per row; the same kernel over the
//                   selected rows stores the residuals v - f instead
//
// Both are dense contractions on the matrix cores (16x16x32 MFMAs, lane =
// (c = lane % 16, g = lane / 16)).  Operand index order: every 16-row MFMA
// tile t of a 128-wide index (rank, head dimension, hidden unit) holds, in
// its row m, the index 32 (t / 2) + 8 (m / 4) + 4 (t % 2) + m % 4.  Then the
// accumulators a lane holds for tiles 2a and 2a + 1 cover the 8 consecutive
// indices 32 a + 8 g + [0, 8), which are exactly the K values of the lane's
// operand fragment in the next contraction (16-byte loads and stores, no
// shuffles between the chained products).
//
// Precision.  The projection input X is fp32 after the inverse rotation; it
// is split as X = hi + lo with hi, lo bf16 and both halves go through the
// MFMA (the basis is exact in bf16), so the coefficients carry fp32
// accuracy before they are rounded for storage.  The scoring pass and the
// residual pass split the rebuilt keys and the hidden activations the same
// way and use the exact-erf GELU; int4 coefficients enter the rebuild as
// exact bf16 pairs of code * scale.  The scores that decide the selection
// and the stored residuals v - f thus carry near-fp32 accuracy.
#include <algorithm>
#include <type_traits>

#include "lowram_internal.h"
#include "mfma_common.h"

namespace lowram {
namespace {

using namespace mfma;

constexpr int kD = 128;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

// index x in [0, 128 k) -> operand row 16 t + m (see the header comment)
__device__ __forceinline__ int tile_row(int x) {
  return (x & ~127) + 16 * (2 * ((x >> 5) & 3) + ((x >> 2) & 1)) + 4 * ((x >> 3) & 3) + (x & 3);
}

// bf16 pair split of 8 fp32 values: hi = bf16(x), lo = bf16(x - hi)
__device__ __forceinline__ void split8(f32x4 a, f32x4 b, bf16x8 *hi, bf16x8 *lo) {
  const bf16x8 h = pack8_bf16(a, b);
  f32x4 ra, rb;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ra[e] = a[e] - static_cast<float>(h[e]);
    rb[e] = b[e] - static_cast<float>(h[4 + e]);
  }
  *hi = h;
  *lo = pack8_bf16(ra, rb);
}

// int4 codes (nibble e of w, two's complement) times the fp16 group scale,
// in fp32 (exact: a code of at most 3 magnitude bits times an 11-bit scale
// has at most 14 significant bits), as a bf16 pair hi + lo, which holds them
// exactly too (16 significant bits): the rebuild then multiplies the stored
// coefficients exactly against the bf16 basis
__device__ __forceinline__ void dequant8_pair(uint32_t w, uint32_t scale_bits, bf16x8 *hi, bf16x8 *lo) {
  const float sc = f16_to_f32(static_cast<uint16_t>(scale_bits));
  f32x4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    a[e] = static_cast<float>(static_cast<int32_t>(w << (28 - 4 * e)) >> 28) * sc;
    b[e] = static_cast<float>(static_cast<int32_t>(w << (12 - 4 * e)) >> 28) * sc;
  }
  split8(a, b, hi, lo);
}

// symmetric int4 quantiser of one 32-value group spread over the four lanes
// g = 0..3 of a column (8 values each): fp16 scale max|x| / 7, codes
// clamp(rne(x / scale), -7, 7), all-zero group -> scale 0, codes 0.
// Returns the 8 codes as nibbles (value e in bits 4 e); every lane of the
// wave must call it.
__device__ __forceinline__ uint32_t quant8_int4(const float *x, uint16_t *scale_bits) {
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
  amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
  uint16_t sb = f32_to_f16(amax / 7.0f);
  if ((sb & 0x7fff) >= 0x7c00) sb = 0x7bff;       // saturate to the largest finite fp16
  const float sc = f16_to_f32(sb);
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    int code = 0;
    if (sc > 0.f) code = static_cast<int>(fminf(fmaxf(rintf(x[e] / sc), -7.f), 7.f));
    w |= static_cast<uint32_t>(code & 0xF) << (4 * e);
  }
  *scale_bits = sb;
  return w;
}

__device__ __forceinline__ uint4 pack8_bits(const float *x) {
  uint4 o;
  o.x = f32_to_bf16(x[0]) | (static_cast<uint32_t>(f32_to_bf16(x[1])) << 16);
  o.y = f32_to_bf16(x[2]) | (static_cast<uint32_t>(f32_to_bf16(x[3])) << 16);
  o.z = f32_to_bf16(x[4]) | (static_cast<uint32_t>(f32_to_bf16(x[5])) << 16);
  o.w = f32_to_bf16(x[6]) | (static_cast<uint32_t>(f32_to_bf16(x[7])) << 16);
  return o;
}

__device__ __forceinline__ void unpack8_bf16(uint4 v, float *x) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    x[2 * q] = __uint_as_float(w[q] << 16);
    x[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
  }
}

// =====================================================================
// project_kernel: C[t, k] = sum_c B[k, c] X[t, c] for one sequence
//
// Workgroup tile: 256 ranks x 128 tokens, 8 waves of 64 ranks x 64 tokens.
// The contraction runs over the D = G * Hkv * d columns in blocks of 64: a
// block holds, of one (layer, head), the columns j and j + 64 for
// j in [32 q, 32 q + 32), so the rotation pairs (j, j + 64) meet in the
// thread that stages them.  Per block the workgroup stages in LDS
//   X hi, X lo  [128 tokens][8 chunks of 16 B]   (bf16 halves of X)
//   basis       [256 ranks][8 chunks of 16 B]
// where chunk (kk, g) of a row holds the columns {j0 .. j0 + 3, j0 + 64 ..
// j0 + 67}, j0 = 32 q + 16 kk + 4 g: the K values of k-step kk for lane
// group g.  Chunks are XOR-swizzled by the row's low 3 bits.  Two stages
// alternate: the next block's global loads are issued before the current
// block's MFMAs and written to the other stage after them.
// =====================================================================

constexpr int kPRanks = 256;
constexpr int kPTok = 128;
constexpr int kPRow = 128;                            // bytes per staged row
constexpr int kPStage = (2 * kPTok + kPRanks) * kPRow; // 64 KiB

struct ProjArgs {
  PrefillArgs a;
  double inv_freq[64];      // theta^(-2 i / d)
  int n_tok_tiles, n_rank_tiles, n_items;
  int n_ksplit;             // splits of the contraction over (layer, head) column blocks
  float *partial;           // [n_ksplit, B, N, r] fp32 partial coefficients when n_ksplit > 1
};

__device__ __forceinline__ int prow_off(int row, int q8) { return row * kPRow + ((q8 ^ (row & 7)) << 4); }

template <bool kInt4Coef>
__global__ void __launch_bounds__(kThreads, 1) project_kernel(ProjArgs pa) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const PrefillArgs &a = pa.a;
  const Dims &s = a.s;
  const int r = s.r, N = s.N, H = s.H, G = s.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;

  // ---- workgroup -> (b, token tile, rank tile).  Each XCD (ids equal mod 8)
  // takes a contiguous run: the rank tiles of a token tile read the same key
  // rows, and the token tiles of a sequence the same basis, from its L2.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per_xcd = (pa.n_items + 7) / 8;
  const int item = xcd * per_xcd + slot;
  if (slot >= per_xcd || item >= pa.n_items) return;
  const int ks = item % pa.n_ksplit;                  // contraction split
  const int tile = item / pa.n_ksplit;
  const int rt = tile % pa.n_rank_tiles;
  const int tt = (tile / pa.n_rank_tiles) % pa.n_tok_tiles;
  const int b = tile / (pa.n_rank_tiles * pa.n_tok_tiles);
  const bool split = pa.n_ksplit > 1;
  const int tok0 = tt * kPTok, rank0 = rt * kPRanks;
  const int nb = min(a.n_body[b], N);
  const int wr = wave & 3, wt = wave >> 2;            // wave: ranks 64 wr.., tokens 64 wt..

  // ---- per-lane output location of the epilogue
  auto store_tile = [&](const f32x4 (*acc)[4], bool zero) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int t = tok0 + 64 * wt + 16 * nt + c;
      const bool tok_ok = t < N;
      const bool keep = !zero && t < nb;
#pragma unroll
      for (int a2 = 0; a2 < 2; ++a2) {
        const int r0 = rank0 + 64 * wr + 32 * a2 + 8 * g;
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = keep ? acc[2 * a2][nt][i] : 0.f;
          x[4 + i] = keep ? acc[2 * a2 + 1][nt][i] : 0.f;
        }
        if (split) {                        // fp32 partial sums; the reduce kernel stores
          if (tok_ok && r0 < r) {
            float4 *dst = reinterpret_cast<float4 *>(pa.partial + (((int64_t)ks * pa.a.s.B + b) * N + t) * r + r0);
            dst[0] = make_float4(x[0], x[1], x[2], x[3]);
            dst[1] = make_float4(x[4], x[5], x[6], x[7]);
          }
        } else if constexpr (kInt4Coef) {
          uint16_t sb;
          const uint32_t w = quant8_int4(x, &sb);
          if (tok_ok && r0 < r) {
            const int64_t crow = (int64_t)b * N + t;
            *reinterpret_cast<uint32_t *>(reinterpret_cast<uint8_t *>(a.coef) + crow * (r / 2) + r0 / 2) = w;
            if (g == 0) reinterpret_cast<uint16_t *>(a.coef_scale)[crow * (r / 32) + r0 / 32] = sb;
          }
        } else {
          if (tok_ok && r0 < r)
            *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(a.coef) + ((int64_t)b * N + t) * r + r0) = pack8_bits(x);
        }
      }
    }
  };

  if (tok0 >= nb) {                     // padding rows only: zero coefficients
    if (split) return;                  // (the reduce kernel writes them)
    f32x4 z[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) z[mt][nt] = f32x4{0, 0, 0, 0};
    store_tile(z, true);
    return;
  }

  // ---- staging assignment: thread -> (row slot, chunk q8 = 4 kk + gq)
  const int q8 = tid & 7, kk_s = q8 >> 2, gq = q8 & 3;
  const int srow = tid >> 3;                          // 0..63
  // X items: tokens srow and srow + 64; their rotation cos / sin for the
  // columns j0 + i of both blocks q = 0, 1 of a head (fixed for the whole loop)
  float csv[2][2][4], snv[2][2][4];
  int64_t xrow[2];
  bool xok[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int t = tok0 + srow + 64 * e;
    xok[e] = t < nb;
    const int tc = xok[e] ? t : 0;
    const int p = a.pos ? a.pos[(int64_t)b * N + tc] : tc;
    xrow[e] = tc;
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) rope_cs(p, pa.inv_freq[32 * q + 16 * kk_s + 4 * gq + i], &csv[e][q][i], &snv[e][q][i]);
  }
  // basis items: ranks srow + 64 e, e = 0..3 (clamped rows are zeroed when staged)
  const uint16_t *bas = reinterpret_cast<const uint16_t *>(a.basis) + (int64_t)b * r * s.D;
  const uint16_t *kp = reinterpret_cast<const uint16_t *>(a.k_post);

  uint2 xr[2][2][2], br[2][4][2];                    // [register set][item][half]
  auto gload = [&](int kb, int set) {
    const int lh = kb >> 1, q = kb & 1;
    const int l = lh / H, h = lh - l * H;
    const int j0 = 32 * q + 16 * kk_s + 4 * gq;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint16_t *p = kp + ((((int64_t)b * G + l) * N + xrow[e]) * H + h) * kD + j0;
      xr[set][e][0] = *reinterpret_cast<const uint2 *>(p);
      xr[set][e][1] = *reinterpret_cast<const uint2 *>(p + 64);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rk = min(rank0 + srow + 64 * e, r - 1);
      const uint16_t *p = bas + (int64_t)rk * s.D + (int64_t)lh * kD + j0;
      br[set][e][0] = *reinterpret_cast<const uint2 *>(p);
      br[set][e][1] = *reinterpret_cast<const uint2 *>(p + 64);
    }
  };
  auto stage = [&](int buf, int q, int set) {
    char *st = lds + buf * kPStage;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      float y[8], x[8];
      const uint4 raw = {xr[set][e][0].x, xr[set][e][0].y, xr[set][e][1].x, xr[set][e][1].y};
      unpack8_bf16(raw, y);           // y[0..3] = columns j0.., y[4..7] = j0 + 64..
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float cs = q ? csv[e][1][i] : csv[e][0][i];
        const float sn = q ? snv[e][1][i] : snv[e][0][i];
        x[i] = xok[e] ? y[i] * cs + y[4 + i] * sn : 0.f;
        x[4 + i] = xok[e] ? y[4 + i] * cs - y[i] * sn : 0.f;
      }
      bf16x8 hi, lo;
      split8(f32x4{x[0], x[1], x[2], x[3]}, f32x4{x[4], x[5], x[6], x[7]}, &hi, &lo);
      const int row = srow + 64 * e;
      *reinterpret_cast<bf16x8 *>(st + prow_off(row, q8)) = hi;
      *reinterpret_cast<bf16x8 *>(st + kPTok * kPRow + prow_off(row, q8)) = lo;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rl = srow + 64 * e;
      const uint32_t keep = (rank0 + rl < r) ? ~0u : 0u;    // ranks past r stage as zeros
      const uint4 v = {br[set][e][0].x & keep, br[set][e][0].y & keep, br[set][e][1].x & keep,
                       br[set][e][1].y & keep};
      *reinterpret_cast<uint4 *>(st + 2 * kPTok * kPRow + prow_off(tile_row(rl), q8)) = v;
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0, 0, 0, 0};
  const bool wave_on = rank0 + 64 * wr < r;           // uniform per wave

  auto mfma_block = [&](int buf) {
    const char *st = lds + buf * kPStage;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int qq = 4 * kk + g;
      bf16x8 af[4], bh[4], bl[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        af[mt] = *reinterpret_cast<const bf16x8 *>(st + 2 * kPTok * kPRow + prow_off(64 * wr + 16 * mt + c, qq));
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int row = 64 * wt + 16 * nt + c;
        bh[nt] = *reinterpret_cast<const bf16x8 *>(st + prow_off(row, qq));
        bl[nt] = *reinterpret_cast<const bf16x8 *>(st + kPTok * kPRow + prow_off(row, qq));
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          acc[mt][nt] = mfma_bf16(af[mt], bh[nt], acc[mt][nt]);
          acc[mt][nt] = mfma_bf16(af[mt], bl[nt], acc[mt][nt]);
        }
    }
  };

  // Global loads run two blocks ahead: register set (kb & 1) holds block
  // kb from its request (two blocks earlier) until it is staged.  Requests
  // past the last block re-read the last block (unused), so the loop has no
  // branches around its loads.
  const int hps = G * H / pa.n_ksplit;                // (layer, head) blocks of this split
  const int kb0 = 2 * hps * ks, nkb = 2 * hps * (ks + 1);   // block range [kb0, nkb), even length
  gload(kb0, 0);
  gload(kb0 + 1, 1);
  stage(0, 0, 0);
  __syncthreads();
  for (int kb = kb0; kb < nkb; kb += 2) {
    // block kb (LDS stage 0) on the matrix cores; set 1 holds block kb + 1
    gload(min(kb + 2, nkb - 1), 0);
    __builtin_amdgcn_sched_barrier(0);
    if (wave_on) mfma_block(0);
    __builtin_amdgcn_sched_barrier(0);
    stage(1, 1, 1);
    __syncthreads();
    // block kb + 1 (LDS stage 1); set 0 holds block kb + 2
    gload(min(kb + 3, nkb - 1), 1);
    __builtin_amdgcn_sched_barrier(0);
    if (wave_on) mfma_block(1);
    __builtin_amdgcn_sched_barrier(0);
    if (kb + 2 < nkb) stage(0, 0, 0);
    __syncthreads();
  }
  if (wave_on) store_tile(acc, false);
}

// Sum of the contraction splits, in split order, and the coefficient store:
// one thread per (sequence, row, 8 ranks), the four threads of a 32-rank
// int4 group adjacent in the wave; padding rows get zeros.
template <bool kInt4Coef>
__global__ void __launch_bounds__(256) proj_reduce_kernel(ProjArgs pa) {
  const PrefillArgs &a = pa.a;
  const int r = a.s.r, N = a.s.N, n8 = r / 8;
  const int64_t n_all = (int64_t)a.s.B * N * n8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool in = gid < n_all;
  const int64_t gc = in ? gid : n_all - 1;             // the tail re-reads the last chunk
  const int c8 = static_cast<int>(gc % n8);
  const int64_t row = gc / n8;                        // b * N + t
  const int b = static_cast<int>(row / N), t = static_cast<int>(row % N);
  const bool keep = t < min(a.n_body[b], N);
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = 0.f;
  if (keep) {
    for (int k = 0; k < pa.n_ksplit; ++k) {
      const float4 *src = reinterpret_cast<const float4 *>(pa.partial + ((int64_t)k * a.s.B * N + row) * r + 8 * c8);
      const float4 v0 = src[0], v1 = src[1];
      x[0] += v0.x; x[1] += v0.y; x[2] += v0.z; x[3] += v0.w;
      x[4] += v1.x; x[5] += v1.y; x[6] += v1.z; x[7] += v1.w;
    }
  }
  if constexpr (kInt4Coef) {
    // the quantiser of quant8_int4 over the group's four adjacent lanes
    // (r / 8 is a multiple of 4, so a group never straddles rows or waves)
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    uint16_t sb = f32_to_f16(amax / 7.0f);
    if ((sb & 0x7fff) >= 0x7c00) sb = 0x7bff;
    const float sc = f16_to_f32(sb);
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int code = 0;
      if (sc > 0.f) code = static_cast<int>(fminf(fmaxf(rintf(x[e] / sc), -7.f), 7.f));
      w |= static_cast<uint32_t>(code & 0xF) << (4 * e);
    }
    if (in) {
      *reinterpret_cast<uint32_t *>(reinterpret_cast<uint8_t *>(a.coef) + row * (r / 2) + 4 * c8) = w;
      if ((c8 & 3) == 0) reinterpret_cast<uint16_t *>(a.coef_scale)[row * (r / 32) + c8 / 4] = sb;
    }
  } else if (in) {
    *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(a.coef) + row * r + 8 * c8) = pack8_bits(x);
  }
}

// =====================================================================
// project_small_kernel: the same coefficients C = X B^T for calls with few
// rows per sequence (the fold of an exact tail into the body), where the
// tiles of project_kernel would need a split contraction whose fp32 partial
// sums pass through HBM.  One workgroup per (sequence, 32-token tile,
// 64-rank tile) runs the whole contraction: wave w takes the (layer, head)
// column blocks w, w + 8, ..., with its operands loaded from global memory
// straight into registers (16 bytes per lane and fragment), and the eight
// wave tiles are summed in LDS in wave order (deterministic) before the
// store.
//
// k-steps: per (layer, head) block two units kq = 0, 1; unit kq's lane
// group g holds the columns j0 .. j0 + 7 (k-step 2 kq) and j0 + 64 ..
// j0 + 71 (k-step 2 kq + 1), j0 = 32 kq + 8 g, so each rotation pair
// (j, j + 64) meets in one lane.  A = basis rows (ranks 16 mt + c), B = the
// keys with their rotation undone (tokens 16 nt + c), split into bf16
// halves as in project_kernel.  The (cos, sin) of every (token, frequency)
// of the tile are formed once, into LDS.
// =====================================================================

constexpr int kSTok = 32;                      // tokens per workgroup
constexpr int kSRanks = 64;                    // ranks per workgroup
constexpr int kSCsRow = 64 * 8 + 16;           // bytes per token row of (cos, sin) pairs (padded)
constexpr int kSRedRow = kSRanks + 4;          // floats per token row of a wave's tile (padded)
constexpr size_t kSmallLds = (size_t)kSTok * kSCsRow + (size_t)kWaves * kSTok * kSRedRow * 4;

template <bool kInt4Coef>
__global__ void __launch_bounds__(kThreads, 1) project_small_kernel(ProjArgs pa) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const PrefillArgs &a = pa.a;
  const Dims &s = a.s;
  const int r = s.r, N = s.N, H = s.H, G = s.G, GH = s.G * s.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;

  // ---- workgroup -> (b, token tile, rank tile); each XCD takes a
  // contiguous run (the rank tiles of a token tile read the same keys, the
  // token tiles of a sequence the same basis)
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per_xcd = (pa.n_items + 7) / 8;
  const int item = xcd * per_xcd + slot;
  if (slot >= per_xcd || item >= pa.n_items) return;
  const int rt = item % pa.n_rank_tiles;
  const int tt = (item / pa.n_rank_tiles) % pa.n_tok_tiles;
  const int b = item / (pa.n_rank_tiles * pa.n_tok_tiles);
  const int tok0 = tt * kSTok, rank0 = rt * kSRanks;
  const int nb = min(max(a.n_body[b], 0), N);

  char *csl = lds;                                                    // [kSTok][kSCsRow]
  float *red = reinterpret_cast<float *>(lds + (size_t)kSTok * kSCsRow);   // [kWaves][kSTok][kSRedRow]

  // ---- store of 8 consecutive ranks of one token (threads 0..255: token
  // tid / 8, ranks 8 (tid % 8) ..; the four threads of a 32-rank int4 group
  // are adjacent lanes)
  auto store8 = [&](int tok, int r8, float *x) {
    const int t = tok0 + tok;
    const int64_t crow = (int64_t)b * N + t;
    const int rk = rank0 + 8 * r8;
    if constexpr (kInt4Coef) {
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      uint16_t sb = f32_to_f16(amax / 7.0f);
      if ((sb & 0x7fff) >= 0x7c00) sb = 0x7bff;
      const float sc = f16_to_f32(sb);
      uint32_t w = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int code = 0;
        if (sc > 0.f) code = static_cast<int>(fminf(fmaxf(rintf(x[e] / sc), -7.f), 7.f));
        w |= static_cast<uint32_t>(code & 0xF) << (4 * e);
      }
      if (t < N) {
        *reinterpret_cast<uint32_t *>(reinterpret_cast<uint8_t *>(a.coef) + crow * (r / 2) + rk / 2) = w;
        if ((r8 & 3) == 0) reinterpret_cast<uint16_t *>(a.coef_scale)[crow * (r / 32) + rk / 32] = sb;
      }
    } else {
      if (t < N) *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(a.coef) + crow * r + rk) = pack8_bits(x);
    }
  };

  if (tok0 >= nb) {                                   // padding rows only: zero coefficients
    if (tid < kSTok * 8) {
      float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      store8(tid >> 3, tid & 7, z);
    }
    return;
  }

  // ---- (cos, sin) of frequency f at the position of token tok0 + i; both
  // zero for tokens past the body, whose keys then enter as zeros (thread:
  // token tid / 16, frequencies 4 (tid % 16) ..)
  {
    static_assert(kSTok * 16 == kThreads, "one thread per token and 4 frequencies");
    const int i = tid >> 4, f0 = 4 * (tid & 15);
    const int t = tok0 + i;
    const bool ok = t < nb;
    const int p = ok ? (a.pos ? a.pos[(int64_t)b * N + t] : t) : 0;
    double fr[4];                                     // requested together, before the first use
#pragma unroll
    for (int q = 0; q < 4; ++q) fr[q] = pa.inv_freq[f0 + q];
    float4 cs2[2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float cv, sv;
      rope_cs(p, fr[q], &cv, &sv);
      if (!ok) cv = sv = 0.f;
      if (q & 1) { cs2[q >> 1].z = cv; cs2[q >> 1].w = sv; } else { cs2[q >> 1].x = cv; cs2[q >> 1].y = sv; }
    }
    float4 *dst = reinterpret_cast<float4 *>(csl + i * kSCsRow + 8 * f0);
    dst[0] = cs2[0];
    dst[1] = cs2[1];
  }
  __syncthreads();

  // ---- this lane's rows: basis ranks rank0 + 16 mt + c, tokens 16 nt + c
  const uint16_t *bas = reinterpret_cast<const uint16_t *>(a.basis) + ((int64_t)b * r + rank0 + c) * s.D + 8 * g;
  const uint16_t *kp = reinterpret_cast<const uint16_t *>(a.k_post);
  int xrow[2];                                        // rows past the body read row 0 (zero rotation)
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) xrow[nt] = (tok0 + 16 * nt + c < nb) ? tok0 + 16 * nt + c : 0;

  struct Unit {
    uint4 bs[4][2];     // [mt][half]: basis columns j0 + 64 half + [0, 8)
    uint4 x[2][2];      // [nt][half]: keys, the same columns
  };
  const int n_blk = (GH - wave + kWaves - 1) / kWaves;    // (layer, head) blocks of this wave
  const int n_units = 2 * n_blk;
  // loads past the last unit re-read the last one (unused): no branches around the loads
  auto load_unit = [&](int u, Unit &U) {
    const int uu = min(u, n_units - 1);
    const int lh = wave + kWaves * (uu >> 1), kq = uu & 1;
    const int l = lh / H, h = lh - l * H;
    const uint16_t *bp = bas + (int64_t)lh * kD + 32 * kq;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      U.bs[mt][0] = *reinterpret_cast<const uint4 *>(bp + (int64_t)16 * mt * s.D);
      U.bs[mt][1] = *reinterpret_cast<const uint4 *>(bp + (int64_t)16 * mt * s.D + 64);
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const uint16_t *xp = kp + ((((int64_t)b * G + l) * N + xrow[nt]) * H + h) * kD + 32 * kq + 8 * g;
      U.x[nt][0] = *reinterpret_cast<const uint4 *>(xp);
      U.x[nt][1] = *reinterpret_cast<const uint4 *>(xp + 64);
    }
  };

  f32x4 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) { acc[mt][0] = f32x4{0, 0, 0, 0}; acc[mt][1] = f32x4{0, 0, 0, 0}; }

  auto compute_unit = [&](int u, const Unit &U) {
    const int kq = u & 1;
    bf16x8 bh[2][2], bl[2][2];                        // [nt][half]
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float4 *cp = reinterpret_cast<const float4 *>(csl + (16 * nt + c) * kSCsRow + 8 * (32 * kq + 8 * g));
      float cv[8], sv[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = cp[q];
        cv[2 * q] = v.x; sv[2 * q] = v.y; cv[2 * q + 1] = v.z; sv[2 * q + 1] = v.w;
      }
      float y0[8], y1[8], x0[8], x1[8];
      unpack8_bf16(U.x[nt][0], y0);
      unpack8_bf16(U.x[nt][1], y1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x0[e] = y0[e] * cv[e] + y1[e] * sv[e];
        x1[e] = y1[e] * cv[e] - y0[e] * sv[e];
      }
      split8(f32x4{x0[0], x0[1], x0[2], x0[3]}, f32x4{x0[4], x0[5], x0[6], x0[7]}, &bh[nt][0], &bl[nt][0]);
      split8(f32x4{x1[0], x1[1], x1[2], x1[3]}, f32x4{x1[4], x1[5], x1[6], x1[7]}, &bh[nt][1], &bl[nt][1]);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 af = as_bf16x8(U.bs[mt][half]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          acc[mt][nt] = mfma_bf16(af, bh[nt][half], acc[mt][nt]);
          acc[mt][nt] = mfma_bf16(af, bl[nt][half], acc[mt][nt]);
        }
      }
  };

  // two units in flight: register set u % 2 holds unit u from its request
  // (two units earlier) until its products; the scheduling barriers keep
  // each request after the products of the unit it replaces, so the memory
  // waits before a unit's products cover only that unit's requests
  if (n_units > 0) {
    Unit U0, U1;
    load_unit(0, U0);
    load_unit(1, U1);
    for (int u = 0; u < n_units; u += 2) {       // n_units is even
      __builtin_amdgcn_sched_barrier(0);
      compute_unit(u, U0);
      __builtin_amdgcn_sched_barrier(0);
      load_unit(u + 2, U0);
      __builtin_amdgcn_sched_barrier(0);
      compute_unit(u + 1, U1);
      __builtin_amdgcn_sched_barrier(0);
      load_unit(u + 3, U1);
    }
  }

  // ---- the wave tiles (rank 16 mt + 4 g + i, token 16 nt + c) to LDS, then
  // summed in wave order and stored
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      *reinterpret_cast<f32x4 *>(red + ((size_t)wave * kSTok + 16 * nt + c) * kSRedRow + 16 * mt + 4 * g) =
          acc[mt][nt];
  __syncthreads();
  if (tid < kSTok * 8) {
    const int tok = tid >> 3, r8 = tid & 7;
    float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float4 *src = reinterpret_cast<const float4 *>(red + ((size_t)w * kSTok + tok) * kSRedRow + 8 * r8);
      const float4 v0 = src[0], v1 = src[1];
      x[0] += v0.x; x[1] += v0.y; x[2] += v0.z; x[3] += v0.w;
      x[4] += v1.x; x[5] += v1.y; x[6] += v1.z; x[7] += v1.w;
    }
    if (tok0 + tok >= nb) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    store8(tok, r8, x);
  }
}

// =====================================================================
// score_kernel: rebuild, predict, score (or store residuals)
//
// One workgroup (8 waves) per (sequence b, layer-head lh, split of the rows);
// the workgroup keeps the (lh) slice of the basis in LDS as [j][rank]
// (rows in operand order, XOR-swizzled 16-byte chunks) and W1 of the head
// as [u][j] (rows in operand order, halved: the GELU takes x / 2).  Each
// wave takes 32-row tiles:
//   1. K^T[j, t] = sum_k B^T[j, k] C^T[k, t]   (A = basis from LDS, B =
//      coefficient rows from HBM, four k-steps in flight)
//   2. H^T[u, t] = W1 K^T + b1, GELU           (A = W1 from LDS, B = K^T
//      from the accumulators: rows 32 a + 8 g + [0, 8) of tiles 2a, 2a+1)
//   3. F^T[j, t] = W2 H^T + b2                 (A = W2 rows from L2, B = H^T
//      from registers)
//   4. e[t] = sum_j (v[t, j] - F[t, j])^2, or the residual v - F of the
//      selected rows (kResid: rows come from the selected index lists)
// With kPairs the activation operands of products 2 and 3 (the rebuilt key
// and the hidden layer) are split into bf16 pairs x = hi + lo,
// |x - hi - lo| <= 2^-16 |x|, each product runs on both halves against the
// exact bf16 weights, and the GELU is the exact-erf form: the scores then
// carry near-fp32 accuracy, so the selection they decide differs from the
// exact one only between rows whose exact scores lie within that accuracy.
// Without it the operands are single bf16 values (2^-8) and the GELU the
// half-argument tail polynomial, as in decode.
// =====================================================================

struct ScoreArgs {
  PrefillArgs a;
  int S;             // splits per (b, lh)
  int split_rows;    // rows (residual slots with kResid) per split, a multiple of 32
  int n_items;
};

constexpr int kTile = 32;
constexpr int kTileRows = kTile * kWaves;

template <bool kInt4Coef, bool kResid, bool kPairs, bool kStoreAll = false>
__global__ void __launch_bounds__(kThreads, 1) score_kernel(ScoreArgs sa) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const PrefillArgs &a = sa.a;
  const Dims &s = a.s;
  const int r = s.r, N = s.N, H = s.H, G = s.G, GH = s.G * s.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;

  // ---- workgroup -> (b, split, lh); the heads of one (b, split) read the
  // same coefficient rows and run on one XCD
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per_xcd = (sa.n_items + 7) / 8;
  const int item = xcd * per_xcd + slot;
  if (slot >= per_xcd || item >= sa.n_items) return;
  const int lh = item % GH, split = (item / GH) % sa.S, b = item / (GH * sa.S);
  const int l = lh / H, h = lh - l * H;
  const int nb = min(a.n_body[b], N);
  const int n_rows = kResid ? s.m : N;
  const int i0 = split * sa.split_rows;
  const int i1 = min(n_rows, i0 + sa.split_rows);
  if (i0 >= i1) return;
  const int64_t elh = (int64_t)b * GH + lh;           // (b, l, h) index of err / residual arrays
  if (!kResid && i0 >= nb) {                          // padding rows only
    for (int t = i0 + tid; t < i1; t += kThreads) a.err[elh * N + t] = 0.f;
    return;
  }

  // ---- stage the basis slice (columns lh * 128 + j) rank-chunk major: the
  // 16-byte chunk of ranks 8 kb .. 8 kb + 7 of operand row x = tile_row(j)
  // sits at kb * 2048 + 16 * ((x & ~15) | ((x & 15) ^ (kb & 15))), so a
  // k-step's fragment of 16 rows is one 256-byte run (no bank conflict) and
  // the other column tiles are fixed offsets from it; the 16 lanes that
  // write one instruction's chunks take 16 consecutive kb, so their slots
  // differ as well
  {
    const uint16_t *basis = reinterpret_cast<const uint16_t *>(a.basis) + (int64_t)b * r * s.D + (int64_t)lh * kD;
    const int nkb = r / 8;
    const int nblk = (nkb + 15) / 16 * 256;     // blocks (kb / 16, jb, kb % 16) of 8 ranks x 8 columns
    for (int blk = tid; blk < nblk; blk += kThreads) {
      const int kb = 16 * (blk >> 8) + (blk & 15), jb = (blk >> 4) & 15;
      if (kb >= nkb) continue;
      uint4 v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        v[q] = *reinterpret_cast<const uint4 *>(basis + (int64_t)(8 * kb + q) * s.D + 8 * jb);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        uint16_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t w = (jj >> 1) == 0 ? v[q].x : (jj >> 1) == 1 ? v[q].y : (jj >> 1) == 2 ? v[q].z : v[q].w;
          uint16_t x = static_cast<uint16_t>((jj & 1) ? (w >> 16) : (w & 0xffff));
          // fp16 operands for the int4 path with single operands; the pair
          // path multiplies bf16 pairs against the bf16 basis
          if (kInt4Coef && !kPairs) x = f32_to_f16(bf16_to_f32(x));
          e[q] = x;
        }
        uint4 o;
        o.x = e[0] | (static_cast<uint32_t>(e[1]) << 16);
        o.y = e[2] | (static_cast<uint32_t>(e[3]) << 16);
        o.z = e[4] | (static_cast<uint32_t>(e[5]) << 16);
        o.w = e[6] | (static_cast<uint32_t>(e[7]) << 16);
        const int x = tile_row(8 * jb + jj);
        *reinterpret_cast<uint4 *>(lds + kb * 2048 + 16 * ((x & ~15) | ((x & 15) ^ (kb & 15)))) = o;
      }
    }
  }
  // ---- W1 of the head, halved, rows in operand order, chunk ch of row x at (ch ^ (x & 15))
  char *w1l = lds + (size_t)r * kD * 2;
  const int pb = s.pred_shared ? 0 : b;
  const int64_t who = ((int64_t)pb * G + l) * H + h;
  {
    const uint16_t *w1 = reinterpret_cast<const uint16_t *>(a.w1) + who * kD * kD;
    for (int q = tid; q < kD * (kD / 8); q += kThreads) {
      const int u = q >> 4, ch = q & 15;
      float x[8];
      unpack8_bf16(*reinterpret_cast<const uint4 *>(w1 + (int64_t)u * kD + 8 * ch), x);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= 0.5f;
      const int row = tile_row(u);
      *reinterpret_cast<uint4 *>(w1l + row * (2 * kD) + ((ch ^ (row & 15)) << 4)) = pack8_bits(x);
    }
  }
  __syncthreads();

  // biases in the accumulator order: b1 of hidden rows 32 (ut/2) + 8 g +
  // 4 (ut%2) + i, b2 of output rows 32 a + 8 g + [0, 8) (read per tile from
  // L1, like the W2 rows, rather than held in registers)
  const uint16_t *b1p = reinterpret_cast<const uint16_t *>(a.b1) + who * kD;
  const uint16_t *b2p = reinterpret_cast<const uint16_t *>(a.b2) + who * kD;
  const uint16_t *w2 = reinterpret_cast<const uint16_t *>(a.w2) + who * kD * kD;
  const uint16_t *vbase = reinterpret_cast<const uint16_t *>(a.v);
  const int32_t *ridx = kResid ? a.resid_idx + elh * s.m : nullptr;

  // coefficient buffer resources over the sequence's rows
  __amdgpu_buffer_rsrc_t crs, srs;
  if constexpr (kInt4Coef) {
    crs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(reinterpret_cast<const uint8_t *>(a.coef)) + (int64_t)b * N * (r / 2), 0,
        static_cast<int>((int64_t)N * (r / 2)), 0x00020000);
    srs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(reinterpret_cast<const uint16_t *>(a.coef_scale)) + (int64_t)b * N * (r / 32), 0,
        static_cast<int>((int64_t)N * (r / 32) * 2), 0x00020000);
  } else {
    crs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(reinterpret_cast<const uint16_t *>(a.coef)) + (int64_t)b * N * r, 0,
        static_cast<int>((int64_t)N * r * 2), 0x00020000);
    srs = crs;
  }
  // basis fragment of k-step kk = ks + u (ks a multiple of 4), column tile
  // jt, lane (c, g): chunk 4 kk + g of row 16 jt + c, at
  // bo[u] + 8192 kk + 256 jt with a per-lane part that depends on u only
  int bo[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) bo[u] = 2048 * g + 16 * (c ^ (4 * u + g));
  const int nks = r / 32;                             // even: r is a multiple of 64

  for (int t0 = i0 + kTile * wave; t0 < i1; t0 += kTileRows) {
    const int nvalid = min(kTile, i1 - t0);
    if (!kResid && t0 >= nb) {                        // padding rows: score 0
      if (g == 0)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          if (16 * tt + c < nvalid) a.err[elh * N + t0 + 16 * tt + c] = 0.f;
      continue;
    }
    // rows of this lane's two tokens (16 tt + c); invalid ones read row 0
    int row[2];
    bool ok[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tl = 16 * tt + c;
      int rw = t0 + tl;
      bool v = tl < nvalid;
      if (kResid) rw = v ? ridx[rw] : 0;
      v = v && rw >= 0 && rw < nb;
      row[tt] = v ? rw : 0;
      ok[tt] = v;
    }

    // ---- 1. rebuild K^T
    f32x4 acc[8][2];
#pragma unroll
    for (int jt = 0; jt < 8; ++jt) { acc[jt][0] = f32x4{0, 0, 0, 0}; acc[jt][1] = f32x4{0, 0, 0, 0}; }
    {
      typedef typename std::conditional<kInt4Coef, uint2, uint4>::type Frag;
      int vo[2], so[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        if constexpr (kInt4Coef) {
          vo[tt] = row[tt] * (r / 2) + 4 * g;
          so[tt] = row[tt] * (r / 32) * 2;
        } else {
          vo[tt] = (row[tt] * r + 8 * g) * 2;
          so[tt] = 0;
        }
      }
      auto ldc = [&](int tt, int kk) -> Frag {
        if constexpr (kInt4Coef) {
          return uint2{__builtin_amdgcn_raw_buffer_load_b32(crs, vo[tt], 16 * kk, 0),
                       static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(srs, so[tt], 2 * kk, 0))};
        } else {
          return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(crs, vo[tt], 64 * kk, 0));
        }
      };
      auto kstep = [&](int ks, int u, const Frag &f0, const Frag &f1) {
        const char *fb = lds + bo[u] + 8192 * (ks + u);
        if constexpr (kInt4Coef && kPairs) {
          bf16x8 h0, l0, h1, l1;
          dequant8_pair(f0.x, f0.y, &h0, &l0);
          dequant8_pair(f1.x, f1.y, &h1, &l1);
          bf16x8 af[8];
#pragma unroll
          for (int jt = 0; jt < 8; ++jt)
            af[jt] = as_bf16x8(*reinterpret_cast<const uint4 *>(fb + 256 * jt));
#pragma unroll
          for (int jt = 0; jt < 8; ++jt) {
            acc[jt][0] = mfma_bf16(af[jt], h0, acc[jt][0]);
            acc[jt][0] = mfma_bf16(af[jt], l0, acc[jt][0]);
            acc[jt][1] = mfma_bf16(af[jt], h1, acc[jt][1]);
            acc[jt][1] = mfma_bf16(af[jt], l1, acc[jt][1]);
          }
        } else if constexpr (kInt4Coef) {
          const f16x8 cb0 = dequant8(f0.x, f0.y), cb1 = dequant8(f1.x, f1.y);
          f16x8 af[8];
#pragma unroll
          for (int jt = 0; jt < 8; ++jt)
            af[jt] = as_f16x8(*reinterpret_cast<const uint4 *>(fb + 256 * jt));
#pragma unroll
          for (int jt = 0; jt < 8; ++jt) {
            acc[jt][0] = mfma_f16(af[jt], cb0, acc[jt][0]);
            acc[jt][1] = mfma_f16(af[jt], cb1, acc[jt][1]);
          }
        } else {
          const bf16x8 cb0 = as_bf16x8(f0), cb1 = as_bf16x8(f1);
          bf16x8 af[8];
#pragma unroll
          for (int jt = 0; jt < 8; ++jt)
            af[jt] = as_bf16x8(*reinterpret_cast<const uint4 *>(fb + 256 * jt));
#pragma unroll
          for (int jt = 0; jt < 8; ++jt) {
            acc[jt][0] = mfma_bf16(af[jt], cb0, acc[jt][0]);
            acc[jt][1] = mfma_bf16(af[jt], cb1, acc[jt][1]);
          }
        }
      };
      Frag p0[4], p1[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        p0[u] = ldc(0, min(u, nks - 1));
        p1[u] = ldc(1, min(u, nks - 1));
      }
      int ks = 0;
      for (; ks + 8 <= nks; ks += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          kstep(ks, u, p0[u], p1[u]);
          p0[u] = ldc(0, ks + u + 4);
          p1[u] = ldc(1, ks + u + 4);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (nks - ks >= 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          kstep(ks, u, p0[u], p1[u]);
          if (ks + u + 4 < nks) {
            p0[u] = ldc(0, ks + u + 4);
            p1[u] = ldc(1, ks + u + 4);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        ks += 4;
      }
      if (ks < nks) {
        kstep(ks, 0, p0[0], p1[0]);
        kstep(ks, 1, p0[1], p1[1]);
      }
    }

    // Per-tile copies of the lane's operand offsets, opaque to the compiler:
    // the W1 / W2 / bias reads do not depend on the tile, and hoisting all
    // of them out of the loop would hold ~300 registers.
    int wofs = 8 * g, wrow0 = c;
    asm volatile("" : "+v"(wofs), "+v"(wrow0));
    // W2 A-operand row of lane c in tile jt: output j = 32 (jt/2) + 8 (c/4) + 4 (jt%2) + c%4
    auto w2frag = [&](int jt, int ks) -> bf16x8 {
      const int j = 32 * (jt >> 1) + 8 * (wrow0 >> 2) + 4 * (jt & 1) + (wrow0 & 3);
      return as_bf16x8(*reinterpret_cast<const uint4 *>(w2 + j * kD + 32 * ks + wofs));
    };

    // values of the lane's tokens: j = 32 aa + 8 g + [0, 8).  The bf16
    // scoring requests them here, ahead of the MLP; the pair-split
    // arithmetic (twice the operand registers) after the hidden layer.
    uint4 vq[2][4];
    auto load_v = [&]() {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const uint16_t *vp = vbase + ((((int64_t)b * G + l) * N + row[tt]) * H + h) * kD + 8 * g;
#pragma unroll
        for (int aa = 0; aa < 4; ++aa) vq[tt][aa] = *reinterpret_cast<const uint4 *>(vp + 32 * aa);
      }
    };
    if (!kPairs) load_v();
    // W2 fragments are software-pipelined one j tile ahead in the bf16
    // arithmetic: tile 0's are requested here, tile jt + 1's before tile
    // jt's MFMAs (the pair-split arithmetic has no registers to spare for it)
    bf16x8 wq[2][4];
    if (!kPairs) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) wq[0][ks] = w2frag(0, ks);
    }

    // ---- 2. hidden layer H^T = W1 K^T + b1 and GELU, two u tiles at a time
    // (tiles 2 ks and 2 ks + 1 form the K-step ks operand of the next product)
    bf16x8 kh[2][4], kl[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (kPairs) split8(acc[2 * ks][tt], acc[2 * ks + 1][tt], &kh[tt][ks], &kl[tt][ks]);
        else kh[tt][ks] = pack8_bf16(acc[2 * ks][tt], acc[2 * ks + 1][tt]);
      }
    bf16x8 hh[2][4], hl[2][4];
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2) {
      float b1f[8];
      unpack8_bf16(*reinterpret_cast<const uint4 *>(b1p + 32 * ks2 + wofs), b1f);
      f32x4 hc[2][2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int ut = 2 * ks2 + hf;
        const f32x4 init = {0.5f * b1f[4 * hf], 0.5f * b1f[4 * hf + 1], 0.5f * b1f[4 * hf + 2], 0.5f * b1f[4 * hf + 3]};
        hc[hf][0] = init;
        hc[hf][1] = init;
        const int wrow = 16 * ut + wrow0;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 wf = as_bf16x8(*reinterpret_cast<const uint4 *>(w1l + wrow * (2 * kD) + (((4 * ks + (wofs >> 3)) ^ (wrow & 15)) << 4)));
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            hc[hf][tt] = mfma_bf16(wf, kh[tt][ks], hc[hf][tt]);
            if (kPairs) hc[hf][tt] = mfma_bf16(wf, kl[tt][ks], hc[hf][tt]);
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f32x4 y0, y1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (kPairs) {
            y0[i] = gelu_erf(2.0f * hc[0][tt][i]);
            y1[i] = gelu_erf(2.0f * hc[1][tt][i]);
          } else {
            y0[i] = gelu_half(hc[0][tt][i]);
            y1[i] = gelu_half(hc[1][tt][i]);
          }
        }
        if (kPairs) split8(y0, y1, &hh[tt][ks2], &hl[tt][ks2]);
        else hh[tt][ks2] = pack8_bf16(y0, y1);
      }
    }

    if (kPairs) load_v();

    // ---- 3. F^T = W2 H^T + b2, 4. error or residual, per pair of j tiles
    float esum[2] = {0.f, 0.f};
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) {
      float b2f[8];
      unpack8_bf16(*reinterpret_cast<const uint4 *>(b2p + 32 * aa + wofs), b2f);
      f32x4 fc[2][2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int jt = 2 * aa + hf;
        const f32x4 init = {b2f[4 * hf], b2f[4 * hf + 1], b2f[4 * hf + 2], b2f[4 * hf + 3]};
        fc[hf][0] = init;
        fc[hf][1] = init;
        if (!kPairs && jt + 1 < 8) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) wq[(jt + 1) & 1][ks] = w2frag(jt + 1, ks);
        }
        if (!kPairs) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const bf16x8 wf = kPairs ? w2frag(jt, ks) : wq[jt & 1][ks];
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            fc[hf][tt] = mfma_bf16(wf, hh[tt][ks], fc[hf][tt]);
            if (kPairs) fc[hf][tt] = mfma_bf16(wf, hl[tt][ks], fc[hf][tt]);
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float v[8], d8[8];
        unpack8_bf16(vq[tt][aa], v);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          d8[i] = v[i] - fc[0][tt][i];
          d8[4 + i] = v[4 + i] - fc[1][tt][i];
        }
        if constexpr (kResid) {
          const int slot_i = t0 + 16 * tt + c;
          const bool in = 16 * tt + c < nvalid;
          float x8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x8[e] = ok[tt] ? d8[e] : 0.f;
          const int64_t e0 = (elh * s.m + slot_i) * kD + 32 * aa + 8 * g;
          if (s.resid_store == LOWRAM_STORE_INT4_G32) {
            uint16_t sb;
            const uint32_t w = quant8_int4(x8, &sb);
            if (in) {
              *reinterpret_cast<uint32_t *>(reinterpret_cast<uint8_t *>(a.resid_val) + (e0 >> 1)) = w;
              if (g == 0) reinterpret_cast<uint16_t *>(a.resid_scale)[e0 >> 5] = sb;
            }
          } else if (in) {
            *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(a.resid_val) + e0) = pack8_bits(x8);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) esum[tt] += d8[e] * d8[e];
          if constexpr (kStoreAll) {          // every row's residual, stored as the residual pass would
            const bool in = 16 * tt + c < nvalid;
            float x8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x8[e] = ok[tt] ? d8[e] : 0.f;
            const int64_t e0 = (elh * N + t0 + 16 * tt + c) * kD + 32 * aa + 8 * g;
            if (s.resid_store == LOWRAM_STORE_INT4_G32) {
              uint16_t sb;
              const uint32_t w = quant8_int4(x8, &sb);
              if (in) {
                *reinterpret_cast<uint32_t *>(reinterpret_cast<uint8_t *>(a.all_resid) + (e0 >> 1)) = w;
                if (g == 0) reinterpret_cast<uint16_t *>(a.all_resid_scale)[e0 >> 5] = sb;
              }
            } else if (in) {
              *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(a.all_resid) + e0) = pack8_bits(x8);
            }
          }
        }
      }
    }
    if constexpr (!kResid) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float e = esum[tt];
        e += __shfl_xor(e, 16, 64);
        e += __shfl_xor(e, 32, 64);
        const int tl = 16 * tt + c;
        if (g == 0 && tl < nvalid) a.err[elh * N + t0 + tl] = ok[tt] ? e : 0.f;
      }
    }
  }
}

int ceil_div(int x, int y) { return (x + y - 1) / y; }

// Calls with at most this many rows per sequence (the fold of an exact tail)
// take project_small_kernel.
constexpr int kSmallMaxN = 256;
bool proj_small(const Dims &s) { return s.N <= kSmallMaxN; }

// Splits of the projection's contraction: 1 when the output tiles alone give
// 256 workgroups, else doubled (over whole (layer, head) blocks) until they do.
int proj_ksplit(const Dims &s) {
  const int items = s.B * ceil_div(s.N, kPTok) * ceil_div(s.r, kPRanks);
  const int GH = s.G * s.H;
  int ks = 1;
  while (items * ks < 256 && GH % (2 * ks) == 0) ks *= 2;
  return ks;
}

}  // namespace

size_t prefill_mfma_scratch(const Dims &s) {
  if (proj_small(s)) return 0;
  const int ks = proj_ksplit(s);
  return ks > 1 ? (size_t)ks * s.B * s.N * s.r * sizeof(float) : 0;
}

bool prefill_mfma_supports(const Dims &s) {
  return s.dtype == LOWRAM_BF16 && s.d == kD && s.r % 64 == 0 && s.r <= 512 &&
         (int64_t)s.N * s.r * 2 < ((int64_t)1 << 31);
}

hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t st) {
  const Dims &s = a.s;
  const bool ic = s.coef_store == LOWRAM_STORE_INT4_G32;
  hipError_t e;
  // coefficients
  if (proj_small(s)) {
    ProjArgs pa{};
    pa.a = a;
    for (int i = 0; i < 64; ++i) pa.inv_freq[i] = pow(s.theta, -2.0 * i / s.d);
    pa.n_tok_tiles = ceil_div(s.N, kSTok);
    pa.n_rank_tiles = s.r / kSRanks;
    pa.n_ksplit = 1;
    pa.n_items = s.B * pa.n_tok_tiles * pa.n_rank_tiles;
    const int n_wg = 8 * ceil_div(pa.n_items, 8);
    auto kfn = ic ? project_small_kernel<true> : project_small_kernel<false>;
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void *>(kfn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)kSmallLds)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(kfn, dim3(n_wg), dim3(kThreads), kSmallLds, st, pa);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else {
    ProjArgs pa{};
    pa.a = a;
    for (int i = 0; i < 64; ++i) pa.inv_freq[i] = pow(s.theta, -2.0 * i / s.d);
    pa.n_tok_tiles = ceil_div(s.N, kPTok);
    pa.n_rank_tiles = ceil_div(s.r, kPRanks);
    pa.n_ksplit = proj_ksplit(s);
    pa.partial = a.scratch;
    if (pa.n_ksplit > 1 && !pa.partial) return hipErrorInvalidValue;
    pa.n_items = s.B * pa.n_tok_tiles * pa.n_rank_tiles * pa.n_ksplit;
    const int n_wg = 8 * ceil_div(pa.n_items, 8);
    const size_t lds = 2 * kPStage;
    auto kfn = ic ? project_kernel<true> : project_kernel<false>;
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void *>(kfn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)lds)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(kfn, dim3(n_wg), dim3(kThreads), lds, st, pa);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (pa.n_ksplit > 1) {
      const int64_t n = (int64_t)s.B * s.N * (s.r / 8);
      auto rfn = ic ? proj_reduce_kernel<true> : proj_reduce_kernel<false>;
      hipLaunchKernelGGL(rfn, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, pa);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  // scores, then selection, then residuals of the selected rows
  const size_t lds = (size_t)s.r * kD * 2 + (size_t)kD * kD * 2;
  const int GH = s.G * s.H;
  auto run_score = [&](bool resid) -> hipError_t {
    ScoreArgs sa{};
    sa.a = a;
    const int rows = resid ? s.m : s.N;
    const int max_s = std::max(1, ceil_div(rows, kTileRows));
    sa.S = std::min(max_s, std::max(1, ceil_div(256, s.B * GH)));
    sa.split_rows = kTile * ceil_div(ceil_div(rows, sa.S), kTile);
    sa.n_items = s.B * sa.S * GH;
    const int n_wg = 8 * ceil_div(sa.n_items, 8);
    // both passes multiply bf16 pairs and take the exact-erf GELU, so the
    // scores that decide the selection carry near-fp32 accuracy
    auto kfn = resid ? (ic ? score_kernel<true, true, true> : score_kernel<false, true, true>)
                     : a.all_resid ? (ic ? score_kernel<true, false, true, true> : score_kernel<false, false, true, true>)
                                   : (ic ? score_kernel<true, false, true> : score_kernel<false, false, true>);
    hipError_t e2 = hipFuncSetAttribute(reinterpret_cast<const void *>(kfn),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e2 != hipSuccess) return e2;
    hipLaunchKernelGGL(kfn, dim3(n_wg), dim3(kThreads), lds, st, sa);
    return hipGetLastError();
  };
  if ((e = run_score(false)) != hipSuccess) return e;
  if (s.m == 0) return hipSuccess;
  if (a.no_select) return a.all_resid ? hipSuccess : hipErrorInvalidValue;
  if ((e = launch_select(a, st)) != hipSuccess) return e;
  return a.all_resid ? hipSuccess : run_score(true);   // every row's residual is already stored
}

}  // namespace lowram
