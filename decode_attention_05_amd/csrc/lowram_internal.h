// Internal declarations of the LowRAM library: device helpers shared by the
// kernels, the checked argument bundles, and the launchers that the C entry
// points call.  Not part of the public ABI (see include/lowram.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lowram.h"

namespace lowram {

// ----------------------------------------------------------------- argument bundles

struct Dims {
  int B, G, Hq, H, d, r, N, m, Te, grp;
  int64_t D;          // G * H * d
  double theta;
  int dtype, coef_store, resid_store, pred_shared, algo;
};

struct PrefillArgs {
  Dims s;
  const void *k_post, *v;
  const int32_t *pos, *n_body;
  const void *basis, *w1, *b1, *w2, *b2;
  void *coef, *coef_scale;
  int32_t *resid_idx;
  void *resid_val, *resid_scale;
  float *err;         // never NULL here: err_out or the workspace
  float *scratch;     // workspace of the MFMA projection's split contraction (or NULL)
  // optional (MFMA path): the scoring pass also stores every row's residual
  // v - f(k^) here, [B, G, Hkv, N, d] in the residual storage, and the
  // separate residual pass over the selected rows is skipped
  void *all_resid, *all_resid_scale;
  // with all_resid: stop after the scoring pass (the caller selects the
  // residual rows from err itself)
  bool no_select;
};

// order-preserving key of a non-negative score: NaN above +inf, -0 as +0
// (the residual selection ranks rows by (key descending, row ascending))
__device__ __forceinline__ uint32_t score_key(float e) {
  uint32_t u = __float_as_uint(e);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fffffffu;
  if (u & 0x80000000u) return 0u;                 // -0 (scores are never negative)
  return u;
}

// appending exact rows to the compressed body: the cache arrays (in/out)
// and the workspace buffers of the small prefill of the new rows
struct AppendArgs {
  int B, GH, N, m, r, d, el, n_new, m_new;   // el: bytes per native-stored element
  bool int4_coef, int4_res;
  int32_t *n_body;            // [B] in/out
  const int32_t *pos_new;     // [B, n_new] or NULL (then n_body[b] + t)
  int32_t *pos;               // [B, N] or NULL
  void *coef, *coef_scale;
  int32_t *resid_idx;
  void *resid_val, *resid_scale;
  int32_t *nb_old, *n_new_arr, *pos_tmp;     // workspace
  void *coef_tmp, *coef_scale_tmp;
  int32_t *idx_tmp;
  void *val_tmp, *val_scale_tmp;
  bool val_by_row;            // val_tmp holds every new row's residual ([list][n_new]), else the chosen ones ([list][m_new])
  // the merge selects each list's m_new rows from the scores itself (no
  // separate selection launch; n_new <= kMergeSelectMax), else they come
  // from idx_tmp
  bool select_in_merge;
  const float *err_tmp;       // [list][n_new] scores of the new rows
};
// (at 512 new rows the merge's 256 threads ranking 512 x 512 pairs took
// 52 us against 24 + 16 us for the separate 1024-thread selection and merge)
constexpr int kMergeSelectMax = 256;

// predictor fitting: the caller's arrays and hyperparameters
struct FitArgs {
  Dims s;
  const void *coef, *coef_scale, *basis, *v;
  const int32_t *n_body;
  void *w1, *b1, *w2, *b2;    // in: initial weights, out: fitted weights
  float *loss_out, *grad_out; // optional
  int steps;
  double lr, beta1, beta2, eps;
  void *workspace;
};

// workspace of the fit (byte offsets) and its partition of the rows
struct FitLayout {
  int NC;                     // 64-row chunks per sequence
  int64_t NP;                 // NC * 64
  int S;                      // row splits per (sequence, head)
  int npar;                   // parameters per predictor: 2 d^2 + 2 d
  int ps;                     // floats per partial-gradient slot
  size_t kh, kt, vt, master, mom1, mom2, wc, part, total;
};

// what the fit kernels read and write (workspace pointers resolved)
struct FitDev {
  int B, G, H, N, r, Bp, NC, S, npar, ps, pred_shared;
  int64_t NP;
  const void *coef, *coef_scale, *basis, *v;
  const int32_t *n_body;
  void *w1, *b1, *w2, *b2;
  float *loss_out, *grad_out;
  uint16_t *kh;               // [B*G*H][2][NP][d] rebuilt keys, bf16 pairs
  uint16_t *kt;               // [B*G*H][NC][2][d][64] the same per chunk, transposed
  float *vt;                  // [B*G*H][NC][d][64] values, transposed
  float *master, *mom1, *mom2;  // [Bp*G*H][npar] weights (W1, b1, W2, b2) and Adam moments
  uint16_t *wc;               // [Bp*G*H][6][d][d] bf16 pairs of W1, W2, W2^T
  float *part;                // [B*G*H][S][ps] partial gradient sums, loss at npar
  float lr, beta1, beta2, eps;
};

struct DecodeArgs {
  Dims s;
  int layer;
  const void *q;
  lowram_cache c;
  const int32_t *sub_off, *sub_idx;
  void *out;
  float *lse;
  float *partials;    // [B, Hq, n_splits, PART_STRIDE(d)]
  int n_splits;       // body splits + 1 tail split
  int split_rows;     // attended rows per body split
  // caller events recorded right before / after the body-row kernel
  // (lowram_decode_attn_timed); both null otherwise
  hipEvent_t ev_before, ev_after;
};

struct DenseArgs {
  int B, Hq, H, d, T, grp;
  const void *q, *k, *v;
  const int32_t *ctx_len;
  void *out;
  float *lse;
  float *partials;
  int n_splits, split_rows;
  int64_t kv_b_stride;  // elements between sequences of k / v
  int64_t kv_off;       // elements added to every sequence's base
  int split_base;       // first split index written in partials
};

// per-(b, qh, split) partial record: M, L, acc1, pad, acc_h[d], acc_v[d]
__host__ __device__ constexpr int part_stride(int d) { return 4 + 2 * d; }

// ----------------------------------------------------------------- launchers

// Caller events of a timed decode call, recorded around its main kernel.
inline hipError_t mark_kernel_start(const DecodeArgs &a, hipStream_t st) {
  return a.ev_before ? hipEventRecord(a.ev_before, st) : hipSuccess;
}
inline hipError_t mark_kernel_end(const DecodeArgs &a, hipStream_t st) {
  return a.ev_after ? hipEventRecord(a.ev_after, st) : hipSuccess;
}

hipError_t launch_prefill_plain(const PrefillArgs &a, hipStream_t st);
hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t st);
bool prefill_mfma_supports(const Dims &s);
// bytes of fp32 partial coefficients the MFMA prefill needs for shape s (0: none)
size_t prefill_mfma_scratch(const Dims &s);
// exact top-m selection of every (sequence, layer, head) from a.err into a.resid_idx
hipError_t launch_select(const PrefillArgs &a, hipStream_t st);
// setup, the prefill of the new rows (mini), and the merge into the cache
hipError_t launch_append(const AppendArgs &p, const PrefillArgs &mini, bool mfma, hipStream_t st);
FitLayout fit_layout(const Dims &s);
size_t fit_grad_lds(int d);
hipError_t launch_fit(const FitArgs &a, hipStream_t st);
hipError_t launch_decode_plain(const DecodeArgs &a, hipStream_t st);
hipError_t launch_decode_mfma(const DecodeArgs &a, hipStream_t st);
bool decode_mfma_supports(const Dims &s);
int decode_mfma_split_rows(const Dims &s);
int decode_mfma_n_splits(const Dims &s);
size_t decode_mfma_workspace(const Dims &s);
hipError_t launch_tail(const DecodeArgs &a, int split_index, int split_rows, int n_tail_splits,
                       hipStream_t st);
// arguments of the exact-tail splits of a decode call (records split_index ...)
DenseArgs tail_args(const DecodeArgs &a, int split_index, int split_rows);
hipError_t launch_combine(const DecodeArgs &a, bool hoisted, hipStream_t st);
// the device scratch array of the allocation-free decode entry: its size,
// and its address on the current device (looked up once per device)
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void **ptr);
hipError_t launch_dense(const DenseArgs &a, hipStream_t st);

// ----------------------------------------------------------------- device helpers

struct bf16_t {
  uint16_t x;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even; NaN -> canonical quiet NaN
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float ldf(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ldf(const bf16_t *p, int64_t i) { return bf16_to_f32(p[i].x); }
__device__ __forceinline__ void stf(float *p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void stf(bf16_t *p, int64_t i, float v) { p[i].x = f32_to_bf16(v); }

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return static_cast<float>(v);
}

__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  _Float16 v = static_cast<_Float16>(f);  // round to nearest even
  uint16_t h;
  __builtin_memcpy(&h, &v, 2);
  return h;
}

// signed nibble e of a packed int4 array
__device__ __forceinline__ int int4_at(const uint8_t *p, int64_t e) {
  int byte = p[e >> 1];
  int nib = (e & 1) ? (byte >> 4) : (byte & 0xF);
  return nib >= 8 ? nib - 16 : nib;
}

// exact-erf GELU
__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

// cos / sin of pos * theta^(-2i/d): the angle is formed and reduced to
// [-pi, pi] in fp64, then evaluated in fp32.
__device__ __forceinline__ void rope_cs(int pos, double inv_freq, float *c, float *s) {
  const double two_pi = 6.283185307179586476925286766559;
  double a = static_cast<double>(pos) * inv_freq;
  double k = rint(a / two_pi);
  float red = static_cast<float>(fma(-k, two_pi, a));
  sincosf(red, s, c);
}

// First index i in [0, n) with list[i] >= key in an ascending int32 list (n
// if there is none), found by the 64 lanes of a wave probing evenly spaced
// positions: every round narrows the range to one interval between probes
// (about two rounds for a few thousand entries).  Every lane returns it.
__device__ __forceinline__ int wave_lower_bound(const int32_t *list, int n, int key) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = n;                      // the answer lies in [lo, hi]
  while (lo < hi) {
    const int step = (hi - lo + 63) / 64;
    const int p = lo + lane * step;
    const bool below = p < hi && list[p] < key;
    const int cnt = __popcll(__ballot(below));   // probes below the key: a prefix of the lanes
    if (cnt == 0) return lo;
    const int nlo = lo + (cnt - 1) * step + 1;
    hi = min(lo + cnt * step, hi);
    lo = nlo;
  }
  return lo;
}

}  // namespace lowram
