// Prefill: compress the prompt body of one layer group.
//
// LowRAM (arXiv:2611.07025), "LowRAM Paper: Amortised Values and Low-Rank
// Keys for KV Compression": "Step-by-step mental model for one decoding
// session" item 1, "Asymmetric key compression with xKV" and "Value cache
// amortisation in plain language"; arXiv listing, Abstract (residuals only
// for the worst-reconstructed tokens).
//
//   prefill_rows_kernel   per body row: undo RoPE, project the concatenated
//                         pre-RoPE keys on the basis, store the coefficients,
//                         rebuild the keys from the stored coefficients, run
//                         every (layer, head) predictor and write the squared
//                         prediction error
//   select_kernel         per (sequence, layer, head): exact radix selection
//                         of the m largest errors (ties to the lower row),
//                         written in ascending row order
//   residual_kernel       per selected row: value minus prediction, stored
#include "lowram_internal.h"

namespace lowram {
namespace {

constexpr int kRowsThreads = 256;
constexpr int kMaxD = 8192;     // D = G * Hkv * d held in LDS per row
constexpr int kMaxR = 1024;

struct Freqs {
  double w[64];
};

// int4 quantisation of one group of 32 values held by 32 consecutive lanes
// (lane & 31 = element).  Returns the code; *scale gets the fp16 bits.
__device__ __forceinline__ int quant_int4_lane32(float x, uint16_t *scale_bits, float *deq) {
  float amax = fabsf(x);
  for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
  uint16_t sb = f32_to_f16(amax / 7.0f);
  if ((sb & 0x7fff) >= 0x7c00) sb = 0x7bff;       // saturate to the largest finite fp16
  const float sc = f16_to_f32(sb);
  int code = 0;
  if (sc > 0.f) code = static_cast<int>(fminf(fmaxf(rintf(x / sc), -7.f), 7.f));
  *scale_bits = sb;
  *deq = static_cast<float>(code) * sc;
  return code;
}

template <typename DT, bool kInt4Coef>
__global__ void __launch_bounds__(kRowsThreads) prefill_rows_kernel(PrefillArgs a, Freqs fr) {
  const Dims s = a.s;
  const int t = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int d = s.d, half = d / 2, H = s.H, G = s.G;
  const int64_t D = s.D;
  __shared__ float X[kMaxD];        // pre-RoPE keys, then rebuilt keys
  __shared__ float C[kMaxR];        // stored (dequantised) coefficients
  __shared__ float red[kRowsThreads / 64];
  __shared__ float hid[kRowsThreads];

  const int nb = a.n_body[b];
  const int64_t crow = (int64_t)b * s.N + t;
  if (t >= nb) {                                  // padding row
    if (kInt4Coef) {
      uint8_t *cp = reinterpret_cast<uint8_t *>(a.coef) + crow * (s.r / 2);
      uint16_t *sp = reinterpret_cast<uint16_t *>(a.coef_scale) + crow * (s.r / 32);
      for (int k = tid; k < s.r / 2; k += blockDim.x) cp[k] = 0;
      for (int k = tid; k < s.r / 32; k += blockDim.x) sp[k] = 0;
    } else {
      for (int k = tid; k < s.r; k += blockDim.x) stf(reinterpret_cast<DT *>(a.coef), crow * s.r + k, 0.f);
    }
    for (int lh = tid; lh < G * H; lh += blockDim.x)
      a.err[((int64_t)b * G * H + lh) * s.N + t] = 0.f;
    return;
  }
  const DT *kp = reinterpret_cast<const DT *>(a.k_post);
  const DT *basis = reinterpret_cast<const DT *>(a.basis) + (int64_t)b * s.r * D;
  const int p = a.pos ? a.pos[crow] : t;

  // 1. undo RoPE: x_i = y_i cos + y_{i+d/2} sin,  x_{i+d/2} = y_{i+d/2} cos - y_i sin
  for (int64_t c = tid; c < D; c += blockDim.x) {
    const int j = static_cast<int>(c % d);
    const int64_t lh = c / d;
    const int l = static_cast<int>(lh / H), h = static_cast<int>(lh % H);
    const int64_t base = ((((int64_t)b * G + l) * s.N + t) * H + h) * d;
    float cs, sn;
    rope_cs(p, fr.w[j < half ? j : j - half], &cs, &sn);
    const float y = ldf(kp, base + j);
    X[c] = j < half ? y * cs + ldf(kp, base + j + half) * sn : y * cs - ldf(kp, base + j - half) * sn;
  }
  __syncthreads();

  // 2. project: c[k] = sum_c basis[k, c] x[c]  (one wave per rank, lanes over c)
  const int lane = tid & 63, wave = tid >> 6, nwave = blockDim.x >> 6;
  for (int k = wave; k < s.r; k += nwave) {
    float acc = 0.f;
    for (int64_t c = lane; c < D; c += 64) acc += ldf(basis, (int64_t)k * D + c) * X[c];
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) C[k] = acc;
  }
  __syncthreads();

  // store, keeping the stored value for the rebuild
  if (kInt4Coef) {
    uint8_t *cp = reinterpret_cast<uint8_t *>(a.coef) + crow * (s.r / 2);
    uint16_t *sp = reinterpret_cast<uint16_t *>(a.coef_scale) + crow * (s.r / 32);
    for (int k0 = wave * 64; k0 < s.r; k0 += nwave * 64) {
      const int k = k0 + lane;
      const bool ok = k < s.r;
      uint16_t sb;
      float deq;
      const int code = quant_int4_lane32(ok ? C[k] : 0.f, &sb, &deq);
      const int hi = __shfl_down(code, 1, 64);
      if (ok && (k & 1) == 0) cp[k >> 1] = static_cast<uint8_t>((code & 0xF) | ((hi & 0xF) << 4));
      if (ok && (k & 31) == 0) sp[k >> 5] = sb;
      if (ok) C[k] = deq;
    }
  } else {
    DT *cp = reinterpret_cast<DT *>(a.coef) + crow * s.r;
    for (int k = tid; k < s.r; k += blockDim.x) {
      stf(cp, k, C[k]);
      C[k] = ldf(cp, k);            // the stored (rounded) value
    }
  }
  __syncthreads();

  // 3. rebuild: x^[c] = sum_k c[k] basis[k, c]
  for (int64_t c = tid; c < D; c += blockDim.x) {
    float acc = 0.f;
    for (int k = 0; k < s.r; ++k) acc += C[k] * ldf(basis, (int64_t)k * D + c);
    X[c] = acc;
  }
  __syncthreads();

  // 4. predict and score every (layer, head): threads (pair, j), pairs per pass = 256 / d
  const int per = kRowsThreads / d;
  const int sub = tid / d, j = tid % d;
  const DT *vv = reinterpret_cast<const DT *>(a.v);
  const int pb = s.pred_shared ? 0 : b;
  for (int lh0 = 0; lh0 < G * H; lh0 += per) {
    const int lh = lh0 + sub;
    const bool act = lh < G * H;
    const int l = act ? lh / H : 0, h = act ? lh % H : 0;
    const int64_t wo = ((int64_t)pb * G + l) * H + h;
    const DT *W1 = reinterpret_cast<const DT *>(a.w1) + wo * d * d;
    const DT *W2 = reinterpret_cast<const DT *>(a.w2) + wo * d * d;
    float hs = 0.f;
    if (act) {
      hs = ldf(reinterpret_cast<const DT *>(a.b1), wo * d + j);
      for (int u = 0; u < d; ++u) hs += ldf(W1, (int64_t)j * d + u) * X[(int64_t)lh * d + u];
    }
    hid[tid] = gelu_erf(hs);
    __syncthreads();
    float diff = 0.f;
    if (act) {
      float f = ldf(reinterpret_cast<const DT *>(a.b2), wo * d + j);
      for (int u = 0; u < d; ++u) f += ldf(W2, (int64_t)j * d + u) * hid[sub * d + u];
      const float vj = ldf(vv, ((((int64_t)b * G + l) * s.N + t) * H + h) * d + j);
      diff = (vj - f) * (vj - f);
    }
    for (int o = 32; o > 0; o >>= 1) diff += __shfl_xor(diff, o, 64);
    if (lane == 0) red[wave] = diff;
    __syncthreads();
    if (act && j == 0) {
      float e = 0.f;
      for (int w = 0; w < d / 64; ++w) e += red[sub * (d / 64) + w];
      a.err[((int64_t)b * G * H + lh) * s.N + t] = e;
    }
    __syncthreads();
  }
}

constexpr int kSelThreads = 1024;
constexpr int kSelSmall = 512;        // lists up to this length are ranked directly

__global__ void __launch_bounds__(kSelThreads) select_kernel(const float *err, const int32_t *n_body,
                                                              int N, int m, int GH, int32_t *idx_out) {
  const int bid = blockIdx.x, b = bid / GH;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwave = blockDim.x >> 6;
  const int n = min(n_body[b], N);
  const float *e = err + (int64_t)bid * N;
  int32_t *out = idx_out + (int64_t)bid * m;
  const int me = min(m, n);
  for (int i = me + tid; i < m; i += blockDim.x) out[i] = 0x7fffffff;
  if (me <= 0) return;
  if (me == n) {
    for (int i = tid; i < n; i += blockDim.x) out[i] = i;
    return;
  }
  __shared__ int wsum_sel[kSelThreads / 64], wsum_eq[kSelThreads / 64];
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (n <= kSelSmall) {
    // short lists: the rank of every row by (key desc, row asc), counted
    // directly, then the chosen rows written in ascending row order
    __shared__ uint32_t keys[kSelSmall];
    const int i = tid;
    const uint32_t k = i < n ? score_key(e[i]) : 0u;
    if (i < n) keys[i] = k;
    __syncthreads();
    int rank = 0;
    if (i < n)
      for (int j = 0; j < n; ++j) {
        const uint32_t kj = keys[j];
        rank += (kj > k || (kj == k && j < i)) ? 1 : 0;
      }
    const bool sel = i < n && rank < me;
    const uint64_t bsel = __ballot(sel);
    if (lane == 0) wsum_sel[wave] = __popcll(bsel);
    __syncthreads();
    int pos = __popcll(bsel & lt);
    for (int w = 0; w < wave; ++w) pos += wsum_sel[w];
    if (sel) out[pos] = i;
    return;
  }
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_prefix, sh_kk;
  if (tid == 0) { sh_prefix = 0; sh_kk = me; }
  __syncthreads();
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = sh_prefix;
    const uint32_t mask = (shift + 8 >= 32) ? 0u : (0xffffffffu << (shift + 8));
    for (int i = tid; i < n; i += blockDim.x) {
      const uint32_t k = score_key(e[i]);
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t kk = sh_kk, cum = 0;
      int dg = 255;
      for (; dg > 0; --dg) {
        if (cum + hist[dg] >= kk) break;
        cum += hist[dg];
      }
      sh_kk = kk - cum;
      sh_prefix = prefix | (static_cast<uint32_t>(dg) << shift);
    }
    __syncthreads();
  }
  const uint32_t T = sh_prefix;
  const int need_eq = static_cast<int>(sh_kk);
  // compaction in row order: every key above T, then the first need_eq keys equal to T
  int sel_base = 0, eq_base = 0;
  for (int c0 = 0; c0 < n; c0 += blockDim.x) {
    const int i = c0 + tid;
    const uint32_t k = i < n ? score_key(e[i]) : 0u;
    const bool is_eq = i < n && k == T;
    const bool is_gt = i < n && k > T;
    const uint64_t beq = __ballot(is_eq);
    if (lane == 0) wsum_eq[wave] = __popcll(beq);
    __syncthreads();
    int eq_before = eq_base + __popcll(beq & lt);
    for (int w = 0; w < wave; ++w) eq_before += wsum_eq[w];
    const bool sel = is_gt || (is_eq && eq_before < need_eq);
    const uint64_t bsel = __ballot(sel);
    if (lane == 0) wsum_sel[wave] = __popcll(bsel);
    __syncthreads();
    int pos = sel_base + __popcll(bsel & lt);
    for (int w = 0; w < wave; ++w) pos += wsum_sel[w];
    if (sel) out[pos] = i;
    int tot_sel = 0, tot_eq = 0;
    for (int w = 0; w < nwave; ++w) { tot_sel += wsum_sel[w]; tot_eq += wsum_eq[w]; }
    sel_base += tot_sel;
    eq_base += tot_eq;
    __syncthreads();
  }
}

template <typename DT, bool kInt4Coef, bool kInt4Res>
__global__ void __launch_bounds__(128) residual_kernel(PrefillArgs a) {
  const Dims s = a.s;
  const int slot = blockIdx.x, lh = blockIdx.y, b = blockIdx.z;
  const int l = lh / s.H, h = lh % s.H, d = s.d, j = threadIdx.x;
  __shared__ float kt[128], hid[128];
  const int64_t rrow = ((int64_t)b * s.G * s.H + lh) * s.m + slot;
  const int t = a.resid_idx[rrow];
  const bool valid = t >= 0 && t < min(a.n_body[b], s.N);
  float res = 0.f;
  if (valid) {
    const int64_t crow = (int64_t)b * s.N + t;
    const DT *basis = reinterpret_cast<const DT *>(a.basis) + (int64_t)b * s.r * s.D;
    const int64_t col = (int64_t)lh * d + j;
    float acc = 0.f;
    if (kInt4Coef) {
      const uint8_t *cp = reinterpret_cast<const uint8_t *>(a.coef) + crow * (s.r / 2);
      const uint16_t *sp = reinterpret_cast<const uint16_t *>(a.coef_scale) + crow * (s.r / 32);
      for (int k = 0; k < s.r; ++k)
        acc += (static_cast<float>(int4_at(cp, k)) * f16_to_f32(sp[k >> 5])) * ldf(basis, (int64_t)k * s.D + col);
    } else {
      const DT *cp = reinterpret_cast<const DT *>(a.coef) + crow * s.r;
      for (int k = 0; k < s.r; ++k) acc += ldf(cp, k) * ldf(basis, (int64_t)k * s.D + col);
    }
    kt[j] = acc;
  }
  __syncthreads();
  if (valid) {
    const int pb = s.pred_shared ? 0 : b;
    const int64_t wo = ((int64_t)pb * s.G + l) * s.H + h;
    const DT *W1 = reinterpret_cast<const DT *>(a.w1) + wo * d * d;
    float hs = ldf(reinterpret_cast<const DT *>(a.b1), wo * d + j);
    for (int u = 0; u < d; ++u) hs += ldf(W1, (int64_t)j * d + u) * kt[u];
    hid[j] = gelu_erf(hs);
  }
  __syncthreads();
  if (valid) {
    const int pb = s.pred_shared ? 0 : b;
    const int64_t wo = ((int64_t)pb * s.G + l) * s.H + h;
    const DT *W2 = reinterpret_cast<const DT *>(a.w2) + wo * d * d;
    float f = ldf(reinterpret_cast<const DT *>(a.b2), wo * d + j);
    for (int u = 0; u < d; ++u) f += ldf(W2, (int64_t)j * d + u) * hid[u];
    const DT *vv = reinterpret_cast<const DT *>(a.v);
    res = ldf(vv, ((((int64_t)b * s.G + l) * s.N + t) * s.H + h) * d + j) - f;
  }
  const int64_t e = rrow * d + j;
  if (kInt4Res) {
    uint16_t sb;
    float deq;
    const int code = quant_int4_lane32(res, &sb, &deq);
    const int hi = __shfl_down(code, 1, 64);
    if ((j & 1) == 0) reinterpret_cast<uint8_t *>(a.resid_val)[e >> 1] = static_cast<uint8_t>((code & 0xF) | ((hi & 0xF) << 4));
    if ((j & 31) == 0) reinterpret_cast<uint16_t *>(a.resid_scale)[e >> 5] = sb;
  } else {
    stf(reinterpret_cast<DT *>(a.resid_val), e, res);
  }
}

Freqs make_freqs(int d, double theta) {
  Freqs f{};
  for (int i = 0; i < d / 2 && i < 64; ++i) f.w[i] = pow(theta, -2.0 * i / d);
  return f;
}

template <typename DT, bool IC>
hipError_t launch_rows(const PrefillArgs &a, const Freqs &fr, hipStream_t st) {
  dim3 grid(a.s.N, a.s.B);
  hipLaunchKernelGGL((prefill_rows_kernel<DT, IC>), grid, dim3(kRowsThreads), 0, st, a, fr);
  return hipGetLastError();
}

template <typename DT, bool IC, bool IR>
hipError_t launch_resid(const PrefillArgs &a, hipStream_t st) {
  dim3 grid(a.s.m, a.s.G * a.s.H, a.s.B);
  hipLaunchKernelGGL((residual_kernel<DT, IC, IR>), grid, dim3(a.s.d), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const PrefillArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(select_kernel, dim3(a.s.B * a.s.G * a.s.H), dim3(kSelThreads), 0, st,
                     a.err, a.n_body, a.s.N, a.s.m, a.s.G * a.s.H, a.resid_idx);
  return hipGetLastError();
}

hipError_t launch_prefill_plain(const PrefillArgs &a, hipStream_t st) {
  const Freqs fr = make_freqs(a.s.d, a.s.theta);
  const bool ic = a.s.coef_store == LOWRAM_STORE_INT4_G32;
  const bool ir = a.s.resid_store == LOWRAM_STORE_INT4_G32;
  hipError_t e;
  if (a.s.N > 0) {
    if (a.s.dtype == LOWRAM_F32) e = launch_rows<float, false>(a, fr, st);
    else if (ic) e = launch_rows<bf16_t, true>(a, fr, st);
    else e = launch_rows<bf16_t, false>(a, fr, st);
    if (e != hipSuccess) return e;
  }
  if (a.s.m == 0) return hipSuccess;
  if ((e = launch_select(a, st)) != hipSuccess) return e;
  if (a.s.dtype == LOWRAM_F32) return launch_resid<float, false, false>(a, st);
  if (ic && ir) return launch_resid<bf16_t, true, true>(a, st);
  if (ic) return launch_resid<bf16_t, true, false>(a, st);
  if (ir) return launch_resid<bf16_t, false, true>(a, st);
  return launch_resid<bf16_t, false, false>(a, st);
}

}  // namespace lowram
