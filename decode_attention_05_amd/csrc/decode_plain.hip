// Plain decode kernel: one attended row at a time, one thread per head-dim
// element.  It handles every supported shape and storage mode (fp32 and
// bf16, native and int4, d = 64 or 128) and is the fp32 path; the MFMA kernel
// is the fast bf16 path.
//
// Steps (LowRAM, arXiv:2611.07025; "LowRAM Paper: Amortised Values and
// Low-Rank Keys for KV Compression", sections "Asymmetric key compression
// with xKV" and "Value cache amortisation in plain language"):
//   rebuild the pre-RoPE key of (layer, head) from the row's coefficients and
//   the shared basis, rotate it to the row's position, score it against the
//   group's queries, regenerate the value with the per-head MLP, add the
//   stored residual when the row has one, and fold the row into an online
//   softmax.  The exact tail rows form one extra split.  Splits write
//   (max, sum, accumulator) records that the combine kernel merges.
#include "lowram_internal.h"

namespace lowram {
namespace {

constexpr int kMaxGrp = 8;

struct Freqs {
  double w[64];
};

template <typename DT, bool kInt4Coef, bool kInt4Res>
__global__ void __launch_bounds__(128) decode_plain_kernel(DecodeArgs a, Freqs fr) {
  const Dims s = a.s;
  const int d = s.d, half = d / 2;
  const int j = threadIdx.x;               // head-dim element
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int l = a.layer;
  const int grp = s.grp;

  __shared__ float sh_kt[128];             // pre-RoPE key
  __shared__ float sh_hid[128];            // MLP hidden
  __shared__ float sh_red[kMaxGrp][2];     // per-wave partial scores

  const DT *q = reinterpret_cast<const DT *>(a.q);
  float qv[kMaxGrp];
  for (int g = 0; g < grp; ++g) qv[g] = ldf(q, ((int64_t)b * s.Hq + h * grp + g) * d + j);

  float M[kMaxGrp], L[kMaxGrp], acc[kMaxGrp];
  for (int g = 0; g < kMaxGrp; ++g) { M[g] = -INFINITY; L[g] = 0.f; acc[g] = 0.f; }
  const float scale = rsqrtf(static_cast<float>(d));
  const int lane = j & 63, wave = j >> 6, nwave = (d + 63) / 64;

  // score one row: returns s_g for every g (block-wide reduction)
  auto scores = [&](float kj, float *sg) {
    for (int g = 0; g < grp; ++g) {
      float p = qv[g] * kj;
      for (int o = 32; o > 0; o >>= 1) p += __shfl_xor(p, o, 64);
      if (lane == 0) sh_red[g][wave] = p;
    }
    __syncthreads();
    for (int g = 0; g < grp; ++g) {
      float t = 0.f;
      for (int w = 0; w < nwave; ++w) t += sh_red[g][w];
      sg[g] = t * scale;
    }
    __syncthreads();
  };
  auto fold = [&](const float *sg, float vj) {
    for (int g = 0; g < grp; ++g) {
      float mn = fmaxf(M[g], sg[g]);
      float c = __expf(M[g] - mn);      // exp(-inf) = 0 on the first row
      float p = __expf(sg[g] - mn);
      acc[g] = acc[g] * c + p * vj;
      L[g] = L[g] * c + p;
      M[g] = mn;
    }
  };

  const int body_splits = a.n_splits - 1;
  if (split < body_splits) {
    // ---- body rows of this split (n_body clamped to [0, n_body_max], so no
    // row past the allocation is read whatever the array holds)
    const int nb = min(max(a.c.n_body[b], 0), s.N);
    int64_t i0 = (int64_t)split * a.split_rows, i1;
    const int32_t *rows = nullptr;
    if (a.sub_off) {
      const int64_t o0 = a.sub_off[b], o1 = a.sub_off[b + 1];
      i1 = min<int64_t>(o1 - o0, i0 + a.split_rows);
      rows = a.sub_idx + o0;
    } else {
      i1 = min<int64_t>(nb, i0 + a.split_rows);
    }
    const DT *basis = reinterpret_cast<const DT *>(a.c.basis) + (int64_t)b * s.r * s.D;
    const int64_t col = ((int64_t)l * s.H + h) * d;
    const int pb = s.pred_shared ? 0 : b;
    const int64_t wo = (((int64_t)pb * s.G + l) * s.H + h);
    const DT *W1 = reinterpret_cast<const DT *>(a.c.w1) + wo * d * d;
    const DT *W2 = reinterpret_cast<const DT *>(a.c.w2) + wo * d * d;
    const DT *B1 = reinterpret_cast<const DT *>(a.c.b1) + wo * d;
    const DT *B2 = reinterpret_cast<const DT *>(a.c.b2) + wo * d;
    const int64_t rbase = (((int64_t)b * s.G + l) * s.H + h) * s.m;
    const int32_t *ridx = a.c.resid_idx + (s.m ? rbase : 0);
    // first residual slot that can match a row of this split
    int slot = 0;
    if (i0 < i1 && s.m > 0) {
      int first = rows ? rows[i0] : (int)i0;
      int lo = 0, hi = s.m;
      while (lo < hi) { int mid = (lo + hi) >> 1; if (ridx[mid] < first) lo = mid + 1; else hi = mid; }
      slot = lo;
    }
    const int fi = j < half ? j : j - half;
    for (int64_t i = i0; i < i1; ++i) {
      const int t = rows ? rows[i] : (int)i;
      if (t < 0 || t >= nb) continue;                 // out-of-range subset entry
      // rebuild k~[j] = sum_k c[t,k] basis[k, col+j]
      float kt = 0.f;
      if (kInt4Coef) {
        const uint8_t *cp = reinterpret_cast<const uint8_t *>(a.c.coef) + ((int64_t)b * s.N + t) * (s.r / 2);
        const uint16_t *sp = reinterpret_cast<const uint16_t *>(a.c.coef_scale) + ((int64_t)b * s.N + t) * (s.r / 32);
        for (int k = 0; k < s.r; ++k)
          kt += (static_cast<float>(int4_at(cp, k)) * f16_to_f32(sp[k >> 5])) * ldf(basis, (int64_t)k * s.D + col + j);
      } else {
        const DT *cp = reinterpret_cast<const DT *>(a.c.coef) + ((int64_t)b * s.N + t) * s.r;
        for (int k = 0; k < s.r; ++k) kt += ldf(cp, k) * ldf(basis, (int64_t)k * s.D + col + j);
      }
      sh_kt[j] = kt;
      __syncthreads();
      // rotate to the row's original position
      const int p = a.c.pos ? a.c.pos[(int64_t)b * s.N + t] : t;
      float cs, sn;
      rope_cs(p, fr.w[fi], &cs, &sn);
      const float kr = j < half ? kt * cs - sh_kt[j + half] * sn : kt * cs + sh_kt[j - half] * sn;
      float sg[kMaxGrp];
      scores(kr, sg);
      // value: W2 gelu(W1 k~ + b1) + b2 (+ residual)
      float hsum = ldf(B1, j);
      for (int u = 0; u < d; ++u) hsum += ldf(W1, (int64_t)j * d + u) * sh_kt[u];
      sh_hid[j] = gelu_erf(hsum);
      __syncthreads();
      float vj = ldf(B2, j);
      for (int u = 0; u < d; ++u) vj += ldf(W2, (int64_t)j * d + u) * sh_hid[u];
      while (slot < s.m && ridx[slot] < t) ++slot;
      if (slot < s.m && ridx[slot] == t) {
        const int64_t e = (rbase + slot) * d + j;
        if (kInt4Res) {
          const uint8_t *rp = reinterpret_cast<const uint8_t *>(a.c.resid_val);
          const uint16_t *rs = reinterpret_cast<const uint16_t *>(a.c.resid_scale);
          vj += static_cast<float>(int4_at(rp, e)) * f16_to_f32(rs[e >> 5]);
        } else {
          vj += ldf(reinterpret_cast<const DT *>(a.c.resid_val), e);
        }
      }
      fold(sg, vj);
      __syncthreads();
    }
  } else {
    // ---- exact tail rows
    const int tl = a.c.tail_len[b];
    const DT *tk = reinterpret_cast<const DT *>(a.c.tail_k);
    const DT *tv = reinterpret_cast<const DT *>(a.c.tail_v);
    for (int t = 0; t < tl && t < s.Te; ++t) {
      const int64_t e = ((((int64_t)b * s.G + l) * s.Te + t) * s.H + h) * d + j;
      float sg[kMaxGrp];
      scores(ldf(tk, e), sg);
      fold(sg, ldf(tv, e));
    }
  }
  // ---- partial record
  const int ps = part_stride(d);
  for (int g = 0; g < grp; ++g) {
    float *rec = a.partials + (((int64_t)b * s.Hq + h * grp + g) * a.n_splits + split) * ps;
    if (j == 0) { rec[0] = M[g]; rec[1] = L[g]; rec[2] = 0.f; rec[3] = 0.f; }
    rec[4 + j] = 0.f;
    rec[4 + d + j] = acc[g];
  }
}

Freqs make_freqs(int d, double theta) {
  Freqs f{};
  for (int i = 0; i < d / 2 && i < 64; ++i) f.w[i] = pow(theta, -2.0 * i / d);
  return f;
}

}  // namespace

hipError_t launch_decode_plain(const DecodeArgs &a, hipStream_t st) {
  dim3 grid(a.n_splits, a.s.H, a.s.B), block(a.s.d);
  Freqs fr = make_freqs(a.s.d, a.s.theta);
  const bool ic = a.s.coef_store == LOWRAM_STORE_INT4_G32;
  const bool ir = a.s.resid_store == LOWRAM_STORE_INT4_G32;
  hipError_t e = mark_kernel_start(a, st);
  if (e != hipSuccess) return e;
  if (a.s.dtype == LOWRAM_F32) {
    hipLaunchKernelGGL((decode_plain_kernel<float, false, false>), grid, block, 0, st, a, fr);
  } else if (!ic && !ir) {
    hipLaunchKernelGGL((decode_plain_kernel<bf16_t, false, false>), grid, block, 0, st, a, fr);
  } else if (ic && ir) {
    hipLaunchKernelGGL((decode_plain_kernel<bf16_t, true, true>), grid, block, 0, st, a, fr);
  } else if (ic) {
    hipLaunchKernelGGL((decode_plain_kernel<bf16_t, true, false>), grid, block, 0, st, a, fr);
  } else {
    hipLaunchKernelGGL((decode_plain_kernel<bf16_t, false, true>), grid, block, 0, st, a, fr);
  }
  e = hipGetLastError();
  return e != hipSuccess ? e : mark_kernel_end(a, st);
}

}  // namespace lowram
