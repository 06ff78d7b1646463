// The shared key basis of a layer group on the GPU: randomized subspace
// iteration (Halko, Martinsson and Tropp, "Finding structure with
// randomness", SIAM Review 2011, Algorithm 4.4) on the pre-RoPE key matrix
// X [n, D] of each sequence, from a caller-given Gaussian start.
//
// Per round:  P = X Q^T;  P~ = orth(P);  Y = X^T P~ (kept as rows, Y^T);
//             Q = orth(Y).  A last orth of Q restores fp32 orthogonality.
// orth(M) is QR by Cholesky of the Gram matrix (CholeskyQR): G = M^T M in
// fp64, G = L L^T in fp64 with a pivot test that skips dependent columns,
// then M L^{-T}.  Only the last orthonormalisation needs to be accurate:
// the earlier ones change the iterate by upper-triangular factors, which
// leave the final QR factor alone.
//
// Kernels: the inverse rotation (X, fp32), one tiled matrix-product kernel
// on the matrix cores for every product (fp32 operands and accumulation
// with v_mfma_f32_16x16x4f32; the Gram matrices with fp64 accumulation on
// v_mfma_f64_16x16x4f64), a one-workgroup-per-sequence Cholesky in fp64, the
// triangular inverse in fp64 one column block per workgroup, and the final
// conversion.
#include <algorithm>
#include <cmath>

#include "basis_internal.h"

namespace lowram {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Acc;
template <> struct Acc<float> { typedef f32x4 type; };
template <> struct Acc<double> { typedef f64x4 type; };

__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f64x4 mma(double a, double b, f64x4 c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

constexpr int kBK = 16;       // contraction step of the product kernel
constexpr int kW = 32;        // panel width of the Cholesky and the inverse
constexpr int kPW = kW + 1;   // padded LDS row (doubles) of a panel
constexpr double kDropTau = 1e-10;   // pivot <= tau * max diagonal: dependent column

// ----------------------------------------------------------------- inverse rotation

struct PrepArgs {
  const void *k_post;
  const int32_t *pos, *n_body;
  float *x;
  int B, G, H, d, N;
  int64_t NP, D;
  double inv_freq[64];
};

// X[b, t, (l H + h) d + j]: the key of row t of (l, h) turned back by
// -pos * theta^(-2i/d) on the pair (i, i + d/2); rows t >= n_body[b] are 0.
// One workgroup per row (b, t): thread i < d/2 forms its angle once and
// turns pair i of every (layer, head).
template <typename TK>
__global__ void __launch_bounds__(256) basis_prep_kernel(PrepArgs p) {
  const int half = p.d >> 1, GH = p.G * p.H;
  const int64_t row_id = blockIdx.x;
  const int b = (int)(row_id / p.NP);
  const int64_t t = row_id % p.NP;
  const TK *kp = static_cast<const TK *>(p.k_post);
  float *row = p.x + row_id * p.D;
  const int nb = min(p.n_body[b], p.N);
  const int i = threadIdx.x % half, h0 = threadIdx.x / half, hstep = blockDim.x / half;
  if (t >= nb) {
    for (int h = h0; h < GH; h += hstep) {
      row[h * p.d + i] = 0.0f;
      row[h * p.d + i + half] = 0.0f;
    }
    return;
  }
  const int ps = p.pos ? p.pos[(int64_t)b * p.N + t] : (int)t;
  float c, sn;
  rope_cs(ps, p.inv_freq[i], &c, &sn);
  for (int lh = h0; lh < GH; lh += hstep) {
    const int l = lh / p.H, h = lh % p.H;
    const int64_t src = ((((int64_t)b * p.G + l) * p.N + t) * p.H + h) * p.d;
    const float k0 = ldf(kp, src + i), k1 = ldf(kp, src + i + half);
    row[lh * p.d + i] = fmaf(k0, c, k1 * sn);
    row[lh * p.d + i + half] = fmaf(-k0, sn, k1 * c);
  }
}

// ----------------------------------------------------------------- products

struct GemmArgs {
  const float *A, *B;
  void *C;
  int M, N, K, Kc, S;         // Kc: contraction length per split (multiple of kBK)
  int lower;                  // 1: only tiles touching the lower triangle (n <= m)
  int nx, ny, nz, per_xcd;    // tiles along N, M and batch x split; workgroups per XCD
  int64_t lda, ldb, ldc;
  int64_t sA, sB, sC, sSplit; // batch strides (elements) and split stride of C
};

// C[b][s][m][n] = sum over k in split s of A_b(m, k) B_b(n, k), with
// A_b(m, k) = A[m lda + k] if AK else A[k lda + m] (B likewise).  M, N and
// every leading dimension are multiples of 4, K of kBK; tiles past M or N
// are masked.  256 threads = 2 x 2 waves, each wave a (16 WM) x (16 WN)
// block of 16 x 16 MFMA tiles; operands staged through LDS as [k][m].  Both
// MFMAs take lane l's operands at row (or column) l % 16 and k = l / 16.
template <typename T, bool AK, bool BK, int WM, int WN>
__global__ void __launch_bounds__(256) gemm_kernel(GemmArgs g) {
  typedef typename Acc<T>::type AccT;
  constexpr bool kF64 = sizeof(T) == 8;
  constexpr int BM = 32 * WM, BN = 32 * WN;
  constexpr int PA = BM + 4, PB = BN + 4;
  constexpr int LA = BM / 64, LB = BN / 64;   // float4 loads per thread and step
  __shared__ T As[kBK][PA];
  __shared__ T Bs[kBK][PB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // workgroup ids are dealt to the 8 XCDs by id mod 8: the tile order is
  // remapped so that consecutive tiles (those sharing a row block of A)
  // run on one XCD and share its L2
  const int lid = (int)(blockIdx.x & 7) * g.per_xcd + (int)(blockIdx.x >> 3);
  if (lid >= g.nx * g.ny * g.nz) return;
  const int tx = lid % g.nx, ty = (lid / g.nx) % g.ny, tz = lid / (g.nx * g.ny);
  const int b = tz / g.S, s = tz % g.S;
  const int m0 = ty * BM, n0 = tx * BN;
  if (g.lower && n0 >= m0 + BM) return;       // the whole tile lies above the diagonal
  const int k_begin = s * g.Kc, k_end = min(g.K, k_begin + g.Kc);
  const float *A = g.A + b * g.sA, *Bm = g.B + b * g.sB;

  float4 ra[LA], rb[LB];
  auto load = [&](int k) {
#pragma unroll
    for (int u = 0; u < LA; ++u) {
      const int f = tid + 256 * u;
      int row, kk;
      if (AK) { row = f >> 2; kk = (f & 3) * 4; } else { kk = f / (BM / 4); row = (f % (BM / 4)) * 4; }
      const bool ok = m0 + row < g.M;
      ra[u] = ok ? *reinterpret_cast<const float4 *>(AK ? A + (int64_t)(m0 + row) * g.lda + k + kk
                                                        : A + (int64_t)(k + kk) * g.lda + m0 + row)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int f = tid + 256 * u;
      int row, kk;
      if (BK) { row = f >> 2; kk = (f & 3) * 4; } else { kk = f / (BN / 4); row = (f % (BN / 4)) * 4; }
      const bool ok = n0 + row < g.N;
      rb[u] = ok ? *reinterpret_cast<const float4 *>(BK ? Bm + (int64_t)(n0 + row) * g.ldb + k + kk
                                                        : Bm + (int64_t)(k + kk) * g.ldb + n0 + row)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int u = 0; u < LA; ++u) {
      const int f = tid + 256 * u;
      const float v[4] = {ra[u].x, ra[u].y, ra[u].z, ra[u].w};
      if (AK) {
        const int row = f >> 2, kk = (f & 3) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) As[kk + e][row] = static_cast<T>(v[e]);
      } else {
        const int kk = f / (BM / 4), row = (f % (BM / 4)) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) As[kk][row + e] = static_cast<T>(v[e]);
      }
    }
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      const int f = tid + 256 * u;
      const float v[4] = {rb[u].x, rb[u].y, rb[u].z, rb[u].w};
      if (BK) {
        const int row = f >> 2, kk = (f & 3) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) Bs[kk + e][row] = static_cast<T>(v[e]);
      } else {
        const int kk = f / (BN / 4), row = (f % (BN / 4)) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e) Bs[kk][row + e] = static_cast<T>(v[e]);
      }
    }
  };

  AccT acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = AccT{0, 0, 0, 0};

  if (k_begin < k_end) load(k_begin);
  for (int k = k_begin; k < k_end; k += kBK) {
    __syncthreads();
    stage();
    __syncthreads();
    if (k + kBK < k_end) load(k + kBK);
#pragma unroll
    for (int kq = 0; kq < kBK / 4; ++kq) {
      const int kr = kq * 4 + (lane >> 4);
      T av[WM], bv[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i) av[i] = As[kr][wm * 16 * WM + i * 16 + (lane & 15)];
#pragma unroll
      for (int j = 0; j < WN; ++j) bv[j] = Bs[kr][wn * 16 * WN + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = mma(av[i], bv[j], acc[i][j]);
    }
  }

  T *C = static_cast<T *>(g.C) + b * g.sC + s * g.sSplit;
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      const int n = n0 + wn * 16 * WN + j * 16 + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // output row of accumulator e: 4 (lane / 16) + e for the fp32 MFMA,
        // lane / 16 + 4 e for the fp64 one (measured on gfx950)
        const int rw = kF64 ? (lane >> 4) + 4 * e : 4 * (lane >> 4) + e;
        const int m = m0 + wm * 16 * WM + i * 16 + rw;
        if (m < g.M && n < g.N) C[(int64_t)m * g.ldc + n] = acc[i][j][e];
      }
    }
}

// out[b][i] = sum over s of part[b][s][i], i < n
__global__ void __launch_bounds__(256) sum_splits_kernel(const float *part, float *out, int B, int S,
                                                          int64_t n) {
  const int64_t total = (int64_t)B * n;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = e / n, i = e % n;
    const float *p = part + b * S * n + i;
    float a = 0.0f;
    for (int s = 0; s < S; ++s) a += p[(int64_t)s * n];
    out[e] = a;
  }
}

// ----------------------------------------------------------------- Cholesky and inverse

struct CholArgs {
  const double *gpart;        // [B][S][r][r] Gram partial sums
  double *lw;                 // [B][r][r] fp64 factor (lower triangle)
  double *dinv;               // [B][r][kW] inverses of the diagonal blocks
  float *linv;                // [B][r][r] L^{-1}, rows of skipped columns zero
  int32_t *drop;              // [B][r] 1 where a column was skipped
  int r, S;
};

// lower triangle of the Gram matrix = sum of the split partial sums
__global__ void __launch_bounds__(256) gram_sum_kernel(CholArgs a, int B) {
  const int r = a.r;
  const int64_t rr = (int64_t)r * r, total = (int64_t)B * rr;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = e / rr, k = e % rr;
    if (k % r > k / r) continue;
    const double *g = a.gpart + b * a.S * rr + k;
    double v = 0.0;
    for (int s = 0; s < a.S; ++s) v += g[s * rr];
    a.lw[e] = v;
  }
}

// inverses of the kW x kW diagonal blocks of L (grid r / kW x B, 64
// threads): thread c < kW solves column c by forward substitution
__global__ void __launch_bounds__(64) dinv_kernel(CholArgs a) {
  __shared__ double ld[kW][kPW];
  __shared__ double x[kW][kPW];
  const int r = a.r, I = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const double *L = a.lw + (int64_t)b * r * r + (int64_t)(I * kW) * r + I * kW;
  for (int e = tid; e < kW * kW; e += 64) ld[e / kW][e % kW] = L[(int64_t)(e / kW) * r + e % kW];
  __syncthreads();
  if (tid < kW) {
    const int c = tid;
    for (int i = 0; i < kW; ++i) {
      double v = 0.0;
      if (i >= c) {
        v = (i == c) ? 1.0 : 0.0;
        for (int k = c; k < i; ++k) v -= ld[i][k] * x[k][c];
        v /= ld[i][i];
      }
      x[i][c] = v;
    }
  }
  __syncthreads();
  double *Dv = a.dinv + (int64_t)b * r * kW + (int64_t)(I * kW) * kW;
  for (int e = tid; e < kW * kW; e += 64) Dv[e] = x[e / kW][e % kW];
}

constexpr int kCT = 512;      // threads of the Cholesky workgroup: one per panel row

// One workgroup per sequence: L L^T = sum of the partials, right-looking
// with kW-wide panels in LDS.  A pivot d_j <= kDropTau * max_i G_ii (or not a
// number) marks column j dependent on the ones before it: L gets a unit
// column and a zero row there, so L^{-1} is L_kept^{-1} on the kept indices
// and the unit vector at j (whose row inv_kernel writes as zero).
__global__ void __launch_bounds__(kCT) chol_kernel(CholArgs a) {
  extern __shared__ double lds[];
  double *pt = lds;                      // [kW][r]: the current panel, column-major
  __shared__ int drop[512];
  __shared__ double red[16];
  const int r = a.r, tid = threadIdx.x, b = blockIdx.x;
  double *L = a.lw + (int64_t)b * r * r;

  // the largest diagonal entry of the Gram matrix
  double md = 0.0;
  for (int i = tid; i < r; i += kCT) md = fmax(md, L[(int64_t)i * r + i]);
  for (int o = 32; o > 0; o >>= 1) md = fmax(md, __shfl_xor(md, o));
  if ((tid & 63) == 0) red[tid >> 6] = md;
  __syncthreads();
  if (tid == 0) {
    double m = 0.0;
    for (int w = 0; w < kCT / 64; ++w) m = fmax(m, red[w]);
    red[0] = m;
  }
  __syncthreads();
  const double lim = kDropTau * red[0];

  __shared__ double s_piv;
  __shared__ double s_col[kW];
  for (int p0 = 0; p0 < r; p0 += kW) {
    const int rows = r - p0;
    // thread i holds row i of the panel in registers
    const int i = tid;
    double v[kW];
    if (i < rows) {
      const double2 *src = reinterpret_cast<const double2 *>(L + (int64_t)(p0 + i) * r + p0);
#pragma unroll
      for (int c = 0; c < kW; c += 2) {
        const double2 x = src[c / 2];
        v[c] = (c <= i) ? x.x : 0.0;
        v[c + 1] = (c + 1 <= i) ? x.y : 0.0;
      }
    }
#pragma unroll
    for (int j = 0; j < kW; ++j) {
      if (i == j) s_piv = v[j];
      __syncthreads();
      const double dj = s_piv;
      const bool dep = !(dj > lim);
      const double lj = dep ? 1.0 : sqrt(dj), inv = dep ? 0.0 : 1.0 / lj;
      if (i == j) {
        v[j] = lj;
        drop[p0 + j] = dep ? 1 : 0;
      } else if (i > j && i < rows) {
        v[j] *= inv;
        if (i < kW) s_col[i] = v[j];
      }
      __syncthreads();
      // rank-1 update of the later columns of the panel (c <= i)
      if (i > j && i < rows) {
#pragma unroll
        for (int c = j + 1; c < kW; ++c)
          if (c <= i) v[c] -= v[j] * s_col[c];
      }
    }
    __syncthreads();
    // a skipped column's row inside the diagonal block is zero
    if (i < kW && drop[p0 + i]) {
#pragma unroll
      for (int c = 0; c < kW; ++c)
        if (c < i) v[c] = 0.0;
    }
    if (i < rows) {
      double2 *dst = reinterpret_cast<double2 *>(L + (int64_t)(p0 + i) * r + p0);
#pragma unroll
      for (int c = 0; c < kW; c += 2) {
        pt[c * r + i] = v[c];
        pt[(c + 1) * r + i] = v[c + 1];
        if (c + 1 <= i) dst[c / 2] = make_double2(v[c], v[c + 1]);
        else if (c <= i) L[(int64_t)(p0 + i) * r + p0 + c] = v[c];
      }
    }
    __syncthreads();
    // trailing update L22 -= L21 L21^T on the fp64 matrix cores: each wave
    // takes 16 x 16 tiles of the lower triangle, the panel (column-major in
    // LDS) supplying both operands; the tile's old values are requested one
    // tile ahead
    const int t0 = p0 + kW, nt = r - t0;
    if (nt > 0) {
      const int nb16 = nt / 16, ntile = nb16 * (nb16 + 1) / 2;
      const int wave = tid >> 6, lane = tid & 63, lm = lane & 15, lg = lane >> 4;
      auto tile_of = [](int e, int &bi, int &bc) {
        bi = (int)((sqrt(8.0 * e + 1.0) - 1.0) * 0.5);
        while ((bi + 1) * (bi + 2) / 2 <= e) ++bi;
        while (bi * (bi + 1) / 2 > e) --bi;
        bc = e - bi * (bi + 1) / 2;
      };
      auto load_old = [&](int e, double *o) {
        if (e < ntile) {
          int bi, bc;
          tile_of(e, bi, bc);
          const double *src = L + (int64_t)(t0 + 16 * bi + lg) * r + t0 + 16 * bc + lm;
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] = src[(int64_t)4 * q * r];
        }
      };
      double nold[4] = {0.0, 0.0, 0.0, 0.0};
      load_old(wave, nold);
      for (int e = wave; e < ntile; e += kCT / 64) {
        int bi, bc;
        tile_of(e, bi, bc);
        const double old[4] = {nold[0], nold[1], nold[2], nold[3]};
        load_old(e + kCT / 64, nold);
        f64x4 acc = {0.0, 0.0, 0.0, 0.0};
        const double *pa = pt + kW + 16 * bi + lm, *pb = pt + kW + 16 * bc + lm;
#pragma unroll
        for (int kq = 0; kq < kW; kq += 4) acc = mma(pa[(kq + lg) * r], pb[(kq + lg) * r], acc);
        double *dst = L + (int64_t)(t0 + 16 * bi + lg) * r + t0 + 16 * bc + lm;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (bc < bi || lm <= lg + 4 * q) dst[(int64_t)4 * q * r] = old[q] - acc[q];
      }
    }
    __syncthreads();
  }
  // rows of skipped columns are zero left of their panel (inside it the
  // panel step cleared them)
  for (int i = tid; i < r; i += kCT)
    if (drop[i])
      for (int c = 0; c < (i / kW) * kW; ++c) L[(int64_t)i * r + c] = 0.0;
  for (int i = tid; i < r; i += kCT) a.drop[(int64_t)b * r + i] = drop[i];
}

// L^{-1}, one kW-column block J per workgroup (grid r / kW x B): block
// forward substitution X_I = Dinv_I (E_IJ - sum_{J <= K < I} L_IK X_K) with
// the column block X in LDS and one kW x kW block of L at a time.
__global__ void __launch_bounds__(1024) inv_kernel(CholArgs a) {
  extern __shared__ double lds[];
  const int r = a.r, J = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int c0 = J * kW, nb = r / kW, ri = tid / kW, cc = tid % kW;
  double *X = lds;                       // [r - c0][kPW]: rows c0.. of the column block
  double *lb = X + (r - c0) * kPW;       // [kW][kPW]: a block of L, then of Dinv
  double *tt = lb + kW * kPW;            // [kW][kPW]
  const double *L = a.lw + (int64_t)b * r * r;
  const double *Dv = a.dinv + (int64_t)b * r * kW;
  const int32_t *dp = a.drop + (int64_t)b * r;
  float *Li = a.linv + (int64_t)b * r * r;
  for (int I = J; I < nb; ++I) {
    const double *Lrow = L + (int64_t)(I * kW + ri) * r + cc;
    double t = (I == J && ri == cc) ? 1.0 : 0.0;
    double nxt = (J < I) ? Lrow[J * kW] : 0.0;
    for (int K = J; K < I; ++K) {
      __syncthreads();
      lb[ri * kPW + cc] = nxt;
      __syncthreads();
      if (K + 1 < I) nxt = Lrow[(K + 1) * kW];
      const double *xk = X + (K * kW - c0) * kPW + cc;
#pragma unroll 8
      for (int k = 0; k < kW; ++k) t -= lb[ri * kPW + k] * xk[k * kPW];
    }
    tt[ri * kPW + cc] = t;
    __syncthreads();
    lb[ri * kPW + cc] = Dv[(int64_t)(I * kW + ri) * kW + cc];
    __syncthreads();
    double x = 0.0;
    for (int k = 0; k <= ri; ++k) x += lb[ri * kPW + k] * tt[k * kPW + cc];
    X[(I * kW + ri - c0) * kPW + cc] = x;
    __syncthreads();
  }
  for (int e = tid; e < r * kW; e += 1024) {
    const int i = e / kW, c = e % kW;
    const float v = (i < c0 || dp[i]) ? 0.0f : static_cast<float>(X[(i - c0) * kPW + c]);
    Li[(int64_t)i * r + c0 + c] = v;
  }
}

template <typename TO>
__global__ void __launch_bounds__(256) basis_store_kernel(const float *y, TO *out, int64_t n) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x)
    stf(out, e, y[e]);
}

// ----------------------------------------------------------------- host side

int cdiv(int64_t x, int64_t y) { return (int)((x + y - 1) / y); }

// split count and per-split length of a contraction of length K (multiple of
// kBK) so that tiles * B * S reaches about `want` workgroups, each split at
// least 256 long
void plan_split(int64_t K, int64_t tiles, int B, int want, int *S, int *Kc) {
  int s = std::max(1, cdiv(want, tiles * B));
  s = std::min<int64_t>(s, std::max<int64_t>(1, K / 256));
  int kc = cdiv(cdiv(K, s), kBK) * kBK;
  *S = std::max(1, cdiv(K, std::max(kc, kBK)));
  *Kc = std::max(kc, kBK);
}

template <typename T, bool AK, bool BK, int WM, int WN>
hipError_t gemm(const float *A, int64_t lda, int64_t sA, const float *Bm, int64_t ldb, int64_t sB,
                void *C, int64_t ldc, int64_t sC, int64_t sSplit, int M, int N, int K, int S, int Kc,
                int B, hipStream_t st, int lower = 0) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const int nx = cdiv(N, 32 * WN), ny = cdiv(M, 32 * WM), nz = B * S;
  const int64_t tiles = (int64_t)nx * ny * nz;
  const int per = (int)((tiles + 7) / 8);
  GemmArgs g{A, Bm, C, M, N, K, Kc, S, lower, nx, ny, nz, per, lda, ldb, ldc, sA, sB, sC, sSplit};
  hipLaunchKernelGGL((gemm_kernel<T, AK, BK, WM, WN>), dim3(8 * per), dim3(256), 0, st, g);
  return hipGetLastError();
}

// workgroups aimed at by a Gram product's split (about half of them return
// at once: their tile lies above the diagonal)
constexpr int kGramWant = 4096;

size_t chol_lds(int r) { return (size_t)kW * r * sizeof(double); }
size_t inv_lds(int r) { return (size_t)(r + 2 * kW) * kPW * sizeof(double); }

}  // namespace

BasisLayout basis_layout(const Dims &s) {
  BasisLayout L{};
  L.NP = ((int64_t)s.N + 127) / 128 * 128;
  const int r = s.r;
  const int64_t gt = (int64_t)cdiv(r, 64) * cdiv(r, 64);
  int kc;
  plan_split(std::max<int64_t>(L.NP, kBK), gt, s.B, kGramWant, &L.sgp, &kc);
  plan_split(s.D, gt, s.B, kGramWant, &L.sgq, &kc);
  plan_split(std::max<int64_t>(L.NP, kBK), (int64_t)cdiv(r, 128) * cdiv(s.D, 128), s.B, 1024, &L.sy, &kc);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = (off + bytes + 255) & ~(size_t)255;
    return at;
  };
  L.x = take((size_t)s.B * L.NP * s.D * 4);
  L.p = take((size_t)s.B * L.NP * r * 4);
  L.pt = take((size_t)s.B * L.NP * r * 4);
  L.y = take((size_t)s.B * r * s.D * 4);
  L.q = take((size_t)s.B * r * s.D * 4);
  L.yp = take(L.sy > 1 ? (size_t)s.B * L.sy * r * s.D * 4 : 0);
  L.g = take((size_t)s.B * std::max(L.sgp, L.sgq) * r * r * 8);
  L.lw = take((size_t)s.B * r * r * 8);
  L.dinv = take((size_t)s.B * r * kW * 8);
  L.linv = take((size_t)s.B * r * r * 4);
  L.drop = take((size_t)s.B * r * 4);
  L.total = off;
  return L;
}

hipError_t launch_basis(const BasisArgs &a, hipStream_t st) {
  const Dims &s = a.s;
  const BasisLayout Ly = basis_layout(s);
  char *ws = static_cast<char *>(a.workspace);
  float *X = reinterpret_cast<float *>(ws + Ly.x);
  float *P = reinterpret_cast<float *>(ws + Ly.p);
  float *Pt = reinterpret_cast<float *>(ws + Ly.pt);
  float *Y = reinterpret_cast<float *>(ws + Ly.y);
  float *Q = reinterpret_cast<float *>(ws + Ly.q);
  float *Yp = reinterpret_cast<float *>(ws + Ly.yp);
  double *Gp = reinterpret_cast<double *>(ws + Ly.g);
  double *Lw = reinterpret_cast<double *>(ws + Ly.lw);
  double *Dv = reinterpret_cast<double *>(ws + Ly.dinv);
  float *Li = reinterpret_cast<float *>(ws + Ly.linv);
  const int B = s.B, r = s.r;
  const int64_t D = s.D, NP = Ly.NP, rr = (int64_t)r * r;
  hipError_t e;

  PrepArgs pa{};
  pa.k_post = a.k_post; pa.pos = a.pos; pa.n_body = a.n_body; pa.x = X;
  pa.B = B; pa.G = s.G; pa.H = s.H; pa.d = s.d; pa.N = s.N; pa.NP = NP; pa.D = D;
  for (int i = 0; i < s.d / 2; ++i) pa.inv_freq[i] = std::pow(s.theta, -2.0 * i / s.d);
  if (B * NP > 0) {               // one workgroup per row; d / 2 divides 256
    if (s.dtype == LOWRAM_BF16)
      hipLaunchKernelGGL(basis_prep_kernel<bf16_t>, dim3((unsigned)(B * NP)), dim3(256), 0, st, pa);
    else
      hipLaunchKernelGGL(basis_prep_kernel<float>, dim3((unsigned)(B * NP)), dim3(256), 0, st, pa);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }

  const size_t lds = chol_lds(r), lds_inv = inv_lds(r);
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void *>(&chol_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) != hipSuccess)
    return e;
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void *>(&inv_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_inv)) != hipSuccess)
    return e;
  int32_t *Dp = reinterpret_cast<int32_t *>(ws + Ly.drop);
  const int64_t gt = (int64_t)cdiv(r, 64) * cdiv(r, 64);
  int sgp, kgp, sgq, kgq, sy, ky;
  plan_split(NP, gt, B, kGramWant, &sgp, &kgp);
  plan_split(D, gt, B, kGramWant, &sgq, &kgq);
  plan_split(NP, (int64_t)cdiv(r, 128) * cdiv(D, 128), B, 1024, &sy, &ky);

  // orth of the r vectors held as rows of V [r][D] (rows = true) or as the
  // columns of V [NP][r]: Gram, factor, then out = V L^{-T} / L^{-1} V
  auto factor = [&](const float *V, bool rows) -> hipError_t {
    hipError_t er;
    if (rows)
      er = gemm<double, true, true, 2, 2>(V, D, r * D, V, D, r * D, Gp, r, sgq * rr, rr, r, r, (int)D,
                                          sgq, kgq, B, st, 1);
    else
      er = gemm<double, false, false, 2, 2>(V, r, NP * r, V, r, NP * r, Gp, r, sgp * rr, rr, r, r, (int)NP,
                                            sgp, kgp, B, st, 1);
    if (er != hipSuccess) return er;
    CholArgs ca{Gp, Lw, Dv, Li, Dp, r, rows ? sgq : sgp};
    hipLaunchKernelGGL(gram_sum_kernel, dim3((int)std::min<int64_t>(cdiv(B * rr, 256), 16384)), dim3(256), 0, st,
                       ca, B);
    if ((er = hipGetLastError()) != hipSuccess) return er;
    hipLaunchKernelGGL(chol_kernel, dim3(B), dim3(kCT), lds, st, ca);
    if ((er = hipGetLastError()) != hipSuccess) return er;
    hipLaunchKernelGGL(dinv_kernel, dim3(r / kW, B), dim3(64), 0, st, ca);
    if ((er = hipGetLastError()) != hipSuccess) return er;
    hipLaunchKernelGGL(inv_kernel, dim3(r / kW, B), dim3(1024), lds_inv, st, ca);
    return hipGetLastError();
  };

  const float *Qsrc = a.start;
  for (int round = 0; round <= a.power_iters; ++round) {
    // P = X Q^T  [NP][r]
    if ((e = gemm<float, true, true, 4, 4>(X, D, NP * D, Qsrc, D, r * D, P, r, NP * r, 0, (int)NP, r, (int)D,
                                           1, (int)D, B, st)) != hipSuccess) return e;
    // P~ = P L^{-T}
    if ((e = factor(P, false)) != hipSuccess) return e;
    if ((e = gemm<float, true, true, 4, 4>(P, r, NP * r, Li, r, rr, Pt, r, NP * r, 0, (int)NP, r, r, 1, r,
                                           B, st)) != hipSuccess) return e;
    // Y^T = P~^T X  [r][D]
    if (sy > 1) {
      if ((e = gemm<float, false, false, 4, 4>(Pt, r, NP * r, X, D, NP * D, Yp, D, sy * r * D, r * D, r, (int)D,
                                               (int)NP, sy, ky, B, st)) != hipSuccess) return e;
      const int64_t n = (int64_t)r * D;
      hipLaunchKernelGGL(sum_splits_kernel, dim3((int)std::min<int64_t>(cdiv(B * n, 256), 65536)), dim3(256), 0,
                         st, Yp, Y, B, sy, n);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    } else if ((e = gemm<float, false, false, 4, 4>(Pt, r, NP * r, X, D, NP * D, Y, D, r * D, 0, r, (int)D,
                                                    (int)NP, 1, (int)NP, B, st)) != hipSuccess) return e;
    // Q = L^{-1} Y^T
    if ((e = factor(Y, true)) != hipSuccess) return e;
    if ((e = gemm<float, true, false, 4, 4>(Li, r, rr, Y, D, r * D, Q, D, r * D, 0, r, (int)D, r, 1, r, B,
                                            st)) != hipSuccess) return e;
    Qsrc = Q;
  }
  // last orthonormalisation of Q, into Y
  if ((e = factor(Q, true)) != hipSuccess) return e;
  if ((e = gemm<float, true, false, 4, 4>(Li, r, rr, Q, D, r * D, Y, D, r * D, 0, r, (int)D, r, 1, r, B,
                                          st)) != hipSuccess) return e;
  const int64_t n = (int64_t)B * r * D;
  const int blocks = (int)std::min<int64_t>(cdiv(n, 256), 65536);
  if (s.dtype == LOWRAM_BF16)
    hipLaunchKernelGGL(basis_store_kernel<bf16_t>, dim3(blocks), dim3(256), 0, st, Y,
                       static_cast<bf16_t *>(a.basis_out), n);
  else
    hipLaunchKernelGGL(basis_store_kernel<float>, dim3(blocks), dim3(256), 0, st, Y,
                       static_cast<float *>(a.basis_out), n);
  return hipGetLastError();
}

}  // namespace lowram
