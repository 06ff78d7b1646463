// Appending exact rows to the compressed body (the fold of the exact tail).
//
// LowRAM (arXiv:2611.07025), "LowRAM Paper: Amortised Values and Low-Rank
// Keys for KV Compression": "Asymmetric key compression with xKV", last
// paragraph (newly decoded tokens keep exact K/V); folding some of them into
// the compressed body applies the prefill steps ("Step-by-step mental model
// for one decoding session" item 1) to those rows with the sequence's
// existing basis and predictor.
//
// The call runs in three steps on its stream:
//   append_setup_kernel   copies n_body (the old body lengths) and forms the
//                         new rows' positions (given, or n_body[b] + t)
//   the prefill kernels   on a small cache in the workspace: n_new rows per
//                         sequence, m_new residual rows chosen among them
//   append_merge_kernel   copies the new coefficient rows (and positions)
//                         behind the body, appends each (b, layer, head)'s
//                         chosen rows after the entries already stored,
//                         with their residuals, and sets the new n_body
#include <algorithm>

#include "lowram_internal.h"

namespace lowram {
namespace {

constexpr int kAppendThreads = 256;

__global__ void __launch_bounds__(kAppendThreads) append_setup_kernel(AppendArgs p) {
  const int B = p.B, n_new = p.n_new;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid < B) {
    p.nb_old[gid] = min(max(p.n_body[gid], 0), p.N);
    p.n_new_arr[gid] = n_new;
  }
  if (gid < (int64_t)B * n_new) {
    const int b = static_cast<int>(gid / n_new), t = static_cast<int>(gid % n_new);
    // the old length is read from n_body itself here (nb_old may not be written yet)
    const int n0 = min(max(p.n_body[b], 0), p.N);
    p.pos_tmp[gid] = p.pos_new ? p.pos_new[gid] : n0 + t;
  }
}

// copy n2 16-bit units
__device__ __forceinline__ void copy_u16(uint16_t *dst, const uint16_t *src, int64_t n2, int tid, int nt) {
  for (int64_t i = tid; i < n2; i += nt) dst[i] = src[i];
}

// blocks [0, n_row_blocks): coefficient rows (and positions); blocks after:
// one (b, l, h) residual list each
__global__ void __launch_bounds__(kAppendThreads) append_merge_kernel(AppendArgs p, int n_row_blocks) {
  const int tid = threadIdx.x;
  const int r = p.r, d = p.d, N = p.N, m = p.m, n_new = p.n_new, m_new = p.m_new;
  if ((int)blockIdx.x < n_row_blocks) {
    // rows (b, t): one row per pass of the block
    for (int64_t row = blockIdx.x; row < (int64_t)p.B * n_new; row += n_row_blocks) {
      const int b = static_cast<int>(row / n_new), t = static_cast<int>(row % n_new);
      const int dst = p.nb_old[b] + t;
      if (dst >= N) continue;                           // past the rows allocated: dropped
      const int64_t drow = (int64_t)b * N + dst;
      if (p.int4_coef) {
        copy_u16(reinterpret_cast<uint16_t *>(static_cast<uint8_t *>(p.coef) + drow * (r / 2)),
                 reinterpret_cast<const uint16_t *>(static_cast<const uint8_t *>(p.coef_tmp) + row * (r / 2)),
                 r / 4, tid, blockDim.x);
        copy_u16(static_cast<uint16_t *>(p.coef_scale) + drow * (r / 32),
                 static_cast<const uint16_t *>(p.coef_scale_tmp) + row * (r / 32), r / 32, tid, blockDim.x);
      } else {
        const int u = r * p.el / 2;                     // 16-bit units per row
        copy_u16(static_cast<uint16_t *>(p.coef) + drow * u,
                 static_cast<const uint16_t *>(p.coef_tmp) + row * u, u, tid, blockDim.x);
      }
      if (p.pos && tid == 0) p.pos[drow] = p.pos_tmp[row];
    }
    if (blockIdx.x == 0) {
      __syncthreads();
      for (int b = tid; b < p.B; b += blockDim.x) p.n_body[b] = min(p.nb_old[b] + n_new, N);
    }
    return;
  }
  // residual list of (b, l, h)
  const int64_t lst = blockIdx.x - n_row_blocks;         // (b * G + l) * H + h
  const int b = static_cast<int>(lst / p.GH);
  const int n0 = p.nb_old[b];
  int32_t *idx = p.resid_idx + lst * m;
  __shared__ int count;
  if (tid == 0) {
    // entries are ascending with INT32_MAX padding: first entry >= n0
    int lo = 0, hi = m;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (idx[mid] < n0) lo = mid + 1;
      else hi = mid;
    }
    count = lo;
  }
  __syncthreads();
  const int32_t *nidx = p.idx_tmp + lst * m_new;
  for (int j = 0; j < m_new; ++j) {
    const int e = nidx[j];
    if (e < 0 || e >= n_new) break;                     // the chosen rows form a prefix
    const int slot = count + j;
    if (slot >= m || n0 + e >= N) break;                // no room: dropped
    const int64_t ds = lst * m + slot, ss = lst * m_new + j;
    if (tid == 0) idx[slot] = n0 + e;
    if (p.int4_res) {
      copy_u16(reinterpret_cast<uint16_t *>(static_cast<uint8_t *>(p.resid_val) + ds * (d / 2)),
               reinterpret_cast<const uint16_t *>(static_cast<const uint8_t *>(p.val_tmp) + ss * (d / 2)),
               d / 4, tid, blockDim.x);
      copy_u16(static_cast<uint16_t *>(p.resid_scale) + ds * (d / 32),
               static_cast<const uint16_t *>(p.val_scale_tmp) + ss * (d / 32), d / 32, tid, blockDim.x);
    } else {
      const int u = d * p.el / 2;
      copy_u16(static_cast<uint16_t *>(p.resid_val) + ds * u, static_cast<const uint16_t *>(p.val_tmp) + ss * u, u,
               tid, blockDim.x);
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs &p, const PrefillArgs &mini, bool mfma, hipStream_t st) {
  hipError_t e;
  const int64_t n_setup = std::max<int64_t>((int64_t)p.B * p.n_new, p.B);
  hipLaunchKernelGGL(append_setup_kernel, dim3((unsigned)((n_setup + kAppendThreads - 1) / kAppendThreads)),
                     dim3(kAppendThreads), 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (p.n_new > 0) {
    e = mfma ? launch_prefill_mfma(mini, st) : launch_prefill_plain(mini, st);
    if (e != hipSuccess) return e;
  }
  const int n_row_blocks = (int)std::min<int64_t>(std::max<int64_t>((int64_t)p.B * p.n_new, 1), 4096);
  const int n_lists = (p.m_new > 0) ? p.B * p.GH : 0;
  hipLaunchKernelGGL(append_merge_kernel, dim3(n_row_blocks + n_lists), dim3(kAppendThreads), 0, st, p,
                     n_row_blocks);
  return hipGetLastError();
}

}  // namespace lowram
