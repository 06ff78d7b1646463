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

// blocks [0, n_row_blocks): coefficient rows (and positions), 16 bytes a
// thread; blocks after: one (b, l, h) residual list each
__global__ void __launch_bounds__(kAppendThreads) append_merge_kernel(AppendArgs p, int n_row_blocks) {
  const int tid = threadIdx.x;
  const int r = p.r, d = p.d, N = p.N, m = p.m, n_new = p.n_new, m_new = p.m_new;
  if ((int)blockIdx.x < n_row_blocks) {
    // row (b, t) is 16-byte piece range [row * cw, (row + 1) * cw)
    const int cw = p.int4_coef ? r / 32 : r * p.el / 16;          // 16-byte pieces per row
    const int64_t total = (int64_t)p.B * n_new * cw;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + tid; i < total; i += (int64_t)n_row_blocks * blockDim.x) {
      const int64_t row = i / cw;
      const int piece = static_cast<int>(i % cw);
      const int b = static_cast<int>(row / n_new), t = static_cast<int>(row % n_new);
      const int dst = p.nb_old[b] + t;
      if (dst >= N) continue;                           // past the rows allocated: dropped
      const int64_t drow = (int64_t)b * N + dst;
      reinterpret_cast<uint4 *>(static_cast<uint8_t *>(p.coef) + drow * cw * 16)[piece] =
          reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(p.coef_tmp) + row * cw * 16)[piece];
      if (piece == 0) {
        if (p.int4_coef)
          for (int k = 0; k < r / 32; ++k)
            static_cast<uint16_t *>(p.coef_scale)[drow * (r / 32) + k] =
                static_cast<const uint16_t *>(p.coef_scale_tmp)[row * (r / 32) + k];
        if (p.pos) p.pos[drow] = p.pos_tmp[row];
      }
    }
    if (blockIdx.x == 0) {
      __syncthreads();
      for (int b = tid; b < p.B; b += blockDim.x) p.n_body[b] = min(p.nb_old[b] + n_new, N);
    }
    return;
  }
  // residual list of (b, l, h): the chosen rows (ascending, INT32_MAX
  // padding after them) follow the entries already stored (those < n0)
  const int64_t lst = blockIdx.x - n_row_blocks;         // (b * G + l) * H + h
  const int b = static_cast<int>(lst / p.GH);
  const int n0 = p.nb_old[b];
  int32_t *idx = p.resid_idx + lst * m;
  const int32_t *nidx = p.idx_tmp + lst * m_new;
  __shared__ int count, k_end;
  if (p.select_in_merge) {
    // The list's m_new rows: the top m_new of the new rows' scores by (key
    // descending, row ascending), each row's rank counted directly (n_new <=
    // kMergeSelectMax), the chosen rows written in ascending row order.
    __shared__ uint32_t skey[kMergeSelectMax];
    __shared__ int32_t srow[kMergeSelectMax];
    __shared__ int wsel[kAppendThreads / 64];
    const float *e = p.err_tmp + lst * n_new;
    for (int i = tid; i < n_new; i += kAppendThreads) skey[i] = score_key(e[i]);
    __syncthreads();
    const int lane = tid & 63, wave = tid >> 6;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int base = 0;
    for (int c0 = 0; c0 < n_new; c0 += kAppendThreads) {   // uniform trip count
      const int i = c0 + tid;
      bool sel = false;
      if (i < n_new) {
        const uint32_t k = skey[i];
        int rank = 0;
        for (int j = 0; j < n_new; ++j) {
          const uint32_t kj = skey[j];
          rank += (kj > k || (kj == k && j < i)) ? 1 : 0;
        }
        sel = rank < m_new;
      }
      const uint64_t bs = __ballot(sel);
      if (lane == 0) wsel[wave] = __popcll(bs);
      __syncthreads();
      int pos = base + __popcll(bs & lt);
      for (int w = 0; w < wave; ++w) pos += wsel[w];
      if (sel) srow[pos] = i;
      for (int w = 0; w < kAppendThreads / 64; ++w) base += wsel[w];
      __syncthreads();
    }
    nidx = srow;
  }
  if (tid < 64) {
    // first slot past the stored entries, and how many chosen rows fit: the
    // leading entries that are rows of the call and have a slot and a row
    const int c0 = wave_lower_bound(idx, m, n0);
    int kend = m_new;
    for (int j0 = 0; j0 < m_new; j0 += 64) {
      const int j = j0 + tid;
      bool ok = j >= m_new;                             // past the list: no bound here
      if (j < m_new) {
        const int e = nidx[j];
        ok = e >= 0 && e < n_new && c0 + j < m && n0 + e < N;
      }
      const uint64_t bad = ~__ballot(ok);
      if (bad) { kend = min(kend, j0 + static_cast<int>(__builtin_ctzll(bad))); break; }
    }
    if (tid == 0) { count = c0; k_end = kend; }
  }
  __syncthreads();
  const int c0 = count, kend = k_end;
  for (int j = tid; j < kend; j += blockDim.x) idx[c0 + j] = n0 + nidx[j];
  // residual rows: 16-byte pieces (int4 scales in 16-bit units)
  const int rw = p.int4_res ? d / 32 : d * p.el / 16;           // 16-byte pieces per residual row
  // source of chosen entry j: its row's residual (every new row stored) or
  // the j-th chosen one
  auto src_row = [&](int j) -> int64_t { return p.val_by_row ? lst * n_new + nidx[j] : lst * m_new + j; };
  for (int i = tid; i < kend * rw; i += blockDim.x) {
    const int j = i / rw, piece = i % rw;
    const int64_t ds = lst * m + c0 + j, ss = src_row(j);
    reinterpret_cast<uint4 *>(static_cast<uint8_t *>(p.resid_val) + ds * rw * 16)[piece] =
        reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(p.val_tmp) + ss * rw * 16)[piece];
  }
  if (p.int4_res)
    for (int i = tid; i < kend * (d / 32); i += blockDim.x) {
      const int j = i / (d / 32), k = i % (d / 32);
      static_cast<uint16_t *>(p.resid_scale)[(lst * m + c0 + j) * (d / 32) + k] =
          static_cast<const uint16_t *>(p.val_scale_tmp)[src_row(j) * (d / 32) + k];
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
  const int64_t pieces = (int64_t)p.B * p.n_new * (p.int4_coef ? p.r / 32 : p.r * p.el / 16);
  const int n_row_blocks = (int)std::min<int64_t>(std::max<int64_t>((pieces + kAppendThreads - 1) / kAppendThreads, 1), 4096);
  const int n_lists = (p.m_new > 0) ? p.B * p.GH : 0;
  hipLaunchKernelGGL(append_merge_kernel, dim3(n_row_blocks + n_lists), dim3(kAppendThreads), 0, st, p,
                     n_row_blocks);
  return hipGetLastError();
}

}  // namespace lowram
