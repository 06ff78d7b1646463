// C entry points of the LowRAM library: host-side argument checks, workspace
// planning and kernel dispatch.  No device code lives here; every check runs
// before anything is launched, so a malformed call returns an error without
// touching the GPU.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "basis_internal.h"
#include "lowram_basis.h"
#include "lowram_subset.h"
#include "lowram_timing.h"
#include "subset_internal.h"
#include "lowram_internal.h"

namespace lowram {
namespace {

thread_local std::string g_err;

int32_t fail(int32_t code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int32_t hip_fail(hipError_t e, const char *where) {
  return fail(LOWRAM_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int kMaxGrp = 8;
constexpr int kMaxSplitRecords = 4096;   // the combine kernel stages one weight per record in LDS

int32_t check_shape(const lowram_shape *sh, Dims *out) {
  if (!sh) return fail(LOWRAM_E_ARG, "shape is NULL");
  if (sh->struct_size != sizeof(lowram_shape))
    return fail(LOWRAM_E_ARG, "shape.struct_size %u != %zu", sh->struct_size, sizeof(lowram_shape));
  Dims s{};
  s.B = sh->batch; s.G = sh->group_layers; s.Hq = sh->n_q_heads; s.H = sh->n_kv_heads;
  s.d = sh->head_dim; s.r = sh->rank; s.N = sh->n_body_max; s.m = sh->n_resid; s.Te = sh->tail_max;
  s.theta = sh->rope_theta; s.dtype = sh->dtype; s.coef_store = sh->coef_store;
  s.resid_store = sh->resid_store; s.pred_shared = sh->predictor_shared; s.algo = sh->algo;
  if (s.B < 1 || s.G < 1 || s.H < 1 || s.Hq < 1) return fail(LOWRAM_E_ARG, "batch, group_layers and head counts must be >= 1");
  if (s.Hq % s.H) return fail(LOWRAM_E_ARG, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", s.Hq, s.H);
  s.grp = s.Hq / s.H;
  if (s.N < 0 || s.m < 0 || s.Te < 0) return fail(LOWRAM_E_ARG, "n_body_max, n_resid and tail_max must be >= 0");
  if (s.m > s.N) return fail(LOWRAM_E_ARG, "n_resid (%d) > n_body_max (%d)", s.m, s.N);
  if (!(s.theta > 0.0) || !std::isfinite(s.theta)) return fail(LOWRAM_E_ARG, "rope_theta must be finite and > 0");
  if (s.dtype != LOWRAM_F32 && s.dtype != LOWRAM_BF16) return fail(LOWRAM_E_ARG, "unknown dtype %d", s.dtype);
  for (int st : {s.coef_store, s.resid_store})
    if (st != LOWRAM_STORE_NATIVE && st != LOWRAM_STORE_INT4_G32) return fail(LOWRAM_E_ARG, "unknown store mode %d", st);
  if (s.pred_shared != 0 && s.pred_shared != 1) return fail(LOWRAM_E_ARG, "predictor_shared must be 0 or 1");
  if (s.algo < LOWRAM_ALGO_AUTO || s.algo > LOWRAM_ALGO_MFMA) return fail(LOWRAM_E_ARG, "unknown algo %d", s.algo);
  if (sh->reserved != 0) return fail(LOWRAM_E_ARG, "reserved must be 0");
  s.D = (int64_t)s.G * s.H * s.d;
  if (s.r < 1 || s.r % 32) return fail(LOWRAM_E_ARG, "rank (%d) must be a positive multiple of 32", s.r);
  if (s.r > s.D) return fail(LOWRAM_E_ARG, "rank (%d) > G*Hkv*d (%lld)", s.r, (long long)s.D);
  // supported by the built kernels
  if (s.d != 64 && s.d != 128) return fail(LOWRAM_E_UNSUPPORTED, "head_dim %d (supported: 64, 128)", s.d);
  if (s.grp > kMaxGrp) return fail(LOWRAM_E_UNSUPPORTED, "n_q_heads / n_kv_heads = %d > %d", s.grp, kMaxGrp);
  if (s.D > 8192) return fail(LOWRAM_E_UNSUPPORTED, "G*Hkv*d = %lld > 8192", (long long)s.D);
  if (s.r > 1024) return fail(LOWRAM_E_UNSUPPORTED, "rank %d > 1024", s.r);
  if (s.dtype == LOWRAM_F32 && (s.coef_store != LOWRAM_STORE_NATIVE || s.resid_store != LOWRAM_STORE_NATIVE))
    return fail(LOWRAM_E_UNSUPPORTED, "int4 storage needs dtype bf16");
  if ((int64_t)s.B * s.N * s.r >= (int64_t)1 << 40 || (int64_t)s.B * s.G * s.H * ((int64_t)s.m + s.N) * s.d >= (int64_t)1 << 40)
    return fail(LOWRAM_E_UNSUPPORTED, "arrays too large");
  *out = s;
  return LOWRAM_OK;
}

struct DecodePlan {
  int algo, split_rows, n_splits;
};

DecodePlan plan_decode(const Dims &s) {
  DecodePlan p{};
  p.algo = s.algo;
  if (p.algo == LOWRAM_ALGO_AUTO) p.algo = decode_mfma_supports(s) ? LOWRAM_ALGO_MFMA : LOWRAM_ALGO_PLAIN;
  p.split_rows = (p.algo == LOWRAM_ALGO_MFMA) ? decode_mfma_split_rows(s) : 64;
  const int body = s.N > 0 ? (s.N + p.split_rows - 1) / p.split_rows : 0;
  p.n_splits = body + 1;                          // + the exact-tail split
  if (p.algo == LOWRAM_ALGO_MFMA) p.n_splits = decode_mfma_n_splits(s);   // body splits + tail splits
  return p;
}

size_t decode_ws(const Dims &s, const DecodePlan &p) {
  if (p.algo == LOWRAM_ALGO_MFMA) return decode_mfma_workspace(s);
  return (size_t)s.B * s.Hq * p.n_splits * part_stride(s.d) * sizeof(float);
}

// prefill kernels for shape s: LOWRAM_ALGO_MFMA or _PLAIN
int prefill_algo(const Dims &s) {
  if (s.algo == LOWRAM_ALGO_AUTO) return prefill_mfma_supports(s) ? LOWRAM_ALGO_MFMA : LOWRAM_ALGO_PLAIN;
  return s.algo;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// prefill workspace: the scores (used when err_out is NULL), then the MFMA
// projection's partial sums when its contraction is split
size_t prefill_err_bytes(const Dims &s) { return align256((size_t)s.B * s.G * s.H * s.N * sizeof(float)); }
size_t prefill_scratch_bytes(const Dims &s) {
  return (prefill_algo(s) == LOWRAM_ALGO_MFMA && prefill_mfma_supports(s)) ? prefill_mfma_scratch(s) : 0;
}
size_t prefill_ws(const Dims &s) { return prefill_err_bytes(s) + prefill_scratch_bytes(s); }

// workspace of lowram_append_body: the small prefill of the new rows
struct AppendPlan {
  size_t nb, nn, pos, coef, coef_scale, idx, val, val_scale, err, scratch, total;
};

AppendPlan plan_append(const Dims &s, int n_new, int m_new) {
  AppendPlan p{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = (off + bytes + 255) & ~(size_t)255;
    return at;
  };
  const size_t el = s.dtype == LOWRAM_F32 ? 4 : 2;
  const size_t GH = (size_t)s.G * s.H;
  p.nb = take((size_t)s.B * 4);
  p.nn = take((size_t)s.B * 4);
  p.pos = take((size_t)s.B * n_new * 4);
  if (s.coef_store == LOWRAM_STORE_INT4_G32) {
    p.coef = take((size_t)s.B * n_new * (s.r / 2));
    p.coef_scale = take((size_t)s.B * n_new * (s.r / 32) * 2);
  } else {
    p.coef = take((size_t)s.B * n_new * s.r * el);
    p.coef_scale = p.coef;
  }
  p.idx = take((size_t)s.B * GH * m_new * 4);
  // residuals of every new row (the MFMA path stores them while scoring;
  // the plain path uses the first m_new rows of each list for the chosen ones)
  if (s.resid_store == LOWRAM_STORE_INT4_G32) {
    p.val = take((size_t)s.B * GH * n_new * (s.d / 2));
    p.val_scale = take((size_t)s.B * GH * n_new * (s.d / 32) * 2);
  } else {
    p.val = take((size_t)s.B * GH * n_new * s.d * el);
    p.val_scale = p.val;
  }
  p.err = take((size_t)s.B * GH * n_new * 4);
  Dims ms = s;                                        // the small prefill of the new rows
  ms.N = n_new;
  ms.m = m_new;
  p.scratch = take(n_new > 0 ? prefill_scratch_bytes(ms) : 0);
  p.total = off;
  return p;
}

int32_t check_append_counts(const Dims &s, int32_t n_new, int32_t m_new) {
  if (n_new < 0 || n_new > s.N) return fail(LOWRAM_E_ARG, "n_new (%d) outside [0, n_body_max = %d]", n_new, s.N);
  if (m_new < 0 || m_new > n_new || m_new > s.m)
    return fail(LOWRAM_E_ARG, "m_new (%d) outside [0, min(n_new, n_resid)] = [0, %d]", m_new, std::min(n_new, s.m));
  return LOWRAM_OK;
}

// Host checks of a decode call's index arrays (host copies): the
// preconditions that the kernels assume and do not check.
int32_t check_indices(const Dims &s, const int32_t *n_body, const int32_t *tail_len, const int32_t *pos,
                      const int32_t *resid_idx, const int32_t *sub_off, const int32_t *sub_idx) {
  for (int b = 0; b < s.B; ++b) {
    if (n_body[b] < 0 || n_body[b] > s.N)
      return fail(LOWRAM_E_ARG, "n_body[%d] = %d outside [0, n_body_max = %d]", b, n_body[b], s.N);
    if (tail_len && (tail_len[b] < 0 || tail_len[b] > s.Te))
      return fail(LOWRAM_E_ARG, "tail_len[%d] = %d outside [0, tail_max = %d]", b, tail_len[b], s.Te);
  }
  if (pos)
    for (int b = 0; b < s.B; ++b)
      for (int t = 0; t < n_body[b]; ++t)
        if (pos[(int64_t)b * s.N + t] < 0) return fail(LOWRAM_E_ARG, "pos[%d][%d] = %d < 0", b, t, pos[(int64_t)b * s.N + t]);
  if (resid_idx && s.m > 0)
    for (int b = 0; b < s.B; ++b)
      for (int lh = 0; lh < s.G * s.H; ++lh) {
        const int32_t *x = resid_idx + ((int64_t)b * s.G * s.H + lh) * s.m;
        bool pad = false;
        for (int i = 0; i < s.m; ++i) {
          if (x[i] == INT32_MAX) { pad = true; continue; }
          if (pad)
            return fail(LOWRAM_E_ARG, "resid_idx[%d][%d][%d][%d] = %d follows a padding slot", b, lh / s.H,
                        lh % s.H, i, x[i]);
          if (x[i] < 0 || x[i] >= n_body[b])
            return fail(LOWRAM_E_ARG, "resid_idx[%d][%d][%d][%d] = %d outside [0, n_body = %d)", b, lh / s.H,
                        lh % s.H, i, x[i], n_body[b]);
          if (i > 0 && x[i] <= x[i - 1])
            return fail(LOWRAM_E_ARG, "resid_idx[%d][%d][%d] not strictly ascending at slot %d (%d after %d)",
                        b, lh / s.H, lh % s.H, i, x[i], x[i - 1]);
        }
      }
  if (sub_off) {
    if (sub_off[0] != 0) return fail(LOWRAM_E_ARG, "subset_off[0] = %d, not 0", sub_off[0]);
    // offsets first: non-decreasing offsets stay within [0, subset_off[B]],
    // the number of entries subset_idx holds
    for (int b = 0; b < s.B; ++b)
      if (sub_off[b + 1] < sub_off[b])
        return fail(LOWRAM_E_ARG, "subset_off decreases at %d (%d after %d)", b + 1, sub_off[b + 1], sub_off[b]);
    for (int b = 0; b < s.B; ++b) {
      for (int i = sub_off[b]; i < sub_off[b + 1]; ++i) {
        if (sub_idx[i] < 0 || sub_idx[i] >= n_body[b])
          return fail(LOWRAM_E_ARG, "subset entry %d of sequence %d = %d outside [0, n_body = %d)", i - sub_off[b], b,
                      sub_idx[i], n_body[b]);
        if (i > sub_off[b] && sub_idx[i] <= sub_idx[i - 1])
          return fail(LOWRAM_E_ARG, "subset of sequence %d not strictly ascending at entry %d (%d after %d)", b,
                      i - sub_off[b], sub_idx[i], sub_idx[i - 1]);
      }
    }
  }
  return LOWRAM_OK;
}

bool validate_enabled() {
  const char *v = std::getenv("LOWRAM_VALIDATE");
  return v && std::strcmp(v, "1") == 0;
}

// LOWRAM_VALIDATE=1: copy a decode call's index arrays to the host (on the
// call's stream, then wait for it) and check them before any launch.
int32_t validate_decode(const Dims &s, const lowram_cache &c, const int32_t *sub_off, const int32_t *sub_idx,
                        hipStream_t st) {
  auto fetch = [&](const int32_t *src, size_t n, std::vector<int32_t> &dst) -> hipError_t {
    dst.assign(n, 0);
    return n ? hipMemcpyAsync(dst.data(), src, n * sizeof(int32_t), hipMemcpyDeviceToHost, st) : hipSuccess;
  };
  std::vector<int32_t> nb, tl, pos, ridx, off, idx;
  hipError_t e;
  if ((e = fetch(c.n_body, s.B, nb)) != hipSuccess) return hip_fail(e, "validate: n_body");
  if ((e = fetch(c.tail_len, s.B, tl)) != hipSuccess) return hip_fail(e, "validate: tail_len");
  if (c.pos && (e = fetch(c.pos, (size_t)s.B * s.N, pos)) != hipSuccess) return hip_fail(e, "validate: pos");
  if (s.m > 0 && (e = fetch(c.resid_idx, (size_t)s.B * s.G * s.H * s.m, ridx)) != hipSuccess)
    return hip_fail(e, "validate: resid_idx");
  if (sub_off && (e = fetch(sub_off, (size_t)s.B + 1, off)) != hipSuccess) return hip_fail(e, "validate: subset_off");
  if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_fail(e, "validate: synchronise");
  if (sub_off) {
    if (off[0] != 0 || off[s.B] < 0) return fail(LOWRAM_E_ARG, "subset_off[0] = %d, subset_off[B] = %d", off[0], off[s.B]);
    if ((e = fetch(sub_idx, (size_t)off[s.B], idx)) != hipSuccess) return hip_fail(e, "validate: subset_idx");
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_fail(e, "validate: synchronise");
  }
  return check_indices(s, nb.data(), tl.data(), c.pos ? pos.data() : nullptr, s.m > 0 ? ridx.data() : nullptr,
                       sub_off ? off.data() : nullptr, idx.data());
}

}  // namespace
}  // namespace lowram

using namespace lowram;

extern "C" {

const char *lowram_status_string(int32_t st) {
  switch (st) {
    case LOWRAM_OK: return "LOWRAM_OK";
    case LOWRAM_E_ARG: return "LOWRAM_E_ARG";
    case LOWRAM_E_UNSUPPORTED: return "LOWRAM_E_UNSUPPORTED";
    case LOWRAM_E_WORKSPACE: return "LOWRAM_E_WORKSPACE";
    case LOWRAM_E_HIP: return "LOWRAM_E_HIP";
    default: return "LOWRAM_E_UNKNOWN";
  }
}

const char *lowram_last_error(void) { return g_err.c_str(); }

int32_t lowram_check_decode_indices(const lowram_shape *shape, const int32_t *n_body, const int32_t *tail_len,
                                    const int32_t *pos, const int32_t *resid_idx, const int32_t *subset_off,
                                    const int32_t *subset_idx) {
  g_err.clear();
  Dims s;
  int32_t st = check_shape(shape, &s);
  if (st) return st;
  if (!n_body) return fail(LOWRAM_E_ARG, "n_body is required");
  if (s.m > 0 && !resid_idx) return fail(LOWRAM_E_ARG, "resid_idx is required when n_resid > 0");
  if (subset_off && !subset_idx && subset_off[s.B] > 0) return fail(LOWRAM_E_ARG, "subset_idx is required with subset_off");
  return check_indices(s, n_body, tail_len, pos, resid_idx, subset_off, subset_idx);
}

int32_t lowram_workspace_size(const lowram_shape *shape, int32_t op, size_t *bytes) {
  g_err.clear();
  Dims s;
  int32_t st = check_shape(shape, &s);
  if (st) return st;
  if (!bytes) return fail(LOWRAM_E_ARG, "bytes is NULL");
  if (op == 0) *bytes = prefill_ws(s);
  else if (op == 1) *bytes = decode_ws(s, plan_decode(s));
  else return fail(LOWRAM_E_ARG, "op must be 0 (prefill) or 1 (decode)");
  return LOWRAM_OK;
}

int32_t lowram_compress_prefill(const lowram_shape *shape, const void *k_post, const void *v,
                                const int32_t *pos, const int32_t *n_body, const void *basis,
                                const void *w1, const void *b1, const void *w2, const void *b2,
                                void *coef_out, void *coef_scale_out, int32_t *resid_idx_out,
                                void *resid_val_out, void *resid_scale_out, float *err_out,
                                void *workspace, size_t workspace_bytes, void *hip_stream) {
  g_err.clear();
  Dims s;
  int32_t st = check_shape(shape, &s);
  if (st) return st;
  if (!n_body || !basis || !w1 || !b1 || !w2 || !b2)
    return fail(LOWRAM_E_ARG, "n_body, basis and predictor pointers are required");
  if (s.N > 0 && (!k_post || !v || !coef_out)) return fail(LOWRAM_E_ARG, "k_post, v and coef_out are required");
  if (s.coef_store == LOWRAM_STORE_INT4_G32 && s.N > 0 && !coef_scale_out)
    return fail(LOWRAM_E_ARG, "coef_scale_out is required with int4 coefficients");
  if (s.m > 0 && (!resid_idx_out || !resid_val_out)) return fail(LOWRAM_E_ARG, "resid_idx_out and resid_val_out are required when n_resid > 0");
  if (s.m > 0 && s.resid_store == LOWRAM_STORE_INT4_G32 && !resid_scale_out)
    return fail(LOWRAM_E_ARG, "resid_scale_out is required with int4 residuals");
  const int algo = prefill_algo(s);
  if (algo == LOWRAM_ALGO_MFMA && !prefill_mfma_supports(s))
    return fail(LOWRAM_E_UNSUPPORTED, "the MFMA prefill needs bf16, head_dim 128 and rank a multiple of 64, at most 512");
  if (s.N == 0) return LOWRAM_OK;
  const size_t scratch = prefill_scratch_bytes(s);
  const size_t need = (err_out && scratch == 0) ? 0 : prefill_ws(s);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(LOWRAM_E_WORKSPACE, "prefill needs %zu workspace bytes (got %zu)", need, workspace ? workspace_bytes : 0);
  char *ws = static_cast<char *>(workspace);
  float *err = err_out ? err_out : reinterpret_cast<float *>(ws);
  PrefillArgs a{};
  a.s = s; a.k_post = k_post; a.v = v; a.pos = pos; a.n_body = n_body; a.basis = basis;
  a.w1 = w1; a.b1 = b1; a.w2 = w2; a.b2 = b2; a.coef = coef_out; a.coef_scale = coef_scale_out;
  a.resid_idx = resid_idx_out; a.resid_val = resid_val_out; a.resid_scale = resid_scale_out; a.err = err;
  a.scratch = scratch ? reinterpret_cast<float *>(ws + prefill_err_bytes(s)) : nullptr;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  hipError_t e = (algo == LOWRAM_ALGO_MFMA) ? launch_prefill_mfma(a, stream) : launch_prefill_plain(a, stream);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return LOWRAM_OK;
}

int32_t lowram_append_workspace_size(const lowram_shape *shape, int32_t n_new, int32_t m_new, size_t *bytes) {
  g_err.clear();
  Dims s;
  int32_t st = check_shape(shape, &s);
  if (st) return st;
  if ((st = check_append_counts(s, n_new, m_new))) return st;
  if (!bytes) return fail(LOWRAM_E_ARG, "bytes is NULL");
  *bytes = plan_append(s, n_new, m_new).total;
  return LOWRAM_OK;
}

int32_t lowram_append_body(const lowram_shape *shape, int32_t n_new, int32_t m_new, const void *k_post_new,
                           const void *v_new, const int32_t *pos_new, const void *basis, const void *w1,
                           const void *b1, const void *w2, const void *b2, int32_t *n_body, int32_t *pos,
                           void *coef, void *coef_scale, int32_t *resid_idx, void *resid_val, void *resid_scale,
                           float *err_out, void *workspace, size_t workspace_bytes, void *hip_stream) {
  g_err.clear();
  Dims s;
  int32_t st = check_shape(shape, &s);
  if (st) return st;
  if ((st = check_append_counts(s, n_new, m_new))) return st;
  if (!n_body || !basis || !w1 || !b1 || !w2 || !b2)
    return fail(LOWRAM_E_ARG, "n_body, basis and predictor pointers are required");
  if (n_new > 0 && (!k_post_new || !v_new || !coef)) return fail(LOWRAM_E_ARG, "k_post_new, v_new and coef are required");
  if (n_new > 0 && s.coef_store == LOWRAM_STORE_INT4_G32 && !coef_scale)
    return fail(LOWRAM_E_ARG, "coef_scale is required with int4 coefficients");
  if (m_new > 0 && (!resid_idx || !resid_val)) return fail(LOWRAM_E_ARG, "resid_idx and resid_val are required when m_new > 0");
  if (m_new > 0 && s.resid_store == LOWRAM_STORE_INT4_G32 && !resid_scale)
    return fail(LOWRAM_E_ARG, "resid_scale is required with int4 residuals");
  if (pos && !pos_new && n_new > 0) return fail(LOWRAM_E_ARG, "a cache with positions needs pos_new");
  const AppendPlan pl = plan_append(s, n_new, m_new);
  if (!workspace || workspace_bytes < pl.total)
    return fail(LOWRAM_E_WORKSPACE, "append needs %zu workspace bytes (got %zu)", pl.total, workspace ? workspace_bytes : 0);
  Dims ms = s;                                        // the small prefill of the new rows
  ms.N = n_new;
  ms.m = m_new;
  int algo = s.algo;
  if (algo == LOWRAM_ALGO_AUTO) algo = prefill_mfma_supports(ms) ? LOWRAM_ALGO_MFMA : LOWRAM_ALGO_PLAIN;
  if (algo == LOWRAM_ALGO_MFMA && n_new > 0 && !prefill_mfma_supports(ms))
    return fail(LOWRAM_E_UNSUPPORTED, "the MFMA prefill needs bf16, head_dim 128 and rank a multiple of 64, at most 512");
  char *ws = static_cast<char *>(workspace);
  AppendArgs p{};
  p.B = s.B; p.GH = s.G * s.H; p.N = s.N; p.m = s.m; p.r = s.r; p.d = s.d;
  p.el = s.dtype == LOWRAM_F32 ? 4 : 2; p.n_new = n_new; p.m_new = m_new;
  p.int4_coef = s.coef_store == LOWRAM_STORE_INT4_G32; p.int4_res = s.resid_store == LOWRAM_STORE_INT4_G32;
  p.n_body = n_body; p.pos_new = pos_new; p.pos = pos; p.coef = coef; p.coef_scale = coef_scale;
  p.resid_idx = resid_idx; p.resid_val = resid_val; p.resid_scale = resid_scale;
  p.nb_old = reinterpret_cast<int32_t *>(ws + pl.nb);
  p.n_new_arr = reinterpret_cast<int32_t *>(ws + pl.nn);
  p.pos_tmp = reinterpret_cast<int32_t *>(ws + pl.pos);
  p.coef_tmp = ws + pl.coef; p.coef_scale_tmp = ws + pl.coef_scale;
  p.idx_tmp = reinterpret_cast<int32_t *>(ws + pl.idx);
  p.val_tmp = ws + pl.val; p.val_scale_tmp = ws + pl.val_scale;
  PrefillArgs a{};
  a.s = ms; a.k_post = k_post_new; a.v = v_new; a.pos = p.pos_tmp; a.n_body = p.n_new_arr; a.basis = basis;
  a.w1 = w1; a.b1 = b1; a.w2 = w2; a.b2 = b2; a.coef = p.coef_tmp; a.coef_scale = p.coef_scale_tmp;
  a.resid_idx = p.idx_tmp; a.resid_val = p.val_tmp; a.resid_scale = p.val_scale_tmp;
  a.err = err_out ? err_out : reinterpret_cast<float *>(ws + pl.err);
  a.scratch = reinterpret_cast<float *>(ws + pl.scratch);
  if (algo == LOWRAM_ALGO_MFMA && m_new > 0) {       // residuals stored by the scoring pass, by row
    a.all_resid = p.val_tmp;
    a.all_resid_scale = p.val_scale_tmp;
    p.val_by_row = true;
    if (n_new <= kMergeSelectMax) {                  // the merge ranks the scores itself
      a.no_select = true;
      p.select_in_merge = true;
      p.err_tmp = a.err;
    }
  }
  hipError_t e = launch_append(p, a, algo == LOWRAM_ALGO_MFMA, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return LOWRAM_OK;
}

int32_t lowram_fit_workspace_size(const lowram_shape *shape, size_t *bytes) {
  g_err.clear();
  Dims s;
  int32_t st = check_shape(shape, &s);
  if (st) return st;
  if (!bytes) return fail(LOWRAM_E_ARG, "bytes is NULL");
  *bytes = fit_layout(s).total;
  return LOWRAM_OK;
}

int32_t lowram_fit_predictor(const lowram_shape *shape, const void *coef, const void *coef_scale,
                             const int32_t *n_body, const void *basis, const void *v,
                             const lowram_fit_params *params, void *w1, void *b1, void *w2, void *b2,
                             float *loss_out, float *grad_out, void *workspace, size_t workspace_bytes,
                             void *hip_stream) {
  g_err.clear();
  Dims s;
  int32_t st = check_shape(shape, &s);
  if (st) return st;
  if (!params) return fail(LOWRAM_E_ARG, "params is NULL");
  if (params->struct_size != sizeof(lowram_fit_params))
    return fail(LOWRAM_E_ARG, "params.struct_size %u != %zu", params->struct_size, sizeof(lowram_fit_params));
  const lowram_fit_params &fp = *params;
  if (fp.steps < 0) return fail(LOWRAM_E_ARG, "steps (%d) must be >= 0", fp.steps);
  if (!(fp.lr > 0.0) || !std::isfinite(fp.lr)) return fail(LOWRAM_E_ARG, "lr must be finite and > 0");
  if (!(fp.beta1 >= 0.0 && fp.beta1 < 1.0) || !(fp.beta2 >= 0.0 && fp.beta2 < 1.0))
    return fail(LOWRAM_E_ARG, "beta1 and beta2 must lie in [0, 1)");
  if (!(fp.eps > 0.0) || !std::isfinite(fp.eps)) return fail(LOWRAM_E_ARG, "eps must be finite and > 0");
  if (!n_body || !basis || !w1 || !b1 || !w2 || !b2)
    return fail(LOWRAM_E_ARG, "n_body, basis and predictor pointers are required");
  if (s.N > 0 && (!coef || !v)) return fail(LOWRAM_E_ARG, "coef and v are required");
  if (s.N > 0 && s.coef_store == LOWRAM_STORE_INT4_G32 && !coef_scale)
    return fail(LOWRAM_E_ARG, "coef_scale is required with int4 coefficients");
  const FitLayout L = fit_layout(s);
  if (!workspace || workspace_bytes < L.total)
    return fail(LOWRAM_E_WORKSPACE, "fit needs %zu workspace bytes (got %zu)", L.total, workspace ? workspace_bytes : 0);
  if (fp.steps == 0) return LOWRAM_OK;
  FitArgs a{};
  a.s = s; a.coef = coef; a.coef_scale = coef_scale; a.basis = basis; a.v = v; a.n_body = n_body;
  a.w1 = w1; a.b1 = b1; a.w2 = w2; a.b2 = b2; a.loss_out = loss_out; a.grad_out = grad_out;
  a.steps = fp.steps; a.lr = fp.lr; a.beta1 = fp.beta1; a.beta2 = fp.beta2; a.eps = fp.eps;
  a.workspace = workspace;
  hipError_t e = launch_fit(a, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "fit launch");
  return LOWRAM_OK;
}

int32_t lowram_basis_workspace_size(const lowram_shape *shape, size_t *bytes) {
  g_err.clear();
  Dims s;
  int32_t st = check_shape(shape, &s);
  if (st) return st;
  if (!bytes) return fail(LOWRAM_E_ARG, "bytes is NULL");
  if (s.r > 512) return fail(LOWRAM_E_UNSUPPORTED, "the basis computation supports rank <= 512 (got %d)", s.r);
  *bytes = basis_layout(s).total;
  return LOWRAM_OK;
}

int32_t lowram_compute_basis(const lowram_shape *shape, const void *k_post, const int32_t *pos,
                             const int32_t *n_body, const float *start, int32_t power_iters,
                             void *basis_out, void *workspace, size_t workspace_bytes, void *hip_stream) {
  g_err.clear();
  Dims s;
  int32_t st = check_shape(shape, &s);
  if (st) return st;
  if (power_iters < 0 || power_iters > 64) return fail(LOWRAM_E_ARG, "power_iters (%d) outside [0, 64]", power_iters);
  if (!n_body || !start || !basis_out) return fail(LOWRAM_E_ARG, "n_body, start and basis_out are required");
  if (s.N > 0 && !k_post) return fail(LOWRAM_E_ARG, "k_post is required");
  if (reinterpret_cast<uintptr_t>(start) % 16) return fail(LOWRAM_E_ARG, "start must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(workspace) % 16) return fail(LOWRAM_E_ARG, "workspace must be 16-byte aligned");
  if (s.r > 512) return fail(LOWRAM_E_UNSUPPORTED, "the basis computation supports rank <= 512 (got %d)", s.r);
  const BasisLayout L = basis_layout(s);
  if (!workspace || workspace_bytes < L.total)
    return fail(LOWRAM_E_WORKSPACE, "basis needs %zu workspace bytes (got %zu)", L.total, workspace ? workspace_bytes : 0);
  BasisArgs a{};
  a.s = s; a.k_post = k_post; a.pos = pos; a.n_body = n_body; a.start = start; a.power_iters = power_iters;
  a.basis_out = basis_out; a.workspace = workspace;
  hipError_t e = launch_basis(a, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "basis launch");
  return LOWRAM_OK;
}

int32_t lowram_subset_capacity(int32_t batch, int32_t n_body_max, const lowram_subset_policy *policy,
                               int64_t *entries) {
  g_err.clear();
  if (!policy || !entries) return fail(LOWRAM_E_ARG, "policy and entries are required");
  if (policy->struct_size != sizeof(lowram_subset_policy))
    return fail(LOWRAM_E_ARG, "policy.struct_size %u != %zu", policy->struct_size, sizeof(lowram_subset_policy));
  if (batch < 1 || n_body_max < 0) return fail(LOWRAM_E_ARG, "batch must be >= 1 and n_body_max >= 0");
  if (policy->n_sink < 0 || policy->n_recent < 0 || policy->stride < 0)
    return fail(LOWRAM_E_ARG, "n_sink, n_recent and stride must be >= 0");
  *entries = (int64_t)batch * subset_count(n_body_max, policy->n_sink, policy->n_recent, policy->stride);
  return LOWRAM_OK;
}

int32_t lowram_select_subset(int32_t batch, const int32_t *n_body, int32_t n_body_max,
                             const lowram_subset_policy *policy, int32_t *subset_off, int32_t *subset_idx,
                             int64_t capacity, void *hip_stream) {
  int64_t need = 0;
  int32_t st = lowram_subset_capacity(batch, n_body_max, policy, &need);
  if (st) return st;
  if (!n_body || !subset_off || (!subset_idx && need > 0))
    return fail(LOWRAM_E_ARG, "n_body, subset_off and subset_idx are required");
  if (need > INT32_MAX) return fail(LOWRAM_E_ARG, "the subset would exceed 2^31 entries");
  if (capacity < need) return fail(LOWRAM_E_ARG, "subset_idx holds %lld entries, the bound is %lld",
                                   (long long)capacity, (long long)need);
  hipError_t e = launch_subset(n_body, n_body_max, batch, policy->n_sink, policy->n_recent, policy->stride,
                               subset_off, subset_idx, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "subset launch");
  return LOWRAM_OK;
}

static int32_t decode_call(const lowram_shape *shape, int32_t layer, const void *q, const lowram_cache *cache,
                           const int32_t *subset_off, const int32_t *subset_idx, void *out, float *lse_out,
                           void *workspace, size_t workspace_bytes, void *hip_stream, hipEvent_t ev_before,
                           hipEvent_t ev_after, bool noalloc = false) {
  g_err.clear();
  Dims s;
  int32_t st = check_shape(shape, &s);
  if (st) return st;
  if (layer < 0 || layer >= s.G) return fail(LOWRAM_E_ARG, "layer %d outside [0, %d)", layer, s.G);
  if (!q || !out || !cache) return fail(LOWRAM_E_ARG, "q, out and cache are required");
  const lowram_cache &c = *cache;
  if (!c.n_body || !c.basis || !c.w1 || !c.b1 || !c.w2 || !c.b2 || !c.tail_len)
    return fail(LOWRAM_E_ARG, "cache.n_body, basis, predictor and tail_len are required");
  if (s.N > 0 && !c.coef) return fail(LOWRAM_E_ARG, "cache.coef is required");
  if (s.N > 0 && s.coef_store == LOWRAM_STORE_INT4_G32 && !c.coef_scale)
    return fail(LOWRAM_E_ARG, "cache.coef_scale is required with int4 coefficients");
  if (s.m > 0 && (!c.resid_idx || !c.resid_val)) return fail(LOWRAM_E_ARG, "cache residual arrays are required when n_resid > 0");
  if (s.m > 0 && s.resid_store == LOWRAM_STORE_INT4_G32 && !c.resid_scale)
    return fail(LOWRAM_E_ARG, "cache.resid_scale is required with int4 residuals");
  if (s.Te > 0 && (!c.tail_k || !c.tail_v)) return fail(LOWRAM_E_ARG, "cache.tail_k and tail_v are required when tail_max > 0");
  if (subset_off && !subset_idx) return fail(LOWRAM_E_ARG, "subset_idx is required with subset_off");
  const DecodePlan p = plan_decode(s);
  if (p.algo == LOWRAM_ALGO_MFMA && !decode_mfma_supports(s))
    return fail(LOWRAM_E_UNSUPPORTED, "the MFMA kernel needs bf16, head_dim 128 and rank a multiple of 64");
  if (p.n_splits > kMaxSplitRecords)
    return fail(LOWRAM_E_UNSUPPORTED, "%d split records per query head > %d", p.n_splits, kMaxSplitRecords);
  const size_t need = decode_ws(s, p);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (noalloc) {
    if (need > noalloc_scratch_bytes())
      return fail(LOWRAM_E_WORKSPACE, "this decode call needs %zu bytes of scratch, more than the %zu the "
                  "allocation-free entry holds: use lowram_decode_attn with a workspace", need,
                  noalloc_scratch_bytes());
    hipError_t e = noalloc_scratch(&workspace);
    if (e != hipSuccess) return hip_fail(e, "scratch address");
    workspace_bytes = noalloc_scratch_bytes();
  } else {
    if (!workspace || workspace_bytes < need)
      return fail(LOWRAM_E_WORKSPACE, "decode needs %zu workspace bytes (got %zu)", need,
                  workspace ? workspace_bytes : 0);
    if (validate_enabled() && (st = validate_decode(s, c, subset_off, subset_idx, stream))) return st;
  }
  DecodeArgs a{};
  a.s = s; a.layer = layer; a.q = q; a.c = c; a.sub_off = subset_off; a.sub_idx = subset_idx;
  a.out = out; a.lse = lse_out; a.partials = static_cast<float *>(workspace);
  a.n_splits = p.n_splits; a.split_rows = p.split_rows;
  a.ev_before = ev_before; a.ev_after = ev_after;
  // the MFMA path merges the splits inside its own launches
  hipError_t e = (p.algo == LOWRAM_ALGO_MFMA) ? launch_decode_mfma(a, stream) : launch_decode_plain(a, stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (p.algo != LOWRAM_ALGO_MFMA) {
    e = launch_combine(a, false, stream);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
  }
  return LOWRAM_OK;
}

int32_t lowram_decode_attn(const lowram_shape *shape, int32_t layer, const void *q, const lowram_cache *cache,
                           const int32_t *subset_off, const int32_t *subset_idx, void *out, float *lse_out,
                           void *workspace, size_t workspace_bytes, void *hip_stream) {
  return decode_call(shape, layer, q, cache, subset_off, subset_idx, out, lse_out, workspace, workspace_bytes,
                     hip_stream, nullptr, nullptr);
}

int32_t lowram_decode_attn_noalloc(const lowram_shape *shape, int32_t layer, const void *q,
                                   const lowram_cache *cache, const int32_t *subset_off, const int32_t *subset_idx,
                                   void *out, float *lse_out, void *hip_stream) {
  return decode_call(shape, layer, q, cache, subset_off, subset_idx, out, lse_out, nullptr, 0, hip_stream, nullptr,
                     nullptr, true);
}

int32_t lowram_decode_attn_timed(const lowram_shape *shape, int32_t layer, const void *q,
                                 const lowram_cache *cache, const int32_t *subset_off, const int32_t *subset_idx,
                                 void *out, float *lse_out, void *workspace, size_t workspace_bytes,
                                 void *hip_stream, void *before_event, void *after_event) {
  if (!before_event || !after_event) {
    g_err.clear();
    return fail(LOWRAM_E_ARG, "both timing events are required");
  }
  return decode_call(shape, layer, q, cache, subset_off, subset_idx, out, lse_out, workspace, workspace_bytes,
                     hip_stream, static_cast<hipEvent_t>(before_event), static_cast<hipEvent_t>(after_event));
}

static int32_t dense_check(int32_t B, int32_t Hq, int32_t H, int32_t d, int32_t T) {
  if (B < 1 || Hq < 1 || H < 1 || T < 0) return fail(LOWRAM_E_ARG, "batch and heads must be >= 1, max_ctx >= 0");
  if (Hq % H) return fail(LOWRAM_E_ARG, "n_q_heads must be a multiple of n_kv_heads");
  if (d != 64 && d != 128) return fail(LOWRAM_E_UNSUPPORTED, "head_dim %d (supported: 64, 128)", d);
  if (Hq / H > kMaxGrp) return fail(LOWRAM_E_UNSUPPORTED, "n_q_heads / n_kv_heads > %d", kMaxGrp);
  if (T > 0 && (T + 511) / 512 > kMaxSplitRecords) return fail(LOWRAM_E_UNSUPPORTED, "max_ctx too large");
  return LOWRAM_OK;
}

// Rows per comparator split: 2048 (long row runs per workgroup keep the
// loads of many waves in flight), halved while the grid would have fewer
// than 512 workgroups, down to 512.
static int dense_split_rows(int32_t B, int32_t H, int32_t T) {
  int split = 2048;
  while (split > 512 && (int64_t)B * H * ((T + split - 1) / split) < 512) split /= 2;
  return split;
}

int32_t lowram_dense_workspace_size(int32_t B, int32_t Hq, int32_t H, int32_t d, int32_t T, size_t *bytes) {
  g_err.clear();
  int32_t st = dense_check(B, Hq, H, d, T);
  if (st) return st;
  if (!bytes) return fail(LOWRAM_E_ARG, "bytes is NULL");
  const int split = dense_split_rows(B, H, T);
  const int ns = T > 0 ? (T + split - 1) / split : 1;
  *bytes = (size_t)B * Hq * ns * part_stride(d) * sizeof(float);
  return LOWRAM_OK;
}

int32_t lowram_dense_decode_attn(int32_t B, int32_t Hq, int32_t H, int32_t d, int32_t T,
                                 const void *q, const void *k, const void *v, const int32_t *ctx_len,
                                 void *out, float *lse_out, void *workspace, size_t workspace_bytes,
                                 void *hip_stream) {
  g_err.clear();
  int32_t st = dense_check(B, Hq, H, d, T);
  if (st) return st;
  if (!q || !out || !ctx_len || (T > 0 && (!k || !v))) return fail(LOWRAM_E_ARG, "q, k, v, ctx_len and out are required");
  size_t need;
  lowram_dense_workspace_size(B, Hq, H, d, T, &need);
  if (!workspace || workspace_bytes < need)
    return fail(LOWRAM_E_WORKSPACE, "dense decode needs %zu workspace bytes (got %zu)", need, workspace ? workspace_bytes : 0);
  DenseArgs a{};
  a.B = B; a.Hq = Hq; a.H = H; a.d = d; a.T = T; a.grp = Hq / H; a.q = q; a.k = k; a.v = v;
  a.ctx_len = ctx_len; a.out = out; a.lse = lse_out; a.partials = static_cast<float *>(workspace);
  a.split_rows = dense_split_rows(B, H, T); a.n_splits = T > 0 ? (T + a.split_rows - 1) / a.split_rows : 1;
  a.kv_b_stride = (int64_t)T * H * d; a.kv_off = 0; a.split_base = 0;
  hipError_t e = launch_dense(a, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "dense launch");
  return LOWRAM_OK;
}

}  // extern "C"
