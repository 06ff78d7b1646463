/*
 * lowram_basis.h — the shared key basis of a layer group, computed on the
 * GPU (the step before lowram_compress_prefill).  Conventions, notation and
 * status codes are those of lowram.h.
 *
 * [EXPL] "Asymmetric key compression with xKV": adjacent layers share their
 * dominant key subspaces, so a layer group stores one shared basis plus
 * small per-token factors, computed on the keys with the rotary embedding
 * undone; "Step-by-step mental model ...", item 1 (prefill compresses the
 * keys with shared low-rank bases).  The pages name no algorithm for the
 * basis.  The dominant r-dimensional subspace of the rows of the pre-RoPE
 * key matrix X (its top-r right singular subspace) is what the stored
 * factors c = basis x lose least of; this call computes an orthonormal basis
 * of it by randomized subspace iteration (Halko, Martinsson and Tropp,
 * "Finding structure with randomness", SIAM Review 53(2), 2011,
 * Algorithm 4.4).
 */
#ifndef LOWRAM_BASIS_H
#define LOWRAM_BASIS_H

#include "lowram.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of workspace lowram_compute_basis needs for this shape: the pre-RoPE
 * keys (4 N' D bytes per sequence, N' = n_body_max rounded up to 128), two
 * N' x r and two r x D fp32 iterates (at small batch also partial sums of
 * X^T P), fp64 Gram partial sums and factors, the fp32 inverse factor. */
int32_t lowram_basis_workspace_size(const lowram_shape *shape, size_t *bytes);

/*
 * lowram_compute_basis — per sequence b, with X the n_body[b] x D matrix of
 * pre-RoPE keys (row t = the keys of body row t of every (layer, head) with
 * the rotation at pos[t] undone, column (l*Hkv + h)*d + j, as prefill's
 * steps 1-2 form it):
 *   Q = start[b];  repeat power_iters + 1 times:
 *       P = orth(X Q^T);   Q = orth(X^T P)^T;
 *   basis[b] = Q   (r orthonormal rows spanning the computed subspace)
 * where orth(M) keeps the column order of Gram-Schmidt: the Q factor of
 * M = Q R with R's diagonal positive.  A column whose residual against the
 * kept columns before it has norm <= 1e-5 times the largest column norm of
 * M is treated as dependent: it yields a zero vector and takes no further
 * part; so rows past the numerical rank of X (e.g. when n_body[b] < r) are
 * zero.  No Rayleigh-Ritz step: the rows span the subspace but are not the
 * individual singular vectors.  Every step runs on the GPU; the random
 * numbers are the caller's (start).
 * Arithmetic: fp32 keys and products (matrix cores, fp32 accumulation);
 * Gram matrices, Cholesky factors and their inverses in fp64; the last Q is
 * orthonormalised twice.
 *
 * k_post     [B,G,N,Hkv,d] dtype   keys as the model produced them (post RoPE)
 * pos        [B,N] int32 or NULL   original positions (NULL: pos = t)
 * n_body     [B] int32             rows t >= n_body[b] are not part of X
 * start      [B,r,D] fp32          the starting matrix (e.g. i.i.d. standard
 *                                  normal), 16-byte aligned
 * power_iters  0 .. 64             rounds beyond the first
 * basis_out  [B,r,D] dtype         the basis, rows as in lowram_cache.basis
 * workspace  lowram_basis_workspace_size(shape) bytes, 16-byte aligned
 * Shape fields used: batch, group_layers, n_kv_heads, head_dim, rank
 * (r <= 512), n_body_max, rope_theta, dtype; the others are checked as
 * everywhere but not used.
 * Errors: LOWRAM_E_ARG (shape, power_iters, NULL required pointer,
 * misaligned start or workspace), _UNSUPPORTED (r > 512), _WORKSPACE, _HIP.
 */
int32_t lowram_compute_basis(const lowram_shape *shape, const void *k_post,
                             const int32_t *pos, const int32_t *n_body,
                             const float *start, int32_t power_iters,
                             void *basis_out, void *workspace,
                             size_t workspace_bytes, void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* LOWRAM_BASIS_H */
