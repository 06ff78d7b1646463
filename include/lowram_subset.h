/*
 * lowram_subset.h — a structured choice of the body rows decode attends
 * (the subset passed to lowram_decode_attn).  Conventions and status codes
 * are those of lowram.h.
 *
 * [ABS] and [WIKI] flowchart: only a selected subset of the KV pairs is
 * rebuilt at each decode step; [EXPL] "Value cache amortisation in plain
 * language" (selective reconstruction, so decode touches only a subset).
 * The pages do not say how the subset is chosen.  This call builds the
 * plainest structured one, from position alone: the first n_sink rows
 * (attention sinks, the eviction family [EXPL] "The bottleneck LowRAM
 * targets" names), the last n_recent rows, and every stride-th row in
 * between.  It reads no scores, so it never needs the rows it skips.
 */
#ifndef LOWRAM_SUBSET_H
#define LOWRAM_SUBSET_H

#include "lowram.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  uint32_t struct_size;       /* = sizeof(lowram_subset_policy)             */
  int32_t n_sink;             /* >= 0: rows 0 .. n_sink-1 are attended      */
  int32_t n_recent;           /* >= 0: the last n_recent body rows          */
  int32_t stride;             /* >= 0: rows n_sink + k*stride in between;
                                 0 = none                                   */
} lowram_subset_policy;

/* Upper bound of the subset size of a batch (entries of subset_idx):
 * batch * count(n_body_max), count being non-decreasing in n_body. */
int32_t lowram_subset_capacity(int32_t batch, int32_t n_body_max,
                               const lowram_subset_policy *policy,
                               int64_t *entries);

/*
 * lowram_select_subset — per sequence b with n = n_body[b] clamped to
 * [0, n_body_max]:
 *   A_b = { t < n : t < n_sink  or  t >= n - n_recent
 *                   or (stride > 0 and (t - n_sink) % stride == 0) }
 * written as CSR, sorted ascending: subset_off[0] = 0,
 * subset_off[b+1] = subset_off[b] + |A_b|, subset_idx[subset_off[b] + k]
 * = the k-th row of A_b.  The result is what lowram_decode_attn takes as
 * its subset (shared by every head and layer of the group).
 * n_body      [B] int32 (device)
 * subset_off  [B+1] int32 (device), written
 * subset_idx  [capacity] int32 (device), written (capacity from
 *             lowram_subset_capacity; entries past subset_off[B] untouched)
 * Errors: LOWRAM_E_ARG (batch < 1, n_body_max < 0, negative policy fields,
 * struct size, NULL pointer, capacity below the bound), _HIP.
 */
int32_t lowram_select_subset(int32_t batch, const int32_t *n_body,
                             int32_t n_body_max,
                             const lowram_subset_policy *policy,
                             int32_t *subset_off, int32_t *subset_idx,
                             int64_t capacity, void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* LOWRAM_SUBSET_H */
