// Internal declarations of the key-basis computation (randomized subspace
// iteration on the pre-RoPE keys): the checked arguments, the workspace
// plan and the launcher called by lowram_compute_basis.
#pragma once

#include "lowram_internal.h"

namespace lowram {

struct BasisArgs {
  Dims s;
  const void *k_post;         // [B, G, N, H, d] dtype
  const int32_t *pos;         // [B, N] or NULL
  const int32_t *n_body;      // [B]
  const float *start;         // [B, r, D]
  int power_iters;
  void *basis_out;            // [B, r, D] dtype
  void *workspace;
};

// workspace of the basis computation (byte offsets) and its split choices
struct BasisLayout {
  int64_t NP;                 // rows of X and P: N rounded up to 128
  int sgp, sgq;               // split counts of the Gram products over rows / over D
  int sy;                     // split count of X^T P over rows
  size_t x, p, pt, y, q, yp, g, lw, dinv, linv, drop, total;
};

BasisLayout basis_layout(const Dims &s);
hipError_t launch_basis(const BasisArgs &a, hipStream_t st);

}  // namespace lowram
