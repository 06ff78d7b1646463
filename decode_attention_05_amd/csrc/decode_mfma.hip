// MFMA decode kernel (bf16, head_dim 128).
#include "lowram_internal.h"

namespace lowram {

bool decode_mfma_supports(const Dims &) { return false; }
int decode_mfma_split_rows(const Dims &) { return 256; }
hipError_t launch_decode_mfma(const DecodeArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace lowram
