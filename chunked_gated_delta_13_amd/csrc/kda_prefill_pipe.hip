// Instantiations of the two-role (look-ahead) chunk-prefill kernel: bf16, d_k = d_v = 128,
// 64-token chunks, fp32 log alpha or the fused bounded gate; 8 chunk waves.
#include "kda_prefill_pipe.h"

namespace kda {

hipError_t launch_prefill_bf16_pipe(int ncw, const PrefillArgs& a, hipStream_t s) {
    if (ncw == 8) return a.gate ? launch_prefill_pipe<8, true>(a, s) : launch_prefill_pipe<8, false>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace kda
