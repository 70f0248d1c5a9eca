// bf16-input instantiations of the fused chunk-prefill kernel: a 128-column slice at d_k = 128 runs
// on 8 waves (16 columns each), every other slice on 4.
#include "kda_prefill_kernel.h"

namespace kda {

hipError_t launch_prefill_bf16(int dk, int dvw, int nw, int chunk, const PrefillArgs& a, hipStream_t s) {
    using T = __bf16;
    if (dk == 128 && dvw == 128 && nw == 8) {
        if (chunk == 64) return launch_prefill_cfg<PrefillCfg<128, 1, 64, T, 8>>(a, s);
        if (chunk == 32) return launch_prefill_cfg<PrefillCfg<128, 1, 32, T, 8>>(a, s);
        if (chunk == 16) return launch_prefill_cfg<PrefillCfg<128, 1, 16, T, 8>>(a, s);
    }
    if (dk == 128 && dvw == 64) {
        if (chunk == 64) return launch_prefill_cfg<PrefillCfg<128, 1, 64, T, 4>>(a, s);
        if (chunk == 32) return launch_prefill_cfg<PrefillCfg<128, 1, 32, T, 4>>(a, s);
        if (chunk == 16) return launch_prefill_cfg<PrefillCfg<128, 1, 16, T, 4>>(a, s);
    }
    if (dk == 64 && dvw == 64) {
        if (chunk == 64) return launch_prefill_cfg<PrefillCfg<64, 1, 64, T, 4>>(a, s);
        if (chunk == 32) return launch_prefill_cfg<PrefillCfg<64, 1, 32, T, 4>>(a, s);
        if (chunk == 16) return launch_prefill_cfg<PrefillCfg<64, 1, 16, T, 4>>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_bf16_dual(int dk, int dvw, int nw, int chunk, const PrefillArgs& a, hipStream_t s) {
    using T = __bf16;
    if (dk == 128 && dvw == 128 && nw == 8) {
        if (chunk == 64) return launch_prefill_cfg<PrefillCfg<128, 1, 64, T, 8>, true>(a, s);
        if (chunk == 32) return launch_prefill_cfg<PrefillCfg<128, 1, 32, T, 8>, true>(a, s);
        if (chunk == 16) return launch_prefill_cfg<PrefillCfg<128, 1, 16, T, 8>, true>(a, s);
    }
    return hipErrorInvalidValue;
}

// Gate mode (bf16 raw gate pre-activation in place of fp32 log alpha), 8-wave shapes only.
hipError_t launch_prefill_bf16_gate(int dk, int dvw, int nw, int chunk, bool dual, const PrefillArgs& a,
                                    hipStream_t s) {
    using T = __bf16;
    if (dk == 128 && dvw == 128 && nw == 8) {
        if (dual) {
            if (chunk == 64) return launch_prefill_cfg<PrefillCfg<128, 1, 64, T, 8>, true, true>(a, s);
            if (chunk == 32) return launch_prefill_cfg<PrefillCfg<128, 1, 32, T, 8>, true, true>(a, s);
            if (chunk == 16) return launch_prefill_cfg<PrefillCfg<128, 1, 16, T, 8>, true, true>(a, s);
        } else {
            if (chunk == 64) return launch_prefill_cfg<PrefillCfg<128, 1, 64, T, 8>, false, true>(a, s);
            if (chunk == 32) return launch_prefill_cfg<PrefillCfg<128, 1, 32, T, 8>, false, true>(a, s);
            if (chunk == 16) return launch_prefill_cfg<PrefillCfg<128, 1, 16, T, 8>, false, true>(a, s);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
