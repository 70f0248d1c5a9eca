// Allocation-free sequence-split prefill: kda_chunk_prefill_ex with the caller's workspace replaced
// by one fixed device array per GPU (for callers that cannot allocate device memory).
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

// The transitions, increments and entry states of a split.  Each GPU the library runs on holds
// its own copy until the process ends.  In host code `scratch` names a host-side stand-in, not
// device memory: kernels and runtime calls only ever get the device address looked up below.
static __device__ __align__(256) char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch` per device

// Device address of this device's `scratch`, looked up once per device with the device current.
kda_status_t scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return KDA_ERR_DEVICE;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return KDA_ERR_DEVICE;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KDA_OK;
}

}  // namespace

extern "C" kda_status_t kda_chunk_prefill_noalloc(const void* q, const void* k, const void* v,
                                                  const float* log_alpha, const float* beta, const float* S0,
                                                  void* o, float* S_T, int B, int T, int H, int dk, int dv,
                                                  int chunk, kda_dtype_t dt, int seg_len, int n_vs, void* stream) {
    // 0 for a shape the prefill rejects or does not split: the call below then validates or runs
    // it without any scratch
    const size_t need = kda_chunk_prefill_workspace_bytes_ex(B, T, H, dk, dv, chunk, dt, seg_len);
    if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        const kda_status_t st = scratch_address(&ws);
        if (st != KDA_OK) return st;
    }
    return kda::prefill_on_stream(q, k, v, log_alpha, beta, S0, o, S_T, B, T, H, dk, dv, chunk, dt, seg_len, n_vs,
                                  ws, need > 0 ? (size_t)KDA_NOALLOC_SCRATCH_BYTES : 0, stream);
}
