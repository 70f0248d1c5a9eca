// Host side of libkda: argument validation, the sequence-split planner and
// kernel launches on the caller's stream.  Nothing here allocates memory or
// synchronises the host with the device.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace kda {
hipError_t launch_prefill_bf16(int dk, int dvw, int nw, int chunk, const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_f32(int dk, int dvw, int nw, int chunk, const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_bf16_dual(int dk, int dvw, int nw, int chunk, const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_bf16_pipe(int ncw, const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_bf16_gate(int dk, int dvw, int nw, int chunk, bool dual, const PrefillArgs& a,
                                    hipStream_t s);
}  // namespace kda

namespace {

using kda::PrefillArgs;

// Shortest segment worth a split at T tokens.  Over n segments the two passes take about
// 2.3 T / n chunk-times (5.3 us per 64-token chunk) and the scan n steps of about 13 us, least
// near T / n = 8 sqrt(T) (measured on the MI355X at T = 4096 .. 16384: 512- to 1024-token
// segments, up to 2.2x faster than one unsplit pass); never below 512 tokens.
long long min_segment(long long T) {
    const long long l = (long long)(8.0 * sqrt((double)T));
    return l > 512 ? l : 512;
}
constexpr int kSliceWaves = 8;        // waves per workgroup for 128-column bf16 slices
constexpr int kPipeChunkWaves = 8;    // chunk waves of the two-role prefill kernel

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void* p, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return {lo, lo + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

bool mul_ok(long long a, long long b, long long* out) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > (1LL << 62) / a) return false;
    *out = a * b;
    return true;
}

// A second stream per device for work that overlaps the caller's stream (created once, default
// priority, never destroyed), with the two events that fork it from and join it back to the
// caller's stream.  Callers hold g_side_mu while they enqueue a fork ... join sequence.
struct SideStream {
    hipStream_t stream;
    hipEvent_t fork, join;
};
std::mutex g_side_mu;
SideStream* side_stream() {
    static SideStream side[64];
    static bool made[64] = {false};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (!made[dev]) {
        SideStream x;
        if (hipStreamCreateWithFlags(&x.stream, hipStreamNonBlocking) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        if (hipEventCreateWithFlags(&x.fork, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&x.join, hipEventDisableTiming) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        side[dev] = x;
        made[dev] = true;
    }
    return &side[dev];
}

int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            n = 256;
        }
        cached[dev] = n;
    }
    return cached[dev];
}

// Chunk length the kernels run for a caller's chunk.  fp32 operands of a 64-token chunk do not fit
// the 160 KiB of LDS of one workgroup, so an fp32 call with chunk 64 runs as 32-token chunks: the
// result of the method does not depend on the chunk length beyond rounding, and every length the
// caller may pass with chunk 64 (segment length, checkpoint spacing) is a multiple of 32.
int kernel_chunk(int chunk, kda_dtype_t dt) { return (dt == KDA_F32 && chunk == 64) ? 32 : chunk; }

// Shape checks shared by the prefill entry points.
kda_status_t check_prefill_shape(int B, int T, int H, int dk, int dv, int chunk, kda_dtype_t dt) {
    if (B < 0 || T < 0 || H < 0) return KDA_ERR_INVALID_ARGUMENT;
    if (dt != KDA_BF16 && dt != KDA_F32) return KDA_ERR_INVALID_ARGUMENT;
    if (dk <= 0 || dv <= 0 || chunk <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if (dk != dv || (dk != 64 && dk != 128)) return KDA_ERR_UNSUPPORTED;
    if (chunk != 16 && chunk != 32 && chunk != 64) return KDA_ERR_UNSUPPORTED;
    if (!kda::prefill_supported(dk, dv, kernel_chunk(chunk, dt), dt == KDA_F32)) return KDA_ERR_UNSUPPORTED;
    long long n = 0;
    if (!mul_ok((long long)B * T, (long long)H * dk, &n)) return KDA_ERR_INVALID_ARGUMENT;
    // lane offsets inside one chunk are 32-bit byte offsets: 64 token rows of H * dk fp32 values
    if ((long long)H * dk > (1LL << 22)) return KDA_ERR_UNSUPPORTED;
    if ((long long)B * H > (1LL << 27)) return KDA_ERR_UNSUPPORTED;   // units fit the launch grid
    return KDA_OK;
}

// Drafted blocks up to this many tokens run as a token loop on the decode kernel (state read
// once, tokens in order on chip); longer blocks run as a chunked prefill.
constexpr int kSpecTokenLoopMax = kda::kDecodeMaxTokens;

// Shape, pointer, alignment and overlap checks of a speculative block (token-loop path).
// o (verify) or accepted (commit) is the one of the two that is not NULL.
kda_status_t check_spec_pointers(const void* q, const void* k, const void* v, const float* log_alpha,
                                 const float* beta, const float* S, const void* o, const int* accepted, int N,
                                 int m, int H, int dk, int dv, kda_dtype_t dt) {
    if (dt != KDA_BF16 && dt != KDA_F32) return KDA_ERR_INVALID_ARGUMENT;
    if (dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if (dk != dv || (dk != 64 && dk != 128)) return KDA_ERR_UNSUPPORTED;
    long long ntok_ll = 0, nh = 0;
    if (!mul_ok((long long)N * m, H, &ntok_ll) || !mul_ok(N, H, &nh)) return KDA_ERR_INVALID_ARGUMENT;
    if (nh * (dk / 64) > 0x7fffffffLL) return KDA_ERR_UNSUPPORTED;
    if (N == 0 || H == 0) return KDA_OK;
    if (!q || !k || !v || !log_alpha || !beta || !S || (!o && !accepted)) return KDA_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(log_alpha, 16) || !aligned(S, 16) ||
        !aligned(beta, 4) || (o && !aligned(o, 16)) || (accepted && !aligned(accepted, 4)))
        return KDA_ERR_INVALID_ARGUMENT;
    const size_t esz = dt == KDA_BF16 ? 2 : 4;
    const size_t ntok = (size_t)ntok_ll;
    const Range rs = range_of(S, (size_t)nh * dk * dv * sizeof(float));
    const Range ins[] = {range_of(q, ntok * dk * esz), range_of(k, ntok * dk * esz), range_of(v, ntok * dv * esz),
                         range_of(log_alpha, ntok * dk * sizeof(float)), range_of(beta, ntok * sizeof(float))};
    if (o) {   // verify: o must not overlap any input or the state
        const Range ro = range_of(o, ntok * dv * esz);
        for (const Range& r : ins)
            if (overlap(ro, r)) return KDA_ERR_INVALID_ARGUMENT;
        if (overlap(ro, rs)) return KDA_ERR_INVALID_ARGUMENT;
    } else {   // commit: the state is written and must not overlap any input
        for (const Range& r : ins)
            if (overlap(rs, r)) return KDA_ERR_INVALID_ARGUMENT;
        if (overlap(rs, range_of(accepted, (size_t)N * sizeof(int)))) return KDA_ERR_INVALID_ARGUMENT;
    }
    return KDA_OK;
}

// Chunk length for an m-token speculative block: the smallest supported chunk that holds it.
int spec_chunk(int m, kda_dtype_t dt) {
    if (m <= 16) return 16;
    if (m <= 32 || dt == KDA_F32) return 32;
    return 64;
}

// Segments of a split: segment 0 holds seg_len + shift tokens, every later one seg_len (the last
// one possibly fewer).
long long segment_count(long long T, long long seg_len, long long shift) {
    if (T <= seg_len + shift) return 1;
    return 1 + (T - seg_len - shift + seg_len - 1) / seg_len;
}

// The automatic plan: column slices first (no extra work beyond the shared per-chunk tiles),
// then segments when even that leaves most compute units idle.  The widest step of a split runs
// every segment at once (segment 0 from S0 beside the zero-start runs of the others), one
// workgroup per unit and segment, and it never takes every compute unit (on the MI355X, launches
// that needed all 256 at once ran up to 13% slower at times).  Segments are of equal length (the
// last one possibly shorter): every step runs the same work on each of them.
void auto_plan(int B, int T, int H, int dk, int dv, int chunk, bool f32, int* seg_len, int* n_vs,
               long long* shift) {
    const long long cus = cu_count();
    const long long bh = (long long)B * H;
    // Two column slices only pay where a 128-column workgroup has 4 waves (32 columns each):
    // halving the columns then halves the state products of every chunk.  With 8 waves a slice
    // already holds 16 columns per wave, and a second slice would only repeat the decay and
    // intra-chunk work; the sequence split below is what shortens the chain of chunks.
    const bool eight = kda::prefill_waves(dk, dv, f32) == 8;
    int vs = (dv == 128 && !eight && 2 * bh <= cus) ? 2 : 1;
    long long seg = T;
    const long long units = bh * vs;
    const long long lmin = min_segment(T);
    if (units > 0 && 2 * units <= cus && (long long)T >= 3 * lmin) {
        long long n = (cus - 1) / units;   // segments
        if (n > T / lmin) n = T / lmin;
        if (n >= 3) {
            // whole chunks, rounded up so that n segments cover the sequence
            long long L = ((long long)T + n - 1) / n;
            L = (L + chunk - 1) / chunk * chunk;
            seg = L;
        }
    }
    if (seg_len) *seg_len = (int)(seg > 0 ? seg : chunk);
    if (n_vs) *n_vs = vs;
    if (shift) *shift = 0;
}

// Resolve an explicit or automatic plan.  n_seg == 1 means no split.  An explicit seg_len gives
// segments of equal length (shift 0).
kda_status_t resolve_plan(int B, int T, int H, int dk, int dv, int chunk, kda_dtype_t dt,
                          int seg_len_in, int n_vs_in, long long* seg_len, int* n_seg, int* n_vs,
                          long long* shift) {
    if (seg_len_in < 0 || (seg_len_in > 0 && seg_len_in % chunk != 0)) return KDA_ERR_INVALID_ARGUMENT;
    // segment lengths are whole chunks of the caller's length (multiples of the kernels' chunk too)
    int a_seg = 0, a_vs = 0;
    long long a_sh = 0;
    auto_plan(B, T, H, dk, dv, chunk, dt == KDA_F32, &a_seg, &a_vs, &a_sh);
    long long sl = seg_len_in > 0 ? seg_len_in : a_seg;
    long long sh = seg_len_in > 0 ? 0 : a_sh;
    int vs = n_vs_in > 0 ? n_vs_in : a_vs;
    if (n_vs_in < 0 || vs > 2 || (vs == 2 && dv != 128)) return KDA_ERR_INVALID_ARGUMENT;
    if (!kda::prefill_supported(dk, dv / vs, kernel_chunk(chunk, dt), dt == KDA_F32)) return KDA_ERR_UNSUPPORTED;
    if (sl <= 0 || sl + sh >= T) {
        sl = T > 0 ? T : chunk;
        sh = 0;
    }
    const long long ns = T > 0 ? segment_count(T, sl, sh) : 1;
    if (ns > (1 << 20)) return KDA_ERR_UNSUPPORTED;
    // every launch of a split counts its units (b, h, segment, slice) in an int
    if ((long long)B * H * ns * vs > (1LL << 30)) return KDA_ERR_UNSUPPORTED;
    *seg_len = sl;
    *n_seg = (int)ns;
    *n_vs = vs;
    if (shift) *shift = sh;
    return KDA_OK;
}

// Split workspace: transitions M [B*H, n_seg-1, dk, dk] (slot s for segment s; slot 0 unused),
// increments H [B*H, n_seg-1, dk, dv] (likewise), entry states S_in [B*H, n_seg, dk, dv] (slot s
// for segment s >= 1; slot 0 holds the last segment's increment), then the transition pass's
// chunk counts [B*H, n_seg-1, n_vs] int32 in a region sized for two column slices, padded to 16 bytes.
size_t workspace_for(int B, int H, int dk, int dv, int n_seg) {
    if (n_seg <= 1) return 0;
    const size_t bh = (size_t)B * H;
    const size_t mats = (size_t)(n_seg - 1) * ((size_t)dk * dk + (size_t)dk * dv) + (size_t)n_seg * dk * dv;
    const size_t counts = (bh * (size_t)(n_seg - 1) * 2 * sizeof(int) + 15) / 16 * 16;
    return bh * mats * sizeof(float) + counts;
}

// A launch description with every optional part off.
PrefillArgs blank_prefill_args() {
    PrefillArgs a;
    memset(&a, 0, sizeof(a));
    a.out_seg = -1;
    a.tail_seg = -1;
    return a;
}

kda_status_t prefill_entry(const void* q, const void* k, const void* v, const float* log_alpha, const void* gate,
                           bool gmode, const float* beta, const float* S0, void* o, float* S_T, int B, int T, int H, int dk,
                           int dv, int chunk, kda_dtype_t dt, int ckpt_every, float* S_ckpt, int seg_len,
                           int n_vs, void* workspace, size_t workspace_bytes, void* stream, bool side_ok = true);

}  // namespace

namespace kda {


bool prefill_supported(int dk, int dvw, int chunk, bool f32) {
    if (dk != 64 && dk != 128) return false;
    if (dvw != 64 && dvw != 128) return false;
    if (dvw > dk) return false;
    if (chunk != 16 && chunk != 32 && chunk != 64) return false;
    if (f32 && chunk == 64) return false;   // fp32 operands of a 64-token chunk exceed 160 KiB of LDS
    return true;
}

// Waves per workgroup of the single-role kernel: 8 for a 128-column bf16 slice at d_k = 128 (16
// columns per wave, two waves per SIMD), else 4.
int prefill_waves(int dk, int dvw, bool f32) {
    if (f32 || dk != 128 || dvw != 128) return 4;
    return kSliceWaves;
}

// Chunk waves of the two-role look-ahead kernel, or 0 when a launch does not run on it.  It takes
// bf16, d_k = d_v = 128 in one slice, 64-token chunks, no per-sequence lengths and real values.
static int pipe_chunk_waves(int dk, int dvw, int chunk, bool f32, const PrefillArgs& a) {
    const bool fits = !f32 && dk == 128 && dvw == 128 && chunk == 64 && a.n_vs == 1 && !a.lens &&
                      !a.zero_values && prefill_waves(dk, dvw, f32) == 8;
    return fits ? kPipeChunkWaves : 0;
}

hipError_t launch_prefill(int dk, int dvw, int chunk, bool f32, const PrefillArgs& a, hipStream_t s) {
    if (!prefill_supported(dk, dvw, chunk, f32)) return hipErrorInvalidValue;
    if (const int ncw = pipe_chunk_waves(dk, dvw, chunk, f32, a)) return launch_prefill_bf16_pipe(ncw, a, s);
    const int nw = prefill_waves(dk, dvw, f32);
    if (a.gate) return f32 ? hipErrorInvalidValue : launch_prefill_bf16_gate(dk, dvw, nw, chunk, false, a, s);
    return f32 ? launch_prefill_f32(dk, dvw, nw, chunk, a, s) : launch_prefill_bf16(dk, dvw, nw, chunk, a, s);
}

bool prefill_dual_supported(int dk, int dvw, int chunk, bool f32) {
    return prefill_supported(dk, dvw, chunk, f32) && !f32 && prefill_waves(dk, dvw, f32) == 8;
}

hipError_t launch_prefill_dual(int dk, int dvw, int chunk, bool f32, const PrefillArgs& a, hipStream_t s) {
    if (!prefill_dual_supported(dk, dvw, chunk, f32)) return hipErrorInvalidValue;
    if (a.gate) return launch_prefill_bf16_gate(dk, dvw, prefill_waves(dk, dvw, f32), chunk, true, a, s);
    return launch_prefill_bf16_dual(dk, dvw, prefill_waves(dk, dvw, f32), chunk, a, s);
}

}  // namespace kda

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(kda_status_t s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT: bad shape, NULL pointer, misalignment or overlap";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: head size, chunk or dtype not implemented";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
        case KDA_ERR_DEVICE: return "KDA_ERR_DEVICE: HIP runtime call or kernel launch failed";
    }
    return "KDA: unknown status";
}

kda_status_t kda_chunk_prefill_plan(int B, int T, int H, int dk, int dv, int chunk, kda_dtype_t dt,
                                    int* seg_len, int* n_vs) {
    const kda_status_t st = check_prefill_shape(B, T, H, dk, dv, chunk, dt);
    if (st != KDA_OK) return st;
    long long sl = 0;
    int ns = 0, vs = 0;
    const kda_status_t st2 = resolve_plan(B, T, H, dk, dv, chunk, dt, 0, 0, &sl, &ns, &vs, nullptr);
    if (st2 != KDA_OK) return st2;
    if (seg_len) *seg_len = (int)sl;
    if (n_vs) *n_vs = vs;
    return KDA_OK;
}

size_t kda_chunk_prefill_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk, kda_dtype_t dt) {
    return kda_chunk_prefill_workspace_bytes_ex(B, T, H, dk, dv, chunk, dt, 0);
}

size_t kda_chunk_prefill_workspace_bytes_ex(int B, int T, int H, int dk, int dv, int chunk, kda_dtype_t dt,
                                            int seg_len) {
    if (check_prefill_shape(B, T, H, dk, dv, chunk, dt) != KDA_OK) return 0;
    long long sl = 0;
    int ns = 0, vs = 0;
    if (resolve_plan(B, T, H, dk, dv, chunk, dt, seg_len, 0, &sl, &ns, &vs, nullptr) != KDA_OK) return 0;
    return workspace_for(B, H, dk, dv, ns);
}

kda_status_t kda_chunk_prefill_ex(const void* q, const void* k, const void* v, const float* log_alpha,
                                  const float* beta, const float* S0, void* o, float* S_T, int B, int T,
                                  int H, int dk, int dv, int chunk, kda_dtype_t dt, int seg_len, int n_vs,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    return kda_chunk_prefill_ckpt(q, k, v, log_alpha, beta, S0, o, S_T, B, T, H, dk, dv, chunk, dt, 0, nullptr,
                                  seg_len, n_vs, workspace, workspace_bytes, stream);
}

kda_status_t kda_chunk_prefill_ckpt(const void* q, const void* k, const void* v, const float* log_alpha,
                                    const float* beta, const float* S0, void* o, float* S_T, int B, int T,
                                    int H, int dk, int dv, int chunk, kda_dtype_t dt, int ckpt_every,
                                    float* S_ckpt, int seg_len, int n_vs, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    return prefill_entry(q, k, v, log_alpha, nullptr, false, beta, S0, o, S_T, B, T, H, dk, dv, chunk, dt, ckpt_every,
                         S_ckpt, seg_len, n_vs, workspace, workspace_bytes, stream);
}

kda_status_t kda_chunk_prefill_gate(const void* q, const void* k, const void* v, const void* gate,
                                    const float* beta, const float* S0, void* o, float* S_T, int B, int T,
                                    int H, int dk, int dv, int chunk, kda_dtype_t dt, int seg_len, int n_vs,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_entry(q, k, v, nullptr, gate, true, beta, S0, o, S_T, B, T, H, dk, dv, chunk, dt, 0, nullptr,
                         seg_len, n_vs, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Every prefill entry point: the decay input is log_alpha (fp32) or, with gmode, gate (bf16 raw
// gate pre-activation).  side_ok = false keeps a sequence split entirely on `stream` (segment 0
// inside the zero-start launch of the other segments; no stream or event of the library's).
kda_status_t prefill_entry(const void* q, const void* k, const void* v, const float* log_alpha, const void* gate,
                           bool gmode, const float* beta, const float* S0, void* o, float* S_T, int B, int T, int H, int dk,
                           int dv, int chunk, kda_dtype_t dt, int ckpt_every, float* S_ckpt, int seg_len,
                           int n_vs, void* workspace, size_t workspace_bytes, void* stream, bool side_ok) {
    kda_status_t st = check_prefill_shape(B, T, H, dk, dv, chunk, dt);
    if (st != KDA_OK) return st;
    if (gmode && (dt != KDA_BF16 || !kda::prefill_dual_supported(dk, dv, chunk, false)))
        return KDA_ERR_UNSUPPORTED;   // 8-wave bf16 shapes only
    if (gmode && n_vs > 1) return KDA_ERR_UNSUPPORTED;
    const void* decay_in = gmode ? gate : static_cast<const void*>(log_alpha);
    const size_t decay_esz = gmode ? 2 : sizeof(float);
    if (ckpt_every < 0 || (ckpt_every > 0 && ckpt_every % chunk != 0)) return KDA_ERR_INVALID_ARGUMENT;
    const int n_ckpt = ckpt_every > 0 ? T / ckpt_every : 0;
    long long sl = 0, shift = 0;
    int ns = 0, vs = 0;
    st = resolve_plan(B, T, H, dk, dv, chunk, dt, seg_len, n_vs, &sl, &ns, &vs, &shift);
    if (st != KDA_OK) return st;
    if (B == 0 || H == 0) return KDA_OK;
    chunk = kernel_chunk(chunk, dt);

    const size_t esz = dt == KDA_BF16 ? 2 : 4;
    const size_t ntok = (size_t)B * T * H;
    const size_t state_bytes = (size_t)B * H * dk * dv * sizeof(float);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);

    // pointers, alignment, aliasing
    if (S0 && !aligned(S0, 16)) return KDA_ERR_INVALID_ARGUMENT;
    if (S_T && !aligned(S_T, 16)) return KDA_ERR_INVALID_ARGUMENT;
    if (S0 && S_T && S0 != S_T && overlap(range_of(S0, state_bytes), range_of(S_T, state_bytes)))
        return KDA_ERR_INVALID_ARGUMENT;
    if (T > 0) {
        if (!q || !k || !v || !decay_in || !beta || !o) return KDA_ERR_INVALID_ARGUMENT;
        if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
            !aligned(decay_in, 16) || !aligned(beta, 4))
            return KDA_ERR_INVALID_ARGUMENT;
        const Range ins[] = {range_of(q, ntok * dk * esz), range_of(k, ntok * dk * esz),
                             range_of(v, ntok * dv * esz), range_of(decay_in, ntok * dk * decay_esz),
                             range_of(beta, ntok * sizeof(float))};
        const Range ro = range_of(o, ntok * dv * esz);
        for (const Range& r : ins) {
            if (overlap(ro, r)) return KDA_ERR_INVALID_ARGUMENT;
            if (S_T && overlap(range_of(S_T, state_bytes), r)) return KDA_ERR_INVALID_ARGUMENT;
        }
        if (S0 && overlap(ro, range_of(S0, state_bytes))) return KDA_ERR_INVALID_ARGUMENT;
        if (S_T && overlap(ro, range_of(S_T, state_bytes))) return KDA_ERR_INVALID_ARGUMENT;
    }
    if (n_ckpt > 0 && B > 0 && H > 0) {   // checkpoints: [B, n_ckpt, H, dk, dv], written only
        if (!S_ckpt || !aligned(S_ckpt, 16)) return KDA_ERR_INVALID_ARGUMENT;
        const Range rc = range_of(S_ckpt, (size_t)B * n_ckpt * H * dk * dv * sizeof(float));
        const Range others[] = {range_of(q, ntok * dk * esz), range_of(k, ntok * dk * esz),
                                range_of(v, ntok * dv * esz), range_of(decay_in, ntok * dk * decay_esz),
                                range_of(beta, ntok * sizeof(float)), range_of(o, ntok * dv * esz)};
        for (const Range& r : others)
            if (overlap(rc, r)) return KDA_ERR_INVALID_ARGUMENT;
        if (S0 && overlap(rc, range_of(S0, state_bytes))) return KDA_ERR_INVALID_ARGUMENT;
        if (S_T && overlap(rc, range_of(S_T, state_bytes))) return KDA_ERR_INVALID_ARGUMENT;
        if (workspace && overlap(rc, range_of(workspace, workspace_for(B, H, dk, dv, ns))))
            return KDA_ERR_INVALID_ARGUMENT;
    }
    const size_t need = workspace_for(B, H, dk, dv, ns);
    if (need > 0) {
        if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return KDA_ERR_WORKSPACE;
        const Range rw = range_of(workspace, need);
        if (overlap(rw, range_of(o, ntok * dv * esz))) return KDA_ERR_INVALID_ARGUMENT;
        if (S_T && overlap(rw, range_of(S_T, state_bytes))) return KDA_ERR_INVALID_ARGUMENT;
        if (S0 && overlap(rw, range_of(S0, state_bytes))) return KDA_ERR_INVALID_ARGUMENT;
    }

    (void)hipGetLastError();  // clear a stale error so a failure below is ours
    if (T == 0) {
        if (S_T && S_T != S0) {
            if (kda::launch_state_copy(S_T, S0, (long long)B * H * dk * dv, s) != hipSuccess)
                return KDA_ERR_DEVICE;
        }
        return KDA_OK;
    }

    const int dvw = dv / vs;
    const bool f32 = dt == KDA_F32;
    const long long SS = (long long)dk * dv;

    PrefillArgs a = blank_prefill_args();
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_alpha = log_alpha;
    a.gate = gate;
    a.beta = beta;
    a.T = T;
    a.B = B;
    a.H = H;
    a.seg_len = sl;
    a.n_vs = vs;

    if (ns == 1) {
        a.o = o;
        a.s_in = S0;
        a.sin_bh_stride = SS;
        a.sin_seg_stride = 0;
        a.init_mode = S0 ? 1 : 0;
        a.s_out = S_T;
        a.sout_bh_stride = SS;
        a.sout_seg_stride = 0;
        a.out_seg = -1;
        a.seg0 = 0;
        a.n_seg_launch = 1;
        a.n_units = B * H;
        a.zero_values = 0;
        if (n_ckpt > 0) {
            a.s_ckpt = S_ckpt;
            a.ckpt_every = ckpt_every;
            a.n_ckpt = n_ckpt;
        }
        if (kda::launch_prefill(dk, dvw, chunk, f32, a, s) != hipSuccess) return KDA_ERR_DEVICE;
        return KDA_OK;
    }

    // ---- sequence split ----
    // Segment s >= 1 depends on its entry state only through the transition M_s, and the entry
    // state's influence dies out along the segment: for unit keys and beta in [0, 2] every token's
    // transition (I - beta k k^T) Diag(alpha) is a contraction, and the decay shrinks it further.
    //  1. A transition pass over segments 1 .. ns-1 (identity start, zero values; for 8-wave shapes
    //     together with the increment H_s) stops once every entry of its transition has fallen below
    //     2^-126, stores the transition as zeros and records how many chunks it ran; a transition
    //     that never dies is formed over the whole segment (count -1).
    //  2. Segments 1 .. ns-1 run with outputs from a zero start (in the shared 8-wave pass, only
    //     those whose transition died: the others have their increment already); their final states
    //     are the increments H_s.  Segment 0 runs from S0 with its outputs, on a side stream beside
    //     steps 1-2, or inside step 2's launch; its final state is the entry state S_in(1).
    //  3. The scan S_in(s+1) = M_s S_in(s) + H_s, s = 1 .. ns-2.
    //  4. Each segment s >= 1 reruns from S_in(s) the chunks its transition pass counted (all of
    //     them for count -1), overwriting those outputs.
    // Past that count the entry state adds less than d_k 2^-126 times its own size to the state,
    // so the zero-start outputs stand (exact up to rounding); where the transition never dies, the
    // steps are the plain two-pass split.  Sources: "Kimi K3's architecture" (orkas.ai), "The bill
    // comes due in the serving stack" (transition and zero-start state combine across segments);
    // "Inside Kimi K3" (academa.ai lecture), sequence paragraph (the diagonal gate scales down
    // what the state keeps from earlier tokens).
    float* ws = reinterpret_cast<float*>(workspace);
    const long long bh = (long long)B * H;
    float* wsM = ws;
    float* wsH = wsM + bh * (ns - 1) * SS;
    float* wsSin = wsH + bh * (ns - 1) * SS;
    int* wsZ = reinterpret_cast<int*>(wsSin + bh * ns * SS);
    a.seg_shift = shift;
    a.n_seg_total = ns;
    const bool dual = kda::prefill_dual_supported(dk, dvw, chunk, f32);

    PrefillArgs pt = a;  // step 1: transitions of segments 1 .. ns-1, early stop
    pt.o = nullptr;
    pt.s_in = nullptr;
    pt.init_mode = 2;
    pt.zero_values = 1;
    pt.s_out = wsM;
    pt.sout_bh_stride = (long long)(ns - 1) * SS;
    pt.sout_seg_stride = SS;
    pt.out_seg = -1;
    pt.seg0 = 1;
    pt.n_seg_launch = ns - 1;
    pt.n_units = (int)(bh * (ns - 1));
    pt.probe = 1;
    pt.z_out = wsZ;
    pt.tail_seg = ns - 1;   // the last segment's transition and increment are not kept
    pt.s_tail = nullptr;
    if (dual) {   // with the increment: the decay and intra-chunk work is shared
        pt.init_mode = 0;
        pt.zero_values = 0;
        pt.s_out = wsH;
        pt.s_aux = wsM;
        pt.saux_bh_stride = (long long)(ns - 1) * SS;
        pt.saux_seg_stride = SS;
    }

    PrefillArgs pz = a;  // step 2: segments from a zero start with outputs; increments H_s
    pz.o = o;
    pz.s_in = S0;
    pz.sin_bh_stride = SS;
    pz.sin_seg_stride = 0;
    pz.init_mode = 0;
    pz.s_out = wsH;
    pz.sout_bh_stride = (long long)(ns - 1) * SS;
    pz.sout_seg_stride = SS;
    pz.out_seg = -1;
    pz.seg0 = 1;
    pz.n_seg_launch = ns - 1;
    pz.n_units = (int)(bh * (ns - 1));
    pz.z_in = wsZ;
    pz.z_gate = dual ? 1 : 0;
    pz.tail_seg = ns - 1;   // the last segment's increment goes to S_in slot 0
    pz.s_tail = wsSin;
    pz.stail_bh_stride = (long long)ns * SS;
    pz.s_head = wsSin + SS;   // segment 0's final state is S_in(1)
    pz.shead_bh_stride = (long long)ns * SS;
    if (n_ckpt > 0) {
        pz.s_ckpt = S_ckpt;
        pz.ckpt_every = ckpt_every;
        pz.n_ckpt = n_ckpt;
    }

    {
        // With a side stream, segment 0 (its own launch) overlaps steps 1-2: fork after the
        // caller's earlier work, join before the scan.  One host thread at a time per library, so
        // the shared fork/join events are recorded and waited in order.
        std::lock_guard<std::mutex> lock(g_side_mu);
        SideStream* side = side_ok ? side_stream() : nullptr;
        if (side) {
            if (hipEventRecord(side->fork, s) != hipSuccess || hipStreamWaitEvent(side->stream, side->fork, 0) != hipSuccess)
                return KDA_ERR_DEVICE;
            PrefillArgs p0 = pz;  // segment 0 alone, from S0
            p0.init_mode = S0 ? 1 : 0;
            p0.seg0 = 0;
            p0.n_seg_launch = 1;
            p0.n_units = (int)bh;
            p0.z_gate = 0;
            if (kda::launch_prefill(dk, dvw, chunk, f32, p0, side->stream) != hipSuccess) return KDA_ERR_DEVICE;
        } else {      // segment 0 joins step 2's launch
            pz.init_mode = S0 ? 3 : 0;
            pz.seg0 = 0;
            pz.n_seg_launch = ns;
            pz.n_units = (int)(bh * ns);
        }
        const hipError_t e1 = dual ? kda::launch_prefill_dual(dk, dvw, chunk, f32, pt, s)
                                   : kda::launch_prefill(dk, dvw, chunk, f32, pt, s);
        if (e1 != hipSuccess) return KDA_ERR_DEVICE;
        if (kda::launch_prefill(dk, dvw, chunk, f32, pz, s) != hipSuccess) return KDA_ERR_DEVICE;
        if (side) {
            if (hipEventRecord(side->join, side->stream) != hipSuccess || hipStreamWaitEvent(s, side->join, 0) != hipSuccess)
                return KDA_ERR_DEVICE;
        }
    }

    kda::ScanArgs sa;   // step 3
    sa.M = wsM;
    sa.Hinc = wsH;
    sa.S0 = S0;
    sa.S_in = wsSin;
    sa.BH = (int)bh;
    sa.n_seg = ns;
    sa.s_first = 1;   // S_in(1) was written by segment 0's pass
    sa.z = wsZ;
    sa.n_vs = vs;
    if (ns > 2 && kda::launch_scan(dk, sa, s) != hipSuccess) return KDA_ERR_DEVICE;

    PrefillArgs pf = a;  // step 4: segments 1 .. ns-1 from their entry states, as far as counted
    pf.o = o;
    pf.s_in = wsSin;
    pf.sin_bh_stride = (long long)ns * SS;
    pf.sin_seg_stride = SS;
    pf.init_mode = 1;
    pf.zero_values = 0;
    pf.s_out = S_T;
    pf.sout_bh_stride = SS;
    pf.sout_seg_stride = 0;
    pf.out_seg = ns - 1;
    pf.seg0 = 1;
    pf.n_seg_launch = ns - 1;
    pf.n_units = (int)(bh * (ns - 1));
    pf.z_in = wsZ;
    pf.z_limit = 1;
    pf.tail_seg = ns - 1;   // cut short: S_T is the last segment's increment
    pf.s_tail = wsSin;
    pf.stail_bh_stride = (long long)ns * SS;
    if (n_ckpt > 0) {
        pf.s_ckpt = S_ckpt;
        pf.ckpt_every = ckpt_every;
        pf.n_ckpt = n_ckpt;
    }
    if (kda::launch_prefill(dk, dvw, chunk, f32, pf, s) != hipSuccess) return KDA_ERR_DEVICE;
    return KDA_OK;
}

}  // namespace

namespace kda {

kda_status_t prefill_on_stream(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                               const float* S0, void* o, float* S_T, int B, int T, int H, int dk, int dv, int chunk,
                               kda_dtype_t dt, int seg_len, int n_vs, void* workspace, size_t workspace_bytes,
                               void* stream) {
    return prefill_entry(q, k, v, log_alpha, nullptr, false, beta, S0, o, S_T, B, T, H, dk, dv, chunk, dt, 0, nullptr,
                         seg_len, n_vs, workspace, workspace_bytes, stream, false);
}

}  // namespace kda

extern "C" {

kda_status_t kda_chunk_prefill(const void* q, const void* k, const void* v, const float* log_alpha,
                               const float* beta, const float* S0, void* o, float* S_T, int B, int T, int H,
                               int dk, int dv, int chunk, kda_dtype_t dt, void* workspace,
                               size_t workspace_bytes, void* stream) {
    return kda_chunk_prefill_ex(q, k, v, log_alpha, beta, S0, o, S_T, B, T, H, dk, dv, chunk, dt, 0, 0,
                                workspace, workspace_bytes, stream);
}

kda_status_t kda_spec_verify(const void* q, const void* k, const void* v, const float* log_alpha,
                             const float* beta, const float* S, void* o, int N, int m, int H, int dk, int dv,
                             kda_dtype_t dt, void* stream) {
    if (N < 0 || H < 0 || m < 1) return KDA_ERR_INVALID_ARGUMENT;
    if (N > 0 && H > 0 && !S) return KDA_ERR_INVALID_ARGUMENT;
    if (m > kSpecTokenLoopMax) {
        // a long block runs from S as one unsplit chunked prefill (one segment as long as the block,
        // so no workspace is needed); no state is written
        const int sc = spec_chunk(m, dt);
        const long long whole = ((long long)m + sc - 1) / sc * sc;
        if (whole > 0x7fffffffLL) return KDA_ERR_UNSUPPORTED;
        return kda_chunk_prefill_ex(q, k, v, log_alpha, beta, S, o, nullptr, N, m, H, dk, dv, sc, dt, (int)whole,
                                    0, nullptr, 0, stream);
    }
    const kda_status_t st = check_spec_pointers(q, k, v, log_alpha, beta, S, o, nullptr, N, m, H, dk, dv, dt);
    if (st != KDA_OK || N == 0 || H == 0) return st;
    (void)hipGetLastError();
    kda::DecodeArgs a;
    memset(&a, 0, sizeof(a));
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_alpha = log_alpha;
    a.beta = beta;
    a.S = const_cast<float*>(S);   // read only: write_state is 0
    a.o = o;
    a.NH = (long long)N * H;
    a.H = H;
    a.m = m;
    a.lens = nullptr;
    a.write_state = 0;
    if (kda::launch_decode(dk, dt == KDA_F32, a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
        return KDA_ERR_DEVICE;
    return KDA_OK;
}

kda_status_t kda_spec_commit(const void* q, const void* k, const void* v, const float* log_alpha,
                             const float* beta, float* S, const int* accepted, int N, int m, int H, int dk,
                             int dv, kda_dtype_t dt, void* stream) {
    if (N < 0 || H < 0 || m < 1) return KDA_ERR_INVALID_ARGUMENT;
    if (m <= kSpecTokenLoopMax) {
        const kda_status_t st0 =
            check_spec_pointers(q, k, v, log_alpha, beta, S, nullptr, accepted, N, m, H, dk, dv, dt);
        if (st0 != KDA_OK || N == 0 || H == 0) return st0;
        (void)hipGetLastError();
        kda::DecodeArgs d;
        memset(&d, 0, sizeof(d));
        d.q = q;
        d.k = k;
        d.v = v;
        d.log_alpha = log_alpha;
        d.beta = beta;
        d.S = S;
        d.o = nullptr;
        d.NH = (long long)N * H;
        d.H = H;
        d.m = m;
        d.lens = accepted;
        d.write_state = 1;
        if (kda::launch_decode(dk, dt == KDA_F32, d, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
            return KDA_ERR_DEVICE;
        return KDA_OK;
    }
    const int chunk = spec_chunk(m, dt);
    kda_status_t st = check_prefill_shape(N, m, H, dk, dv, chunk, dt);
    if (st != KDA_OK) return st;
    // one segment as long as the block: the commit never splits the sequence
    const long long whole = ((long long)m + chunk - 1) / chunk * chunk;
    if (whole > 0x7fffffffLL) return KDA_ERR_UNSUPPORTED;
    long long sl = 0;
    int ns = 0, vs = 0;
    st = resolve_plan(N, m, H, dk, dv, chunk, dt, (int)whole, 0, &sl, &ns, &vs, nullptr);
    if (st != KDA_OK) return st;
    if (ns != 1) return KDA_ERR_UNSUPPORTED;   // unreachable: seg_len >= m
    if (N == 0 || H == 0) return KDA_OK;
    if (!q || !k || !v || !log_alpha || !beta || !S || !accepted) return KDA_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(log_alpha, 16) || !aligned(S, 16) ||
        !aligned(beta, 4) || !aligned(accepted, 4))
        return KDA_ERR_INVALID_ARGUMENT;
    const size_t esz = dt == KDA_BF16 ? 2 : 4;
    const size_t ntok = (size_t)N * m * H;
    const Range rs = range_of(S, (size_t)N * H * dk * dv * sizeof(float));
    const Range ins[] = {range_of(q, ntok * dk * esz), range_of(k, ntok * dk * esz), range_of(v, ntok * dv * esz),
                         range_of(log_alpha, ntok * dk * sizeof(float)), range_of(beta, ntok * sizeof(float)),
                         range_of(accepted, (size_t)N * sizeof(int))};
    for (const Range& r : ins)
        if (overlap(rs, r)) return KDA_ERR_INVALID_ARGUMENT;

    (void)hipGetLastError();
    const long long SS = (long long)dk * dv;
    PrefillArgs a = blank_prefill_args();
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_alpha = log_alpha;
    a.beta = beta;
    a.o = nullptr;            // the outputs were produced by the verify call
    a.s_in = S;               // each workgroup reads its own columns of S before it writes them
    a.sin_bh_stride = SS;
    a.init_mode = 1;
    a.s_out = S;
    a.sout_bh_stride = SS;
    a.out_seg = -1;
    a.T = m;
    a.B = N;
    a.H = H;
    a.seg_len = m;
    a.n_seg_launch = 1;
    a.n_vs = vs;
    a.n_units = N * H;
    a.lens = accepted;
    if (kda::launch_prefill(dk, dv / vs, chunk, dt == KDA_F32, a, reinterpret_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return KDA_ERR_DEVICE;
    return KDA_OK;
}

kda_status_t kda_decode_step(const void* q, const void* k, const void* v, const float* log_alpha,
                             const float* beta, float* S, void* o, int N, int H, int dk, int dv,
                             kda_dtype_t dt, void* stream) {
    if (N < 0 || H < 0 || dk <= 0 || dv <= 0) return KDA_ERR_INVALID_ARGUMENT;
    if (dt != KDA_BF16 && dt != KDA_F32) return KDA_ERR_INVALID_ARGUMENT;
    if (dk != dv || (dk != 64 && dk != 128)) return KDA_ERR_UNSUPPORTED;
    long long nh = 0;
    if (!mul_ok(N, H, &nh)) return KDA_ERR_INVALID_ARGUMENT;
    if (nh == 0) return KDA_OK;
    if (!q || !k || !v || !log_alpha || !beta || !S || !o) return KDA_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(S, 16) ||
        !aligned(log_alpha, 16) || !aligned(beta, 4))
        return KDA_ERR_INVALID_ARGUMENT;
    const size_t esz = dt == KDA_BF16 ? 2 : 4;
    const Range ro = range_of(o, (size_t)nh * dv * esz);
    const Range rs = range_of(S, (size_t)nh * dk * dv * sizeof(float));
    const Range ins[] = {range_of(q, (size_t)nh * dk * esz), range_of(k, (size_t)nh * dk * esz),
                         range_of(v, (size_t)nh * dv * esz), range_of(log_alpha, (size_t)nh * dk * sizeof(float)),
                         range_of(beta, (size_t)nh * sizeof(float))};
    for (const Range& r : ins)
        if (overlap(ro, r) || overlap(rs, r)) return KDA_ERR_INVALID_ARGUMENT;
    if (overlap(ro, rs)) return KDA_ERR_INVALID_ARGUMENT;

    kda::DecodeArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_alpha = log_alpha;
    a.beta = beta;
    a.S = S;
    a.o = o;
    a.NH = nh;
    a.H = H;
    a.m = 1;
    a.lens = nullptr;
    a.write_state = 1;
    (void)hipGetLastError();
    if (kda::launch_decode(dk, dt == KDA_F32, a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
        return KDA_ERR_DEVICE;
    return KDA_OK;
}

}  // extern "C"
