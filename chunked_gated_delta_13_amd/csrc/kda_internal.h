// Host <-> kernel interface inside libkda (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/kda.h"

namespace kda {

// One launch of the fused chunk kernel over units (b, h, segment, column slice).
struct PrefillArgs {
    const void* q;            // [B, T, H, DK]   bf16 or fp32
    const void* k;            // [B, T, H, DK]
    const void* v;            // [B, T, H, DK]   (d_v == d_k)
    const float* log_alpha;   // [B, T, H, DK]   (nullptr in the gate mode)
    const float* beta;        // [B, T, H]
    void* o;                  // [B, T, H, DK] or nullptr (no output)
    const void* gate;         // [B, T, H, DK] bf16 raw gate pre-activation, or nullptr

    // initial state of a unit (b, h, s): s_in + bh * sin_bh_stride + s * sin_seg_stride
    const float* s_in;
    long long sin_bh_stride;
    long long sin_seg_stride;
    int init_mode;            // 0: zeros, 1: load from s_in, 2: identity columns, 3: segment 0
                              // loads s_in (its entry state), later segments start at zero

    // final state of a unit, written when out_seg < 0 or s == out_seg
    float* s_out;
    long long sout_bh_stride;
    long long sout_seg_stride;
    int out_seg;

    long long T;              // tokens per sequence
    int B, H;
    long long seg_len;        // tokens per segment
    long long seg_shift;      // extra tokens of segment 0: segment s >= 1 starts at s * seg_len + seg_shift
    int seg0;                 // first segment index of this launch
    int n_seg_launch;         // segments per (b, h) in this launch
    int n_vs;                 // state-column slices per unit
    int n_units;              // B * H * n_seg_launch
    int zero_values;          // 1: treat v as zeros (transition pass)

    // dual pass (launch_prefill_dual): s_out receives each unit's increment (zero start, real
    // values) and s_aux its transition (identity columns, zero values); no output rows
    float* s_aux;
    long long saux_bh_stride;
    long long saux_seg_stride;

    // per-sequence token counts (device, [B]; clamped to [0, T]) or nullptr: sequence b then
    // stops after lens[b] tokens, and its final state is the state after those tokens
    const int* lens;

    // checkpoints [B, n_ckpt, H, DK, DK] or nullptr: the state after every ckpt_every tokens
    // (a multiple of the chunk), i.e. after tokens ckpt_every * (i + 1), i < n_ckpt
    float* s_ckpt;
    int ckpt_every;
    int n_ckpt;

    // ---- short cut of the sequence split: an entry state's influence dies out ----
    // Chunk counts per (b, h, segment s >= 1, column slice) at
    //   z[((bh * (n_seg_total - 1)) + s - 1) * n_vs + vs]:
    // the chunks a transition pass ran before every entry of its transition columns fell below
    // 2^-126 (it then stops and stores the transition as zeros), or -1 if they never did.
    int probe;                // 1: this transition pass stops early and writes z_out
    int* z_out;
    const int* z_in;          // counts of an earlier probe, read by the gate and the limit
    int z_gate;               // 1: skip a unit s >= 1 whose count is -1 (the probe formed its increment)
    int z_limit;              // 1: a unit s >= 1 runs only its count of chunks (all of them when -1)
    int n_seg_total;          // segments per (b, h) of the whole split
    // final state of the last segment (tail_seg): written to s_tail instead of s_out, or, with
    // z_limit, copied from s_tail to s_out when the unit was cut short
    float* s_tail;
    long long stail_bh_stride;
    int tail_seg;             // -1: none
    // final state of segment 0, when set: written to s_head instead of s_out
    float* s_head;
    long long shead_bh_stride;
};

struct ScanArgs {
    const float* M;           // [B*H, n_seg-1, DK, DK]
    const float* Hinc;        // [B*H, n_seg-1, DK, DK]
    const float* S0;          // [B*H, DK, DK] or nullptr
    float* S_in;              // [B*H, n_seg, DK, DK]  (out; with s_first = 1, S_in(1) is an input)
    int BH;
    int n_seg;
    int s_first;              // 0: start from S0; 1: start from S_in(1), already in place
    // the transition pass's chunk counts (layout as in PrefillArgs, n_seg segments) or nullptr:
    // a step whose transition died (count >= 0, stored as zeros) is S_in(s+1) = H_s, no product
    const int* z;
    int n_vs;
};

// Decode step (m = 1) or a block of m <= kDecodeMaxTokens tokens per (sequence, head) run from
// the state on chip.
constexpr int kDecodeMaxTokens = 16;
struct DecodeArgs {
    const void* q;            // [N, m, H, DK]
    const void* k;
    const void* v;            // [N, m, H, DK]
    const float* log_alpha;   // [N, m, H, DK]
    const float* beta;        // [N, m, H]
    float* S;                 // [N, H, DK, DK]
    void* o;                  // [N, m, H, DK] or nullptr (no outputs)
    long long NH;             // N * H
    int H;
    int m;                    // tokens per block
    const int* lens;          // per-sequence token counts (device, clamped to [0, m]) or nullptr
    int write_state;          // 1: write the state after the block back to S
};

// dvw = state columns per workgroup (d_v / column slices).
bool prefill_supported(int dk, int dvw, int chunk, bool f32);
// Waves per workgroup that launch_prefill uses for a slice of dvw state columns.
int prefill_waves(int dk, int dvw, bool f32);
hipError_t launch_prefill(int dk, int dvw, int chunk, bool f32, const PrefillArgs& a,
                          hipStream_t stream);
// Transition and increment of every unit in one pass (shapes with 8-wave workgroups only).
bool prefill_dual_supported(int dk, int dvw, int chunk, bool f32);
hipError_t launch_prefill_dual(int dk, int dvw, int chunk, bool f32, const PrefillArgs& a,
                               hipStream_t stream);
hipError_t launch_scan(int dk, const ScanArgs& a, hipStream_t stream);
hipError_t launch_decode(int dk, bool f32, const DecodeArgs& a, hipStream_t stream);
// dst[i] = src ? src[i] : 0 for n floats
hipError_t launch_state_copy(float* dst, const float* src, long long n, hipStream_t stream);

// kda_chunk_prefill_ex with every launch of a sequence split on `stream` itself (no second stream
// of the library, nothing created or allocated); the workspace is the caller's.
kda_status_t prefill_on_stream(const void* q, const void* k, const void* v, const float* log_alpha, const float* beta,
                               const float* S0, void* o, float* S_T, int B, int T, int H, int dk, int dv, int chunk,
                               kda_dtype_t dt, int seg_len, int n_vs, void* workspace, size_t workspace_bytes,
                               void* stream);

}  // namespace kda
