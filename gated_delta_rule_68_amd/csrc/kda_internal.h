// Private interface between the host entry points (kda_api.cpp) and the HIP
// kernels. Nothing here is part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Everything one mixer call needs, already validated by the host entry point.
struct MixerArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    const float* conv_w;
    float* ring;
    const float* state_in;
    float* state_out;
    const void* z;
    const float* norm_w;
    void* out;
    float* o_core;  // may be null
    int B, T, H, D, K;
    float scale, rms_eps;
    bool bf16;  // activations are bf16 (else fp32)
    bool gdn;   // scalar gate per (token, head) and SiLU output gate
    void* ws;
    size_t ws_bytes;
    hipStream_t stream;
    // Rows of each sequence in memory for the activation inputs (q, k, v, g, beta):
    // T except for a rollback replay, which walks the first T of tp stored rows.
    int tp;
    // Whether the readout (z, norm_w in; out, o_core out) is produced; a rollback
    // replay only rebuilds the state and the ring (the sequential arms honour it).
    bool readout;
    // Gate activation (GATE_*): GATE_GIVEN means g and beta hold the log gate and beta;
    // otherwise they hold their pre-activations and every arm applies the activation
    // in fp32 as it reads them.
    int gate_form;
    const float* gate_a;     // [H]: A_log (GATE_SIGMOID) or the multiplier a (GATE_SOFTPLUS)
    const float* gate_bias;  // [H*D] (KDA) or [H] (GDN)
    float gate_lb;           // lower bound of the log gate
    // Query / key heads (GDN grouped heads; H for KDA and plain GDN). H is the number
    // of value heads, a multiple of Hk, and value head h reads query / key head
    // h % Hk. q and k rows are Hk*D wide; v, z, out, o_core rows H*D; the conv
    // weight and ring planes are q (Hk*D rows), k (Hk*D), v (H*D), in that order.
    int Hk;
    // Packed variable-length batch (null: B sequences of T rows each). Sequence b holds
    // rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of the [T][...] activations, T being the
    // total row count; its ring and state slots are b as usual.
    const int* cu_seqlens;
    // Packed batches: the sequences longest first (a permutation of 0..B-1 written by
    // launch_seq_order), so that the first workgroups dispatched take the longest work;
    // null: in index order.
    const int* seq_order;
    // Segmented chunked prefill (ARM_SEGMENTED): segment count, rows of segment 0 and
    // of the others (seg_plan), the pass a launch runs (1 or 3) and the workspace
    // holding the segment states (SegLayout).
    int seg_n, seg_len0, seg_len, seg_pass;
    float* seg_ws;
};

// Segmented chunked prefill. The state map of a run of tokens is affine in its
// entry state, S_out = M S_in + B: the recurrence's decay and delta-rule update act
// on the key index by left multiplication and add a term that does not depend on S.
// Each sequence is cut into n segments: segment 0 of len0 rows, then segments of len
// rows (the last one takes the rest). Pass 1 runs segment 0 from the given state
// and, for every middle segment s, the same tokens twice: from a zero state (its
// final state is B_s) and from the identity with v = 0 (its final state is M_s). A
// scan then forms the entry states S_{s+1} = M_s S_s + B_s, and pass 3 runs
// segments 1 .. n-1 from them with readout.
//
// One workgroup fills a compute unit. Pass 3 must fit one wave over the 256 units,
// (n-1) pairs <= 256. In pass 1 the pairs' segment-0 runs hold `pairs` units and the
// 2 (n-2) pairs middle runs take the other 256 - pairs units in r rounds (workgroups
// start in index order as units free up, the segment-0 runs first). The plan
// minimises the time of the critical path, pass 1 (the longer of segment 0 and r
// rounds of middle runs), the scan and pass 3, over n <= kSegMax and segment lengths
// (in 64-row units) of at least min_chunks units.
// - timed (AUTO): the cost model below, in hundredths of the time of one 32-row chunk
//   with readout on a fully loaded chip (measured on the 32-row kernel, KDA and GDN
//   alike). A run costs its chunks plus kSegRunFixed (its state load, the pipeline's
//   fill and drain and the final stores: 3 to 3.7 chunk times measured; the plans of
//   the measured workloads are the same anywhere in 2.5 .. 3.7); a chunk of a run
//   without readout costs kSegNoReadout of one with readout (the kernel leaves out the
//   query side, P, O and the gated norm there); a scan step costs kSegScanStep, and a
//   second round of middle runs starts kSegGap after the first round's runs end.
// - untimed (the explicit mode): 64-row units of the critical path, max(len0, r len)
//   + len, with no fixed costs, so short sequences still take several segments.
// The 64-row kernel (conv kernels of more than 4 taps) shares the plan.
constexpr int kSegMax = 32;
constexpr int kSegCUs = 256;
constexpr int kSegRunFixed = 370, kSegNoReadout = 69, kSegScanStep = 140, kSegGap = 40;
struct SegPlan {
    int n, len0, len;  // segment count; rows of segment 0 and of the others
    long cost;         // critical path (timed: hundredths of a 32-row chunk time; untimed: 64-row units)
};
// Critical path of the unsegmented chunked arm (one run of T rows) in the timed units.
__host__ __device__ inline long seg_chunked_cost(int T) { return (((long)T + 31) / 32) * 100 + kSegRunFixed; }
__host__ __device__ inline SegPlan seg_plan(long pairs, int T, int min_chunks, bool timed) {
    const long nch = ((long)T + 63) / 64;  // 64-row units
    SegPlan best{1, T, 0, timed ? seg_chunked_cost(T) : nch};
    if (min_chunks < 1) min_chunks = 1;
    if (pairs >= kSegCUs) return best;
    const long free_cu = kSegCUs - pairs;
    for (int n = 3; n <= kSegMax && (long)(n - 1) * pairs <= kSegCUs; ++n) {
        const long mid = 2 * pairs * (n - 2);
        const long r = (mid + free_cu - 1) / free_cu;
        if (!timed) {
            const long x0 = nch / (r + n - 1);
            for (long x = x0; x <= x0 + 1; ++x) {
                const long l0 = nch - (n - 1) * x;
                if (x < min_chunks || l0 < 1) continue;
                const long cost = (l0 > r * x ? l0 : r * x) + x;
                if (cost < best.cost) best = SegPlan{n, (int)(l0 * 64), (int)(x * 64), cost};
            }
            continue;
        }
        // x (units per segment after the first) that balances the two sides of pass 1
        const long x0 = (200 * nch + kSegRunFixed - r * kSegRunFixed - (r - 1) * kSegGap) /
                        (200 * (n - 1) + 2 * r * kSegNoReadout);
        for (long i = 0; i < 5; ++i) {  // around the balance, and the shortest segments
            const long x = i < 4 ? x0 - 1 + i : min_chunks;
            const long l0 = nch - (n - 1) * x;
            if (x < min_chunks || l0 < 1) continue;
            const long seg0 = 200 * l0 + kSegRunFixed;
            const long mids = r * (2 * kSegNoReadout * x + kSegRunFixed) + (r - 1) * kSegGap;
            const long cost = (seg0 > mids ? seg0 : mids) + (long)kSegScanStep * (n - 2) + 200 * x + kSegRunFixed;
            if (cost < best.cost) best = SegPlan{n, (int)(l0 * 64), (int)(x * 64), cost};
        }
    }
    return best;
}
// Byte offsets of the segmented arm's workspace: a zero block (also the zero v row of
// the M runs), the identity, a dummy output row for runs without readout, then the
// fp32 D x D state blocks [slot][pair] of S_1 .. S_{n-1}, M_1 .. M_{n-2},
// B_1 .. B_{n-2} (state layout [value][key]).
struct SegLayout {
    size_t zero, ident, dummy, slots, total;
};
__host__ __device__ inline SegLayout seg_layout(long pairs, int H, int D, int n) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t blk = (size_t)D * D * 4, row = (size_t)H * D * 4;
    SegLayout l;
    l.zero = 0;
    l.ident = al(blk > row ? blk : row);
    l.dummy = l.ident + al(blk);
    l.slots = l.dummy + al(row);
    const size_t nslot = n >= 2 ? (size_t)(n - 1) + 2 * (size_t)(n >= 3 ? n - 2 : 0) : 0;
    l.total = l.slots + nslot * (size_t)pairs * blk;
    return l;
}

// Sequence processed by the workgroups of dispatch rank r.
__device__ inline int seq_of(const MixerArgs& a, int r) { return a.seq_order ? a.seq_order[r] : r; }

// Activation rows of all sequences of a call.
__host__ __device__ inline size_t total_rows(const MixerArgs& a) {
    return a.cu_seqlens ? (size_t)a.T : (size_t)a.B * a.T;
}
// First row and row count of sequence b. Offsets of a packed batch are clamped into
// [0, T] and made non-decreasing, so a malformed table cannot send a kernel outside
// the activations (its results are then meaningless, but every access stays in bounds).
__device__ inline void seq_span(const MixerArgs& a, int b, size_t* start, int* len) {
    if (a.cu_seqlens) {
        const int s0 = min(max(a.cu_seqlens[b], 0), a.T);
        const int s1 = min(max(a.cu_seqlens[b + 1], s0), a.T);
        *start = (size_t)s0;
        *len = s1 - s0;
    } else {
        *start = (size_t)b * a.tp;
        *len = a.T;
    }
}

// Conv-weight / ring row of channel ch of plane (0 q, 1 k, 2 v) for value head h.
__host__ __device__ inline size_t plane_row(const MixerArgs& a, int plane, int h, int ch) {
    const size_t kw = (size_t)a.Hk * a.D;
    return plane < 2 ? plane * kw + (size_t)(h % a.Hk) * a.D + ch : 2 * kw + (size_t)h * a.D + ch;
}
// Whether the segmented arm's last segment writes the new conv ring itself, with no ring
// roll launch: the 32-row chunk kernel runs the arm (bf16, D = 128, K <= 4), the call
// has at least K-1 rows (the new ring is then input rows only) and at least two
// segments (the old ring's readers, the segment-0 runs of pass 1, have all finished when
// pass 3 writes it).
__host__ __device__ inline bool seg_ring_fused(const MixerArgs& a) {
    return a.bf16 && a.D == 128 && a.K <= 4 && a.T >= a.K - 1 && a.seg_n >= 2 && !a.cu_seqlens;
}
// Ring rows (= conv-weight rows) of one sequence.
__host__ __device__ inline size_t ring_rows(const MixerArgs& a) { return (size_t)(2 * a.Hk + a.H) * a.D; }

// Values of the KDA_GATE_* codes of the public header.
enum GateForm { GATE_GIVEN = 0, GATE_SIGMOID = 1, GATE_SOFTPLUS = 2 };

// Arms (values match the KDA_ARM_* codes of the public header).
enum Arm { ARM_SEQ_FUSED = 1, ARM_SEQ_SPLIT = 2, ARM_CHUNKED = 3, ARM_SEGMENTED = 4 };

// Workspace carve-up of the split sequential arm: fp32 arrays, each starting on a
// 256-byte boundary.
struct SplitWorkspace {
    size_t qh, kh, vh, eg, kq, o, total;  // byte offsets and total size
};
SplitWorkspace split_workspace(int B, int T, int H, int Hk, int D, bool gdn);

// Whether this build carries the chunked prefill arm.
extern const bool kChunkedArmBuilt;

// Workspace of the chunked arm: nseq sequences of H heads, rows activation rows in all.
size_t chunked_workspace_bytes(int nseq, size_t rows, int H, int D);

// Workspace of the segmented arm for B sequences of H heads cut into n segments.
size_t segmented_workspace_bytes(int B, int H, int D, int n);

// The static scratch buffer of the allocation-free prefill (kda_scratch.hip): its size,
// and its device address on the device of `stream` (looked up once per device).
size_t static_scratch_bytes();
hipError_t static_scratch(hipStream_t stream, void** ptr);

// Launchers: enqueue on a.stream, return the first launch error (hipSuccess if none).
hipError_t launch_seq_fused(const MixerArgs& a);
hipError_t launch_seq_split(const MixerArgs& a);
hipError_t launch_chunked(const MixerArgs& a);
// Segmented chunked prefill; a.seg_n / a.seg_len hold the plan and a.ws its
// workspace (seg_layout).
hipError_t launch_segmented(const MixerArgs& a);
// The 32-row chunk kernel (kda_c32.hip): bf16 activations, D = 128, K <= 4. The
// chunked and segmented arms run it wherever it fits, the 64-row kernel otherwise.
bool chunked32_fits(const MixerArgs& a);
hipError_t launch_chunked32(const MixerArgs& a);
// One pass of the segmented arm on the 32-row kernel (a.seg_pass, grid as planned).
hipError_t launch_seg_pass32(const MixerArgs& a, int grid);
// Gated RMSNorm of a fp32 pre-norm output o [B][T][H*D] into a.out.
hipError_t launch_norm(const MixerArgs& a, const float* o);
// Rank the B sequences of a packed batch by length, longest first (ties by index),
// into order[0..B-1].
hipError_t launch_seq_order(const MixerArgs& a, int* order);
// Roll every sequence's ring to the last K-1 raw rows of its T input rows (q, k and
// v planes, or with qk_only the q and k planes alone).
hipError_t launch_ring_roll(const MixerArgs& a, bool qk_only);

}  // namespace kda
