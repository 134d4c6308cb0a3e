// Sequential arms of the KDA / GDN mixer for gfx950 (wave64).
//
// Fused arm: one workgroup of 8*D threads per (sequence, head) runs the whole path
// for all T tokens - conv + SiLU (q, k, v), l2 (q, k), the delta-rule scan on
// register-resident state, the gated RMSNorm, and the ring roll - so decode is a
// single kernel that streams each 64 KiB head state from HBM once and back once.
//
// Split arm (prefill with few (b, h) pairs): a pre-kernel over (b, h, 32-token
// block) writes the conv/l2 results to the workspace, a scan kernel splits each
// head's value columns over D/32 workgroups (the columns of the delta rule are
// independent given q, k, v, g, beta), and a norm kernel finishes the rows.
//
// Both arms call the same device helpers with the same lane mapping, so they are
// bit-identical to each other and to chained T = 1 calls.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int TB_FUSED = 4;   // tokens staged in LDS per pass of the fused kernel
constexpr int TB_PRE = 32;    // tokens per pre-kernel workgroup
constexpr int TB_SCAN = 32;   // tokens staged in LDS per pass of the split scan

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ------------------------------------------------------------------ fused arm
// Value columns per thread of the fused kernel at D = 128. Two columns (512
// threads, ~117 VGPRs, two workgroups per CU) measured fastest on the decode step:
// one column (1024 threads) keeps too little state in flight per CU, four or eight
// columns raise the register count until occupancy drops.
template <int D>
constexpr int fused_cpt() { return D >= 128 ? 2 : 1; }
template <int D>
constexpr int fused_threads() { return 8 * D / fused_cpt<D>(); }

template <int D, bool BF, bool GDN>
__global__ __launch_bounds__(fused_threads<D>()) void seq_fused_kernel(MixerArgs a) {
    constexpr int CPT = fused_cpt<D>();
    constexpr int NT = fused_threads<D>();
    constexpr int NG = NT / 8;  // 8-lane column groups; column of (group g, slot c) = g + c*NG
    constexpr int NW = NT / 64;
    constexpr int KPL = D / 8;
    constexpr int EW = GDN ? 1 : D;
    __shared__ float pre[3][TB_FUSED][D];  // conv outputs q, k, v (q, k l2-normalised in place)
    __shared__ float es[TB_FUSED][EW];     // exp(g)
    __shared__ float os[TB_FUSED][D];      // scan readout
    __shared__ float bs[TB_FUSED], kqs[TB_FUSED];
    __shared__ float wins[3 * D][KMAX - 1];  // conv windows between token blocks

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
    const int H = a.H, T = a.T, K = a.K;
    const size_t qkv = (size_t)H * D;
    const size_t head_off = (size_t)h * D;
    const int grp = wave * 8 + (lane >> 3), s = lane & 7;

    // Issue the state loads first so their HBM latency overlaps the conv / l2 work.
    float S[CPT][KPL];
#pragma unroll
    for (int c = 0; c < CPT; ++c)
        load_keys<D>(S[c], a.state_in + ((size_t)bh * D + grp + c * NG) * D, s);

    // The gate column of this thread is fixed (NT is a multiple of D); its activation
    // parameters arrive with the ring rows, which are waited for right below (read
    // before the state, their pointers' scalar load would hold the state loads back).
    static_assert(NT % D == 0, "one gate column per thread");
    const GateCol gp = gate_col(a, h, GDN ? h : head_off + tid % D);

    // Conv windows of this head's 3*D (plane, channel) rows start as the old ring.
    for (int r = tid; r < 3 * D; r += NT) {
        const int plane = r / D, ch = r % D;
        const float* ring_row = a.ring + ((size_t)b * 3 * qkv + plane * qkv + head_off + ch) * (K - 1);
        ConvChannel cc;
        conv_window_from_ring(cc, ring_row, K);
#pragma unroll
        for (int e = 0; e < KMAX - 1; ++e) wins[r][e] = cc.win[e];
    }

    for (int t0 = 0; t0 < T; t0 += TB_FUSED) {
        const int nt = min(TB_FUSED, T - t0);
        const size_t row0 = (size_t)b * a.tp + t0;  // tp == T whenever the readout is produced
        for (int r = tid; r < 3 * D; r += NT) {
            const int plane = r / D, ch = r % D;
            const void* xsrc = plane == 0 ? a.q : (plane == 1 ? a.k : a.v);
            ConvChannel cc;
            conv_load_taps(cc, a.conv_w + (plane * qkv + head_off + ch) * K, K);
#pragma unroll
            for (int e = 0; e < KMAX - 1; ++e) cc.win[e] = wins[r][e];
            for (int tt = 0; tt < nt; ++tt) {
                const float x = ld_act<BF>(xsrc, (row0 + tt) * qkv + head_off + ch);
                pre[plane][tt][ch] = silu_f(conv_push(cc, x));
            }
#pragma unroll
            for (int e = 0; e < KMAX - 1; ++e) wins[r][e] = cc.win[e];
        }
        if constexpr (GDN) {
            if (tid < nt) es[tid][0] = exp_f(gate_in(a, gp, ld_act<BF>(a.g, (row0 + tid) * H + h)));
        } else {
            for (int idx = tid; idx < nt * D; idx += NT) {
                const int tt = idx / D, i = idx % D;
                es[tt][i] = exp_f(gate_in(a, gp, ld_act<BF>(a.g, (row0 + tt) * qkv + head_off + i)));
            }
        }
        if (tid < nt) bs[tid] = beta_in(a, ld_act<BF>(a.beta, (row0 + tid) * H + h));
        __syncthreads();
        for (int tt = wave; tt < nt; tt += NW) l2_qk_row<D>(pre[0][tt], pre[1][tt], lane, &kqs[tt]);
        __syncthreads();
        for (int tt = 0; tt < nt; ++tt) {
            float vj[CPT], o[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) vj[c] = pre[2][tt][grp + c * NG];
            scan_step_cols<D, GDN, CPT>(S, pre[0][tt], pre[1][tt], es[tt], vj, bs[tt], kqs[tt],
                                        a.scale, s, o);
            if (s == 0) {
#pragma unroll
                for (int c = 0; c < CPT; ++c) os[tt][grp + c * NG] = o[c];
            }
        }
        __syncthreads();
        if (a.readout) {
            for (int tt = wave; tt < nt; tt += NW) {
                const size_t off = (row0 + tt) * qkv + head_off;
                const GateRow gz = load_gate_row<D, BF>(a, off, lane);
                gated_rmsnorm_row<D, BF, GDN>(os[tt], gz, a, off, lane, a.o_core);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int c = 0; c < CPT; ++c)
        store_keys<D>(a.state_out + ((size_t)bh * D + grp + c * NG) * D, S[c], s);
    // Each ring row was read only by this workgroup (window init); the windows now hold
    // the last K-1 raw inputs of [old ring ++ x].
    for (int r = tid; r < 3 * D; r += NT) {
        const int plane = r / D, ch = r % D;
        float* ring_row = a.ring + ((size_t)b * 3 * qkv + plane * qkv + head_off + ch) * (K - 1);
        ConvChannel cc;
#pragma unroll
        for (int e = 0; e < KMAX - 1; ++e) cc.win[e] = wins[r][e];
        conv_window_to_ring(cc, ring_row, K);
    }
}

// ------------------------------------------------------------------ split arm
template <int D>
constexpr int pre_threads() { return ((3 * D + 63) / 64) * 64; }

template <int D, bool BF, bool GDN>
__global__ __launch_bounds__(pre_threads<D>()) void pre_kernel(MixerArgs a, float* qh, float* kh,
                                                               float* vh, float* eg, float* kqv) {
    constexpr int NT = pre_threads<D>();
    constexpr int NW = NT / 64;
    __shared__ float pre[3][TB_PRE][D];
    __shared__ float kqs[TB_PRE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
    const int H = a.H, T = a.T, K = a.K;
    const int t0 = blockIdx.y * TB_PRE;
    const int nt = min(TB_PRE, T - t0);
    const size_t qkv = (size_t)H * D;
    const size_t head_off = (size_t)h * D;
    const size_t row0 = (size_t)b * T + t0;      // workspace rows
    const size_t rin0 = (size_t)b * a.tp + t0;   // input rows

    static_assert(NT % D == 0, "one gate column per thread");
    const GateCol gp = gate_col(a, h, GDN ? h : head_off + tid % D);
    const bool conv_thread = tid < 3 * D;
    const int plane = tid / D, ch = tid % D;
    const size_t cf = (size_t)plane * qkv + head_off + ch;
    float* ring_row = a.ring + ((size_t)b * 3 * qkv + cf) * (K - 1);
    const void* xsrc = plane == 0 ? a.q : (plane == 1 ? a.k : a.v);
    auto raw_at = [&](int pos) -> float {  // x~[K-1+pos]: raw input at token pos (< 0: ring)
        return pos >= 0 ? ld_act<BF>(xsrc, ((size_t)b * a.tp + pos) * qkv + head_off + ch)
                        : ring_row[pos + K - 1];
    };
    if (conv_thread) {
        ConvChannel cc;
        conv_load_taps(cc, a.conv_w + cf * K, K);
#pragma unroll
        for (int d = 1; d < KMAX; ++d) cc.win[KMAX - 1 - d] = (d <= K - 1) ? raw_at(t0 - d) : 0.0f;
        for (int tt = 0; tt < nt; ++tt)
            pre[plane][tt][ch] = silu_f(conv_push(cc, ld_act<BF>(xsrc, (rin0 + tt) * qkv + head_off + ch)));
        // Only the first token block reads the old ring (TB_PRE >= KMAX - 1), so it
        // alone rolls it, after its own reads: new slot K-1-d = raw input at T-d.
        if (blockIdx.y == 0) {
            float nr[KMAX - 1];
#pragma unroll
            for (int d = 1; d < KMAX; ++d) nr[KMAX - 1 - d] = (d <= K - 1) ? raw_at(T - d) : 0.0f;
#pragma unroll
            for (int d = 1; d < KMAX; ++d)
                if (d <= K - 1) ring_row[K - 1 - d] = nr[KMAX - 1 - d];
        }
    }
    if constexpr (GDN) {
        if (tid < nt) eg[(row0 + tid) * H + h] = exp_f(gate_in(a, gp, ld_act<BF>(a.g, (rin0 + tid) * H + h)));
    } else {
        for (int idx = tid; idx < nt * D; idx += NT) {
            const size_t col = head_off + idx % D;
            eg[(row0 + idx / D) * qkv + col] = exp_f(gate_in(a, gp, ld_act<BF>(a.g, (rin0 + idx / D) * qkv + col)));
        }
    }
    __syncthreads();
    for (int tt = wave; tt < nt; tt += NW) l2_qk_row<D>(pre[0][tt], pre[1][tt], lane, &kqs[tt]);
    __syncthreads();
    for (int idx = tid; idx < nt * D; idx += NT) {
        const int tt = idx / D, i = idx % D;
        const size_t off = (row0 + tt) * qkv + head_off + i;
        qh[off] = pre[0][tt][i];
        kh[off] = pre[1][tt][i];
        vh[off] = pre[2][tt][i];
    }
    if (tid < nt) kqv[(row0 + tid) * H + h] = kqs[tid];
}

template <int D>
constexpr int split_cols() { return D < 32 ? D : 32; }

template <int D, bool BF, bool GDN>
__global__ __launch_bounds__(8 * split_cols<D>()) void scan_split_kernel(
    MixerArgs a, const float* qh, const float* kh, const float* vh, const float* eg,
    const float* kqv, float* o) {
    constexpr int COLS = split_cols<D>();
    constexpr int NS = D / COLS;
    constexpr int NT = 8 * COLS;
    constexpr int KPL = D / 8;
    constexpr int EW = GDN ? 1 : D;
    __shared__ float qs[TB_SCAN][D], ks[TB_SCAN][D], es[TB_SCAN][EW];
    __shared__ float vs[TB_SCAN][COLS], os[TB_SCAN][COLS];
    __shared__ float bs[TB_SCAN], kqs[TB_SCAN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bh = blockIdx.x / NS, split = blockIdx.x % NS;
    const int b = bh / a.H, h = bh % a.H;
    const int H = a.H, T = a.T;
    const size_t qkv = (size_t)H * D;
    const size_t head_off = (size_t)h * D;
    const int jl = wave * 8 + (lane >> 3), s = lane & 7;
    const int j = split * COLS + jl;

    float S[1][KPL];
    load_keys<D>(S[0], a.state_in + ((size_t)bh * D + j) * D, s);

    for (int t0 = 0; t0 < T; t0 += TB_SCAN) {
        const int nt = min(TB_SCAN, T - t0);
        const size_t row0 = (size_t)b * T + t0;
        for (int idx = tid; idx < nt * D; idx += NT) {
            const int tt = idx / D, i = idx % D;
            const size_t off = (row0 + tt) * qkv + head_off + i;
            qs[tt][i] = qh[off];
            ks[tt][i] = kh[off];
            if constexpr (!GDN) es[tt][i] = eg[off];
        }
        for (int idx = tid; idx < nt * COLS; idx += NT) {
            const int tt = idx / COLS, c = idx % COLS;
            vs[tt][c] = vh[(row0 + tt) * qkv + head_off + split * COLS + c];
        }
        if (tid < nt) {
            const size_t hr = (row0 + tid) * H + h;
            bs[tid] = beta_in(a, ld_act<BF>(a.beta, ((size_t)b * a.tp + t0 + tid) * H + h));
            kqs[tid] = kqv[hr];
            if constexpr (GDN) es[tid][0] = eg[hr];
        }
        __syncthreads();
        for (int tt = 0; tt < nt; ++tt) {
            const float vj[1] = {vs[tt][jl]};
            float ov[1];
            scan_step_cols<D, GDN, 1>(S, qs[tt], ks[tt], es[tt], vj, bs[tt], kqs[tt], a.scale, s, ov);
            if (s == 0) os[tt][jl] = ov[0];
        }
        __syncthreads();
        for (int idx = tid; idx < nt * COLS; idx += NT) {
            const int tt = idx / COLS, c = idx % COLS;
            o[(row0 + tt) * qkv + head_off + split * COLS + c] = os[tt][c];
        }
    }
    store_keys<D>(a.state_out + ((size_t)bh * D + j) * D, S[0], s);
}

// One wavefront per (b, t, h) row.
template <int D, bool BF, bool GDN>
__global__ __launch_bounds__(256) void norm_kernel(MixerArgs a, const float* o) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const size_t rows = (size_t)a.B * a.T * a.H;
    const size_t row = (size_t)blockIdx.x * 4 + wave;
    if (row >= rows) return;
    const size_t off = (row / a.H) * ((size_t)a.H * D) + (row % a.H) * D;
    const GateRow gz = load_gate_row<D, BF>(a, off, lane);
    gated_rmsnorm_row<D, BF, GDN>(o + off, gz, a, off, lane, nullptr);
}

template <int D, bool BF, bool GDN>
hipError_t fused_launch(const MixerArgs& a) {
    hipLaunchKernelGGL((seq_fused_kernel<D, BF, GDN>), dim3(a.B * a.H), dim3(fused_threads<D>()), 0,
                       a.stream, a);
    return hipGetLastError();
}

template <int D, bool BF, bool GDN>
hipError_t split_launch(const MixerArgs& a) {
    const SplitWorkspace w = split_workspace(a.B, a.T, a.H, a.D, a.gdn);
    char* base = static_cast<char*>(a.ws);
    float* qh = reinterpret_cast<float*>(base + w.qh);
    float* kh = reinterpret_cast<float*>(base + w.kh);
    float* vh = reinterpret_cast<float*>(base + w.vh);
    float* eg = reinterpret_cast<float*>(base + w.eg);
    float* kq = reinterpret_cast<float*>(base + w.kq);
    float* o = a.o_core ? a.o_core : reinterpret_cast<float*>(base + w.o);
    const int nblk = (a.T + TB_PRE - 1) / TB_PRE;
    hipLaunchKernelGGL((pre_kernel<D, BF, GDN>), dim3(a.B * a.H, nblk), dim3(pre_threads<D>()), 0,
                       a.stream, a, qh, kh, vh, eg, kq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int NS = D / split_cols<D>();
    hipLaunchKernelGGL((scan_split_kernel<D, BF, GDN>), dim3(a.B * a.H * NS), dim3(8 * split_cols<D>()),
                       0, a.stream, a, qh, kh, vh, eg, kq, o);
    e = hipGetLastError();
    if (e != hipSuccess || !a.readout) return e;
    const size_t rows = (size_t)a.B * a.T * a.H;
    hipLaunchKernelGGL((norm_kernel<D, BF, GDN>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                       a.stream, a, o);
    return hipGetLastError();
}

template <int D, bool BF, bool GDN>
struct FusedOp {
    static hipError_t run(const MixerArgs& a) { return fused_launch<D, BF, GDN>(a); }
};
template <int D, bool BF, bool GDN>
struct SplitOp {
    static hipError_t run(const MixerArgs& a) { return split_launch<D, BF, GDN>(a); }
};

template <template <int, bool, bool> class Op>
hipError_t dispatch(const MixerArgs& a) {
    if (a.D == 128) {
        if (a.bf16) return a.gdn ? Op<128, true, true>::run(a) : Op<128, true, false>::run(a);
        return a.gdn ? Op<128, false, true>::run(a) : Op<128, false, false>::run(a);
    }
    if (a.D == 16) {
        if (a.bf16) return a.gdn ? Op<16, true, true>::run(a) : Op<16, true, false>::run(a);
        return a.gdn ? Op<16, false, true>::run(a) : Op<16, false, false>::run(a);
    }
    return hipErrorInvalidValue;
}

}  // namespace

SplitWorkspace split_workspace(int B, int T, int H, int D, bool gdn) {
    const size_t act = align256((size_t)B * T * H * D * 4);
    const size_t per_head = align256((size_t)B * T * H * 4);
    SplitWorkspace w;
    w.qh = 0;
    w.kh = w.qh + act;
    w.vh = w.kh + act;
    w.eg = w.vh + act;
    w.kq = w.eg + (gdn ? per_head : act);
    w.o = w.kq + per_head;
    w.total = w.o + act;
    return w;
}

hipError_t launch_seq_fused(const MixerArgs& a) { return dispatch<FusedOp>(a); }

hipError_t launch_norm(const MixerArgs& a, const float* o) {
    const size_t rows = (size_t)a.B * a.T * a.H;
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    if (a.D == 128) {
        if (a.bf16) {
            if (a.gdn) hipLaunchKernelGGL((norm_kernel<128, true, true>), grid, block, 0, a.stream, a, o);
            else hipLaunchKernelGGL((norm_kernel<128, true, false>), grid, block, 0, a.stream, a, o);
        } else {
            if (a.gdn) hipLaunchKernelGGL((norm_kernel<128, false, true>), grid, block, 0, a.stream, a, o);
            else hipLaunchKernelGGL((norm_kernel<128, false, false>), grid, block, 0, a.stream, a, o);
        }
    } else if (a.D == 16) {
        if (a.bf16) {
            if (a.gdn) hipLaunchKernelGGL((norm_kernel<16, true, true>), grid, block, 0, a.stream, a, o);
            else hipLaunchKernelGGL((norm_kernel<16, true, false>), grid, block, 0, a.stream, a, o);
        } else {
            if (a.gdn) hipLaunchKernelGGL((norm_kernel<16, false, true>), grid, block, 0, a.stream, a, o);
            else hipLaunchKernelGGL((norm_kernel<16, false, false>), grid, block, 0, a.stream, a, o);
        }
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
hipError_t launch_seq_split(const MixerArgs& a) { return dispatch<SplitOp>(a); }

}  // namespace kda
