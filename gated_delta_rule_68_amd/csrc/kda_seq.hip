// Sequential arms of the KDA / GDN mixer for gfx950 (wave64).
//
// Fused arm: one workgroup of 8*D threads per (sequence, head) runs the whole path
// for all T tokens - conv + SiLU (q, k, v), l2 (q, k), the delta-rule scan on
// register-resident state, the gated RMSNorm, and the ring roll - so decode is a
// single kernel that streams each 64 KiB head state from HBM once and back once.
// A variant of it for calls of at most 16 tokens (seq_short_kernel) takes the decode
// step and short calls at D = 128.
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

// G value heads per workgroup: G = 1, one workgroup per (sequence, value head); G > 1
// (GDN with G = H / Hk), one workgroup per (sequence, key head) holding every value
// head of that key head, which convolves q / k once and rolls their ring rows itself.
// Each value head's NT1 threads map exactly as the G = 1 kernel's (same arithmetic).
template <int D, bool BF, bool GDN, int G = 1>
__global__ __launch_bounds__(fused_threads<D>() * G) void seq_fused_kernel(MixerArgs a) {
    static_assert(G == 1 || GDN, "grouped value heads are a GDN layout");
    constexpr int CPT = fused_cpt<D>();
    constexpr int NT1 = fused_threads<D>();  // threads per value head
    constexpr int NT = NT1 * G;
    constexpr int NG = NT1 / 8;  // 8-lane column groups; column of (group g, slot c) = g + c*NG
    constexpr int NW = NT / 64;
    constexpr int KPL = D / 8;
    constexpr int EW = GDN ? 1 : D;
    constexpr int NP = 2 + G;                   // conv planes: q, k, and the G value heads
    __shared__ float pre[NP][TB_FUSED][D];      // conv outputs q, k, v (q, k l2-normalised in place)
    __shared__ float es[TB_FUSED][G * EW];      // exp(g), value head hg at hg * EW
    __shared__ float os[TB_FUSED][G * D];       // scan readout
    __shared__ float bs[TB_FUSED][G], kqs[TB_FUSED];
    __shared__ float wins[NP * D][KMAX - 1];    // conv windows between token blocks

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hg = G == 1 ? 0 : tid / NT1;      // value head within the workgroup
    const int tl = G == 1 ? tid : tid % NT1;    // thread within the value head's threads
    const int HB = a.H / G;                     // workgroups per sequence
    const int hx = blockIdx.x % HB, b = seq_of(a, blockIdx.x / HB);
    auto vhead = [&](int g) { return G == 1 ? hx : hx + g * a.Hk; };
    const int h = vhead(hg), bh = b * a.H + h;  // this thread's value head
    const int H = a.H, K = a.K;
    const size_t qkv = (size_t)H * D;
    const size_t head_off = (size_t)h * D;
    const int grp = (tl >> 6) * 8 + (lane >> 3), s = lane & 7;
    // q / k rows are Hk*D wide and value head h reads key head h % Hk
    const size_t kw = (size_t)a.Hk * D, khead = (size_t)(hx % a.Hk) * D;
    const size_t rrow = ring_rows(a);
    auto prow = [&](int plane, int ch) -> size_t {  // conv-weight / ring row
        return plane < 2 ? plane * kw + khead + ch : 2 * kw + (size_t)vhead(plane - 2) * D + ch;
    };

    // Issue the state loads first so their HBM latency overlaps the conv / l2 work.
    float S[CPT][KPL];
#pragma unroll
    for (int c = 0; c < CPT; ++c)
        load_keys<D>(S[c], a.state_in + ((size_t)bh * D + grp + c * NG) * D, s);

    // The gate column of this thread is fixed (NT1 is a multiple of D; GDN: the threads
    // tid < G * TB_FUSED take token tid % TB_FUSED of value head tid / TB_FUSED); its
    // activation parameters arrive with the ring rows, which are waited for right below
    // (read before the state, their pointers' scalar load would hold the state loads back).
    static_assert(NT1 % D == 0, "one gate column per thread");
    const int ge = min(tid / TB_FUSED, G - 1), te = tid % TB_FUSED;  // GDN gate / beta slots
    const GateCol gp = gate_col(a, GDN ? vhead(ge) : h, GDN ? vhead(ge) : head_off + tid % D);

    size_t rstart;  // first activation row of this sequence
    int T;          // its row count
    seq_span(a, b, &rstart, &T);

    // Conv windows of the workgroup's NP*D (plane, channel) rows start as the old ring.
    for (int r = tid; r < NP * D; r += NT) {
        const int plane = r / D, ch = r % D;
        const float* ring_row = a.ring + ((size_t)b * rrow + prow(plane, ch)) * (K - 1);
        ConvChannel cc;
        conv_window_from_ring(cc, ring_row, K);
#pragma unroll
        for (int e = 0; e < KMAX - 1; ++e) wins[r][e] = cc.win[e];
    }

    for (int t0 = 0; t0 < T; t0 += TB_FUSED) {
        const int nt = min(TB_FUSED, T - t0);
        const size_t row0 = rstart + t0;
        for (int r = tid; r < NP * D; r += NT) {
            const int plane = r / D, ch = r % D;
            const void* xsrc = plane == 0 ? a.q : (plane == 1 ? a.k : a.v);
            ConvChannel cc;
            conv_load_taps(cc, a.conv_w + prow(plane, ch) * K, K);
#pragma unroll
            for (int e = 0; e < KMAX - 1; ++e) cc.win[e] = wins[r][e];
            const size_t xw = plane < 2 ? kw : qkv;
            const size_t xc = (plane < 2 ? khead : (size_t)vhead(plane - 2) * D) + ch;
            for (int tt = 0; tt < nt; ++tt) {
                const float x = ld_act<BF>(xsrc, (row0 + tt) * xw + xc);
                pre[plane][tt][ch] = silu_f(conv_push(cc, x));
            }
#pragma unroll
            for (int e = 0; e < KMAX - 1; ++e) wins[r][e] = cc.win[e];
        }
        if constexpr (GDN) {
            if (tid < G * TB_FUSED && te < nt) {
                const int hv = vhead(ge);
                es[te][ge] = exp_f(gate_in(a, gp, ld_act<BF>(a.g, (row0 + te) * H + hv)));
                bs[te][ge] = beta_in(a, ld_act<BF>(a.beta, (row0 + te) * H + hv));
            }
        } else {
            for (int idx = tid; idx < nt * D; idx += NT) {
                const int tt = idx / D, i = idx % D;
                es[tt][i] = exp_f(gate_in(a, gp, ld_act<BF>(a.g, (row0 + tt) * qkv + head_off + i)));
            }
            if (tid < nt) bs[tid][0] = beta_in(a, ld_act<BF>(a.beta, (row0 + tid) * H + h));
        }
        __syncthreads();
        for (int tt = wave; tt < nt; tt += NW) l2_qk_row<D>(pre[0][tt], pre[1][tt], lane, &kqs[tt]);
        __syncthreads();
        for (int tt = 0; tt < nt; ++tt) {
            float vj[CPT], o[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) vj[c] = pre[2 + hg][tt][grp + c * NG];
            scan_step_cols<D, GDN, CPT>(S, pre[0][tt], pre[1][tt], &es[tt][hg * EW], vj, bs[tt][hg], kqs[tt],
                                        a.scale, s, o);
            if (s == 0) {
#pragma unroll
                for (int c = 0; c < CPT; ++c) os[tt][hg * D + grp + c * NG] = o[c];
            }
        }
        __syncthreads();
        if (a.readout) {
            for (int idx = wave; idx < nt * G; idx += NW) {
                const int tt = idx / G, g = idx % G;
                const size_t off = (row0 + tt) * qkv + (size_t)vhead(g) * D;
                const GateRow gz = load_gate_row<D, BF>(a, off, lane);
                gated_rmsnorm_row<D, BF, GDN>(&os[tt][g * D], gz, a, off, lane, a.o_core);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int c = 0; c < CPT; ++c)
        store_keys<D>(a.state_out + ((size_t)bh * D + grp + c * NG) * D, S[c], s);
    // The windows now hold the last K-1 raw inputs of [old ring ++ x]. Each v row was
    // read only by this workgroup (window init); so were the q / k rows unless another
    // workgroup shares the key head (G == 1 with Hk < H), in which case they are rolled
    // by a kernel of their own after this one (that workgroup may still be reading them).
    for (int r = tid; r < NP * D; r += NT) {
        const int plane = r / D, ch = r % D;
        if (plane < 2 && G == 1 && a.Hk != a.H) continue;
        float* ring_row = a.ring + ((size_t)b * rrow + prow(plane, ch)) * (K - 1);
        ConvChannel cc;
#pragma unroll
        for (int e = 0; e < KMAX - 1; ++e) cc.win[e] = wins[r][e];
        conv_window_to_ring(cc, ring_row, K);
    }
}

// Short calls at D = 128, one value head per workgroup (G = 1): the fused kernel's work
// for T <= TM tokens (the decode step is TM = 1; speculative verify and rollback
// replays take TM = 8 or 16), calling the same helpers on the same values in the same
// order, so the bits equal those of the fused and split arms. Every raw row of the call
// is requested at once, right behind the state, and nothing is kept for a later token
// block: with few live registers three 512-thread workgroups share a CU, three 64 KiB
// head states in flight per CU instead of two. The new ring rows are written as soon
// as the conv has read the old ones (each row is read only by its own thread; q / k
// rows shared with other value heads, Hk < H, are left to the roll kernel that runs
// after this one). Rows past T are clamped copies of row T-1 and are not used.
constexpr int SHORT_D = 128, SHORT_THREADS = 512, SHORT_TMAX = 16;
template <bool BF, bool GDN, int TM>
__global__ __launch_bounds__(SHORT_THREADS, 6) void seq_short_kernel(MixerArgs a) {
    constexpr int D = SHORT_D, CPT = 2, NG = SHORT_THREADS / 8, KPL = D / 8, EW = GDN ? 1 : D;
    constexpr int NW = SHORT_THREADS / 64;
    static_assert(fused_cpt<D>() == CPT && fused_threads<D>() == SHORT_THREADS, "the fused kernel's lane map");
    static_assert(SHORT_THREADS % D == 0, "one gate column per thread");
    __shared__ float pre[3][TM][D];  // conv outputs q, k, v (q, k l2-normalised in place)
    __shared__ float es[TM][EW];     // exp(g)
    __shared__ float os[TM][D];      // scan readout
    __shared__ float bs[TM], kqs[TM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = blockIdx.x % a.H, b = seq_of(a, blockIdx.x / a.H);
    const int bh = b * a.H + h, K = a.K;
    const size_t qkv = (size_t)a.H * D, head_off = (size_t)h * D;
    const int grp = (tid >> 6) * 8 + (lane >> 3), s = lane & 7;
    const size_t kw = (size_t)a.Hk * D, khead = (size_t)(h % a.Hk) * D;

    const GateCol gp = gate_col(a, h, GDN ? (size_t)h : head_off + tid % D);
    size_t row0;
    int Tspan;
    seq_span(a, b, &row0, &Tspan);
    const int T = TM == 1 ? 1 : Tspan;  // 1 <= T <= TM (the launch checks it)

    // The conv inputs are requested before the state (vector-memory loads complete in
    // order), so the conv, gates and l2 norms run while the state streams in. Every
    // thread requests valid elements (threads tid >= 3 D those of plane 2, unused), so
    // no branch stands between the requests and the state's.
    // Conv + SiLU of plane tid / D, channel tid % D.
    const int plane = min(tid / D, 2), ch = tid % D;
    const size_t prow = plane < 2 ? plane * kw + khead + ch : 2 * kw + head_off + ch;
    float* ring_row = a.ring + ((size_t)b * ring_rows(a) + prow) * (K - 1);
    ConvChannel cc;
    conv_window_from_ring(cc, ring_row, K);
    conv_load_taps(cc, a.conv_w + prow * K, K);
    const void* xsrc = plane == 0 ? a.q : (plane == 1 ? a.k : a.v);
    const size_t xw = plane < 2 ? kw : qkv, xc = (plane < 2 ? khead : head_off) + ch;
    float x[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) x[t] = ld_act<BF>(xsrc, (row0 + min(t, T - 1)) * xw + xc);
    // gate and beta of row min(tid / EW, T - 1), entry tid % EW (KDA: one channel per
    // thread and row for T <= SHORT_THREADS / D rows, the rest below)
    constexpr int GR = GDN ? TM : (TM * D <= SHORT_THREADS ? TM : SHORT_THREADS / D);
    const int gt = min(GDN ? tid : tid / D, T - 1);
    const float graw = ld_act<BF>(a.g, GDN ? (row0 + gt) * a.H + h : (row0 + gt) * qkv + head_off + tid % D);
    const float braw = ld_act<BF>(a.beta, (row0 + min(tid, T - 1)) * a.H + h);
    asm volatile("" ::: "memory");
    float S[CPT][KPL];
#pragma unroll
    for (int c = 0; c < CPT; ++c) load_keys<D>(S[c], a.state_in + ((size_t)bh * D + grp + c * NG) * D, s);
    asm volatile("" ::: "memory");
    if (tid < 3 * D) {
#pragma unroll
        for (int t = 0; t < TM; ++t)
            if (t < T) pre[plane][t][ch] = silu_f(conv_push(cc, x[t]));
        if (plane == 2 || a.Hk == a.H) conv_window_to_ring(cc, ring_row, K);
    }
    if constexpr (GDN) {
        if (tid < T) {
            es[tid][0] = exp_f(gate_in(a, gp, graw));
            bs[tid] = beta_in(a, braw);
        }
    } else {
        if (tid < GR * D && tid / D < T) es[tid / D][tid % D] = exp_f(gate_in(a, gp, graw));
        for (int idx = GR * D + tid; idx < T * D; idx += SHORT_THREADS) {
            const int t = idx / D, i = idx % D;
            es[t][i] = exp_f(gate_in(a, gp, ld_act<BF>(a.g, (row0 + t) * qkv + head_off + i)));
        }
        if (tid < T) bs[tid] = beta_in(a, braw);
    }
    __syncthreads();
    for (int t = wave; t < T; t += NW) l2_qk_row<D>(pre[0][t], pre[1][t], lane, &kqs[t]);
    __syncthreads();
    for (int t = 0; t < T; ++t) {
        float vj[CPT], o[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) vj[c] = pre[2][t][grp + c * NG];
        scan_step_cols<D, GDN, CPT>(S, pre[0][t], pre[1][t], es[t], vj, bs[t], kqs[t], a.scale, s, o);
        if (s == 0) {
#pragma unroll
            for (int c = 0; c < CPT; ++c) os[t][grp + c * NG] = o[c];
        }
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) store_keys<D>(a.state_out + ((size_t)bh * D + grp + c * NG) * D, S[c], s);
    if (!a.readout) return;
    __syncthreads();
    for (int t = wave; t < T; t += NW) {
        const size_t off = (row0 + t) * qkv + head_off;
        const GateRow gz = load_gate_row<D, BF>(a, off, lane);
        gated_rmsnorm_row<D, BF, GDN>(os[t], gz, a, off, lane, a.o_core);
    }
}

// Longer calls at D = 128, one value head per workgroup (G = 1), packed batches
// included: the short-call kernel's structure over blocks of 16 tokens. A block's raw
// rows and conv taps are all requested at its start; the conv windows carry over in
// LDS between blocks. Same helpers, same values, same order as the
// fused kernel (its bits). At most 80 VGPRs and 51 KiB of LDS: three workgroups per CU.
constexpr int BLOCK_TB = 16;
template <bool BF, bool GDN>
__global__ __launch_bounds__(SHORT_THREADS, 6) void seq_blocks_kernel(MixerArgs a) {
    constexpr int D = SHORT_D, CPT = 2, NG = SHORT_THREADS / 8, KPL = D / 8, EW = GDN ? 1 : D;
    constexpr int NW = SHORT_THREADS / 64, TB = BLOCK_TB, RPW = TB / NW;
    static_assert(fused_cpt<D>() == CPT && fused_threads<D>() == SHORT_THREADS, "the fused kernel's lane map");
    static_assert(TB % NW == 0, "norm rows per wavefront");
    __shared__ float pre[3][TB][D];          // conv outputs q, k, v (q, k l2-normalised in place)
    __shared__ float es[TB][EW];             // exp(g)
    __shared__ float os[TB][D];              // scan readout
    __shared__ float bs[TB], kqs[TB];
    __shared__ float wins[3 * D][KMAX - 1];  // conv windows between blocks

    // The thread index is re-materialised at every phase (an opaque copy): otherwise the
    // compiler hoists every phase's per-thread addresses out of the block loop and keeps
    // them all alive at once, which spills.
    int tid = threadIdx.x;
#define KDA_LAUNDER_TID() asm volatile("" : "+v"(tid))
    const int h = blockIdx.x % a.H, b = seq_of(a, blockIdx.x / a.H);
    const int bh = b * a.H + h, K = a.K;
    const size_t qkv = (size_t)a.H * D, head_off = (size_t)h * D;
    const size_t kw = (size_t)a.Hk * D, khead = (size_t)(h % a.Hk) * D;
    // conv row of threads tid < 3 D: plane tid / D (q, k, v), channel tid % D
    auto ring_row_of = [&](int t) -> float* {
        const int plane = t / D, ch = t % D;
        const size_t prow = plane < 2 ? plane * kw + khead + ch : 2 * kw + head_off + ch;
        return a.ring + ((size_t)b * ring_rows(a) + prow) * (K - 1);
    };
    auto state_row = [&](int t, int c) -> size_t {  // offset of this thread's column c
        return ((size_t)bh * D + (t >> 6) * 8 + ((t & 63) >> 3) + c * NG) * D;
    };

    float S[CPT][KPL];
#pragma unroll
    for (int c = 0; c < CPT; ++c) load_keys<D>(S[c], a.state_in + state_row(tid, c), tid & 7);

    const GateCol gp = gate_col(a, h, GDN ? (size_t)h : head_off + tid % D);
    size_t rstart;
    int T;
    seq_span(a, b, &rstart, &T);

    if (tid < 3 * D) {
        ConvChannel cc;
        conv_window_from_ring(cc, ring_row_of(tid), K);
#pragma unroll
        for (int e = 0; e < KMAX - 1; ++e) wins[tid][e] = cc.win[e];
    }
    for (int t0 = 0; t0 < T; t0 += TB) {
        const int nt = min(TB, T - t0);
        const size_t row0 = rstart + t0;
        KDA_LAUNDER_TID();
        if (tid < 3 * D) {  // conv + SiLU of plane tid / D, channel tid % D
            const int plane = tid / D, ch = tid % D;
            const size_t prow = plane < 2 ? plane * kw + khead + ch : 2 * kw + head_off + ch;
            ConvChannel cc;
            conv_load_taps(cc, a.conv_w + prow * K, K);
            const void* xsrc = plane == 0 ? a.q : (plane == 1 ? a.k : a.v);
            const size_t xw = plane < 2 ? kw : qkv, xc = (plane < 2 ? khead : head_off) + ch;
            float x[TB];
#pragma unroll
            for (int t = 0; t < TB; ++t) x[t] = ld_act<BF>(xsrc, (row0 + min(t, nt - 1)) * xw + xc);
#pragma unroll
            for (int e = 0; e < KMAX - 1; ++e) cc.win[e] = wins[tid][e];
#pragma unroll
            for (int t = 0; t < TB; ++t)
                if (t < nt) pre[plane][t][ch] = silu_f(conv_push(cc, x[t]));
#pragma unroll
            for (int e = 0; e < KMAX - 1; ++e) wins[tid][e] = cc.win[e];
        }
        KDA_LAUNDER_TID();
        if constexpr (GDN) {
            if (tid < nt) {
                es[tid][0] = exp_f(gate_in(a, gp, ld_act<BF>(a.g, (row0 + tid) * a.H + h)));
                bs[tid] = beta_in(a, ld_act<BF>(a.beta, (row0 + tid) * a.H + h));
            }
        } else {
            for (int idx = tid; idx < nt * D; idx += SHORT_THREADS) {
                const int t = idx / D, i = idx % D;
                es[t][i] = exp_f(gate_in(a, gp, ld_act<BF>(a.g, (row0 + t) * qkv + head_off + i)));
            }
            if (tid < nt) bs[tid] = beta_in(a, ld_act<BF>(a.beta, (row0 + tid) * a.H + h));
        }
        __syncthreads();
        KDA_LAUNDER_TID();
        for (int t = tid >> 6; t < nt; t += NW) l2_qk_row<D>(pre[0][t], pre[1][t], tid & 63, &kqs[t]);
        __syncthreads();
        KDA_LAUNDER_TID();
        {
            const int grp = (tid >> 6) * 8 + ((tid & 63) >> 3), s = tid & 7;
            for (int t = 0; t < nt; ++t) {
                float vj[CPT], o[CPT];
#pragma unroll
                for (int c = 0; c < CPT; ++c) vj[c] = pre[2][t][grp + c * NG];
                scan_step_cols<D, GDN, CPT>(S, pre[0][t], pre[1][t], es[t], vj, bs[t], kqs[t], a.scale, s, o);
                if (s == 0) {
#pragma unroll
                    for (int c = 0; c < CPT; ++c) os[t][grp + c * NG] = o[c];
                }
            }
        }
        __syncthreads();
        KDA_LAUNDER_TID();
        if (a.readout) {
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                const int t = (tid >> 6) + r * NW;
                if (t < nt) {
                    const size_t off = (row0 + t) * qkv + head_off;
                    const GateRow gz = load_gate_row<D, BF>(a, off, tid & 63);
                    gated_rmsnorm_row<D, BF, GDN>(os[t], gz, a, off, tid & 63, a.o_core);
                }
            }
        }
        __syncthreads();
    }
    KDA_LAUNDER_TID();
#pragma unroll
    for (int c = 0; c < CPT; ++c) store_keys<D>(a.state_out + state_row(tid, c), S[c], tid & 7);
    // the windows hold the last K-1 raw inputs of [old ring ++ x]; q / k rows shared
    // with other value heads (Hk < H) are rolled by the roll kernel after this one
    if (tid < 3 * D && (tid >= 2 * D || a.Hk == a.H)) {
        ConvChannel cc;
#pragma unroll
        for (int e = 0; e < KMAX - 1; ++e) cc.win[e] = wins[tid][e];
        conv_window_to_ring(cc, ring_row_of(tid), K);
    }
#undef KDA_LAUNDER_TID
}

// Short calls of GDN with two value heads per key head (H = 2 Hk): one 512-thread
// workgroup per (sequence, key head) holds both value heads, each thread two columns
// of each (the fused kernel's column map, once per head), so the q / k conv runs once
// and the workgroup rolls its own q / k ring rows. Two workgroups share a CU: four
// head states in flight per CU, where the 1024-thread fused kernel holds two.
template <bool BF, int TM>
__global__ __launch_bounds__(SHORT_THREADS, 4) void seq_short_pair_kernel(MixerArgs a) {
    constexpr int D = SHORT_D, CPT = 2, NG = SHORT_THREADS / 8, KPL = D / 8, G = 2;
    constexpr int NW = SHORT_THREADS / 64;
    static_assert((2 + G) * D == SHORT_THREADS, "one conv channel per thread");
    __shared__ float pre[2 + G][TM][D];  // conv outputs q, k, v of value head 0, 1
    __shared__ float es[TM][G];          // exp(g) per value head
    __shared__ float os[TM][G * D];      // scan readout
    __shared__ float bs[TM][G], kqs[TM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hx = blockIdx.x % a.Hk, b = seq_of(a, blockIdx.x / a.Hk);
    const int K = a.K;
    const size_t qkv = (size_t)a.H * D, kw = (size_t)a.Hk * D, khead = (size_t)hx * D;
    const int grp = (tid >> 6) * 8 + (lane >> 3), s = lane & 7;
    auto vhead = [&](int g) { return hx + g * a.Hk; };

    float S[G][CPT][KPL];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < CPT; ++c)
            load_keys<D>(S[g][c], a.state_in + ((size_t)(b * a.H + vhead(g)) * D + grp + c * NG) * D, s);

    const int ge = min(tid / TM, G - 1), te = tid % TM;  // gate / beta slot of threads tid < G * TM
    const GateCol gp = gate_col(a, vhead(ge), vhead(ge));
    size_t row0;
    int Tspan;
    seq_span(a, b, &row0, &Tspan);
    const int T = TM == 1 ? 1 : Tspan;  // 1 <= T <= TM (the launch checks it)

    {  // conv + SiLU of plane tid / D (q, k, v of head 0, v of head 1), channel tid % D
        const int plane = tid / D, ch = tid % D;
        const size_t vo = plane < 2 ? 0 : (size_t)vhead(plane - 2) * D;
        const size_t prow = plane < 2 ? plane * kw + khead + ch : 2 * kw + vo + ch;
        float* ring_row = a.ring + ((size_t)b * ring_rows(a) + prow) * (K - 1);
        ConvChannel cc;
        conv_window_from_ring(cc, ring_row, K);
        conv_load_taps(cc, a.conv_w + prow * K, K);
        const void* xsrc = plane == 0 ? a.q : (plane == 1 ? a.k : a.v);
        const size_t xw = plane < 2 ? kw : qkv, xc = (plane < 2 ? khead : vo) + ch;
        float x[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) x[t] = ld_act<BF>(xsrc, (row0 + min(t, T - 1)) * xw + xc);
#pragma unroll
        for (int t = 0; t < TM; ++t)
            if (t < T) pre[plane][t][ch] = silu_f(conv_push(cc, x[t]));
        conv_window_to_ring(cc, ring_row, K);
    }
    if (tid < G * TM && te < T) {
        const int hv = vhead(ge);
        es[te][ge] = exp_f(gate_in(a, gp, ld_act<BF>(a.g, (row0 + te) * a.H + hv)));
        bs[te][ge] = beta_in(a, ld_act<BF>(a.beta, (row0 + te) * a.H + hv));
    }
    __syncthreads();
    for (int t = wave; t < T; t += NW) l2_qk_row<D>(pre[0][t], pre[1][t], lane, &kqs[t]);
    __syncthreads();
    for (int t = 0; t < T; ++t) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float vj[CPT], o[CPT];
#pragma unroll
            for (int c = 0; c < CPT; ++c) vj[c] = pre[2 + g][t][grp + c * NG];
            scan_step_cols<D, true, CPT, true>(S[g], pre[0][t], pre[1][t], &es[t][g], vj, bs[t][g], kqs[t], a.scale, s, o);
            if (s == 0) {
#pragma unroll
                for (int c = 0; c < CPT; ++c) os[t][g * D + grp + c * NG] = o[c];
            }
            if (TM == 1) {  // a one-token call stores head 0's state while head 1 is scanned
#pragma unroll
                for (int c = 0; c < CPT; ++c)
                    store_keys<D>(a.state_out + ((size_t)(b * a.H + vhead(g)) * D + grp + c * NG) * D, S[g][c], s);
            }
        }
    }
    if (TM > 1) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int c = 0; c < CPT; ++c)
                store_keys<D>(a.state_out + ((size_t)(b * a.H + vhead(g)) * D + grp + c * NG) * D, S[g][c], s);
    }
    if (!a.readout) return;
    __syncthreads();
    for (int idx = wave; idx < T * G; idx += NW) {
        const int t = idx / G, g = idx % G;
        const size_t off = (row0 + t) * qkv + (size_t)vhead(g) * D;
        const GateRow gz = load_gate_row<D, BF>(a, off, lane);
        gated_rmsnorm_row<D, BF, true>(&os[t][g * D], gz, a, off, lane, a.o_core);
    }
}

template <bool BF>
hipError_t short_pair_launch(const MixerArgs& a) {
    const dim3 grid(a.B * a.Hk), block(SHORT_THREADS);
    if (a.T == 1)
        hipLaunchKernelGGL((seq_short_pair_kernel<BF, 1>), grid, block, 0, a.stream, a);
    else if (a.T <= 8)
        hipLaunchKernelGGL((seq_short_pair_kernel<BF, 8>), grid, block, 0, a.stream, a);
    else
        hipLaunchKernelGGL((seq_short_pair_kernel<BF, SHORT_TMAX>), grid, block, 0, a.stream, a);
    return hipGetLastError();
}

template <bool BF, bool GDN>
hipError_t short_launch(const MixerArgs& a) {
    const dim3 grid(a.B * a.H), block(SHORT_THREADS);
    if (a.T == 1)
        hipLaunchKernelGGL((seq_short_kernel<BF, GDN, 1>), grid, block, 0, a.stream, a);
    else if (a.T <= 8)
        hipLaunchKernelGGL((seq_short_kernel<BF, GDN, 8>), grid, block, 0, a.stream, a);
    else
        hipLaunchKernelGGL((seq_short_kernel<BF, GDN, SHORT_TMAX>), grid, block, 0, a.stream, a);
    return hipGetLastError();
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
    // Key heads shared by several value heads (Hk < H): the workgroups of value heads
    // h < Hk (key head h) alone convolve, normalise and store q / k and roll their ring
    // rows; every workgroup does its own v.
    const bool qk_owner = h < a.Hk;
    const size_t kw = (size_t)a.Hk * D;
    const int plane = tid / D, ch = tid % D;
    const bool conv_thread = tid < 3 * D && (plane == 2 || qk_owner);
    const size_t cf = plane < 2 ? plane * kw + head_off + ch : 2 * kw + head_off + ch;
    float* ring_row = a.ring + ((size_t)b * ring_rows(a) + cf) * (K - 1);
    const void* xsrc = plane == 0 ? a.q : (plane == 1 ? a.k : a.v);
    const size_t xw = plane < 2 ? kw : qkv;
    auto raw_at = [&](int pos) -> float {  // x~[K-1+pos]: raw input at token pos (< 0: ring)
        return pos >= 0 ? ld_act<BF>(xsrc, ((size_t)b * a.tp + pos) * xw + head_off + ch)
                        : ring_row[pos + K - 1];
    };
    if (conv_thread) {
        ConvChannel cc;
        conv_load_taps(cc, a.conv_w + cf * K, K);
#pragma unroll
        for (int d = 1; d < KMAX; ++d) cc.win[KMAX - 1 - d] = (d <= K - 1) ? raw_at(t0 - d) : 0.0f;
        for (int tt = 0; tt < nt; ++tt)
            pre[plane][tt][ch] = silu_f(conv_push(cc, ld_act<BF>(xsrc, (rin0 + tt) * xw + head_off + ch)));
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
    if (qk_owner)
        for (int tt = wave; tt < nt; tt += NW) l2_qk_row<D>(pre[0][tt], pre[1][tt], lane, &kqs[tt]);
    __syncthreads();
    for (int idx = tid; idx < nt * D; idx += NT) {
        const int tt = idx / D, i = idx % D;
        if (qk_owner) {
            const size_t koff = (row0 + tt) * kw + head_off + i;  // key head h
            qh[koff] = pre[0][tt][i];
            kh[koff] = pre[1][tt][i];
        }
        vh[(row0 + tt) * qkv + head_off + i] = pre[2][tt][i];
    }
    if (qk_owner && tid < nt) kqv[(row0 + tid) * a.Hk + h] = kqs[tid];
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
    const int hk = h % a.Hk;  // key head of this value head
    const size_t kw = (size_t)a.Hk * D, khead = (size_t)hk * D;

    float S[1][KPL];
    load_keys<D>(S[0], a.state_in + ((size_t)bh * D + j) * D, s);

    for (int t0 = 0; t0 < T; t0 += TB_SCAN) {
        const int nt = min(TB_SCAN, T - t0);
        const size_t row0 = (size_t)b * T + t0;
        for (int idx = tid; idx < nt * D; idx += NT) {
            const int tt = idx / D, i = idx % D;
            const size_t koff = (row0 + tt) * kw + khead + i;
            qs[tt][i] = qh[koff];
            ks[tt][i] = kh[koff];
            if constexpr (!GDN) es[tt][i] = eg[(row0 + tt) * qkv + head_off + i];
        }
        for (int idx = tid; idx < nt * COLS; idx += NT) {
            const int tt = idx / COLS, c = idx % COLS;
            vs[tt][c] = vh[(row0 + tt) * qkv + head_off + split * COLS + c];
        }
        if (tid < nt) {
            const size_t hr = (row0 + tid) * H + h;
            bs[tid] = beta_in(a, ld_act<BF>(a.beta, ((size_t)b * a.tp + t0 + tid) * H + h));
            kqs[tid] = kqv[(row0 + tid) * a.Hk + hk];
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
    const size_t rows = total_rows(a) * a.H;
    const size_t row = (size_t)blockIdx.x * 4 + wave;
    if (row >= rows) return;
    const size_t off = (row / a.H) * ((size_t)a.H * D) + (row % a.H) * D;
    const GateRow gz = load_gate_row<D, BF>(a, off, lane);
    gated_rmsnorm_row<D, BF, GDN>(o + off, gz, a, off, lane, nullptr);
}

template <int D, bool BF, bool GDN>
hipError_t fused_launch(const MixerArgs& a) {
    if constexpr (GDN) {
        if (a.H == 2 * a.Hk) {  // both value heads of a key head in one workgroup
            if (D == SHORT_D && a.T >= 1 && a.T <= SHORT_TMAX && !a.cu_seqlens) return short_pair_launch<BF>(a);
            hipLaunchKernelGGL((seq_fused_kernel<D, BF, GDN, 2>), dim3(a.B * a.Hk), dim3(2 * fused_threads<D>()),
                               0, a.stream, a);
            return hipGetLastError();
        }
    }
    hipError_t e;
    if (D == SHORT_D && a.T >= 1 && a.T <= SHORT_TMAX && !a.cu_seqlens) {
        e = short_launch<BF, GDN>(a);
    } else if (D == SHORT_D) {
        hipLaunchKernelGGL((seq_blocks_kernel<BF, GDN>), dim3(a.B * a.H), dim3(SHORT_THREADS), 0, a.stream, a);
        e = hipGetLastError();
    } else {
        hipLaunchKernelGGL((seq_fused_kernel<D, BF, GDN>), dim3(a.B * a.H), dim3(fused_threads<D>()), 0,
                           a.stream, a);
        e = hipGetLastError();
    }
    if (e != hipSuccess || a.Hk == a.H) return e;
    return launch_ring_roll(a, true);  // shared q / k rows, after every reader
}

template <int D, bool BF, bool GDN>
hipError_t split_launch(const MixerArgs& a) {
    if (a.cu_seqlens) return hipErrorInvalidValue;  // packed batches take the fused arm
    const SplitWorkspace w = split_workspace(a.B, a.T, a.H, a.Hk, a.D, a.gdn);
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

SplitWorkspace split_workspace(int B, int T, int H, int Hk, int D, bool gdn) {
    const size_t act = align256((size_t)B * T * H * D * 4);
    const size_t kact = align256((size_t)B * T * Hk * D * 4);
    const size_t per_head = align256((size_t)B * T * H * 4);
    const size_t per_khead = align256((size_t)B * T * Hk * 4);
    SplitWorkspace w;
    w.qh = 0;
    w.kh = w.qh + kact;
    w.vh = w.kh + kact;
    w.eg = w.vh + act;
    w.kq = w.eg + (gdn ? per_head : act);
    w.o = w.kq + per_khead;
    w.total = w.o + act;
    return w;
}

namespace {

// Thread n ranks sequence n: the number of longer sequences plus the number of equally
// long ones before it. Lengths are the clamped spans the mixer kernels use.
__global__ __launch_bounds__(256) void seq_order_kernel(MixerArgs a, int* order) {
    __shared__ int lens[256];
    const int n = blockIdx.x * 256 + threadIdx.x;
    size_t st;
    int len = -1;
    if (n < a.B) seq_span(a, n, &st, &len);
    int rank = 0;
    for (int m0 = 0; m0 < a.B; m0 += 256) {
        const int m = m0 + threadIdx.x;
        int lm = -1;
        if (m < a.B) seq_span(a, m, &st, &lm);
        __syncthreads();
        lens[threadIdx.x] = lm;
        __syncthreads();
        const int cnt = min(256, a.B - m0);
        for (int j = 0; j < cnt; ++j) {
            const int l = lens[j];
            rank += (l > len) || (l == len && m0 + j < n);
        }
    }
    if (n < a.B) order[rank] = n;
}

// One thread per ring row: the K-1 newest raw inputs of [old ring ++ x] (the row's
// old slots are read into registers before any store). Rows of a sequence are
// numbered as the ring: q plane, k plane (Hk*D each), v plane (H*D).
template <bool BF>
__global__ __launch_bounds__(256) void ring_roll_kernel(MixerArgs a, int rows_per_seq) {
    const size_t row = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (row >= (size_t)a.B * rows_per_seq) return;
    const size_t kw = (size_t)a.Hk * a.D, vw = (size_t)a.H * a.D;
    const int b = (int)(row / rows_per_seq);
    const size_t cf = row % rows_per_seq;
    const int plane = cf < kw ? 0 : (cf < 2 * kw ? 1 : 2);
    const size_t ch = plane < 2 ? cf - plane * kw : cf - 2 * kw;
    const size_t xw = plane < 2 ? kw : vw;
    const void* x = plane == 0 ? a.q : (plane == 1 ? a.k : a.v);
    const int K = a.K;
    size_t rstart;
    int T;
    seq_span(a, b, &rstart, &T);
    float* ring_row = a.ring + ((size_t)b * ring_rows(a) + cf) * (K - 1);
    float nr[KMAX - 1];
#pragma unroll
    for (int d = 1; d < KMAX; ++d) {
        const int pos = T - d;
        nr[KMAX - 1 - d] = (d <= K - 1) ? (pos >= 0 ? ld_act<BF>(x, (rstart + pos) * xw + ch)
                                                     : ring_row[pos + K - 1])
                                        : 0.0f;
    }
#pragma unroll
    for (int d = 1; d < KMAX; ++d)
        if (d <= K - 1) ring_row[K - 1 - d] = nr[KMAX - 1 - d];
}

}  // namespace

hipError_t launch_seq_order(const MixerArgs& a, int* order) {
    hipLaunchKernelGGL(seq_order_kernel, dim3((unsigned)((a.B + 255) / 256)), dim3(256), 0, a.stream, a, order);
    return hipGetLastError();
}

hipError_t launch_ring_roll(const MixerArgs& a, bool qk_only) {
    const int rows_per_seq = (int)(qk_only ? (size_t)2 * a.Hk * a.D : ring_rows(a));
    const size_t rows = (size_t)a.B * rows_per_seq;
    const dim3 grid((unsigned)((rows + 255) / 256)), block(256);
    if (a.bf16) hipLaunchKernelGGL((ring_roll_kernel<true>), grid, block, 0, a.stream, a, rows_per_seq);
    else hipLaunchKernelGGL((ring_roll_kernel<false>), grid, block, 0, a.stream, a, rows_per_seq);
    return hipGetLastError();
}

hipError_t launch_seq_fused(const MixerArgs& a) { return dispatch<FusedOp>(a); }

hipError_t launch_norm(const MixerArgs& a, const float* o) {
    const size_t rows = total_rows(a) * a.H;
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
