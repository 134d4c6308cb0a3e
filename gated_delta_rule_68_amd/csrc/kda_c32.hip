// Chunked prefill of the KDA / GDN mixer for gfx950 in chunks of 32 rows: bf16
// activations, D = 128, conv kernels of up to 4 taps, one (sequence, head) per
// workgroup of 16 wavefronts in two specialised groups.
//
// The recurrence is taken in its WY / UT form (memra-engine kda.rs, module notes on the
// chunked twin: a cumulative log gate per channel, k scaled by exp(-Gcum) and q by
// exp(+Gcum), a triangular intra-chunk solve; for GDN one scalar gate per row). Per
// chunk of 32 rows with carried state S (key i x value j), G the inclusive cumulative
// log gate from the chunk start and G_l its value at the last row:
//   L[s][j] = sum_i k_s[i] k_j[i] e^{G_s[i]-G_j[i]}  (j < s),  P the same with q_s, j <= s
//   T  = (I + diag(beta) L)^-1
//   Ub = T diag(beta) (V - K+ S)            K+_j = k_j e^{G_j}
//   O  = scale (Q+ S + P Ub)                Q+_s = q_s e^{G_s}
//   S  = diag(e^{G_l}) S + K_dec^T Ub       K_dec_j = k_j e^{G_l - G_j}
// K+, Q+ and K_dec have factors <= 1. For L and P (KDA) the rows form two 16-row
// blocks; with R_a the cumulative gate before block a and gamma = G - R_a (at most 16
// gates, >= -80 for gates >= -5), k e^{-gamma} <= e^{80} stays inside the bf16 range:
//   L, P block (a, a):  (k, q) e^{gamma}  .  k e^{-gamma}
//   L, P block (1, 0):  (k, q) e^{gamma}  .  (k e^{-gamma}) e^{R_1}
// For GDN the gate is a scalar per row, so L = (k k^T) * E and P = (q k^T) * E with
// E[s][j] = e^{G_s - G_j} taken on the 32 x 32 products, and the row factors of K+,
// Q+ and K_dec are applied to the MFMA results instead of the operands.
//
// Work layout: wavefronts 8..15 (two per SIMD) prepare chunk c+1 while wavefronts 0..7
// (two per SIMD) run chunk c's state-dependent work, so every SIMD holds VALU-heavy
// and MFMA-heavy wavefronts at once, two of each to hide each other's latencies. The
// state group carries the longer chains; it issues first (older wavefronts, raised
// priority). A step has two phases between workgroup barriers:
//   phase  preparing group (chunk c+1)             state group (chunk c)
//   1      conv + SiLU of q, k, l2 norms, gates    v conv, L and P (MFMA), T, Q+ S, K+ S
//   2      decay factors, operand tiles            Ub, O, state update; gated RMSNorm
//                                                  and stores of chunk c-1
// The preparing wavefront w convolves rows 4w .. 4w+3, two channels per lane, straight
// from registers: each lane reads its channels of its rows and of the 3 rows before
// them (the conv history; the old ring before the sequence start), so no raw rows are
// staged in LDS; the l2 norms are sums over the 64 lanes of a wavefront. The state
// lives in the state group's MFMA accumulators, owned by value column (state wavefront
// w holds value columns 16w .. 16w+15 for all 128 keys). Packed to bf16, those
// accumulators are directly the operand of Q+ S and K+ S (keys in the accumulator
// order), and Ub's accumulators directly the operands of P Ub and K_dec^T Ub, so the
// state-dependent work needs no LDS exchange of its own. Tiles whose contraction index
// meets an accumulator are stored with that index permuted within each 32-wide slice
// (perm32), so every MFMA fragment is one 16-byte LDS read. Tiles that one group
// writes while the other reads the previous chunk's are double-buffered.
//
// The segmented arm's runs without readout (from zero and from the identity: only
// their final state is used) take a specialisation of both groups chosen once per
// workgroup: no q rows, q conv or Q+ tiles, no P blocks, Q+ S, O, gated norm or stores.
#include <type_traits>

#include "kda_chunk_common.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int C = 32;            // rows per chunk
constexpr int DK = CHUNK_DK;     // 128
constexpr int NT = 1024;         // 16 wavefronts: 0..7 carry the state, 8..15 prepare
constexpr int GT = 512;          // threads of one group
constexpr int NW = 8;            // wavefronts of one group
constexpr int RW = C / NW;       // rows per preparing (and v conv) wavefront: 4
constexpr int KT = 4;            // conv window of this kernel (K <= 4)
constexpr int HALO = KT - 1;     // conv history rows
constexpr int NR = RW + HALO;    // rows a lane reads per conv plane
constexpr int LDR = DK + 8;      // bf16 pitch of [32][128] tiles
constexpr int LDJ = C + 8;       // bf16 pitch of [128][32] tiles
constexpr int LDT = 20;          // fp32 pitch of the 16 x 16 solve blocks

// Physical position of index k within a 32-wide slice: the accumulator order of two
// stacked 16-row MFMA results (lane q4 holds rows 4 q4 .. +3 of each), so that lane
// q4's 16-byte read at 8 q4 returns exactly the rows its accumulators hold.
__device__ __forceinline__ int perm32(int k) { return ((k & 15) >> 2) * 8 + (k >> 4) * 4 + (k & 3); }
__device__ __forceinline__ int pchan(int c) { return (c & ~31) | perm32(c & 31); }
// Column of the [128][32] tiles (K_dec^T, v^T) as stored: the 16-byte block of
// column col is XORed with bits 4-5 of the row, so the 8-byte stores of a wavefront
// (rows two apart, one column block) spread over the LDS banks; a reader of 16 rows
// r0 .. r0 + 15 applies one constant (r0 a multiple of 16).
__device__ __forceinline__ int swz(int col, int row) { return col ^ (((row >> 4) & 3) << 3); }

template <bool GDN>
struct C32Lds {
    // written in phase 2 by the preparing group, read by the state group in the next
    // step's phase 1
    alignas(16) __bf16 qa[C][LDR];             // KDA: q^ e^{gamma}; GDN: q^ (channels permuted)
    __bf16 ka[C][LDR];             // KDA: k^ e^{gamma}; GDN: k^
    __bf16 kb[GDN ? 1 : C][LDR];   // k^ e^{-gamma}
    __bf16 qp[GDN ? 1 : C][LDR];   // Q+, rows 16..31 (block 0's rows are those of qa)
    __bf16 kp[GDN ? 1 : C][LDR];   // K+, rows 16..31 (block 0's rows are those of ka)
    __bf16 kb1[GDN ? 1 : C / 2][LDR];  // rows 0..15: k^ e^{-gamma} e^{R_1} (L, P block (1, 0))
    // double-buffered by chunk parity
    __bf16 kdt[2][DK][LDJ];        // KDA: K_dec^T; GDN: k^T  ([key][row], rows permuted)
    float beta[2][C];
    float ffn[2][GDN ? 4 : DK];    // KDA: e^{G_l} per key
    float gcum[2][C];              // GDN: G per row (log2 units)
    // the state group's own: L and P written in phase 1 (P read in phase 2), v^T
    // written in phase 1 and read in phase 2
    __bf16 vbt[DK][LDJ];           // v^T (conv output, no beta)
    __bf16 pb[C][LDJ];             // P [s][j] (j permuted)
    float lf10[16][LDT];           // A_10 = diag(beta) L, rows 16.., columns 0..15
    float ltd[2][16 * LDT];        // A_aa transposed: [a][c * LDT + r] = A[16a + r][16a + c]
    float tdiag[2][16][LDT];       // T_aa (fp32), the state group's own
    bf16x8 tfrag[2][64];           // T as the MFMA A fragments of a state wavefront's lanes
    float gsum[NW][DK];            // KDA: gate sums of each wavefront's rows; GDN: [0][r] row prefix, [1][w] totals
    float nrm[NW][8];              // 1 / ||row|| of the l2 norms, per preparing wavefront
    float taps[3][2][64][KT];      // conv taps of the q, k, v planes: [plane][e][lane] for channel 2 lane + e
                                   // (each lane reads back only its own, 16 bytes apart across lanes)
    float normw[DK];               // norm weight (written by the state group, read back by each lane)
    union {
        float hist[3][HALO][DK];   // conv history before the sequence (first chunk)
        float ost[2][C][DK + 4];   // O staging for the norm, by chunk parity
    } u;
    float gpos[2][GDN ? C : 1];    // GDN: e^{G_j} per row
    float gdec[2][GDN ? C : 1];    // GDN: e^{G_l - G_j} per row
    uint32_t tcnt;                 // diagonal blocks T_00 finished (state wavefront 2)
};

__device__ __forceinline__ float lo_bf(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// The value of quad lane src in every lane of its quad (DPP quad_perm [src x 4]; every
// lane reads a lane of its own quad, so no lane keeps an old value); src is a constant
// once the caller's loop is unrolled.
template <int CTRL>
__device__ __forceinline__ float mov_dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float quad_bcast(float x, int src) {
    switch (src) {
        case 0: return mov_dpp<0x00>(x);
        case 1: return mov_dpp<0x55>(x);
        case 2: return mov_dpp<0xAA>(x);
        default: return mov_dpp<0xFF>(x);
    }
}

// Two 16-row accumulator tiles (rows 4 q4 + r of each) as one bf16 operand in the
// perm32 slot order.
__device__ __forceinline__ bf16x8 pack2(f32x4v t0, f32x4v t1) {
    return bf16x8{(__bf16)t0[0], (__bf16)t0[1], (__bf16)t0[2], (__bf16)t0[3],
                  (__bf16)t1[0], (__bf16)t1[1], (__bf16)t1[2], (__bf16)t1[3]};
}

// What one workgroup works on.
struct C32Job {
    size_t rowb;           // first activation row of the run
    int T;                 // its rows
    int lo;                // lowest row index a conv history may read (0 or -HALO)
    int b, h;
    bool ring_start;       // the run starts at the sequence start: history from the ring
    bool readout;          // outputs are written
    uint32_t vbytes;       // range of the v loads: 0 for the segmented arm's M runs (v = 0)
    const float* s_in;
    float* s_out;
    int s_init;            // the entry state: 0 read from s_in, 1 zero, 2 identity
};

// Raw rows of one plane: a lane's two channels (one dword of bf16, `lane_off` bytes into
// the row) of rows RW w - 3 .. RW w + RW - 1 of the chunk at c0, from a clamped row (rows
// past T repeat row T-1, rows before the run clamp to job.lo). Row indices are
// wave-uniform: the buffer starts at the lowest row any wavefront reads, and each row is
// a scalar offset from it. Nothing is consumed before the next chunk, so the loads stay
// in flight.
__device__ __forceinline__ void load_rows(uint32_t (&x)[NR], const void* base, size_t stride, size_t col0,
                                          uint32_t lane_off, uint32_t bytes, const C32Job& j, int c0, int w) {
    const int rb = min(max(c0 - HALO, j.lo), j.T - 1);
    const auto rs = buf_rsrc(static_cast<const __bf16*>(base) + ((size_t)((long long)j.rowb + rb) * stride + col0), bytes);
    const uint32_t pitch = (uint32_t)(stride * sizeof(__bf16));
#pragma unroll
    for (int i = 0; i < NR; ++i) {
        const int rel = min(max(c0 + RW * w - HALO + i, j.lo), j.T - 1);
        x[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)lane_off, (int)((uint32_t)(rel - rb) * pitch), 0);
    }
}

// The conv taps of the lane's channels row and row + 1 (w[e][KT - 1] multiplies the
// newest input). With K = KT the two weight rows are 32 contiguous bytes, requested as
// two 16-byte loads; the lanes of a wavefront then cover 2 KB in 32 requests instead of
// 128 scattered 4-byte ones.
__device__ __forceinline__ void load_taps2(float (&w)[2][KT], const float* conv_w, size_t row, int K) {
    if (K == KT) {
        const f32x4v t0 = ld4f(conv_w + row * KT), t1 = ld4f(conv_w + (row + 1) * KT);
#pragma unroll
        for (int j = 0; j < KT; ++j) {
            w[0][j] = t0[j];
            w[1][j] = t1[j];
        }
    } else {
        load_taps<KT, 2>(w, conv_w, row, K);
    }
}

// conv + SiLU of the lane's two channels over its RW rows: the window starts from the
// halo rows (or, for the first chunk of a run at the sequence start, from the ring
// copy in LDS: `hist` non-null); wt[e][KT-1] multiplies the current input. With L2U
// the taps carry a factor log2(e), so the conv output u is x log2(e) and the result
// u sigmoid(x) = log2(e) SiLU(x) (for rows that are l2-normalised next, where the
// factor cancels).
template <bool L2U = false>
__device__ __forceinline__ void conv_rows(const uint32_t (&x)[NR], const float* hist, const float (&wt)[2][KT],
                                          float (&y)[RW][2]) {
    float win[HALO][2];
#pragma unroll
    for (int i = 0; i < HALO; ++i) {
        win[i][0] = lo_bf(x[i]);
        win[i][1] = hi_bf(x[i]);
    }
    if (hist) {
#pragma unroll
        for (int i = 0; i < HALO; ++i) {
            win[i][0] = hist[i * DK];
            win[i][1] = hist[i * DK + 1];
        }
    }
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const float xc[2] = {lo_bf(x[HALO + r]), hi_bf(x[HALO + r])};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            float acc = 0.0f;
#pragma unroll
            for (int t = 0; t < HALO; ++t) acc = fmaf(wt[e][t], win[t][e], acc);
            acc = fmaf(wt[e][KT - 1], xc[e], acc);
            if constexpr (L2U) y[r][e] = acc * __builtin_amdgcn_rcpf(1.0f + exp2_f(-acc));
            else y[r][e] = silu_f(acc);
        }
#pragma unroll
        for (int t = 0; t < HALO - 1; ++t)
#pragma unroll
            for (int e = 0; e < 2; ++e) win[t][e] = win[t + 1][e];
#pragma unroll
        for (int e = 0; e < 2; ++e) win[HALO - 1][e] = xc[e];
    }
}

// The KDA gates of the lane's two channels over its RW rows, activated (FORM) and in
// log2 units, as running sums gp[r][e]; rows at or past n are zero.
template <int FORM>
__device__ __forceinline__ void kda_gate_prefix(const uint32_t (&g)[RW], int row0, int n, float lb2, float m,
                                                float k1, const float (&k0)[2], float (&gp)[RW][2]) {
    float acc[2] = {0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const float x[2] = {lo_bf(g[r]), hi_bf(g[r])};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            float v;
            if constexpr (FORM == GATE_GIVEN) v = x[e] * LOG2E;
            else v = gate_act_log2<FORM>(lb2, m, k1, k0[e], x[e]);
            acc[e] += row0 + r < n ? v : 0.0f;
            gp[r][e] = acc[e];
        }
    }
}

// ---------------------------------------------------------------------------------
// Wavefronts 8..15: the state-independent preparation of each chunk. RO = false (the
// segmented arm's runs without readout, which only carry the state) leaves out every
// query-side step: the q rows, their conv, SiLU and norm, and the Q+ tiles.
// ---------------------------------------------------------------------------------
template <bool GDN, bool ACT, bool RO>
__device__ __forceinline__ void c32_prepare(C32Lds<GDN>& sm, const MixerArgs& a, const C32Job& jb, int w,
                                            int lane) {
    const int q4 = lane >> 4, l16 = lane & 15, c2 = 2 * lane, K = a.K, H = a.H, h = jb.h;
    const size_t qkv = (size_t)H * DK, hoff = (size_t)h * DK;
    const size_t kw = (size_t)a.Hk * DK, khead = (size_t)(h % a.Hk) * DK;
    const int nch = (jb.T + C - 1) / C;
    const int pr0 = RW * w;  // this wavefront's first row of a chunk

    // raw rows of the first chunk; beta and the GDN gate stay raw bf16 bits until they
    // are used (converting them at the load would wait for every row load before them)
    uint32_t rq[NR], rk[NR], rg[GDN ? 1 : RW];
    uint32_t rbeta = 0, rgs = 0;
    const uint32_t lane_off = 4u * lane;  // the lane's two channels, in bytes
    auto load_chunk = [&](int c0) {
        if constexpr (RO) load_rows(rq, a.q, kw, khead, lane_off, BUF_ALL, jb, c0, w);
        load_rows(rk, a.k, kw, khead, lane_off, BUF_ALL, jb, c0, w);
        const int gb = min(c0 + pr0, jb.T - 1);  // the wavefront's first row, clamped
        if constexpr (!GDN) {
            const auto rs = buf_rsrc(static_cast<const __bf16*>(a.g) + ((jb.rowb + gb) * qkv + hoff), BUF_ALL);
#pragma unroll
            for (int i = 0; i < RW; ++i)
                rg[i] = __builtin_amdgcn_raw_buffer_load_b32(
                    rs, (int)lane_off, (int)((uint32_t)(min(c0 + pr0 + i, jb.T - 1) - gb) * (uint32_t)(qkv * 2)), 0);
        }
        // beta (and the GDN gate) of row pr0 + lane % RW
        const int boff = (min(c0 + pr0 + (lane & (RW - 1)), jb.T - 1) - gb) * H * 2;
        const size_t hr0 = (jb.rowb + gb) * H + h;
        rbeta = __builtin_amdgcn_raw_buffer_load_b16(buf_rsrc(static_cast<const unsigned short*>(a.beta) + hr0, BUF_ALL),
                                                     boff, 0, 0);
        if constexpr (GDN)
            rgs = __builtin_amdgcn_raw_buffer_load_b16(buf_rsrc(static_cast<const unsigned short*>(a.g) + hr0, BUF_ALL),
                                                       boff, 0, 0);
    };
    // Every load of the prologue is requested before the first wait, so the first step
    // starts after one memory round trip: the first chunk's rows, the conv taps of the
    // lane's q and k channels (parked in LDS for the whole run, each lane reading back
    // only what it wrote), the conv history before the sequence start (the old ring;
    // slot K-1-d is d rows back, oldest first: preparing wavefront 0 convolves the q / k
    // planes of the first chunk, state wavefront 0 the v plane in the next step) and the
    // gate-activation constants.
    load_chunk(0);
    float wtq[2][KT] = {}, wtk[2][KT];
    if constexpr (RO) load_taps2(wtq, a.conv_w, khead + c2, K);
    load_taps2(wtk, a.conv_w, kw + khead + c2, K);
    const bool hist0 = jb.ring_start && w == 0;
    float hv[3][HALO][2];
    if (hist0) {
        const float* ring_b = a.ring + (size_t)jb.b * ring_rows(a) * (K - 1);
#pragma unroll
        for (int pl = 0; pl < 3; ++pl)
#pragma unroll
            for (int d = 1; d <= HALO; ++d)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const size_t fr = plane_row(a, pl, h, c2 + e);
                    const float x = ring_b[fr * (K - 1) + max(K - 1 - d, 0)];
                    hv[pl][HALO - d][e] = d <= K - 1 ? x : 0.0f;
                }
    }
    float gm = 0.0f, gbias = 0.0f, k1 = 0.0f, lb2 = 0.0f, k0[2] = {0.0f, 0.0f};
    if constexpr (GDN) {
        if (a.gate_form != GATE_GIVEN) {
            gm = gate_head_factor(a, h);
            gbias = a.gate_bias[h];
        }
    }
    if constexpr (ACT) {
        gm = gate_head_factor(a, h);
        lb2 = a.gate_lb * LOG2E;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float bias = a.gate_bias[hoff + c2 + e];
            if (a.gate_form == GATE_SIGMOID) gate_log2_consts<GATE_SIGMOID>(gm, bias, &k1, &k0[e]);
            else gate_log2_consts<GATE_SOFTPLUS>(gm, bias, &k1, &k0[e]);
        }
    }
    // the q / k taps times log2(e): their conv outputs are l2-normalised, so the factor
    // leaves the normalised rows as they are and saves a multiply in each SiLU
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        *reinterpret_cast<f32x4v*>(&sm.taps[0][e][lane][0]) =
            LOG2E * f32x4v{wtq[e][0], wtq[e][1], wtq[e][2], wtq[e][3]};
        *reinterpret_cast<f32x4v*>(&sm.taps[1][e][lane][0]) =
            LOG2E * f32x4v{wtk[e][0], wtk[e][1], wtk[e][2], wtk[e][3]};
    }
    if (hist0) {
#pragma unroll
        for (int pl = 0; pl < 3; ++pl)
#pragma unroll
            for (int i = 0; i < HALO; ++i)
#pragma unroll
                for (int e = 0; e < 2; ++e) sm.u.hist[pl][i][c2 + e] = hv[pl][i][e];
        lds_wave_sync();
    }
    auto taps_of = [&](int pl, float (&wt)[2][KT]) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const f32x4v t = ld4f(&sm.taps[pl][e][lane][0]);
#pragma unroll
            for (int j = 0; j < KT; ++j) wt[e][j] = t[j];
        }
    };

    // one step per chunk; the state group's last step (chunk nch - 1) follows the loop
    for (int s = 0; s < nch; ++s) {
        const int c0 = s * C, n = min(C, jb.T - c0), par = s & 1;
        // ---- phase 1: conv + SiLU of q and k, l2 norms, gate prefix ----
        float yq[RW][2], yk[RW][2];
        float gp[GDN ? 1 : RW][2];
        {
            const bool from_hist = jb.ring_start && s == 0 && w == 0;
            {
                float wt[2][KT];
                if constexpr (RO) {
                    taps_of(0, wt);
                    conv_rows<true>(rq, from_hist ? &sm.u.hist[0][0][c2] : nullptr, wt, yq);
                } else {
#pragma unroll
                    for (int r = 0; r < RW; ++r) yq[r][0] = yq[r][1] = 0.0f;
                }
                taps_of(1, wt);
                conv_rows<true>(rk, from_hist ? &sm.u.hist[1][0][c2] : nullptr, wt, yk);
            }
            float ps[8];
#pragma unroll
            for (int r = 0; r < RW; ++r) {
                ps[r] = fmaf(yq[r][0], yq[r][0], yq[r][1] * yq[r][1]);
                ps[RW + r] = fmaf(yk[r][0], yk[r][0], yk[r][1] * yk[r][1]);
            }
            const int brow = pr0 + (lane & (RW - 1));
            if constexpr (!GDN) {
                if constexpr (ACT) {
                    if (a.gate_form == GATE_SIGMOID)
                        kda_gate_prefix<GATE_SIGMOID>(rg, pr0, n, lb2, gm, k1, k0, gp);
                    else
                        kda_gate_prefix<GATE_SOFTPLUS>(rg, pr0, n, lb2, gm, k1, k0, gp);
                } else {
                    kda_gate_prefix<GATE_GIVEN>(rg, pr0, n, lb2, gm, k1, k0, gp);
                }
                *reinterpret_cast<float2*>(&sm.gsum[w][c2]) = make_float2(gp[RW - 1][0], gp[RW - 1][1]);
            } else {
                const float gx = __uint_as_float(rgs << 16);
                float gv = a.gate_form != GATE_GIVEN ? gate_act_core(a.gate_form, a.gate_lb, gm, gbias, gx) : gx;
                gv = (lane < RW && brow < n) ? gv * LOG2E : 0.0f;
#pragma unroll
                for (int off = 1; off < RW; off *= 2) {
                    const float t = __shfl_up(gv, off, RW);
                    if ((lane & (RW - 1)) >= off) gv += t;
                }
                if (lane < RW) sm.gsum[0][brow] = gv;
                if (lane == RW - 1) sm.gsum[1][w] = gv;
            }
            const float bval = beta_in(a, __uint_as_float(rbeta << 16));
            if (lane < RW) sm.beta[par][brow] = brow < n ? bval : 0.0f;
            // l2 norms: lane l gets plane (l >> 3) / RW, row (l >> 3) % RW of this wavefront
            const float ss = sum8x64(ps, lane);
            // the rows carry log2(e) (the taps), and the eps its square, so the result is
            // the plain l2 norm's; the q rows also take the attention scale, which O then
            // inherits through Q+ and P
            if ((lane & 7) == 0) {
                const float inv = rsqrtf(ss + L2_EPS * (LOG2E * LOG2E));
                sm.nrm[w][lane >> 3] = lane < 32 ? inv * a.scale : inv;
            }
            // the next chunk's rows (the registers above are consumed)
            asm volatile("" ::: "memory");
            load_chunk(c0 + C);
        }
        lds_barrier();  // B1

        // ---- phase 2: decay factors and operand tiles ----
        {
            float nr[8];
            {
                const f32x4v v0 = ld4f(&sm.nrm[w][0]), v1 = ld4f(&sm.nrm[w][4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    nr[e] = v0[e];
                    nr[4 + e] = v1[e];
                }
            }
            const int pc = pchan(c2);
            if constexpr (!GDN) {
                // gate sums before this wavefront's rows (off), of rows 0..15 (r1) and of
                // the chunk (tot); w is wave-uniform
                float acc[2] = {0.0f, 0.0f}, off[2] = {0.0f, 0.0f}, r1[2] = {0.0f, 0.0f};
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) {
                    if (ww == w) {
                        off[0] = acc[0];
                        off[1] = acc[1];
                    }
                    if (ww == NW / 2) {
                        r1[0] = acc[0];
                        r1[1] = acc[1];
                    }
                    const float2 s2 = *reinterpret_cast<const float2*>(&sm.gsum[ww][c2]);
                    acc[0] += s2.x;
                    acc[1] += s2.y;
                }
                float er1[2];  // e^{R_1}
#pragma unroll
                for (int e = 0; e < 2; ++e) er1[e] = exp2_f(r1[e]);
                if (w == 0) *reinterpret_cast<float2*>(&sm.ffn[par][c2]) = make_float2(exp2_f(acc[0]), exp2_f(acc[1]));
                // Block a's rows: gamma = G - R_a; Q+ and K+ are the block-relative tiles
                // times e^{R_a} (R_0 = 0, so block 0's are its qa and ka rows and only
                // block 1 stores them), and block 0 also stores k e^{-gamma} e^{R_1}, the
                // operand of the L and P block (1, 0).
                auto tiles = [&](auto blk1c) {
                    constexpr bool blk1 = decltype(blk1c)::value;
                    float kd[2][RW], fl[2];  // fl: e^{G_l - R_a}
#pragma unroll
                    for (int e = 0; e < 2; ++e) fl[e] = exp2_f(acc[e] - (blk1 ? r1[e] : 0.0f));
#pragma unroll
                    for (int r = 0; r < RW; ++r) {
                        bf16x2 oqa, oqp, oka, okp, okb, okb1;
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const float gam = off[e] + gp[r][e] - (blk1 ? r1[e] : 0.0f);
                            const float e1 = exp2_f(gam), e2 = exp2_f(-gam);
                            const float qh = yq[r][e] * nr[r], kh = yk[r][e] * nr[RW + r];
                            const float qa = qh * e1, ka = kh * e1, kbv = kh * e2;
                            if constexpr (RO) oqa[e] = (__bf16)qa;
                            oka[e] = (__bf16)ka;
                            okb[e] = (__bf16)kbv;
                            if constexpr (blk1) {
                                if constexpr (RO) oqp[e] = (__bf16)(qa * er1[e]);
                                okp[e] = (__bf16)(ka * er1[e]);
                            } else {
                                okb1[e] = (__bf16)(kbv * er1[e]);
                            }
                            kd[e][r] = kbv * fl[e];
                        }
                        const int row = pr0 + r;
                        if constexpr (RO) st2(&sm.qa[row][pc], oqa);
                        st2(&sm.ka[row][pc], oka);
                        st2(&sm.kb[row][pc], okb);
                        if constexpr (blk1) {
                            if constexpr (RO) st2(&sm.qp[row][pc], oqp);
                            st2(&sm.kp[row][pc], okp);
                        } else {  // block 0: Q+ and K+ are qa and ka themselves (R_0 = 0)
                            st2(&sm.kb1[row][pc], okb1);
                        }
                    }
                    // K_dec^T: the wavefront's 4 rows are contiguous in the permuted order
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const bf16x4 v4{(__bf16)kd[e][0], (__bf16)kd[e][1], (__bf16)kd[e][2], (__bf16)kd[e][3]};
                        *reinterpret_cast<bf16x4*>(&sm.kdt[par][c2 + e][swz(perm32(pr0), c2 + e)]) = v4;
                    }
                };
                if (w >= NW / 2) tiles(std::true_type{});
                else tiles(std::false_type{});
            } else {
                if (w == 0 && lane < C) {
                    float g = sm.gsum[0][lane];
#pragma unroll
                    for (int ww = 0; ww < NW - 1; ++ww)
                        if (ww < lane / RW) g += sm.gsum[1][ww];
                    sm.gcum[par][lane] = g;
                    // the row factors of the state group, once per chunk
                    const float gl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), C - 1));  // G_l
                    sm.gpos[par][lane] = exp2_f(g);
                    sm.gdec[par][lane] = exp2_f(gl - g);
                }
                float kk[2][RW];
#pragma unroll
                for (int r = 0; r < RW; ++r) {
                    bf16x2 oq, ok;
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        oq[e] = (__bf16)(yq[r][e] * nr[r]);
                        kk[e][r] = yk[r][e] * nr[RW + r];
                        ok[e] = (__bf16)kk[e][r];
                    }
                    if constexpr (RO) st2(&sm.qa[pr0 + r][pc], oq);
                    st2(&sm.ka[pr0 + r][pc], ok);
                }
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const bf16x4 v4{(__bf16)kk[e][0], (__bf16)kk[e][1], (__bf16)kk[e][2], (__bf16)kk[e][3]};
                    *reinterpret_cast<bf16x4*>(&sm.kdt[par][c2 + e][swz(perm32(pr0), c2 + e)]) = v4;
                }
            }
        }
        lds_barrier();  // B2

    }
    // the state group's step for the last chunk
    lds_barrier();
    lds_barrier();
}

// One 16 x 16 block of L = diag(beta) strictly-lower(K+ K-^T) or P = lower(Q+ K-^T) of a
// chunk (KDA: block-relative operands; GDN: k^ and q^ with the scalar decay applied per
// entry), jw: 0 L(0,0), 1 P(0,0), 2 L(1,1), 3 P(1,1), 4 L(1,0), 5 P(1,0). L blocks go
// to the solve's arrays (diagonal blocks transposed), P blocks to pb (its block (0,1)
// above the diagonal stays zero from the start of the run).
template <bool GDN>
__device__ __forceinline__ void lp_block(C32Lds<GDN>& sm, int jw, int par, int lane) {
    // the lane-derived LDS addresses are formed here, not held in registers across the
    // caller's loop (the opaque copy keeps them from being hoisted)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int q4 = ln >> 4, l16 = ln & 15;
    const bool doL = (jw & 1) == 0;
    const int ab = jw < 2 ? 0 : 1, bb = (jw == 2 || jw == 3) ? 1 : 0;  // row block, column block
    const int srow = 16 * ab + l16;
    // the column operand: k^ (GDN); k^ e^{-gamma} of block bb, for block (1, 0) times e^{R_1}
    const __bf16* brow_p = GDN ? &sm.ka[16 * bb + l16][0] : (jw >= 4 ? &sm.kb1[l16][0] : &sm.kb[16 * bb + l16][0]);
    const __bf16* arow_p = doL ? &sm.ka[srow][0] : &sm.qa[srow][0];
    f32x4v acc = zero4();  // lane: X[srow][16 bb + 4 q4 + r]
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {  // operands in two batches of two (registers are scarce here)
        bf16x8 bo[2], ao[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            bo[i] = ld8(brow_p + 32 * (2 * kh + i) + 8 * q4);
            ao[i] = ld8(arow_p + 32 * (2 * kh + i) + 8 * q4);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 2; ++i) acc = mfma_bf16(bo[i], ao[i], acc);
    }
    const int j0 = 16 * bb + 4 * q4;
    if (doL) {
        const float bs = sm.beta[par][srow];
        f32x4v lv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = j0 + r;
            float ef = 1.0f;
            if constexpr (GDN) ef = exp2_f(fminf(sm.gcum[par][srow] - sm.gcum[par][j], 0.0f));
            lv[r] = j < srow ? bs * (acc[r] * ef) : 0.0f;
        }
        if (ab == bb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.ltd[ab][(4 * q4 + r) * LDT + l16] = lv[r];
        } else {
            *reinterpret_cast<f32x4v*>(&sm.lf10[l16][4 * q4]) = lv;
        }
    } else {
        bf16x4 pv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = j0 + r;
            float ef = 1.0f;
            if constexpr (GDN) ef = exp2_f(fminf(sm.gcum[par][srow] - sm.gcum[par][j], 0.0f));
            pv[r] = (__bf16)(j <= srow ? acc[r] * ef : 0.0f);
        }
        *reinterpret_cast<bf16x4*>(&sm.pb[srow][perm32(j0)]) = pv;
    }
}

// ---------------------------------------------------------------------------------
// Wavefronts 0..7: the state; in step s the v conv and the state-dependent work of
// chunk s-1. RO = false (runs without readout) carries only the state: no P blocks,
// Q+ S, O, gated norm or output stores.
// ---------------------------------------------------------------------------------
template <bool GDN, bool RO>
__device__ __forceinline__ void c32_state(C32Lds<GDN>& sm, const MixerArgs& a, const C32Job& jb, int w,
                                          int lane) {
    const int tid = w * 64 + lane;  // 0..511 within the group
    const int q4 = lane >> 4, l16 = lane & 15, c2 = 2 * lane, K = a.K;
    const size_t qkv = (size_t)a.H * DK, hoff = (size_t)jb.h * DK;
    const size_t kw = (size_t)a.Hk * DK;
    const int nch = (jb.T + C - 1) / C;
    const int vcol = 16 * w + l16;  // this lane's value column

    // the epilogue's item: row tid / 16, columns c8 .. c8 + 7
    const int c8 = (tid & 15) * 8, erow = tid >> 4;
    // Every load of the prologue is requested before the first wait, so the run starts
    // after one memory round trip: the first chunk's v rows, the norm weight and the
    // conv taps of the lane's v channels (parked in LDS for the whole run, each lane
    // reading back only what it wrote), then the state.
    const uint32_t lane_off = 4u * lane;  // the lane's two v channels, in bytes
    const size_t vstride = (size_t)a.H * DK;
    uint32_t rv[NR];
    load_rows(rv, a.v, vstride, hoff, lane_off, jb.vbytes, jb, 0, w);
    f32x4v n0 = zero4(), n1 = zero4();
    if constexpr (RO) {
        n0 = ld4f(&a.norm_w[c8]);
        n1 = ld4f(&a.norm_w[c8 + 4]);
    }
    float wt[2][KT];
    load_taps<KT, 2>(wt, a.conv_w, 2 * kw + hoff + c2, K);
    // ---- state: accS[kt] holds keys 16 kt + 4 q4 .. +3 of value column vcol ----
    f32x4v accS[8];
    if (jb.s_init == 0) {
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) accS[kt] = ld4f(&jb.s_in[(size_t)vcol * DK + 16 * kt + 4 * q4]);
    } else {  // the segmented arm's runs from zero and from the identity: formed in place
        const float one = jb.s_init == 2 ? 1.0f : 0.0f;
#pragma unroll
        for (int kt = 0; kt < 8; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) accS[kt][r] = 16 * kt + 4 * q4 + r == vcol ? one : 0.0f;
    }
    // The loop below waits for its prefetched v rows behind the three stores of the
    // previous chunk's epilogue and one gate load (vector-memory counters complete in
    // order). Its entry must show the compiler the same order, or the merged count waits
    // for everything: the state has landed (the empty asm reads it, and so everything
    // requested before it has too), then three stores and a load from an empty range (no
    // memory access) follow.
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) asm volatile("" ::"v"(accS[kt]));
    if constexpr (RO) {
        *reinterpret_cast<f32x4v*>(&sm.normw[c8]) = n0;
        *reinterpret_cast<f32x4v*>(&sm.normw[c8 + 4]) = n1;
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) *reinterpret_cast<f32x4v*>(&sm.taps[2][e][lane][0]) = f32x4v{wt[e][0], wt[e][1], wt[e][2], wt[e][3]};
    // the epilogue's z loads and out / o_core stores: row erow of the chunk, columns
    // c8 .. c8 + 7; rows at or past the chunk's end fall outside the buffer's range (no
    // access), and so does every store of a run without readout or of a null o_core
    const uint32_t eoff = (uint32_t)(erow * qkv + c8) * 2u;
    const uint32_t orow = (uint32_t)(qkv * 2);  // bytes of one bf16 row
    const bool ocore = jb.readout && a.o_core;
    bf16x8 zold{};  // the output gates of the chunk whose epilogue runs next
    if constexpr (RO) {
        const auto none = buf_rsrc(a.out, 0u);
        const u32x4v zero{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < 3; ++i) __builtin_amdgcn_raw_buffer_store_b128(zero, none, (int)eoff + 16 * i, 0, 0);
        // and, as each step ends with its gate load, one from an empty range (zeros)
        zold = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(buf_rsrc(a.z, 0u), (int)eoff, 0, 0));
    }

    if (tid == 0) sm.tcnt = 0u;  // before the barriers below; counted per chunk from here
    if (RO && tid < 64) {  // P block (0, 1), above the diagonal: zero for the whole run
        const __bf16 z = (__bf16)0.0f;
        *reinterpret_cast<bf16x4*>(&sm.pb[tid & 15][perm32(16 + 4 * (tid >> 4))]) = bf16x4{z, z, z, z};
    }
    // step 0: the preparing group's first chunk
    lds_barrier();
    lds_barrier();
    f32x4v oacc[2], racc[2];  // [mt] O^T, K+ S
    // Gated RMSNorm and stores of chunk ce (ce < 0: nothing stored) from its O staging;
    // rows at or past the chunk's end fall outside the buffer's range (no access), and
    // so does every store of a run without readout or of a null o_core.
    auto epilogue = [&](int ce, const bf16x8& zg) {
        const int ne = ce >= 0 ? min(C, jb.T - ce * C) : 0;
        const size_t row0e = jb.rowb + (size_t)max(ce, 0) * C;
        float o8[8], w8[8];
        const f32x4v oa = ld4f(&sm.u.ost[ce & 1][erow][c8]), ob = ld4f(&sm.u.ost[ce & 1][erow][c8 + 4]);
        const f32x4v wa = ld4f(&sm.normw[c8]), wb = ld4f(&sm.normw[c8 + 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            w8[e] = wa[e];
            w8[4 + e] = wb[e];
        }
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o8[e] = oa[e];
            o8[4 + e] = ob[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(o8[e], o8[e], ss);
        ss = sum_row16(ss);  // the 16 lanes of a DPP row share erow
        const float inv = rsqrtf(fmaf(ss, 1.0f / DK, a.rms_eps));
        bf16x8 yb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float zf = (float)zg[e];
            const float gate = GDN ? silu_f(zf) : sigmoid_f(zf);
            yb[e] = (__bf16)(((o8[e] * inv) * w8[e]) * gate);
        }
        const uint32_t rows = jb.readout ? (uint32_t)ne : 0u;
        const auto outr = buf_rsrc(static_cast<__bf16*>(a.out) + (row0e * qkv + hoff), rows * orow);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4v, yb), outr, (int)eoff, 0, 0);
        const auto ocr = buf_rsrc(ocore ? a.o_core + (row0e * qkv + hoff) : nullptr, ocore ? (uint32_t)ne * 2u * orow : 0u);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4v{__float_as_uint(o8[0]), __float_as_uint(o8[1]), __float_as_uint(o8[2]), __float_as_uint(o8[3])},
                                               ocr, (int)(2u * eoff), 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4v{__float_as_uint(o8[4]), __float_as_uint(o8[5]), __float_as_uint(o8[6]), __float_as_uint(o8[7])},
                                               ocr, (int)(2u * eoff + 16u), 0, 0);
    };
    for (int c = 0; c < nch; ++c) {
        const int par = c & 1, c0 = c * C, n = min(C, jb.T - c0);
        const size_t row0 = jb.rowb + c0;
        // ---- phase 1: v conv; diagonal blocks of T; Q+ S as O^T and K+ S ----
        {
            float yv[RW][2], wv[2][KT];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const f32x4v t = ld4f(&sm.taps[2][e][lane][0]);
#pragma unroll
                for (int j = 0; j < KT; ++j) wv[e][j] = t[j];
            }
            const bool from_hist = jb.ring_start && c == 0 && w == 0;
            conv_rows(rv, from_hist ? &sm.u.hist[2][0][c2] : nullptr, wv, yv);
            // v^T: the wavefront's 4 rows are contiguous in the permuted order
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const bf16x4 v4{(__bf16)yv[0][e], (__bf16)yv[1][e], (__bf16)yv[2][e], (__bf16)yv[3][e]};
                *reinterpret_cast<bf16x4*>(&sm.vbt[c2 + e][swz(perm32(RW * w), c2 + e)]) = v4;
            }
        }
        if (w == 2 || w == 3) {
            __builtin_amdgcn_s_setprio(3);  // the longest chain of the phase
            // the diagonal block of L this wavefront inverts (wavefront 3 also L(1,0))
            if (w == 2) {
                lp_block<GDN>(sm, 0, par, lane);
            } else {
                lp_block<GDN>(sm, 2, par, lane);
                lp_block<GDN>(sm, 4, par, lane);
            }
            lds_wave_sync();  // read back across lanes below
            // T_aa = (I + A_aa)^-1, block a = w - 2 on this wavefront (the two blocks on two
            // SIMDs): forward substitution in column (axpy) order, all 64 lanes; lane
            // (col = lane / 4, rg = lane % 4) holds rows 4 rg .. 4 rg + 3 of column col.
            // Step cc takes the pivot x[cc] from its owner in the quad (DPP broadcast) and
            // subtracts A[r][cc] x[cc] from every row r. A_aa is strictly lower triangular,
            // so rows r <= cc subtract exact zeros. Column cc of A_aa is row cc of the
            // transposed copy, read one step ahead.
            // this block's lane-derived LDS addresses are formed here, not held in
            // registers across the loop (the opaque copy keeps them from being hoisted)
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const int col = ln >> 2, rg = ln & 3, bq4 = ln >> 4, bl16 = ln & 15;
            const int bb = w - 2;
            float x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = (4 * rg + i == col) ? 1.0f : 0.0f;
            f32x4v nxt = ld4f(&sm.ltd[bb][4 * rg]);
#pragma unroll
            for (int cc = 0; cc < 15; ++cc) {
                const f32x4v cur = nxt;
                if (cc + 1 < 15) nxt = ld4f(&sm.ltd[bb][(cc + 1) * LDT + 4 * rg]);
                const float piv = quad_bcast(x[cc & 3], cc >> 2);  // from the quad lane owning row cc
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = fmaf(-cur[i], piv, x[i]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.tdiag[bb][4 * rg + i][col] = x[i];
            lds_wave_sync();  // the reads below cross lanes of this wavefront
            // T as the A fragments of every state wavefront (lane: rows 16 mt + l16; slots
            // e < 4 -> column 4 q4 + e, e >= 4 -> column 16 + 4 q4 + e - 4)
            const __bf16 z = (__bf16)0.0f;
            if (bb == 0) {
                const f32x4v t00 = ld4f(&sm.tdiag[0][bl16][4 * bq4]);
                sm.tfrag[0][ln] = bf16x8{(__bf16)t00[0], (__bf16)t00[1], (__bf16)t00[2], (__bf16)t00[3], z, z, z, z};
                // T_00 is in place (the wait above): wavefront 3 may read it
                if (ln == 0) __hip_atomic_fetch_add(&sm.tcnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            } else {
                // T_10 = -T_11 A_10 T_00, formed transposed in registers: Y = A_10^T T_11^T
                // (slot k = 4 kk + q4), then T_10^T = T_00^T Y (negated) with Y fed back
                // as the B operand (slot k = 4 q4 + kk); the lane ends with T_10[l16][4 q4 + r].
                float la[4], lb[4], lc[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    la[kk] = sm.lf10[4 * kk + bq4][bl16];
                    lb[kk] = sm.tdiag[1][bl16][4 * kk + bq4];
                }
                const f32x4v t11 = ld4f(&sm.tdiag[1][bl16][4 * bq4]);
                f32x4v y = zero4();
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) y = mfma_f32(la[kk], lb[kk], y);
                // T_00 of this chunk from wavefront 2: its count of finished blocks
                // reaches c + 1. The two solves take the same time; the wait is bounded
                // (about 2 ms of polling), and a wait that ran out poisons T_10 with NaN so
                // the outputs show it instead of holding silently wrong values.
                bool ready = false;
                for (int it = 0; it < (1 << 16) && !ready; ++it) {
                    const uint32_t done = __builtin_amdgcn_readfirstlane(*static_cast<volatile uint32_t*>(&sm.tcnt));
                    ready = done > (uint32_t)c;
                    if (!ready) __builtin_amdgcn_s_sleep(1);
                }
                asm volatile("" ::: "memory");
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) lc[kk] = sm.tdiag[0][4 * bq4 + kk][bl16];
                f32x4v t10 = zero4();
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) t10 = mfma_f32(lc[kk], y[kk], t10);
                if (!ready) t10 = f32x4v{NAN, NAN, NAN, NAN};
                sm.tfrag[1][ln] = bf16x8{(__bf16)(-t10[0]), (__bf16)(-t10[1]), (__bf16)(-t10[2]), (__bf16)(-t10[3]),
                                           (__bf16)t11[0], (__bf16)t11[1], (__bf16)t11[2], (__bf16)t11[3]};
            }
            __builtin_amdgcn_s_setprio(2);
        } else if (RO && (w == 0 || w == 1 || w == 5)) {  // the blocks of P (read in phase 2)
            lp_block<GDN>(sm, w == 0 ? 1 : (w == 1 ? 3 : 5), par, lane);
        }
        // the next chunk's v rows
        asm volatile("" ::: "memory");
        load_rows(rv, a.v, vstride, hoff, lane_off, jb.vbytes, jb, c0 + C, w);
        // O^T (lane: O[16 mt + l16][16 w + 4 q4 + r]) and K+ S (lane: R[16 mt + 4 q4 + r]
        // [vcol]); the state packed to bf16 is the operand with its keys in the
        // accumulator (perm32) order
        {
            bf16x8 sbop[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) sbop[kk] = pack2(accS[2 * kk], accS[2 * kk + 1]);
            // (KDA: block 0's rows of Q+ and K+ are qa and ka, R_0 = 0; block 1's are qp, kp)
            const __bf16* qsrc0 = &sm.qa[0][0];
            const __bf16* ksrc0 = &sm.ka[0][0];
            const __bf16* qsrc1 = GDN ? &sm.qa[0][0] : &sm.qp[0][0];
            const __bf16* ksrc1 = GDN ? &sm.ka[0][0] : &sm.kp[0][0];
            // LDS operands in batches issued together (a scheduling fence keeps the
            // reads ahead of their uses, so each batch costs one round trip)
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                oacc[mt] = zero4();
                racc[mt] = zero4();
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) {
                    bf16x8 qf[2], kf[2];
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const int off = (16 * mt + l16) * LDR + 32 * (2 * kh + i) + 8 * q4;
                        if constexpr (RO) qf[i] = ld8((mt == 0 ? qsrc0 : qsrc1) + off);
                        kf[i] = ld8((mt == 0 ? ksrc0 : ksrc1) + off);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        if constexpr (RO) oacc[mt] = mfma_bf16(sbop[2 * kh + i], qf[i], oacc[mt]);
                        racc[mt] = mfma_bf16(kf[i], sbop[2 * kh + i], racc[mt]);
                    }
                }
            }
            // the decay of the state update, diag(e^{G_l}) S (the old S is packed above)
            if constexpr (GDN) {
                const float fg = sm.gpos[par][C - 1];  // e^{G_l}
#pragma unroll
                for (int kt = 0; kt < 8; ++kt) accS[kt] *= fg;
            } else {
#pragma unroll
                for (int kh = 0; kh < 2; ++kh) {
                    f32x4v d[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) d[i] = ld4f(&sm.ffn[par][16 * (4 * kh + i) + 4 * q4]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) accS[4 * kh + i] *= d[i];
                }
            }
        }
        lds_barrier();  // B1

        // ---- phase 2: Ub = T diag(beta) (V - K+ S), O, state update ----
        {
            const bf16x8 ta0 = sm.tfrag[0][lane], ta1 = sm.tfrag[1][lane];
            const f32x4v be0 = ld4f(&sm.beta[par][4 * q4]), be1 = ld4f(&sm.beta[par][16 + 4 * q4]);
            const bf16x8 vv = ld8(&sm.vbt[vcol][swz(8 * q4, vcol)]);
            __builtin_amdgcn_sched_barrier(0);

            f32x4v gr0 = f32x4v{1.0f, 1.0f, 1.0f, 1.0f}, gr1 = gr0;  // GDN: e^{G_j} of the lane's rows
            if constexpr (GDN) {
                gr0 = ld4f(&sm.gpos[par][4 * q4]);
                gr1 = ld4f(&sm.gpos[par][16 + 4 * q4]);
            }
            bf16x8 xb;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                xb[r] = (__bf16)(be0[r] * ((float)vv[r] - racc[0][r] * gr0[r]));
                xb[4 + r] = (__bf16)(be1[r] * ((float)vv[4 + r] - racc[1][r] * gr1[r]));
            }
            // Ub[16 mt + 4 q4 + r][vcol]
            const f32x4v ub0 = mfma_bf16(ta0, xb, zero4()), ub1 = mfma_bf16(ta1, xb, zero4());
            const bf16x8 ubo = pack2(ub0, ub1);  // Ub as operand
            bf16x8 ubs = ubo;                    // for the state update (GDN: rows times e^{G_l - G_j})
            if constexpr (GDN) {
                const f32x4v d0 = ld4f(&sm.gdec[par][4 * q4]), d1 = ld4f(&sm.gdec[par][16 + 4 * q4]);
                ubs = pack2(ub0 * d0, ub1 * d1);
            }
            // O^T = (Q+ S)^T + Ub^T P^T (GDN: Q+ S is q S with rows times e^{G_s})
            if constexpr (RO) {
                const bf16x8 p0 = ld8(&sm.pb[l16][8 * q4]), p1 = ld8(&sm.pb[16 + l16][8 * q4]);
                if constexpr (GDN) {
                    oacc[0] *= sm.gpos[par][l16];
                    oacc[1] *= sm.gpos[par][16 + l16];
                }
                oacc[0] = mfma_bf16(ubo, p0, oacc[0]);
                oacc[1] = mfma_bf16(ubo, p1, oacc[1]);
            }
            // S = diag(e^{G_l}) S + K_dec^T Ub (the decay was applied in phase 1)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                bf16x8 kd[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) kd[i] = ld8(&sm.kdt[par][16 * (4 * kh + i) + l16][swz(8 * q4, 16 * (4 * kh + i))]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < 4; ++i) accS[4 * kh + i] = mfma_bf16(kd[i], ubs, accS[4 * kh + i]);
            }
            // the previous chunk's epilogue while the matrix cores run the products above,
            // then this chunk's output gates (used by the next step's epilogue)
            if constexpr (RO) {
                epilogue(c - 1, zold);
                const auto zr = buf_rsrc(static_cast<const __bf16*>(a.z) + (row0 * qkv + hoff), (uint32_t)n * orow);
                zold = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(zr, (int)eoff, 0, 0));
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    *reinterpret_cast<f32x4v*>(&sm.u.ost[par][16 * mt + l16][16 * w + 4 * q4]) = oacc[mt];
            }
        }
        lds_barrier();  // B2
    }
    if constexpr (RO) epilogue(nch - 1, zold);

#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
        *reinterpret_cast<f32x4v*>(&jb.s_out[(size_t)vcol * DK + 16 * kt + 4 * q4]) = accS[kt];
}

template <bool GDN, bool ACT, bool SEG>
__global__ __launch_bounds__(NT) void c32_kernel(MixerArgs a) {
    static_assert(!(GDN && ACT), "GDN gates are activated per row at run time");
    __shared__ C32Lds<GDN> sm;

    int bh;
    SegRun sr{};
    if constexpr (SEG) {
        if (!seg_run(a, &sr)) return;  // whole block exits before any barrier
        bh = sr.pair;
    } else {
        bh = blockIdx.x;
        if (bh >= a.B * a.H) return;
        bh = seq_of(a, bh / a.H) * a.H + bh % a.H;  // packed batches: longest sequences first
    }
    C32Job jb;
    jb.b = bh / a.H;
    jb.h = bh % a.H;
    seq_span(a, jb.b, &jb.rowb, &jb.T);
    if constexpr (SEG) {
        jb.rowb += sr.ro;
        jb.T = sr.len;
    }
    jb.ring_start = !SEG || sr.ro == 0;
    jb.lo = jb.ring_start ? 0 : -HALO;
    jb.readout = !SEG || sr.readout;
    const bool zero_v = SEG && sr.zero_v;
    jb.vbytes = zero_v ? 0u : BUF_ALL;
    jb.s_in = SEG ? sr.s_in : a.state_in + (size_t)bh * DK * DK;
    jb.s_init = SEG ? sr.s_init : 0;
    jb.s_out = SEG ? sr.s_out : a.state_out + (size_t)bh * DK * DK;

    const int tid = threadIdx.x, lane = tid & 63;
    // wave-uniform: every row index built from it is scalar arithmetic
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (jb.T == 0) {  // an empty run: the state passes through
        const f32x4v* src = reinterpret_cast<const f32x4v*>(jb.s_in);
        f32x4v* dst = reinterpret_cast<f32x4v*>(jb.s_out);
        for (int i = tid; i < DK * DK / 4; i += NT) {
            if (jb.s_init == 0) {
                dst[i] = src[i];
            } else {  // zero or identity ([value][key]: entry i covers keys 4 (i % 32) .. +3)
                f32x4v x = zero4();
#pragma unroll
                for (int r = 0; r < 4; ++r) x[r] = jb.s_init == 2 && (4 * i + r) / DK == (4 * i + r) % DK ? 1.0f : 0.0f;
                dst[i] = x;
            }
        }
        return;  // uniform over the workgroup, before any barrier
    }
    // The state group carries the critical path of every step, so it issues first: it
    // holds the older wavefronts (the SIMD arbiter favours them) and a raised priority,
    // and the preparing group fills the issue slots it leaves.
    if (wave >= NW) {
        // the segmented arm's runs without readout take the state-only specialisation
        if (!SEG || jb.readout) c32_prepare<GDN, ACT, true>(sm, a, jb, wave - NW, lane);
        else c32_prepare<GDN, ACT, false>(sm, a, jb, wave - NW, lane);
    } else {
        __builtin_amdgcn_s_setprio(2);
        if (!SEG || jb.readout) c32_state<GDN, true>(sm, a, jb, wave, lane);
        else c32_state<GDN, false>(sm, a, jb, wave, lane);
        // The segmented arm's last segment writes the new conv ring (the last K-1 input
        // rows, T >= K-1 there): only pass 1 read the old one, and it has finished. The
        // value head's v rows here; a key head's q / k rows by its first value head only.
        if constexpr (SEG) {
            if (seg_ring_fused(a) && sr.readout && sr.ro > 0 && sr.ro + sr.len == a.T) {
                const int K = a.K;
                const size_t kw = (size_t)a.Hk * DK, vw = (size_t)a.H * DK;
                const int nrow = (jb.h < a.Hk ? 3 : 1) * DK;  // v rows, then q and k rows
                float* ring_b = a.ring + (size_t)jb.b * ring_rows(a) * (K - 1);
                const size_t rlast = jb.rowb - sr.ro + a.T;  // one past the sequence's last row
                for (int i = tid; i < nrow; i += GT) {
                    const int pl = i < DK ? 2 : i / DK - 1, ch = i % DK;
                    const void* x = pl == 0 ? a.q : (pl == 1 ? a.k : a.v);
                    const size_t xw = pl == 2 ? vw : kw, xc = (size_t)(pl == 2 ? jb.h : jb.h % a.Hk) * DK + ch;
                    float* row = ring_b + plane_row(a, pl, jb.h, ch) * (K - 1);
                    for (int d = 1; d <= K - 1; ++d) row[K - 1 - d] = ld_act<true>(x, (rlast - d) * xw + xc);
                }
            }
        }
    }
}

template <bool GDN, bool SEG>
hipError_t c32_launch(const MixerArgs& a, int grid) {
    static_assert(sizeof(C32Lds<GDN>) <= 160 * 1024, "LDS of one workgroup");
    if (grid <= 0) return hipSuccess;
    const dim3 g(grid), blk(NT);
    if (!GDN && a.gate_form != GATE_GIVEN)
        hipLaunchKernelGGL((c32_kernel<GDN, !GDN, SEG>), g, blk, 0, a.stream, a);
    else
        hipLaunchKernelGGL((c32_kernel<GDN, false, SEG>), g, blk, 0, a.stream, a);
    return hipGetLastError();
}

}  // namespace

bool chunked32_fits(const MixerArgs& a) { return a.bf16 && a.D == DK && a.K <= KT; }

hipError_t launch_chunked32(const MixerArgs& a) {
    if (!chunked32_fits(a)) return hipErrorInvalidValue;
    const int grid = a.B * a.H;
    const hipError_t e = a.gdn ? c32_launch<true, false>(a, grid) : c32_launch<false, false>(a, grid);
    if (e != hipSuccess) return e;
    return launch_ring_roll(a, false);
}

hipError_t launch_seg_pass32(const MixerArgs& a, int grid) {
    return a.gdn ? c32_launch<true, true>(a, grid) : c32_launch<false, true>(a, grid);
}

}  // namespace kda
