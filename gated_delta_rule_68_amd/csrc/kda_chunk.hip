// Chunked prefill arm of the KDA / GDN mixer for gfx950 (D = 128, chunks of 64).
//
// The recurrence is taken 64 tokens at a time in its WY / UT form (memra-engine
// kda.rs, module notes on the chunked twin: a per-channel cumulative log gate,
// k scaled by exp(-Gcum) and q by exp(+Gcum), and a triangular intra-chunk solve;
// for GDN the cumulative gate is one scalar per (token, head)). Per chunk of n rows
// with carried state S (key i x value j) and G the inclusive cumulative log gate:
//   L[s][j] = sum_i k_s[i] k_j[i] e^{G_s[i]-G_j[i]}  (j < s)
//   P[s][j] = sum_i q_s[i] k_j[i] e^{G_s[i]-G_j[i]}  (j <= s)
//   T  = (I + diag(beta) L)^-1
//   W  = T diag(beta) (e^{G} * k),   U = T diag(beta) v
//   Ub = U - W S,   O = scale ((e^{G} * q) S + P Ub)
//   S  = diag(e^{G_last}) S + (e^{G_last - G} * k)^T Ub
//
// Decay factorisation. The 64 rows form four 16-row blocks; with B_a = G at the
// first row of block a and gamma_s = G_s - B_{a(s)} (a sum of at most 15 gates), the
// conv stage writes three decayed operand tiles once per chunk,
//   qa = q e^{gamma},  ka = k e^{gamma},  kb = k e^{-gamma},
// and a table of per-block, per-channel factors e^{B_a}, e^{G_last - B_a},
// e^{B_a - B_b} (a > b) and e^{G_last}. Every decayed operand of the chunk is then one
// of these tiles times one table entry:
//   L, P block (a, b):  ka_s (or qa_s) . (e^{B_a - B_b} kb_j)     (the factor is 1 on the diagonal)
//   W row j:            beta_j e^{B_{a(j)}} ka_j
//   O row s:            e^{B_{a(s)}} qa_s
//   S update row j:     e^{G_last - B_{a(j)}} kb_j
// so the exponentials are taken once per (row, channel) instead of once per use.
// Every factor is <= 1 except e^{-gamma} <= e^{75} (15 gates >= -5), inside the
// fp32 / bf16 range; this is why the arm needs g >= -5.
//
// One workgroup of 8 wavefronts owns one (sequence, head, value-column split) and
// walks the chunks in order; the state lives in MFMA accumulator registers as S
// tiles (wavefront w holds key block w). All contractions run on
// v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32 accumulation); the 64x64
// unit-triangular inverse is solved in fp32 (16x16 diagonal blocks by forward
// substitution, off-diagonal blocks with v_mfma_f32_16x16x4f32). conv + SiLU and l2
// run in-kernel on the raw inputs, so the only HBM traffic is the raw activations,
// the gates, the output and the state once in and once out. For bf16 inputs the raw
// rows of chunk c+1 are requested while chunk c computes.
//
// Variants carried by the same kernel: gates given as pre-activations (template flag
// ACT for KDA: activated once per element at the raw-row store, kept as split fp32
// halves; GDN: activated at that store at run time); query / key rows read from key
// head h % Hk (grouped heads); packed batches, whose sequences take their rows from an
// offsets table and are dispatched longest first.
#include "kda_chunk_common.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

const bool kChunkedArmBuilt = true;

namespace {

constexpr int CH = 64;         // chunk length
constexpr int DK = 128;        // head dim of this arm
constexpr int NTHR = 512;      // 8 wavefronts (two per SIMD)
constexpr int LDH = DK + 8;    // bf16 row stride of [*][128] tiles (272 B: 16-byte aligned, skewed banks)
constexpr int LDC = CH + 8;    // bf16 row stride of [*][64] tiles (144 B)
constexpr int LDF = CH + 4;    // fp32 row stride of the 64x64 solve matrices

// Eight consecutive activations from element `off` (a multiple of 8), as bf16.
template <bool BF>
__device__ __forceinline__ bf16x8 ld_act8(const void* p, size_t off) {
    if constexpr (BF) {
        return *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p) + off);
    } else {
        const float4* f = reinterpret_cast<const float4*>(static_cast<const float*>(p) + off);
        const float4 x = f[0], y = f[1];
        return bf16x8{(__bf16)x.x, (__bf16)x.y, (__bf16)x.z, (__bf16)x.w,
                      (__bf16)y.x, (__bf16)y.y, (__bf16)y.z, (__bf16)y.w};
    }
}

// MFMA 16x16x32 operand layout (lane l, q4 = l / 16, l16 = l % 16): an A fragment
// holds A[l16][8*q4 .. 8*q4+7] of a 16x32 tile, a B fragment B[8*q4 .. +7][l16] of a
// 32x16 tile, and the 16x16 result D[4*q4 + r][l16] for r = 0..3. With both operands
// stored "row = M or N index, contiguous = K index" one loader serves A and B.
// Swapping the two fragments yields the transposed tile: mfma(B-frag, A-frag) leaves
// (AB)[l16][4*q4 + r] in lane l, four consecutive columns of one row, which this file
// uses wherever a result is stored row-major so that the store is one vector write.

// Rows of the per-block factor table (one float per channel; GDN uses column 0).
enum : int {
    F_EBR = 0,   // [4] e^{B_a}
    F_ELR = 4,   // [4] e^{G_last - B_a}
    F_DAB = 8,   // [6] e^{B_a - B_b}, a > b, row F_DAB + a(a-1)/2 + b
    F_FN = 14,   // e^{G_last}
    F_TOT = 15,  // [4] sum of the 16 gates of block a, times log2 e
    F_G0 = 19,   // [4] gate of the first row of block a, times log2 e
    NFAC = 23
};
__device__ __forceinline__ int dab_row(int a, int b) { return F_DAB + a * (a - 1) / 2 + b; }

template <bool GDN, int NC, int KT>
struct ChunkLds {
    alignas(16) __bf16 qa[CH][LDH];  // q^ e^{gamma}
    alignas(16) __bf16 ka[CH][LDH];  // k^ e^{gamma}
    alignas(16) __bf16 kb[CH][LDH];  // k^ e^{-gamma}
    alignas(16) __bf16 hist[KT - 1][2 * DK + NC];  // raw rows before the chunk: [d-1] is d rows back
    alignas(16) float beta[CH];
    alignas(16) float fac[NFAC][GDN ? 4 : DK];
    alignas(16) float nrm[8][16];  // per-wave 1/||row|| of the l2 norm
    union {
        struct {
            __bf16 rq[CH][LDH];               // raw q rows of the chunk
            __bf16 rk[CH][LDH];               // raw k rows
            __bf16 rg[GDN ? 1 : CH][LDH];     // raw gates (KDA), zero past row n
            float gs[CH];                     // raw scalar gates (GDN), zero past row n
        } raw;
        struct {
            union {
                struct {
                    float lf[CH][LDF];             // A = beta_s L[s][j], blocks below the diagonal
                    float ltd[4][16 * 16 + 4];     // diagonal blocks of A, transposed: [a][c * 16 + r] = A[16a+r][16a+c]
                    float tdiag[4][16][17];        // diagonal blocks of T in fp32
                } solve;
                __bf16 wneg[CH][LDH];         // -W
                __bf16 ubt[NC][LDC];          // Ub^T [value][row]
            } w;
            __bf16 tb[CH][LDC];               // T in bf16
            __bf16 pb[CH][LDC];               // P (lower incl. diagonal)
        } m;
    } c;
    union {
        struct {
            union {
                __bf16 vbt[NC][LDC];    // (beta v)^T [value][row]
                uint16_t glo[CH][LDH];  // activated KDA gates: low 16 bits (raw store to P1)
            } vb;
            __bf16 rv[CH][NC + 8];   // raw v rows of the split
        } pre;
        __bf16 sb[NC][LDH];  // S^T in bf16 [value][key]
    } e;
};

// Split index / (b, h) of a block: the column splits of one (b, h) share blockIdx % 8,
// so they run on the same XCD and share its L2 for the raw q / k / g rows they all read.
__device__ __forceinline__ void block_coords(int ncol, int nbh, int* bh, int* split) {
    const int x = blockIdx.x;
    const int group = x / (8 * ncol), within = x % (8 * ncol);
    *split = within / 8;
    *bh = group * 8 + within % 8;
    if (*bh >= nbh) *bh = -1;
}

// Raw rows of one chunk held in registers between their load (issued one chunk ahead
// for bf16 inputs, so the HBM latency overlaps the previous chunk's compute) and
// their store into LDS. Item it of thread tid covers row (tid + 512 it) / 16 and the
// 8 channels ((tid + 512 it) % 16) * 8 of q, k and the gate; v items cover the NC
// value channels of the split.
template <bool GDN, int NC>
struct ChunkRaw {
    static constexpr int NI = CH * (DK / 8) / NTHR;               // 2
    static constexpr int VITEMS = CH * (NC / 8);                  // v items of the chunk
    static constexpr int NV = (VITEMS + NTHR - 1) / NTHR;         // 1 or 2
    bf16x8 q[NI], k[NI], g[GDN ? 1 : NI], v[NV];
    float beta, gs;  // rows tid < CH: beta and (GDN) the scalar gate
};

// Every load is unconditional from a clamped, in-bounds row (rows past T repeat row
// T-1) and nothing consumes the values until the next chunk's P1: a load inside a
// divergent branch, or a select right after it, makes the compiler wait for the load
// on the spot, which would stall on the prefetch itself. Rows past T are masked
// where they are stored (gates and beta) or consumed (conv outputs).
// Parts of one chunk's rows, so that the requests can be spread over the phases of
// the previous chunk: a burst of all of them stalls every wavefront at the issue.
enum RawPart { RAW_Q, RAW_K, RAW_G, RAW_V, RAW_BETA };
// rowb, T: first activation row and row count (>= 1) of the sequence. v rows are
// read from vsrc with row stride vstride (a.v and H*D, or a zero row and 0).
template <bool BF, bool GDN, int NC, RawPart PART>
__device__ __forceinline__ void load_raw_part(ChunkRaw<GDN, NC>& cr, const MixerArgs& a, size_t rowb, int T,
                                              int h, int c0, int jv0, int tid, const void* vsrc, size_t vstride) {
    using CR = ChunkRaw<GDN, NC>;
    const int H = a.H;
    const size_t qkv = (size_t)H * DK, head_off = (size_t)h * DK;
    const size_t kw = (size_t)a.Hk * DK, khead = (size_t)(h % a.Hk) * DK;  // q / k: key head
    if constexpr (PART == RAW_Q || PART == RAW_K || PART == RAW_G) {
        if constexpr (PART == RAW_G && GDN) return;
#pragma unroll
        for (int it = 0; it < CR::NI; ++it) {
            const int idx = tid + NTHR * it, r = idx / (DK / 8), c8 = (idx % (DK / 8)) * 8;
            const size_t row = rowb + min(c0 + r, T - 1);
            if constexpr (PART == RAW_Q) cr.q[it] = ld_act8<BF>(a.q, row * kw + khead + c8);
            if constexpr (PART == RAW_K) cr.k[it] = ld_act8<BF>(a.k, row * kw + khead + c8);
            if constexpr (PART == RAW_G && !GDN) cr.g[it] = ld_act8<BF>(a.g, row * qkv + head_off + c8);
        }
    } else if constexpr (PART == RAW_V) {
#pragma unroll
        for (int it = 0; it < CR::NV; ++it) {
            const int idx = min(tid + NTHR * it, CR::VITEMS - 1);
            const int r = idx / (NC / 8), c8 = (idx % (NC / 8)) * 8;
            cr.v[it] = ld_act8<BF>(vsrc, (rowb + min(c0 + r, T - 1)) * vstride + head_off + jv0 + c8);
        }
    } else {
        const int rr = tid & (CH - 1);
        const size_t hr = (rowb + min(c0 + rr, T - 1)) * H + h;
        cr.beta = ld_act<BF>(a.beta, hr);
        cr.gs = GDN ? ld_act<BF>(a.g, hr) : 0.0f;
    }
}
template <bool BF, bool GDN, int NC>
__device__ __forceinline__ void load_raw(ChunkRaw<GDN, NC>& cr, const MixerArgs& a, size_t rowb, int T,
                                         int h, int c0, int jv0, int tid, const void* vsrc, size_t vstride) {
    load_raw_part<BF, GDN, NC, RAW_Q>(cr, a, rowb, T, h, c0, jv0, tid, vsrc, vstride);
    load_raw_part<BF, GDN, NC, RAW_K>(cr, a, rowb, T, h, c0, jv0, tid, vsrc, vstride);
    load_raw_part<BF, GDN, NC, RAW_G>(cr, a, rowb, T, h, c0, jv0, tid, vsrc, vstride);
    load_raw_part<BF, GDN, NC, RAW_V>(cr, a, rowb, T, h, c0, jv0, tid, vsrc, vstride);
    load_raw_part<BF, GDN, NC, RAW_BETA>(cr, a, rowb, T, h, c0, jv0, tid, vsrc, vstride);
}

// The raw rows of a chunk (n valid rows) from registers into LDS; the gates and beta
// are zero past row n, so G stays at G[n-1] and padded rows change nothing. Every
// thread stores every item it loaded (threads with the same clamped item store the
// same value): a store under a branch leaves its load possibly in flight on the
// other path, and the compiler then waits for all memory traffic at the loop head.
// Gate-activation constants of a thread. GDN: the head factor and bias of its head,
// applied at the raw store with the launch's form. KDA with activated gates: the
// folded constants (gate_log2_consts) of the 8 channels the thread stores.
struct ChunkGate {
    float m, gb;    // GDN
    float k1, lb2;  // KDA
    float k0[8];
};

// KDA gates activated once per element as the raw rows are stored, in log2 units and
// fp32, kept as their high (rg) and low (glo) 16 bits; rows at or past n are 0 (masked
// on the packed words, so that no branch is formed around the activation).
template <int FORM, bool GDN, int NC, typename Lds>
__device__ __forceinline__ void store_gates(Lds& sm, const ChunkRaw<GDN, NC>& raw, int n, int tid,
                                            const ChunkGate& cg) {
    using CR = ChunkRaw<GDN, NC>;
#pragma unroll
    for (int it = 0; it < CR::NI; ++it) {
        const int idx = tid + NTHR * it, r = idx / (DK / 8), c8 = (idx % (DK / 8)) * 8;
        const uint32_t keep = r < n ? 0xffffffffu : 0u;
        uint4 hi, lo;
        uint32_t* h = &hi.x;
        uint32_t* l = &lo.x;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t u0 = __float_as_uint(gate_act_log2<FORM>(cg.lb2, cg.m, cg.k1, cg.k0[2 * p],
                                                                    (float)raw.g[it][2 * p]));
            const uint32_t u1 = __float_as_uint(gate_act_log2<FORM>(cg.lb2, cg.m, cg.k1, cg.k0[2 * p + 1],
                                                                    (float)raw.g[it][2 * p + 1]));
            h[p] = (u0 >> 16) | (u1 & 0xffff0000u);
            l[p] = (u0 & 0xffffu) | (u1 << 16);
        }
        if (n < CH) {  // uniform: only the last chunk has rows to clear
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                h[p] &= keep;
                l[p] &= keep;
            }
        }
        *reinterpret_cast<uint4*>(&sm.c.raw.rg[r][c8]) = hi;
        *reinterpret_cast<uint4*>(&sm.e.pre.vb.glo[r][c8]) = lo;
    }
}

template <bool GDN, int NC, bool ACT, typename Lds>
__device__ __forceinline__ void store_raw(Lds& sm, const ChunkRaw<GDN, NC>& raw, int n, int tid,
                                          const MixerArgs& a, const ChunkGate& cg) {
    using CR = ChunkRaw<GDN, NC>;
#pragma unroll
    for (int it = 0; it < CR::NI; ++it) {
        const int idx = tid + NTHR * it, r = idx / (DK / 8), c8 = (idx % (DK / 8)) * 8;
        st8(&sm.c.raw.rq[r][c8], raw.q[it]);
        st8(&sm.c.raw.rk[r][c8], raw.k[it]);
        if constexpr (!GDN && !ACT) st8(&sm.c.raw.rg[r][c8], r < n ? raw.g[it] : zero8());
    }
    if constexpr (!GDN && ACT) {
        if (a.gate_form == GATE_SIGMOID)
            store_gates<GATE_SIGMOID>(sm, raw, n, tid, cg);
        else
            store_gates<GATE_SOFTPLUS>(sm, raw, n, tid, cg);
    }
#pragma unroll
    for (int it = 0; it < CR::NV; ++it) {
        const int idx = min(tid + NTHR * it, CR::VITEMS - 1), r = idx / (NC / 8), c8 = (idx % (NC / 8)) * 8;
        st8(&sm.e.pre.rv[r][c8], raw.v[it]);
    }
    // beta and (GDN) the scalar gates are activated here in fp32
    const int rr = tid & (CH - 1);
    sm.beta[rr] = rr < n ? (GDN ? beta_in(a, raw.beta) : (ACT ? sigmoid_f(raw.beta) : raw.beta)) : 0.0f;
    if constexpr (GDN)
        sm.c.raw.gs[rr] = rr < n ? (a.gate_form != GATE_GIVEN ? gate_act_core(a.gate_form, a.gate_lb, cg.m, cg.gb, raw.gs)
                                                               : raw.gs)
                                 : 0.0f;
}

// Gate prefix of one 16-row block over two channels (KDA), in log2 units: gm[r][e] is
// the gate sum of rows 1..r, g0 the gate of row 0, tot the block's sum. rg points at
// row 0, channel pair e = 0, 1 of the raw gate rows (pitch LDH).
__device__ __forceinline__ void gate_prefix_given(const __bf16* rg, float (&gm)[16][2], float (&g0)[2],
                                                  float (&tot)[2]) {
    const bf16x2 gf = ld2(rg);
    float acc[2] = {0.0f, 0.0f};
#pragma unroll
    for (int r = 1; r < 16; ++r) {
        const bf16x2 gv = ld2(rg + r * LDH);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            acc[e] = fmaf((float)gv[e], LOG2E, acc[e]);
            gm[r][e] = acc[e];
        }
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        g0[e] = (float)gf[e] * LOG2E;
        tot[e] = g0[e] + acc[e];
    }
}
// The same from gates already activated and in log2 units, stored as the high (rg)
// and low (glo, same pitch) 16 bits of their fp32 values: exact, no bf16 rounding.
__device__ __forceinline__ void gate_prefix_split(const __bf16* rg, const uint16_t* glo, float (&gm)[16][2],
                                                  float (&g0)[2], float (&tot)[2]) {
    float acc[2] = {0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const uint32_t hi = *reinterpret_cast<const uint32_t*>(rg + r * LDH);
        const uint32_t lo = *reinterpret_cast<const uint32_t*>(glo + r * LDH);
        const float g[2] = {__uint_as_float((hi << 16) | (lo & 0xffffu)),
                            __uint_as_float((hi & 0xffff0000u) | (lo >> 16))};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            if (r == 0) {
                g0[e] = g[e];
            } else {
                acc[e] += g[e];
                gm[r][e] = acc[e];
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) tot[e] = g0[e] + acc[e];
}

// N consecutive bf16 channels (N = 1 or 2) as floats.
template <int N>
__device__ __forceinline__ void ld_chan(const __bf16* p, float (&x)[N]) {
    if constexpr (N == 2) {
        const bf16x2 v = ld2(p);
        x[0] = (float)v[0];
        x[1] = (float)v[1];
    } else {
        x[0] = (float)*p;
    }
}

// One causal-conv step over N channels: win holds the KT-1 previous raw inputs (oldest
// first), x the current one; returns SiLU of the sum and slides the window. Rows past
// the end of the sequence are not masked here: they hold copies of the last row
// (finite), and with beta = 0 and zero gates on those rows they drop out of A, W, U,
// the state update and the stored outputs.
template <int KT, int N>
__device__ __forceinline__ void conv_step(float (&win)[KT - 1][N], const float (&x)[N], const float (&w)[N][KT],
                                          float (&y)[N]) {
#pragma unroll
    for (int e = 0; e < N; ++e) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < KT - 1; ++j) acc = fmaf(w[e][j], win[j][e], acc);
        acc = fmaf(w[e][KT - 1], x[e], acc);
        y[e] = silu_f(acc);
    }
#pragma unroll
    for (int j = 0; j < KT - 2; ++j)
#pragma unroll
        for (int e = 0; e < N; ++e) win[j][e] = win[j + 1][e];
#pragma unroll
    for (int e = 0; e < N; ++e) win[KT - 2][e] = x[e];
}

// Column block BB of T below the diagonal: T_ab = -T_aa X_ab with
// X_ab = sum_{c=BB}^{a-1} A_ac T_cb, a = BB+1 .. 3 (v_mfma_f32_16x16x4f32; lane l holds
// A[l16][k] and B[k][l16] of each 4-wide k slice). X and the T_cb of this column stay in
// registers in the result layout (lane holds rows 4 q4 .. 4 q4 + 3 of column l16);
// they enter the next product as its B operand with the k slice permuted to
// k = 4 q4 + kk, and the A operand is read from LDS with the same permutation.
template <int BB, typename M>
__device__ __forceinline__ void merge_column(M& m, int lane) {
    const int q4 = lane >> 4, l16 = lane & 15;
    const auto& lf = m.w.solve.lf;
    const auto& td = m.w.solve.tdiag;
    f32x4v tcol[3 - BB];  // T_{BB+1,BB} .. T_{3,BB}
#pragma unroll
    for (int a = BB + 1; a < 4; ++a) {
        f32x4v x = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)  // c = BB: T_bb from LDS, k = 4 kk + q4
            x = mfma_f32(lf[16 * a + l16][16 * BB + 4 * kk + q4], td[BB][4 * kk + q4][l16], x);
#pragma unroll
        for (int c = BB + 1; c < a; ++c)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)  // k = 4 q4 + kk
                x = mfma_f32(lf[16 * a + l16][16 * c + 4 * q4 + kk], tcol[c - BB - 1][kk], x);
        f32x4v y = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) y = mfma_f32(td[a][l16][4 * q4 + kk], x[kk], y);
        tcol[a - BB - 1] = -y;
#pragma unroll
        for (int r = 0; r < 4; ++r) m.tb[16 * a + 4 * q4 + r][16 * BB + l16] = (__bf16)(-y[r]);
    }
}

// ACT (KDA only): the gates arrive as pre-activations and are activated in P1; the
// given-gate kernel carries none of that code. SEG: a workgroup of the segmented arm
// (NC = 128), mapped by seg_run.
template <bool BF, bool GDN, int NC, int KT, bool ACT, bool SEG = false>
__global__ __launch_bounds__(NTHR) void chunk_kernel(MixerArgs a, float* o_buf) {
    static_assert(!(GDN && ACT), "GDN gates are activated where they are stored");
    static_assert(!SEG || NC == DK, "segments run every value column in one workgroup");
    constexpr int NCOL = DK / NC;
    constexpr int NJB = NC / 16;  // value-column 16-blocks of this split
    constexpr int HLD = 2 * DK + NC;
    __shared__ ChunkLds<GDN, NC, KT> sm;
    using CR = ChunkRaw<GDN, NC>;

    int bh, split;
    SegRun sr{};
    if constexpr (SEG) {
        if (!seg_run(a, &sr)) return;  // whole block exits before any barrier
        bh = sr.pair;
        split = 0;
    } else {
        block_coords(NCOL, a.B * a.H, &bh, &split);
        if (bh < 0) return;  // whole block exits before any barrier
        bh = seq_of(a, bh / a.H) * a.H + bh % a.H;  // packed batches: longest sequences first
    }
    const float* s_in = SEG ? sr.s_in : a.state_in + (size_t)bh * DK * DK;
    float* s_out = SEG ? sr.s_out : a.state_out + (size_t)bh * DK * DK;

    int tid = threadIdx.x, lane = tid & 63;
    const int wave = tid >> 6;
    int q4 = lane >> 4, l16 = lane & 15;
    const int b = bh / a.H, h = bh % a.H;
    const int K = a.K;
    size_t rowb;  // first activation row of this sequence
    int T;        // its row count
    seq_span(a, b, &rowb, &T);
    if constexpr (SEG) {
        rowb += sr.ro;
        T = sr.len;
    }
    // Re-materialise the lane indices at every phase: otherwise the compiler hoists
    // each phase's lane-dependent LDS addresses out of the chunk loop and keeps them
    // all alive at once, which overflows the register file.
#define KDA_LAUNDER_LANE()                                                 \
    do {                                                                   \
        asm volatile("" : "+v"(tid), "+v"(lane), "+v"(q4), "+v"(l16));     \
    } while (0)
    const size_t qkv = (size_t)a.H * DK;
    const size_t head_off = (size_t)h * DK;
    const size_t kw = (size_t)a.Hk * DK, khead = (size_t)(h % a.Hk) * DK;  // q / k: key head h % Hk
    const int jv0 = split * NC;  // first value column of this split
    // v rows, and the outputs' base and row stride. Runs without readout skip the
    // output stores (a branch on a workgroup-uniform value, taken the same way in
    // every chunk); the dummy row only keeps their addresses valid.
    const bool zero_v = SEG && sr.zero_v, readout = !SEG || sr.readout;
    char* const seg_ws = reinterpret_cast<char*>(a.seg_ws);
    const void* const vsrc = zero_v ? static_cast<const void*>(seg_ws) : a.v;
    const size_t vstride = zero_v ? 0 : qkv;
    void* const outp = readout ? a.out : static_cast<void*>(seg_ws + (SEG ? seg_layout(0, a.H, DK, 1).dummy : 0));
    float* const obp = readout ? o_buf : static_cast<float*>(outp);
    const size_t orow = readout ? qkv : 0;

    // ---- state: S tiles (key block `wave`, value block jb): lane holds keys
    // 16 wave + 4 q4 .. +3 of value column 16 jb + l16 ----
    f32x4v accS[NJB];
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
        const int jv = jv0 + jb * 16 + l16;
        accS[jb] = ld4f(&s_in[(size_t)jv * DK + 16 * wave + 4 * q4]);
    }
    // Wavefront (sw, hv) = (wave % 4, wave / 4) owns rows 16*sw.. of U / Ub / O and the
    // value blocks [hv*NJB2, (hv+1)*NJB2).
    constexpr int NJB2 = NJB / 2;
    const int sw = wave & 3, hv = wave >> 2;

    // ---- conv history of the first chunk: the old ring (slot K-1-d is d rows back),
    // or for a segment past the sequence start the raw rows before it ----
    if (!SEG || sr.ro == 0) {
        const float* ring_b = a.ring + (size_t)b * ring_rows(a) * (K - 1);
        for (int idx = tid; idx < (KT - 1) * HLD; idx += NTHR) {
            const int d = idx / HLD + 1, col = idx % HLD;
            const size_t fr = col < 2 * DK ? (size_t)(col / DK) * kw + khead + col % DK
                                           : 2 * kw + head_off + jv0 + (col - 2 * DK);
            sm.hist[d - 1][col] = (__bf16)(d <= K - 1 ? ring_b[fr * (K - 1) + K - 1 - d] : 0.0f);
        }
    } else {
        for (int idx = tid; idx < (KT - 1) * HLD; idx += NTHR) {
            const int d = idx / HLD + 1, col = idx % HLD;
            const size_t row = rowb - (size_t)min(d, K - 1);  // segments start >= 64 rows in
            const float x = col < DK       ? ld_act<BF>(a.q, row * kw + khead + col)
                            : col < 2 * DK ? ld_act<BF>(a.k, row * kw + khead + col - DK)
                                           : ld_act<BF>(vsrc, row * vstride + head_off + jv0 + col - 2 * DK);
            sm.hist[d - 1][col] = (__bf16)(d <= K - 1 ? x : 0.0f);
        }
    }

    // Conv roles. q / k (P1): wavefront w convolves both, rows 16 (w % 4) + 8 (w / 4)
    // .. +7 (half of one 16-row block), channels 2 lane and 2 lane + 1, so the l2 norm
    // of a row is a sum over the 64 lanes of one wavefront and the block's gate prefix
    // is a per-thread running sum. v (P3, while wavefronts 0..3 solve for
    // T): items (NVCH channels, 16-row block) on the threads of wavefronts 4..7, NVP
    // per thread, all of the same channels.
    constexpr int NVCH = NC == 128 ? 2 : 1;
    constexpr int NVIT = 4 * NC / NVCH, NVP = (NVIT + NTHR / 2 - 1) / (NTHR / 2);
    static_assert((NTHR / 2) % (NC / NVCH) == 0, "the v items of a thread share its channels");
    const int vt = tid - NTHR / 2;  // >= 0 on wavefronts 4..7
    const int cv = (vt % (NC / NVCH)) * NVCH;

    // Gate-activation constants (unused for given gates), read once: a global load
    // inside the chunk loop would be waited for together with the prefetch.
    ChunkGate cg{};
    if constexpr (GDN) {
        cg.m = gate_head_factor(a, h);
        cg.gb = a.gate_bias[h];
    }
    if constexpr (ACT) {
        const float* bp = a.gate_bias + head_off + (tid % (DK / 8)) * 8;  // the store channels
        const f32x4v b0 = ld4f(bp), b1 = ld4f(bp + 4);
        const float bias[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        cg.m = gate_head_factor(a, h);
        cg.lb2 = a.gate_lb * LOG2E;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (a.gate_form == GATE_SIGMOID)
                gate_log2_consts<GATE_SIGMOID>(cg.m, bias[e], &cg.k1, &cg.k0[e]);
            else
                gate_log2_consts<GATE_SOFTPLUS>(cg.m, bias[e], &cg.k1, &cg.k0[e]);
        }
    }

    if (T == 0) {  // an empty sequence of a packed batch: the state passes through
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
            const int jv = jv0 + jb * 16 + l16;
            *reinterpret_cast<f32x4v*>(&s_out[(size_t)jv * DK + 16 * wave + 4 * q4]) = accS[jb];
        }
        return;  // uniform over the workgroup, before any barrier
    }

    CR raw;
    load_raw<BF, GDN, NC>(raw, a, rowb, T, h, 0, jv0, tid, vsrc, vstride);
    store_raw<GDN, NC, ACT>(sm, raw, min(CH, T), tid, a, cg);
    __syncthreads();

    for (int c0 = 0; c0 < T; c0 += CH) {
        const int n = min(CH, T - c0);
        const size_t row0 = rowb + c0;

        KDA_LAUNDER_LANE();
        // ---- P0: conv taps and norm weight (re-read every chunk: a few L2-resident
        // bytes). They are requested here, before any prefetch of the next chunk:
        // vector-memory counters complete in order, so a small load issued after the
        // prefetch could only be waited for together with all of it.
        float wqk[2][2][KT], wv[NVCH][KT], w8[8];  // wqk[0]: q taps, wqk[1]: k taps
        load_taps<KT, 2>(wqk[0], a.conv_w, khead + 2 * lane, K);
        load_taps<KT, 2>(wqk[1], a.conv_w, kw + khead + 2 * lane, K);
        load_taps<KT, NVCH>(wv, a.conv_w, 2 * kw + head_off + jv0 + max(cv, 0), K);  // used by wavefronts 4..7
        if constexpr (NCOL == 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) w8[e] = a.norm_w[(tid % (DK / 8)) * 8 + e];
        }

        KDA_LAUNDER_LANE();
        // ---- P1: gate prefix, conv + SiLU + l2, decayed operand tiles. The two
        // wavefronts of a SIMD (w and w + 4) share the 16-row block 16 (w % 4): w takes
        // its rows 0..7 and w + 4 rows 8..15, each for both q and k, so the decay
        // exponentials of a (row, channel) serve the q and both k tiles and the two end
        // together. ----
        {
            const int qq = wave & 3, rb = 16 * qq, c2 = 2 * lane, hr = 8 * (wave >> 2);
            constexpr int NG = GDN ? 1 : 2;
            // the gate of row `row`, channel c2 + e, in log2 units, added to acc
            auto add_gate = [&](float acc, int row, int e) -> float {
                if constexpr (GDN) {
                    return fmaf(sm.c.raw.gs[row], LOG2E, acc);
                } else if constexpr (!ACT) {
                    return fmaf((float)ld2(&sm.c.raw.rg[row][c2])[e], LOG2E, acc);
                } else {
                    const uint32_t hi = *reinterpret_cast<const uint32_t*>(&sm.c.raw.rg[row][c2]);
                    const uint32_t lo = *reinterpret_cast<const uint32_t*>(&sm.e.pre.vb.glo[row][c2]);
                    return acc + __uint_as_float(e ? ((hi & 0xffff0000u) | (lo >> 16)) : ((hi << 16) | (lo & 0xffffu)));
                }
            };
            // gamma of this wavefront's rows (gate sum of rows rb+1 .. rb+hr+r)
            float gm[8][NG], acc[NG];
#pragma unroll
            for (int e = 0; e < NG; ++e) acc[e] = 0.0f;
            if (hr) {
#pragma unroll
                for (int i = 1; i <= 8; ++i)
#pragma unroll
                    for (int e = 0; e < NG; ++e) acc[e] = add_gate(acc[e], rb + i, e);
            }
#pragma unroll
            for (int e = 0; e < NG; ++e) gm[0][e] = acc[e];
#pragma unroll
            for (int r = 1; r < 8; ++r)
#pragma unroll
                for (int e = 0; e < NG; ++e) {
                    acc[e] = add_gate(acc[e], rb + hr + r, e);
                    gm[r][e] = acc[e];
                }
            if (!hr) {  // block total and first gate for the factor table
                float g0[NG];
#pragma unroll
                for (int i = 8; i < 16; ++i)
#pragma unroll
                    for (int e = 0; e < NG; ++e) acc[e] = add_gate(acc[e], rb + i, e);
#pragma unroll
                for (int e = 0; e < NG; ++e) g0[e] = add_gate(0.0f, rb, e);
                if constexpr (GDN) {
                    if (lane == 0) {
                        sm.fac[F_TOT + qq][0] = g0[0] + acc[0];
                        sm.fac[F_G0 + qq][0] = g0[0];
                    }
                } else {
                    *reinterpret_cast<float2*>(&sm.fac[F_TOT + qq][c2]) = make_float2(g0[0] + acc[0], g0[1] + acc[1]);
                    *reinterpret_cast<float2*>(&sm.fac[F_G0 + qq][c2]) = make_float2(g0[0], g0[1]);
                }
            }

            // conv + SiLU of 8 rows x 2 channels of q (pl = 0) and k (pl = 1)
            float y[2][8][2], ps[16];
#pragma unroll
            for (int pl = 0; pl < 2; ++pl) {
                const __bf16* rawp = (pl ? &sm.c.raw.rk[0][0] : &sm.c.raw.rq[0][0]) + c2;
                float win[KT - 1][2];
#pragma unroll
                for (int d = 1; d < KT; ++d) {  // row rb + hr - d: in the chunk, or the history
                    const int r = rb + hr - d;
                    const __bf16* src = r >= 0 ? rawp + r * LDH : &sm.hist[-r - 1][(pl ? DK : 0) + c2];
                    const bf16x2 x = ld2(src);
#pragma unroll
                    for (int e = 0; e < 2; ++e) win[KT - 1 - d][e] = (float)x[e];
                }
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const bf16x2 xv = ld2(rawp + (rb + hr + r) * LDH);
                    const float x[2] = {(float)xv[0], (float)xv[1]};
                    conv_step<KT, 2>(win, x, wqk[pl], y[pl][r]);
                    ps[8 * pl + r] = fmaf(y[pl][r][0], y[pl][r][0], y[pl][r][1] * y[pl][r][1]);
                }
            }
            const float ss = sum16x64(ps, lane);  // lane l: plane (l >> 2) / 8, row hr + (l >> 2) % 8
            if ((lane & 3) == 0) sm.nrm[wave][lane >> 2] = rsqrtf(ss + L2_EPS);
            lds_wave_sync();
            float nr[16];
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4v v4 = ld4f(&sm.nrm[wave][4 * r4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) nr[4 * r4 + e] = v4[e];
            }
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                bf16x2 oq, oa, ob;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float g = gm[r][GDN ? 0 : e];
                    const float ep = exp2_f(g), en = exp2_f(-g);
                    const float qh = y[0][r][e] * nr[r], kh = y[1][r][e] * nr[8 + r];
                    oq[e] = (__bf16)(qh * ep);
                    oa[e] = (__bf16)(kh * ep);
                    ob[e] = (__bf16)(kh * en);
                }
                st2(&sm.qa[rb + hr + r][c2], oq);
                st2(&sm.ka[rb + hr + r][c2], oa);
                st2(&sm.kb[rb + hr + r][c2], ob);
            }
        }
        lds_barrier();
        // The last KT-1 raw q / k rows become the next chunk's history (only a full
        // chunk has a successor; the v rows follow in P4, after this chunk's v conv),
        // and the per-block factor table is formed from the block sums.
        if (n == CH) {
            for (int idx = tid; idx < (KT - 1) * (2 * DK / 8); idx += NTHR) {
                const int d = idx / (2 * DK / 8) + 1, col = (idx % (2 * DK / 8)) * 8;
                const __bf16* src = col < DK ? &sm.c.raw.rq[CH - d][col] : &sm.c.raw.rk[CH - d][col - DK];
                st8(&sm.hist[d - 1][col], ld8(src));
            }
        }
        {
            const int c = tid & (DK - 1), part = tid >> 7;
            if (!GDN || c == 0) {
                float tt[4], bs[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) tt[q] = sm.fac[F_TOT + q][c];
                float run = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    bs[q] = run + sm.fac[F_G0 + q][c];  // B_q = G at row 16 q (log2 units)
                    run += tt[q];
                }
                const float gl = run;  // G_last
                if (part == 0) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) sm.fac[F_EBR + q][c] = exp2_f(bs[q]);
                } else if (part == 1) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) sm.fac[F_ELR + q][c] = exp2_f(gl - bs[q]);
                } else if (part == 2) {
                    sm.fac[dab_row(1, 0)][c] = exp2_f(bs[1] - bs[0]);
                    sm.fac[dab_row(2, 0)][c] = exp2_f(bs[2] - bs[0]);
                    sm.fac[dab_row(2, 1)][c] = exp2_f(bs[2] - bs[1]);
                    sm.fac[F_FN][c] = exp2_f(gl);
                } else {
                    sm.fac[dab_row(3, 0)][c] = exp2_f(bs[3] - bs[0]);
                    sm.fac[dab_row(3, 1)][c] = exp2_f(bs[3] - bs[1]);
                    sm.fac[dab_row(3, 2)][c] = exp2_f(bs[3] - bs[2]);
                }
            }
        }
        lds_barrier();

        KDA_LAUNDER_LANE();
        // ---- P2: L and P, 16x16 blocks (a, b). Wavefront w < 4 computes the diagonal
        // block (w, w) (and solves it in P3 without waiting for the others) plus one
        // block below it; wavefronts 4..6 take the remaining blocks below the diagonal
        // before their v conv. Blocks above the diagonal that P6 reads, (0,1) and (2,3),
        // are written as zeros. ----
        {
            const int w = __builtin_amdgcn_readfirstlane(wave);
            // (row block, first column block, second column block or -1)
            const int ab = w < 4 ? w : (w == 4 ? 2 : 3);
            const int bsel[2] = {w < 4 ? w : (w == 4 ? 1 : (w == 5 ? 0 : (w == 6 ? 2 : -1))),
                                 w == 0 ? 1 : (w == 1 || w == 2 ? 0 : (w == 3 ? 1 : (w == 4 ? 3 : -1)))};
            const int ra = 16 * ab, s = ra + l16;
            f32x4v accL[2], accP[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) accL[t] = accP[t] = zero4();
            if (bsel[0] >= 0) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int i0 = 32 * kk + 8 * q4;
                    const bf16x8 ak = ld8(&sm.ka[s][i0]), aq = ld8(&sm.qa[s][i0]);
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const int bb = bsel[t];
                        if (bb < 0 || bb > ab) continue;
                        bf16x8 bk = ld8(&sm.kb[16 * bb + l16][i0]);
                        if (bb < ab) {  // off-diagonal block: rebase from B_b to B_a
                            const float* d = &sm.fac[dab_row(ab, bb)][GDN ? 0 : i0];
#pragma unroll
                            for (int e = 0; e < 8; ++e) bk[e] = (__bf16)((float)bk[e] * d[GDN ? 0 : e]);
                        }
                        accL[t] = mfma_bf16(bk, ak, accL[t]);  // lane: L[ra + l16][16 bb + 4 q4 + r]
                        accP[t] = mfma_bf16(bk, aq, accP[t]);
                    }
                }
            }
            const float bs = sm.beta[s];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int bb = bsel[t], j0 = 16 * bb + 4 * q4;
                if (bb < 0) continue;
                const bool lo = bb <= ab;
                f32x4v lv;
                bf16x4 pv;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    lv[r] = (lo && j0 + r < s) ? bs * accL[t][r] : 0.0f;
                    pv[r] = (__bf16)((lo && j0 + r <= s) ? accP[t][r] : 0.0f);
                }
                if (bb < ab) {
                    *reinterpret_cast<f32x4v*>(&sm.c.m.w.solve.lf[s][j0]) = lv;
                } else if (bb == ab) {  // A[s][16 ab + 4 q4 + r] -> ltd[ab][(4 q4 + r) * 16 + l16]
#pragma unroll
                    for (int r = 0; r < 4; ++r) sm.c.m.w.solve.ltd[ab][(4 * q4 + r) * 16 + l16] = lv[r];
                }
                *reinterpret_cast<bf16x4*>(&sm.c.m.pb[s][j0]) = pv;
            }
        }
        // No barrier here: P3's first step only reads blocks its own wavefront wrote, and
        // the barrier inside P3 orders everything else P2 wrote before its readers.

        // This chunk's output gates z for the norm in P6 are requested here, and the
        // next chunk's raw rows part by part from here to P6; they are stored into LDS
        // at the end of this iteration.
        constexpr int NZ = NCOL == 1 ? CH * (DK / 8) / NTHR : 1;
        bf16x8 zpre[NZ];
        if constexpr (NCOL == 1) {
#pragma unroll
            for (int it = 0; it < NZ; ++it) {
                const int r = (tid + NTHR * it) / (DK / 8), c8 = (tid % (DK / 8)) * 8;
                zpre[it] = ld_act8<BF>(a.z, (row0 + min(r, n - 1)) * qkv + head_off + c8);
            }
        }
        // (unconditional, like the store into LDS at the end of the iteration: past the
        // last chunk the rows clamp to T-1 and are never used, and a branch would make
        // the compiler wait for every outstanding load and store at its join)
        load_raw_part<BF, GDN, NC, RAW_Q>(raw, a, rowb, T, h, c0 + CH, jv0, tid, vsrc, vstride);
        KDA_LAUNDER_LANE();
        // ---- P3: T = (I + A)^-1, A = diag(beta) L, in 16x16 blocks; meanwhile the v conv:
        // rows 0..7 of each 16-row item here, rows 8..15 while wavefronts 0..2 merge the
        // blocks below the diagonal (the other wavefronts would wait there). With the
        // 8-tap window the carried window would spill, so those kernels convolve all 16
        // rows here. ----
        static_assert(NVP == 1, "one v item per thread of wavefronts 4..7");
        constexpr bool VSPLIT = KT <= 4;
        float vwin[KT - 1][NVCH];  // conv window of this thread's v item, kept for rows 8..15
        const int qv = vt / (NC / NVCH), rbv = 16 * qv;
        auto v_half = [&](int r0) {  // conv + SiLU of rows rbv + r0 .. +7, times beta, stored transposed
            float bt[8];
#pragma unroll
            for (int r4 = 0; r4 < 2; ++r4) {
                const f32x4v b4 = ld4f(&sm.beta[rbv + r0 + 4 * r4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) bt[4 * r4 + e] = b4[e];
            }
            bf16x8 o[NVCH];
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                float x[NVCH], y[NVCH];
                ld_chan<NVCH>(&sm.e.pre.rv[rbv + r0 + r][cv], x);
                conv_step<KT, NVCH>(vwin, x, wv, y);
#pragma unroll
                for (int e = 0; e < NVCH; ++e) o[e][r] = (__bf16)(bt[r] * y[e]);
            }
#pragma unroll
            for (int e = 0; e < NVCH; ++e) st8(&sm.e.pre.vb.vbt[cv + e][rbv + r0], o[e]);
        };
        if (wave < 4) {
            lds_wave_sync();  // this wavefront's own diagonal block from P2
            if (q4 == 0) {
                // Diagonal block `wave`, column l16: (I + A_aa) x = e_l16 in column
                // (axpy) order, so each step's 15 - c updates are independent. Column c
                // of A_aa is row c of the transposed copy; the next column is read
                // while this one is applied.
                const float* at = sm.c.m.w.solve.ltd[wave];
                float x[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) x[r] = (r == l16) ? 1.0f : 0.0f;
                f32x4v cur[4], nxt[4];
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) nxt[r4] = ld4f(at + 4 * r4);
#pragma unroll
                for (int c = 0; c < 15; ++c) {
#pragma unroll
                    for (int r4 = 0; r4 < 4; ++r4) cur[r4] = nxt[r4];
                    asm volatile("" ::: "memory");  // at most one column in flight
                    if (c + 1 < 15) {
#pragma unroll
                        for (int r4 = 0; r4 < 4; ++r4) nxt[r4] = ld4f(at + (c + 1) * 16 + 4 * r4);
                    }
#pragma unroll
                    for (int r = c + 1; r < 16; ++r) x[r] = fmaf(-cur[r >> 2][r & 3], x[c], x[r]);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    sm.c.m.w.solve.tdiag[wave][r][l16] = x[r];
                    sm.c.m.tb[16 * wave + r][16 * wave + l16] = (__bf16)x[r];
                }
            }
        } else {
            // zero T's blocks above the diagonal (row block s / 16, column groups of 8)
            for (int idx = vt; idx < CH * (CH / 8); idx += NTHR / 2) {
                const int r = idx / (CH / 8), c8 = (idx % (CH / 8)) * 8;
                if (c8 >= 16 * ((r >> 4) + 1)) st8(&sm.c.m.tb[r][c8], zero8());
            }
            // v: conv + SiLU, times beta, stored transposed (rows 0..7 of the item)
            if (vt < NVIT) {
#pragma unroll
                for (int d = 1; d < KT; ++d) {
                    float x[NVCH];
                    ld_chan<NVCH>(qv > 0 ? &sm.e.pre.rv[rbv - d][cv] : &sm.hist[d - 1][2 * DK + cv], x);
#pragma unroll
                    for (int e = 0; e < NVCH; ++e) vwin[KT - 1 - d][e] = x[e];
                }
                v_half(0);
                if constexpr (!VSPLIT) v_half(8);
            }
        }
        lds_barrier();
        // Blocks below the diagonal, one column block per wavefront:
        // T_ab = -T_aa sum_{c=b}^{a-1} A_ac T_cb for a = b+1 .. 3.
        if (wave == 0) merge_column<0>(sm.c.m, lane);
        else if (wave == 1) merge_column<1>(sm.c.m, lane);
        else if (wave == 2) merge_column<2>(sm.c.m, lane);
        else if (VSPLIT && wave >= 4 && vt < NVIT) v_half(8);
        lds_barrier();

        KDA_LAUNDER_LANE();
        load_raw_part<BF, GDN, NC, RAW_K>(raw, a, rowb, T, h, c0 + CH, jv0, tid, vsrc, vstride);
        // ---- P4: W = T (beta e^{G} k) -> -W in LDS (key block `wave`);
        //      U = T (beta v) in registers (rows 16*sw.., value blocks of half hv) ----
        if (n == CH) {  // the last KT-1 raw v rows become the next chunk's history
            for (int idx = tid; idx < (KT - 1) * (NC / 8); idx += NTHR) {
                const int d = idx / (NC / 8) + 1, col = (idx % (NC / 8)) * 8;
                st8(&sm.hist[d - 1][2 * DK + col], ld8(&sm.e.pre.rv[CH - d][col]));
            }
        }
        f32x4v accU[NJB2];
        {
            const int i = 16 * wave + l16;
            f32x4v accW[4];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) accW[sb] = zero4();
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int j0 = 32 * kk + 8 * q4;
                const float eb = sm.fac[F_EBR + (j0 >> 4)][GDN ? 0 : i];  // e^{B} of the rows' block
                bf16x8 bw;
#pragma unroll
                for (int e = 0; e < 8; ++e) bw[e] = (__bf16)(sm.beta[j0 + e] * eb * (float)sm.ka[j0 + e][i]);
#pragma unroll
                for (int sb = 0; sb < 4; ++sb)  // lane: W[16 sb + l16][16 wave + 4 q4 + r]
                    accW[sb] = mfma_bf16(bw, ld8(&sm.c.m.tb[16 * sb + l16][32 * kk + 8 * q4]), accW[sb]);
            }
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                bf16x4 wv4;
#pragma unroll
                for (int r = 0; r < 4; ++r) wv4[r] = (__bf16)(-accW[sb][r]);
                *reinterpret_cast<bf16x4*>(&sm.c.m.w.wneg[16 * sb + l16][16 * wave + 4 * q4]) = wv4;
            }
#pragma unroll
            for (int t = 0; t < NJB2; ++t) accU[t] = zero4();
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 at = ld8(&sm.c.m.tb[16 * sw + l16][32 * kk + 8 * q4]);
#pragma unroll
                for (int t = 0; t < NJB2; ++t) {
                    const int jb = hv * NJB2 + t;
                    accU[t] = mfma_bf16(at, ld8(&sm.e.pre.vb.vbt[16 * jb + l16][32 * kk + 8 * q4]), accU[t]);
                }
            }
        }
        lds_barrier();

        KDA_LAUNDER_LANE();
        load_raw_part<BF, GDN, NC, RAW_G>(raw, a, rowb, T, h, c0 + CH, jv0, tid, vsrc, vstride);
        // ---- P5: S^T to LDS in bf16, then Ub = U - W S ----
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
            bf16x4 s4;
#pragma unroll
            for (int r = 0; r < 4; ++r) s4[r] = (__bf16)accS[jb][r];
            *reinterpret_cast<bf16x4*>(&sm.e.sb[16 * jb + l16][16 * wave + 4 * q4]) = s4;
        }
        lds_barrier();
        // Ub = U - W S. The state part of P6's output, O = Q+ S (rows 16*sw.., value
        // blocks of half hv), also reads S^T only: from two value blocks per wavefront
        // on (NC >= 64) it is issued here with Ub, whose independent MFMA chain it
        // overlaps (measured 4% off the chunk time there); with one block (NC = 32) it
        // stays in P6.
        constexpr bool O_EARLY = NJB2 >= 2;
        f32x4v accO[NJB2];
#pragma unroll
        for (int t = 0; t < NJB2; ++t) accO[t] = zero4();
        auto o_state_part = [&](int kk, int i0, const bf16x8* sbt) {  // accO += Q+ S, k slice kk
            const bf16x8 qx = ld8(&sm.qa[16 * sw + l16][i0]);
            const float* eb = &sm.fac[F_EBR + sw][GDN ? 0 : i0];  // e^{B} of block sw
            bf16x8 aq;
#pragma unroll
            for (int e = 0; e < 8; ++e) aq[e] = (__bf16)((float)qx[e] * eb[GDN ? 0 : e]);
#pragma unroll
            for (int t = 0; t < NJB2; ++t)  // lane: O[s][16 jb + 4 q4 + r]
                accO[t] = mfma_bf16(sbt[t], aq, accO[t]);
        };
#pragma unroll 2
        for (int kk = 0; kk < 4; ++kk) {
            const int i0 = 32 * kk + 8 * q4;
            const bf16x8 aw = ld8(&sm.c.m.w.wneg[16 * sw + l16][i0]);
            bf16x8 sbt[NJB2];
#pragma unroll
            for (int t = 0; t < NJB2; ++t) {
                sbt[t] = ld8(&sm.e.sb[16 * (hv * NJB2 + t) + l16][i0]);
                accU[t] = mfma_bf16(aw, sbt[t], accU[t]);
            }
            if constexpr (O_EARLY) o_state_part(kk, i0, sbt);
        }
        lds_barrier();  // every read of -W is done before Ub^T overwrites it
#pragma unroll
        for (int t = 0; t < NJB2; ++t) {
            bf16x4 u4;
#pragma unroll
            for (int r = 0; r < 4; ++r) u4[r] = (__bf16)accU[t][r];
            *reinterpret_cast<bf16x4*>(&sm.c.m.w.ubt[16 * (hv * NJB2 + t) + l16][16 * sw + 4 * q4]) = u4;
        }
        lds_barrier();

        KDA_LAUNDER_LANE();
        load_raw_part<BF, GDN, NC, RAW_V>(raw, a, rowb, T, h, c0 + CH, jv0, tid, vsrc, vstride);
        load_raw_part<BF, GDN, NC, RAW_BETA>(raw, a, rowb, T, h, c0 + CH, jv0, tid, vsrc, vstride);
        // ---- P6: O = scale (Q+ S + P Ub), rows 16*sw.., value blocks of half hv ----
        {
            const int s = 16 * sw + l16;
            if constexpr (!O_EARLY) {
#pragma unroll 2
                for (int kk = 0; kk < 4; ++kk) {
                    const int i0 = 32 * kk + 8 * q4;
                    bf16x8 sbt[NJB2];
#pragma unroll
                    for (int t = 0; t < NJB2; ++t) sbt[t] = ld8(&sm.e.sb[16 * (hv * NJB2 + t) + l16][i0]);
                    o_state_part(kk, i0, sbt);
                }
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (32 * kk > 16 * sw + 15) break;  // P is lower triangular
                const bf16x8 ap = ld8(&sm.c.m.pb[s][32 * kk + 8 * q4]);
#pragma unroll
                for (int t = 0; t < NJB2; ++t)
                    accO[t] = mfma_bf16(ld8(&sm.c.m.w.ubt[16 * (hv * NJB2 + t) + l16][32 * kk + 8 * q4]), ap, accO[t]);
            }
        }
        // O goes through LDS (over S^T, no longer needed this chunk) so that every
        // thread then owns 8 consecutive columns of a row: 16-byte z loads and
        // out / o stores.
        constexpr int LDO = NC + 4;
        static_assert(sizeof(sm.e) >= sizeof(float) * CH * LDO, "O staging fits over S^T");
        lds_barrier();
        {
            float* of = reinterpret_cast<float*>(&sm.e);
#pragma unroll
            for (int t = 0; t < NJB2; ++t)
                *reinterpret_cast<f32x4v*>(&of[(16 * sw + l16) * LDO + 16 * (hv * NJB2 + t) + 4 * q4]) =
                    a.scale * accO[t];
        }
        lds_barrier();
        KDA_LAUNDER_LANE();
        // ---- P7: S = diag(e^{G_last}) S + K_dec^T Ub (key block `wave`). Issued ahead of
        // the output epilogue, whose VALU work then runs while the MFMA chain drains
        // (nothing here is read or written by the epilogue). ----
        {
            const int i = 16 * wave + l16;
            const f32x4v dec = GDN ? f32x4v{sm.fac[F_FN][0], sm.fac[F_FN][0], sm.fac[F_FN][0], sm.fac[F_FN][0]}
                                   : ld4f(&sm.fac[F_FN][16 * wave + 4 * q4]);
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) accS[jb] *= dec;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int j0 = 32 * kk + 8 * q4;
                const float el = sm.fac[F_ELR + (j0 >> 4)][GDN ? 0 : i];  // e^{G_last - B} of the rows' block
                bf16x8 bkd;
#pragma unroll
                for (int e = 0; e < 8; ++e) bkd[e] = (__bf16)((float)sm.kb[j0 + e][i] * el);
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb)
                    accS[jb] = mfma_bf16(bkd, ld8(&sm.c.m.w.ubt[16 * jb + l16][32 * kk + 8 * q4]), accS[jb]);
            }
        }
        // Items past the last row (or past the item count) store a copy of the last
        // row's values to the last row: the stores need no branch, and a branch would
        // make the compiler wait for all memory traffic where it joins.
        {
            constexpr int NITEMS = CH * (NC / 8);
            constexpr int NE = (NITEMS + NTHR - 1) / NTHR;  // items per thread
            const float* of = reinterpret_cast<const float*>(&sm.e);
            if constexpr (NCOL == 1) {
                static_assert(NE == NZ && NITEMS == NE * NTHR, "z prefetch covers the epilogue items");
                if (readout) {
                const int c8 = (tid % (NC / 8)) * 8;  // the same columns for every item of a thread
                const bf16x8* zz = zpre;
#pragma unroll
                for (int it = 0; it < NE; ++it) {
                    // the 16 lanes of a DPP row share r
                    const int r = min((tid + NTHR * it) / (NC / 8), n - 1);
                    float o8[8];
                    float ss = 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        o8[e] = of[r * LDO + c8 + e];
                        ss = fmaf(o8[e], o8[e], ss);
                    }
                    ss = sum_row16(ss);
                    const float inv = rsqrtf(fmaf(ss, 1.0f / DK, a.rms_eps));
                    {
                        const size_t off = (row0 + r) * orow + head_off + c8;
                        float y[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float zf = (float)zz[it][e];
                            const float gate = GDN ? silu_f(zf) : sigmoid_f(zf);
                            y[e] = ((o8[e] * inv) * w8[e]) * gate;
                        }
                        if constexpr (BF) {
                            bf16x8 yb;
#pragma unroll
                            for (int e = 0; e < 8; ++e) yb[e] = (__bf16)y[e];
                            st8(static_cast<__bf16*>(outp) + off, yb);
                        } else {
                            float4* d = reinterpret_cast<float4*>(static_cast<float*>(outp) + off);
                            d[0] = make_float4(y[0], y[1], y[2], y[3]);
                            d[1] = make_float4(y[4], y[5], y[6], y[7]);
                        }
                        if (obp) {
                            float4* d = reinterpret_cast<float4*>(obp + off);
                            d[0] = make_float4(o8[0], o8[1], o8[2], o8[3]);
                            d[1] = make_float4(o8[4], o8[5], o8[6], o8[7]);
                        }
                    }
                }
                }
            } else {
#pragma unroll
                for (int it = 0; it < NE; ++it) {
                    const int idx = min(tid + NTHR * it, NITEMS - 1);
                    const int r = min(idx / (NC / 8), n - 1), c8 = (idx % (NC / 8)) * 8;
                    const float* src = of + r * LDO + c8;
                    float4* d = reinterpret_cast<float4*>(o_buf + (row0 + r) * qkv + head_off + jv0 + c8);
                    d[0] = make_float4(src[0], src[1], src[2], src[3]);
                    d[1] = make_float4(src[4], src[5], src[6], src[7]);
                }
            }
        }

        lds_barrier();
        store_raw<GDN, NC, ACT>(sm, raw, max(min(CH, T - c0 - CH), 0), tid, a, cg);
        lds_barrier();
    }

#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
        const int jv = jv0 + jb * 16 + l16;
        *reinterpret_cast<f32x4v*>(&s_out[(size_t)jv * DK + 16 * wave + 4 * q4]) = accS[jb];
    }
}
#undef KDA_LAUNDER_LANE

// The ring roll of the chunked arm: new slot K-1-d = raw input at token T-d (the old
// ring for T-d < 0). Launched after the chunk kernel, which read the old ring.
int chunk_ncol(int B, int H) {
    const long bh = (long)B * H;
    if (bh >= 256) return 1;
    if (bh >= 128) return 2;
    return 4;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <bool BF, bool GDN, int NC>
hipError_t chunk_launch_nc(const MixerArgs& a, float* o_buf) {
    constexpr int NCOL = DK / NC;
    static_assert(sizeof(ChunkLds<GDN, NC, KMAX>) <= 160 * 1024, "LDS budget of one workgroup");
    const int nbh = a.B * a.H;
    const int grid = ((nbh + 7) / 8) * 8 * NCOL;
    const bool act = !GDN && a.gate_form != GATE_GIVEN;
    const dim3 g(grid), blk(NTHR);
    if (a.K == 4) {
        if (act) hipLaunchKernelGGL((chunk_kernel<BF, GDN, NC, 4, !GDN>), g, blk, 0, a.stream, a, o_buf);
        else hipLaunchKernelGGL((chunk_kernel<BF, GDN, NC, 4, false>), g, blk, 0, a.stream, a, o_buf);
    } else {
        if (act) hipLaunchKernelGGL((chunk_kernel<BF, GDN, NC, KMAX, !GDN>), g, blk, 0, a.stream, a, o_buf);
        else hipLaunchKernelGGL((chunk_kernel<BF, GDN, NC, KMAX, false>), g, blk, 0, a.stream, a, o_buf);
    }
    return hipGetLastError();
}

template <bool BF, bool GDN>
hipError_t chunk_launch(const MixerArgs& a) {
    const int ncol = chunk_ncol(a.B, a.H);
    float* o_buf = a.o_core;
    if (ncol > 1 && !o_buf) o_buf = static_cast<float*>(a.ws);
    hipError_t e;
    if (ncol == 1) e = chunk_launch_nc<BF, GDN, 128>(a, o_buf);
    else if (ncol == 2) e = chunk_launch_nc<BF, GDN, 64>(a, o_buf);
    else e = chunk_launch_nc<BF, GDN, 32>(a, o_buf);
    if (e != hipSuccess) return e;
    if (ncol > 1) {
        e = launch_norm(a, o_buf);
        if (e != hipSuccess) return e;
    }
    return launch_ring_roll(a, false);
}

// The constant blocks of the segmented arm's workspace: zeros (state and v row of
// the M runs) and the identity (entry state of the M runs). A kernel rather than a
// memset, so that the call can be captured in a graph.
__global__ void seg_init_kernel(float* zero, size_t nzero, float* ident) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < nzero) zero[i] = 0.0f;
    if (i < (size_t)DK * DK) ident[i] = (i / DK == i % DK) ? 1.0f : 0.0f;
}

// Entry states of the middle segments: S_{s+1} = M_s S_s + B_s for s = 1 .. n-2, on
// the fp32 MFMA (v_mfma_f32_16x16x4f32: exact fp32 products, fp32 accumulation).
// Workgroup (pair, 32-column block cb), four wavefronts; wavefront w computes keys
// 32 w .. +31 (two 16-row blocks) of the block's 32 columns (two 16-column blocks).
// State blocks are [value][key], so M_s (the final state of the run from the identity)
// holds M[i][k] at [k][i]: the A fragment M[i = l16][k = q4] of a 4-wide k slice is a
// 64-byte run per q4. The current state sits in LDS as [k][column] (row pitch 48 floats:
// the four k rows of a B fragment fall in distinct banks). The workgroups of one pair
// share blockIdx % 8, so they run on one XCD and its L2 fetches M_s and B_s once.
constexpr int SCAN_COLS = 32, SCAN_NCB = DK / SCAN_COLS, SCAN_LD = 48;
__global__ __launch_bounds__(256) void seg_scan_kernel(MixerArgs a) {
    const int P = a.B * a.H, n = a.seg_n;
    const int x = blockIdx.x;
    const int pair = (x / (8 * SCAN_NCB)) * 8 + x % 8, cb = (x / 8) % SCAN_NCB;
    if (pair >= P) return;
    const SegSlots sl = seg_slots(a);
    auto S = [&](int s) { return sl.S(s, pair); };
    auto M = [&](int s) { return sl.M(s, pair); };
    auto Bs = [&](int s) { return sl.B(s, pair); };
    __shared__ __align__(16) float sc[DK][SCAN_LD];  // the current entry state [k][column]
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, q4 = lane >> 4, l16 = lane & 15;
    const size_t col0 = (size_t)cb * SCAN_COLS;
    // result tile (rb, cc): keys 32 w + 16 rb + 4 q4 + r, column col0 + 16 cc + l16
    auto tile = [&](float* blkp, int rb, int cc) {
        return blkp + (col0 + 16 * cc + l16) * DK + 32 * w + 16 * rb + 4 * q4;
    };
    // The wavefront's A operands of one step, M[32 w + 16 rb + l16][k = 4 k4 + q4], all
    // requested at once (one memory round trip per step, not one per few k slices); the
    // next step's M_s and B_s are requested as soon as the current ones are consumed.
    float mreg[2][DK / 4];
    auto load_m = [&](int s) {
        const float* m = M(s) + 32 * w + l16;
#pragma unroll
        for (int k4 = 0; k4 < DK / 4; ++k4) {
            const size_t kr = (size_t)(4 * k4 + q4) * DK;
            mreg[0][k4] = m[kr];
            mreg[1][k4] = m[kr + 16];
        }
    };
    f32x4v acc[2][2];
    auto load_b = [&](int s) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) acc[rb][cc] = ld4f(tile(Bs(s), rb, cc));
    };
    if (n >= 3) {
        load_m(1);
        load_b(1);
    }
    {  // S_1 columns col0 .. +31 into LDS: thread t reads keys 16 (t % 8) .. +15 of column t / 8
        const int j = t / 8, k0 = (t % 8) * 16;
        const float* src = S(1) + (col0 + j) * DK + k0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float4 x4 = *reinterpret_cast<const float4*>(src + 4 * v);
            sc[k0 + 4 * v][j] = x4.x;
            sc[k0 + 4 * v + 1][j] = x4.y;
            sc[k0 + 4 * v + 2][j] = x4.z;
            sc[k0 + 4 * v + 3][j] = x4.w;
        }
    }
    for (int s = 1; s <= n - 2; ++s) {
        __syncthreads();
#pragma unroll
        for (int k4 = 0; k4 < DK / 4; ++k4) {
            const float b0 = sc[4 * k4 + q4][l16], b1 = sc[4 * k4 + q4][16 + l16];
            acc[0][0] = mfma_f32(mreg[0][k4], b0, acc[0][0]);
            acc[0][1] = mfma_f32(mreg[0][k4], b1, acc[0][1]);
            acc[1][0] = mfma_f32(mreg[1][k4], b0, acc[1][0]);
            acc[1][1] = mfma_f32(mreg[1][k4], b1, acc[1][1]);
        }
        if (s < n - 2) load_m(s + 1);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
                *reinterpret_cast<f32x4v*>(tile(S(s + 1), rb, cc)) = acc[rb][cc];
        __syncthreads();
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                for (int r = 0; r < 4; ++r) sc[32 * w + 16 * rb + 4 * q4 + r][16 * cc + l16] = acc[rb][cc][r];
        if (s < n - 2) load_b(s + 1);
    }
}

template <bool BF, bool GDN>
hipError_t seg_pass(const MixerArgs& a, int grid) {
    if (grid <= 0) return hipSuccess;
    if (chunked32_fits(a)) return launch_seg_pass32(a, grid);
    const bool act = !GDN && a.gate_form != GATE_GIVEN;
    const dim3 g(grid), blk(NTHR);
    float* ob = a.o_core;
    if (a.K == 4) {
        if (act) hipLaunchKernelGGL((chunk_kernel<BF, GDN, DK, 4, !GDN, true>), g, blk, 0, a.stream, a, ob);
        else hipLaunchKernelGGL((chunk_kernel<BF, GDN, DK, 4, false, true>), g, blk, 0, a.stream, a, ob);
    } else {
        if (act) hipLaunchKernelGGL((chunk_kernel<BF, GDN, DK, KMAX, !GDN, true>), g, blk, 0, a.stream, a, ob);
        else hipLaunchKernelGGL((chunk_kernel<BF, GDN, DK, KMAX, false, true>), g, blk, 0, a.stream, a, ob);
    }
    return hipGetLastError();
}

template <bool BF, bool GDN>
hipError_t seg_launch(MixerArgs a) {
    const int P = a.B * a.H, n = a.seg_n;
    const SegLayout lay = seg_layout(P, a.H, DK, n);
    a.seg_ws = static_cast<float*>(a.ws);
    char* ws = static_cast<char*>(a.ws);
    hipError_t e = hipSuccess;
    if (!chunked32_fits(a)) {  // the 32-row kernel forms the zero and identity states itself
        const size_t nzero = (lay.ident - lay.zero) / 4;
        const size_t ninit = nzero > (size_t)DK * DK ? nzero : (size_t)DK * DK;
        hipLaunchKernelGGL(seg_init_kernel, dim3((unsigned)((ninit + 255) / 256)), dim3(256), 0, a.stream,
                           reinterpret_cast<float*>(ws + lay.zero), nzero, reinterpret_cast<float*>(ws + lay.ident));
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    a.seg_pass = 1;
    const int mid = n >= 3 ? (n - 2) * P : 0;
    e = seg_pass<BF, GDN>(a, P + 16 * ((mid + 7) / 8));
    if (e != hipSuccess) return e;
    if (n >= 3) {
        hipLaunchKernelGGL(seg_scan_kernel, dim3(((P + 7) / 8) * 8 * SCAN_NCB), dim3(256), 0, a.stream, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (n >= 2) {
        a.seg_pass = 3;
        e = seg_pass<BF, GDN>(a, (n - 1) * P);
        if (e != hipSuccess) return e;
    }
    return seg_ring_fused(a) ? hipSuccess : launch_ring_roll(a, false);
}

}  // namespace

size_t segmented_workspace_bytes(int B, int H, int D, int n) {
    if (D != DK) return 0;
    return seg_layout((long)B * H, H, D, n).total;
}

hipError_t launch_segmented(const MixerArgs& a) {
    if (a.D != DK || a.cu_seqlens || a.seg_n < 1 || a.seg_len0 < 1 || (a.seg_n > 1 && a.seg_len < CH) || !a.ws)
        return hipErrorInvalidValue;
    if (!a.bf16) return hipErrorInvalidValue;  // bf16 activations only (refused on the host)
    return a.gdn ? seg_launch<true, true>(a) : seg_launch<true, false>(a);
}

size_t chunked_workspace_bytes(int nseq, size_t rows, int H, int D) {
    if (D != DK || chunk_ncol(nseq, H) == 1) return 0;
    return align256(rows * H * D * 4);  // fp32 pre-norm output of the column splits
}

hipError_t launch_chunked(const MixerArgs& a) {
    if (a.D != DK) return hipErrorInvalidValue;
    if (chunked32_fits(a)) return launch_chunked32(a);
    if (!a.bf16) return hipErrorInvalidValue;  // bf16 activations only (refused on the host)
    return a.gdn ? chunk_launch<true, true>(a) : chunk_launch<true, false>(a);
}

}  // namespace kda
