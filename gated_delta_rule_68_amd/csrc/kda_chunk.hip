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
// Every factor e^{...} that multiplies an MFMA operand is <= 1 except on the
// diagonal 16x16 blocks of L and P, where the decay is rebased to the first row of
// the block (at most 15 steps of g >= -5, so e^{75} at worst, inside fp32/bf16
// range); this is why the arm needs g >= -5.
//
// One workgroup of 8 wavefronts owns one (sequence, head, value-column split) and
// walks the chunks in order; the state lives in MFMA accumulator registers as S^T
// tiles (wavefront w holds key block w). All contractions run on v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32
// accumulation); the 64x64 unit-triangular inverse is solved in fp32 (16x16 diagonal
// blocks by forward substitution, off-diagonal blocks with v_mfma_f32_16x16x4f32).
// conv + SiLU and l2 run in-kernel on the raw inputs, so the only HBM traffic is the
// raw activations, the gates, the output and the state once in and once out. For
// bf16 inputs the raw rows of chunk c+1 are requested while chunk c computes.
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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4v mfma_bf16(bf16x8 a, bf16x8 b, f32x4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4v mfma_f32(float a, float b, f32x4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 ld8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void st8(__bf16* p, bf16x8 v) { *reinterpret_cast<bf16x8*>(p) = v; }
__device__ __forceinline__ f32x4v zero4() { return f32x4v{0.0f, 0.0f, 0.0f, 0.0f}; }

// Workgroup barrier that orders LDS only: it waits for this wave's LDS operations and
// not for its outstanding global loads, so the next chunk's prefetched rows stay in
// flight across the phases of the current chunk. (Every value crossing phases inside
// the chunk loop goes through LDS or registers; global stores are never read back.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ bf16x8 zero8() {
    const __bf16 z = (__bf16)0.0f;
    return bf16x8{z, z, z, z, z, z, z, z};
}

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

template <bool GDN, int NC>
struct ChunkLds {
    alignas(16) float gam[CH][GDN ? 4 : DK];  // inclusive cumulative log gate
    alignas(16) __bf16 qh[CH][LDH];           // l2-normalised SiLU(conv q)
    alignas(16) __bf16 kh[CH][LDH];           // l2-normalised SiLU(conv k)
    alignas(16) __bf16 pb[CH][LDC];           // P (lower incl. diagonal)
    alignas(16) __bf16 hist[KMAX - 1][2 * DK + NC];  // raw rows before the chunk: [d-1] is d rows back
    alignas(16) float beta[CH];
    alignas(16) float fn[DK];                 // e^{G_last}
    alignas(16) float xs[4][16][17];          // 16x16 scratch of the block solve, waves 0..3
    union {
        struct {
            __bf16 rq[CH][LDH];  // raw q rows of the chunk
            __bf16 rk[CH][LDH];  // raw k rows
        } raw;
        struct {
            float lf[CH][LDF];  // beta_s L[s][j], strictly lower
            float tf[CH][LDF];  // T in fp32
        } solve;
        __bf16 wneg[CH][LDH];  // -W
        __bf16 ubt[NC][LDC];   // Ub^T [value][row]
    } c;
    union {
        struct {
            __bf16 vbt[NC][LDC];  // (beta v)^T [value][row]
            union {
                __bf16 rv[CH][NC + 8];  // raw v rows of the split
                __bf16 tb[CH][LDC];     // T in bf16
            } u;
        } pre;
        __bf16 sb[NC][LDH];  // S^T in bf16 [value][key]
    } e;
};

template <bool GDN>
__device__ __forceinline__ float gam_at(const float (*gam)[GDN ? 4 : DK], int r, int i) {
    if constexpr (GDN)
        return gam[r][0];
    else
        return gam[r][i];
}

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
// their store into LDS. Item it of thread tid covers row (tid + 256 it) / 16 and the
// 8 channels ((tid + 256 it) % 16) * 8 of q, k and the gate; v items cover the NC
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
// T-1) and nothing consumes the values until the next chunk's P0: a load inside a
// divergent branch, or a select right after it, makes the compiler wait for the load
// on the spot, which would stall on the prefetch itself. Rows past T are masked
// where they are consumed (gates and beta in P0, conv outputs in P1).
__device__ __forceinline__ bf16x8 sel8(bool keep, bf16x8 x) {
    return keep ? x : zero8();
}

template <bool BF, bool GDN, int NC>
__device__ __forceinline__ void load_raw(ChunkRaw<GDN, NC>& cr, const MixerArgs& a, int b, int h,
                                         int c0, int jv0, int tid) {
    using CR = ChunkRaw<GDN, NC>;
    const int T = a.T, H = a.H;
    const size_t qkv = (size_t)H * DK, head_off = (size_t)h * DK;
    const size_t rowb = (size_t)b * T;
#pragma unroll
    for (int it = 0; it < CR::NI; ++it) {
        const int idx = tid + NTHR * it, r = idx / (DK / 8), c8 = (idx % (DK / 8)) * 8;
        const bool ok = c0 + r < T;
        const size_t off = (rowb + min(c0 + r, T - 1)) * qkv + head_off + c8;
        (void)ok;
        cr.q[it] = ld_act8<BF>(a.q, off);
        cr.k[it] = ld_act8<BF>(a.k, off);
        if constexpr (!GDN) cr.g[it] = ld_act8<BF>(a.g, off);
    }
#pragma unroll
    for (int it = 0; it < CR::NV; ++it) {
        const int idx = min(tid + NTHR * it, CR::VITEMS - 1);
        const int r = idx / (NC / 8), c8 = (idx % (NC / 8)) * 8;
        cr.v[it] = ld_act8<BF>(a.v, (rowb + min(c0 + r, T - 1)) * qkv + head_off + jv0 + c8);
    }
    const int rr = tid & (CH - 1);
    const size_t hr = (rowb + min(c0 + rr, T - 1)) * H + h;
    cr.beta = ld_act<BF>(a.beta, hr);
    cr.gs = GDN ? ld_act<BF>(a.g, hr) : 0.0f;
}

// The raw rows of a chunk (n valid rows) from registers into LDS: q, k to the raw
// staging tiles, v to its staging tile, the gates (zero past row n, so G stays at
// G[n-1]) and beta; for GDN the scalar gates are scanned here (wave 0).
template <bool GDN, int NC, typename Lds>
__device__ __forceinline__ void store_raw(Lds& sm, const ChunkRaw<GDN, NC>& raw, int n, int tid, int lane) {
    using CR = ChunkRaw<GDN, NC>;
#pragma unroll
    for (int it = 0; it < CR::NI; ++it) {
        const int idx = tid + NTHR * it, r = idx / (DK / 8), c8 = (idx % (DK / 8)) * 8;
        *reinterpret_cast<bf16x8*>(&sm.c.raw.rq[r][c8]) = raw.q[it];
        *reinterpret_cast<bf16x8*>(&sm.c.raw.rk[r][c8]) = raw.k[it];
        if constexpr (!GDN) {
            float4* gp = reinterpret_cast<float4*>(&sm.gam[r][c8]);
            const bf16x8 g8 = raw.g[it];
            const bool ok = r < n;
            gp[0] = make_float4(ok ? (float)g8[0] : 0.0f, ok ? (float)g8[1] : 0.0f,
                                ok ? (float)g8[2] : 0.0f, ok ? (float)g8[3] : 0.0f);
            gp[1] = make_float4(ok ? (float)g8[4] : 0.0f, ok ? (float)g8[5] : 0.0f,
                                ok ? (float)g8[6] : 0.0f, ok ? (float)g8[7] : 0.0f);
        }
    }
#pragma unroll
    for (int it = 0; it < CR::NV; ++it) {
        const int idx = tid + NTHR * it, r = idx / (NC / 8), c8 = (idx % (NC / 8)) * 8;
        if (idx < CR::VITEMS) *reinterpret_cast<bf16x8*>(&sm.e.pre.u.rv[r][c8]) = raw.v[it];
    }
    if (tid < CH) sm.beta[tid] = tid < n ? raw.beta : 0.0f;
    if constexpr (GDN) {
        if (tid < CH) {  // wave 0: inclusive scan of the 64 scalar gates
            float gv = tid < n ? raw.gs : 0.0f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float up = __shfl_up(gv, off, 64);
                if (lane >= off) gv += up;
            }
            sm.gam[tid][0] = gv;
            if (tid == CH - 1) sm.fn[0] = exp_f(gv);
        }
    }
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 ld4(const __bf16* p) { return *reinterpret_cast<const bf16x4*>(p); }

// Sliding conv window over 4 channels: raw rows of the chunk come from `raw` (row
// stride ld), earlier rows from `hist` (hist + (d-1)*hld is the row d rows before the
// chunk). step() takes the next raw row and returns SiLU(conv) of its 4 channels; the
// taps w[e][j] multiply x~[r-(KT-1)+j] (taps beyond K are zero), so the sum runs over
// the window in ascending time order.
template <int KT>
struct ConvWin4 {
    float win[KT - 1][4];  // win[KT-2] = previous row

    __device__ __forceinline__ void init(const __bf16* raw, int ld, const __bf16* hist, int hld, int r0) {
#pragma unroll
        for (int d = 1; d < KT; ++d) {
            const int r = r0 - d;
            const bf16x4 x = r >= 0 ? ld4(raw + r * ld) : ld4(hist + (d - r0 - 1) * hld);
#pragma unroll
            for (int e = 0; e < 4; ++e) win[KT - 1 - d][e] = (float)x[e];
        }
    }

    __device__ __forceinline__ void step(bf16x4 x, const float (&w)[4][KT], bool valid, float (&y)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < KT - 1; ++j) acc = fmaf(w[e][j], win[j][e], acc);
            acc = fmaf(w[e][KT - 1], (float)x[e], acc);
            y[e] = valid ? silu_f(acc) : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < KT - 2; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) win[j][e] = win[j + 1][e];
#pragma unroll
        for (int e = 0; e < 4; ++e) win[KT - 2][e] = (float)x[e];
    }
};

// Taps of 4 channels starting at fused conv row `row`, aligned so that w[e][KT-1]
// multiplies the current input (zero for the KT-K oldest slots). KT == 4 is the
// K == 4 kernel; K of 2, 3 and 5..8 run the KT == 8 kernel.
template <int KT>
__device__ __forceinline__ void load_taps4(float (&w)[4][KT], const float* conv_w, size_t row, int K) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < KT; ++j) {
            if constexpr (KT == 4) {  // this instantiation runs only for K == 4
                w[e][j] = conv_w[(row + e) * 4 + j];
            } else {
                const int tap = j - (KT - K);  // index into the K-wide weight row
                const float x = conv_w[(row + e) * K + max(tap, 0)];
                w[e][j] = tap >= 0 ? x : 0.0f;
            }
        }
}

template <bool BF, bool GDN, int NC, int KT>
__global__ __launch_bounds__(NTHR) void chunk_kernel(MixerArgs a, float* o_buf) {
    constexpr int NCOL = DK / NC;
    constexpr int NJB = NC / 16;  // value-column 16-blocks of this split
    constexpr int HLD = 2 * DK + NC;
    __shared__ ChunkLds<GDN, NC> sm;
    using CR = ChunkRaw<GDN, NC>;

    int bh, split;
    block_coords(NCOL, a.B * a.H, &bh, &split);
    if (bh < 0) return;  // whole block exits before any barrier

    int tid = threadIdx.x, lane = tid & 63;
    const int wave = tid >> 6;
    int q4 = lane >> 4, l16 = lane & 15;
    const int b = bh / a.H, h = bh % a.H;
    const int T = a.T, K = a.K;
    // Re-materialise the lane indices at every phase: otherwise the compiler hoists
    // each phase's lane-dependent LDS addresses out of the chunk loop and keeps them
    // all alive at once, which overflows the register file.
#define KDA_LAUNDER_LANE()                                                 \
    do {                                                                   \
        asm volatile("" : "+v"(tid), "+v"(lane), "+v"(q4), "+v"(l16));     \
    } while (0)
    const size_t qkv = (size_t)a.H * DK;
    const size_t head_off = (size_t)h * DK;
    const int jv0 = split * NC;  // first value column of this split

    // ---- state: S^T tiles (value block jb, key block `wave`) ----
    f32x4v accS[NJB];
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int jv = jv0 + jb * 16 + 4 * q4 + r, i = wave * 16 + l16;
            accS[jb][r] = a.state_in[((size_t)bh * DK + jv) * DK + i];
        }
    // Wavefront (sw, hv) = (wave % 4, wave / 4) owns rows 16*sw.. of U / Ub / O and the
    // value blocks [hv*NJB2, (hv+1)*NJB2).
    constexpr int NJB2 = NJB / 2;
    const int sw = wave & 3, hv = wave >> 2;

    // ---- conv history of the first chunk: the old ring (slot K-1-d is d rows back) ----
    {
        const float* ring_b = a.ring + (size_t)b * 3 * qkv * (K - 1);
        for (int idx = tid; idx < (KMAX - 1) * HLD; idx += NTHR) {
            const int d = idx / HLD + 1, col = idx % HLD;
            const size_t fr = col < 2 * DK ? (size_t)(col / DK) * qkv + head_off + col % DK
                                           : 2 * qkv + head_off + jv0 + (col - 2 * DK);
            sm.hist[d - 1][col] = (__bf16)(d <= K - 1 ? ring_b[fr * (K - 1) + K - 1 - d] : 0.0f);
        }
    }

    // Conv roles: thread = (plane q/k, 8-row group, 8-channel group) for q and k; the
    // v channels of the split are 8-row x 8-channel items of threads 0 .. NVI-1, and
    // (KDA) the per-channel gate scans run on threads 128..255 meanwhile.
    // The taps are re-read every chunk (a few L2-resident bytes) rather than held in
    // registers across the whole chunk loop.
    // Conv items are 4 rows x 4 channels: thread tid convolves q rows (tid / 32) * 4..
    // and k rows of the same group, channels (tid % 32) * 4.., and, if tid < NVI, one v
    // item; the 32 lanes of one row group are consecutive, so the l2 norm of a row is a
    // 32-lane reduction.
    const int crg = (tid / 32) % 16, ccg = tid % 32;
    constexpr int NVI = 16 * (NC / 4);
    const bool vthread = tid < NVI;
    const int vrg = tid / (NC / 4), vcg = tid % (NC / 4);

    CR raw;
    load_raw<BF, GDN, NC>(raw, a, b, h, 0, jv0, tid);
    store_raw<GDN, NC>(sm, raw, min(CH, T), tid, lane);
    __syncthreads();

    for (int c0 = 0; c0 < T; c0 += CH) {
        const int n = min(CH, T - c0);
        const size_t row0 = (size_t)b * T + c0;

        KDA_LAUNDER_LANE();
        // ---- P0: conv taps (the chunk's raw rows are already in LDS: the previous
        // iteration, or the prologue, staged them) ----
        float wq[4][KT], wk[4][KT], wv[4][KT];
        load_taps4<KT>(wq, a.conv_w, head_off + ccg * 4, K);
        load_taps4<KT>(wk, a.conv_w, qkv + head_off + ccg * 4, K);
        if (vthread) load_taps4<KT>(wv, a.conv_w, 2 * qkv + head_off + jv0 + vcg * 4, K);

        KDA_LAUNDER_LANE();
        // ---- P1: cumulative gate (4 threads per channel), then conv + SiLU (+ l2 for
        // q, k) of 4-row x 4-channel items ----
        if constexpr (!GDN) {
            const int c = tid >> 2, qq = tid & 3;  // rows 16 qq .. 16 qq + 15 of channel c
            float g16[16], acc = 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                acc += sm.gam[16 * qq + r][c];
                g16[r] = acc;
            }
            // exclusive prefix of the quarter totals over the 4 lanes of the channel
            const float t1 = __shfl_up(acc, 1, 4), t2 = __shfl_up(acc, 2, 4), t3 = __shfl_up(acc, 3, 4);
            const float base = (qq >= 1 ? t1 : 0.0f) + (qq >= 2 ? t2 : 0.0f) + (qq >= 3 ? t3 : 0.0f);
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.gam[16 * qq + r][c] = base + g16[r];
            if (qq == 3) sm.fn[c] = exp_f(base + acc);
        }
#pragma unroll
        for (int plane = 0; plane < 2; ++plane) {
            const __bf16* rawp = (plane == 0 ? &sm.c.raw.rq[0][0] : &sm.c.raw.rk[0][0]) + ccg * 4;
            __bf16* dst = (plane == 0 ? &sm.qh[0][0] : &sm.kh[0][0]) + ccg * 4;
            ConvWin4<KT> cw;
            cw.init(rawp, LDH, &sm.hist[0][plane * DK + ccg * 4], HLD, crg * 4);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = crg * 4 + rr;
                float y[4];
                cw.step(ld4(rawp + r * LDH), plane == 0 ? wq : wk, r < n, y);
                float ss = 0.0f;
#pragma unroll
                for (int e = 0; e < 4; ++e) ss = fmaf(y[e], y[e], ss);
                ss += __shfl_xor(ss, 1, 64);  // the 32 channel groups of the row
                ss += __shfl_xor(ss, 2, 64);
                ss += __shfl_xor(ss, 4, 64);
                ss += __shfl_xor(ss, 8, 64);
                ss += __shfl_xor(ss, 16, 64);
                const float inv = rsqrtf(ss + L2_EPS);
                bf16x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = (__bf16)(y[e] * inv);
                *reinterpret_cast<bf16x4*>(dst + r * LDH) = o;
            }
        }
        if (vthread) {
            const __bf16* rawp = &sm.e.pre.u.rv[0][vcg * 4];
            ConvWin4<KT> cw;
            cw.init(rawp, NC + 8, &sm.hist[0][2 * DK + vcg * 4], HLD, vrg * 4);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int r = vrg * 4 + rr;
                float y[4];
                cw.step(ld4(rawp + r * (NC + 8)), wv, r < n, y);
                const float bt = sm.beta[r];
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.e.pre.vbt[vcg * 4 + e][r] = (__bf16)(bt * y[e]);
            }
        }
        lds_barrier();
        // The last KMAX-1 raw rows become the next chunk's history (only a full chunk
        // has a successor).
        if (n == CH) {
            for (int idx = tid; idx < (KMAX - 1) * (HLD / 8); idx += NTHR) {
                const int d = idx / (HLD / 8) + 1, col = (idx % (HLD / 8)) * 8;
                const __bf16* src = col < DK ? &sm.c.raw.rq[CH - d][col]
                                  : col < 2 * DK ? &sm.c.raw.rk[CH - d][col - DK]
                                                 : &sm.e.pre.u.rv[CH - d][col - 2 * DK];
                st8(&sm.hist[d - 1][col], ld8(src));
            }
        }
        lds_barrier();

        KDA_LAUNDER_LANE();
        // ---- P2: L and P; wavefront (a, p) = (wave / 2, wave % 2) computes block-row a,
        // column blocks p and p + 2; the decay is rebased to row 16a ----
        {
            const int ab = wave >> 1, par = wave & 1, ra = 16 * ab, s = ra + l16;
            f32x4v accL[2], accP[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) accL[t] = accP[t] = zero4();
            if (par <= ab) {
#pragma unroll 1
                for (int kk = 0; kk < 4; ++kk) {
                    const int i0 = 32 * kk + 8 * q4;
                    float gr[8];
                    bf16x8 ak, aq;
                    const bf16x8 kx = ld8(&sm.kh[s][i0]), qx = ld8(&sm.qh[s][i0]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        gr[e] = gam_at<GDN>(sm.gam, ra, i0 + e);
                        const float ea = exp_f(gam_at<GDN>(sm.gam, s, i0 + e) - gr[e]);
                        ak[e] = (__bf16)((float)kx[e] * ea);
                        aq[e] = (__bf16)((float)qx[e] * ea);
                    }
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const int bb = par + 2 * t;
                        if (bb > ab) break;
                        const int j = 16 * bb + l16;
                        const bf16x8 kj = ld8(&sm.kh[j][i0]);
                        bf16x8 bk;
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            bk[e] = (__bf16)((float)kj[e] * exp_f(gr[e] - gam_at<GDN>(sm.gam, j, i0 + e)));
                        accL[t] = mfma_bf16(ak, bk, accL[t]);
                        accP[t] = mfma_bf16(aq, bk, accP[t]);
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int bb = par + 2 * t;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int sr = ra + 4 * q4 + r, j = 16 * bb + l16;
                    const bool lo = bb <= ab;
                    sm.c.solve.lf[sr][j] = (lo && j < sr) ? sm.beta[sr] * accL[t][r] : 0.0f;
                    sm.pb[sr][j] = (__bf16)((lo && j <= sr) ? accP[t][r] : 0.0f);
                }
            }
        }
        lds_barrier();

        // The next chunk's raw rows are requested here and stored at the end of this
        // iteration, and this chunk's output gates z for the norm in P6, so both HBM
        // latencies overlap P3..P6.
        constexpr int NZ = NCOL == 1 ? CH * (DK / 8) / NTHR : 1;
        bf16x8 zpre[NZ];
        if constexpr (NCOL == 1) {
#pragma unroll
            for (int it = 0; it < NZ; ++it) {
                const int r = (tid + NTHR * it) / (DK / 8), c8 = (tid % (DK / 8)) * 8;
                zpre[it] = ld_act8<BF>(a.z, (row0 + min(r, n - 1)) * qkv + head_off + c8);
            }
        }
        if (c0 + CH < T) load_raw<BF, GDN, NC>(raw, a, b, h, c0 + CH, jv0, tid);
        KDA_LAUNDER_LANE();
        // ---- P3: T = (I + A)^-1, A = diag(beta) L, 16x16 blocks ----
        {
            float (*lf)[LDF] = sm.c.solve.lf;
            float (*tf)[LDF] = sm.c.solve.tf;
            const int ab = wave;  // waves 0..3: one 16-row block each
            if (wave < 4 && q4 == 0) {  // diagonal block ab, column l16, forward substitution
                float x[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    // Keep this row's coefficient loads here: hoisting all 120 of them
                    // would hold 120 registers across the solve.
                    asm volatile("" ::: "memory");
                    float acc = (r == l16) ? 1.0f : 0.0f;
#pragma unroll
                    for (int jj = 0; jj < r; ++jj) acc = fmaf(-lf[16 * ab + r][16 * ab + jj], x[jj], acc);
                    x[r] = acc;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) tf[16 * ab + r][16 * ab + l16] = x[r];
            }
            if (wave < 4) {
                for (int idx = lane; idx < 16 * CH; idx += 64) {  // zero the strictly-upper blocks of row block ab
                    const int r = idx / CH, j = idx % CH;
                    if (j >= 16 * (ab + 1)) tf[16 * ab + r][j] = 0.0f;
                }
            }
            lds_barrier();
            // Off-diagonal blocks by distance: T_ab = -T_aa * sum_{c=b}^{a-1} A_ac T_cb.
            for (int d = 1; d < 4; ++d) {
                const int bb = wave < 4 ? ab - d : -1;
                if (bb >= 0) {
                    f32x4v xacc = zero4();
                    for (int cc = bb; cc < ab; ++cc)
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk)
                            xacc = mfma_f32(lf[16 * ab + l16][16 * cc + 4 * kk + q4],
                                            tf[16 * cc + 4 * kk + q4][16 * bb + l16], xacc);
#pragma unroll
                    for (int r = 0; r < 4; ++r) sm.xs[wave][4 * q4 + r][l16] = xacc[r];
                }
                lds_barrier();
                if (bb >= 0) {
                    f32x4v tacc = zero4();
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        tacc = mfma_f32(tf[16 * ab + l16][16 * ab + 4 * kk + q4],
                                        sm.xs[wave][4 * kk + q4][l16], tacc);
#pragma unroll
                    for (int r = 0; r < 4; ++r) tf[16 * ab + 4 * q4 + r][16 * bb + l16] = -tacc[r];
                }
                lds_barrier();
            }
            for (int idx = tid; idx < CH * CH; idx += NTHR) {
                const int r = idx / CH, j = idx % CH;
                sm.e.pre.u.tb[r][j] = (__bf16)tf[r][j];
            }
        }
        lds_barrier();

        KDA_LAUNDER_LANE();
        // ---- P4: W = T (beta e^{G} k) -> -W in LDS (key block `wave`);
        //      U = T (beta v) in registers (rows 16*sw.., value blocks of half hv) ----
        f32x4v accU[NJB2];
        {
            const int i = 16 * wave + l16;
            f32x4v accW[4];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) accW[sb] = zero4();
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 bw;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int j = 32 * kk + 8 * q4 + e;
                    bw[e] = (__bf16)(sm.beta[j] * (float)sm.kh[j][i] * exp_f(gam_at<GDN>(sm.gam, j, i)));
                }
#pragma unroll
                for (int sb = 0; sb < 4; ++sb)
                    accW[sb] = mfma_bf16(ld8(&sm.e.pre.u.tb[16 * sb + l16][32 * kk + 8 * q4]), bw, accW[sb]);
            }
#pragma unroll
            for (int sb = 0; sb < 4; ++sb)
#pragma unroll
                for (int r = 0; r < 4; ++r) sm.c.wneg[16 * sb + 4 * q4 + r][i] = (__bf16)(-accW[sb][r]);
#pragma unroll
            for (int t = 0; t < NJB2; ++t) accU[t] = zero4();
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 at = ld8(&sm.e.pre.u.tb[16 * sw + l16][32 * kk + 8 * q4]);
#pragma unroll
                for (int t = 0; t < NJB2; ++t) {
                    const int jb = hv * NJB2 + t;
                    accU[t] = mfma_bf16(at, ld8(&sm.e.pre.vbt[16 * jb + l16][32 * kk + 8 * q4]), accU[t]);
                }
            }
        }
        lds_barrier();

        KDA_LAUNDER_LANE();
        // ---- P5: S^T to LDS in bf16, then Ub = U - W S ----
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.e.sb[16 * jb + 4 * q4 + r][16 * wave + l16] = (__bf16)accS[jb][r];
        lds_barrier();
#pragma unroll 2
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8 aw = ld8(&sm.c.wneg[16 * sw + l16][32 * kk + 8 * q4]);
#pragma unroll
            for (int t = 0; t < NJB2; ++t) {
                const int jb = hv * NJB2 + t;
                accU[t] = mfma_bf16(aw, ld8(&sm.e.sb[16 * jb + l16][32 * kk + 8 * q4]), accU[t]);
            }
        }
        lds_barrier();  // every read of -W is done before Ub^T overwrites it
#pragma unroll
        for (int t = 0; t < NJB2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sm.c.ubt[16 * (hv * NJB2 + t) + l16][16 * sw + 4 * q4 + r] = (__bf16)accU[t][r];
        lds_barrier();

        KDA_LAUNDER_LANE();
        // ---- P6: O = scale (Q+ S + P Ub), rows 16*sw.., value blocks of half hv ----
        f32x4v accO[NJB2];
        {
            const int s = 16 * sw + l16;
#pragma unroll
            for (int t = 0; t < NJB2; ++t) accO[t] = zero4();
#pragma unroll 1
            for (int kk = 0; kk < 4; ++kk) {
                const int i0 = 32 * kk + 8 * q4;
                const bf16x8 qx = ld8(&sm.qh[s][i0]);
                bf16x8 aq;
#pragma unroll
                for (int e = 0; e < 8; ++e) aq[e] = (__bf16)((float)qx[e] * exp_f(gam_at<GDN>(sm.gam, s, i0 + e)));
#pragma unroll
                for (int t = 0; t < NJB2; ++t)
                    accO[t] = mfma_bf16(aq, ld8(&sm.e.sb[16 * (hv * NJB2 + t) + l16][i0]), accO[t]);
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (32 * kk > 16 * sw + 15) break;  // P is lower triangular
                const bf16x8 ap = ld8(&sm.pb[s][32 * kk + 8 * q4]);
#pragma unroll
                for (int t = 0; t < NJB2; ++t)
                    accO[t] = mfma_bf16(ap, ld8(&sm.c.ubt[16 * (hv * NJB2 + t) + l16][32 * kk + 8 * q4]), accO[t]);
            }
        }
        // O goes through LDS (over S^T, no longer needed this chunk) so that every
        // thread then owns 8 consecutive columns of a row: 16-byte z loads and
        // out / o stores.
        lds_barrier();
        {
            constexpr int LDO = NC + 4;
            float* of = reinterpret_cast<float*>(&sm.e.sb[0][0]);
#pragma unroll
            for (int t = 0; t < NJB2; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    of[(16 * sw + 4 * q4 + r) * LDO + 16 * (hv * NJB2 + t) + l16] = a.scale * accO[t][r];
        }
        lds_barrier();
        {
            constexpr int LDO = NC + 4;
            constexpr int NITEMS = CH * (NC / 8);
            constexpr int NE = (NITEMS + NTHR - 1) / NTHR;  // items per thread
            const float* of = reinterpret_cast<const float*>(&sm.e.sb[0][0]);
            const int c8 = (tid % (NC / 8)) * 8;  // the same columns for every item of a thread
            if constexpr (NCOL == 1) {
                static_assert(NE == NZ, "z prefetch covers the epilogue items");
                const bf16x8* zz = zpre;
                float w8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) w8[e] = a.norm_w[c8 + e];
#pragma unroll
                for (int it = 0; it < NE; ++it) {
                    const int r = (tid + NTHR * it) / (NC / 8);
                    float o8[8];
                    float ss = 0.0f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        o8[e] = of[r * LDO + c8 + e];
                        ss = fmaf(o8[e], o8[e], ss);
                    }
                    ss += __shfl_xor(ss, 1, 64);  // the 16 lanes of one row
                    ss += __shfl_xor(ss, 2, 64);
                    ss += __shfl_xor(ss, 4, 64);
                    ss += __shfl_xor(ss, 8, 64);
                    const float inv = rsqrtf(fmaf(ss, 1.0f / DK, a.rms_eps));
                    if (tid + NTHR * it < NITEMS && r < n) {
                        const size_t off = (row0 + r) * qkv + head_off + c8;
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
                            st8(static_cast<__bf16*>(a.out) + off, yb);
                        } else {
                            float4* d = reinterpret_cast<float4*>(static_cast<float*>(a.out) + off);
                            d[0] = make_float4(y[0], y[1], y[2], y[3]);
                            d[1] = make_float4(y[4], y[5], y[6], y[7]);
                        }
                        if (o_buf) {
                            float4* d = reinterpret_cast<float4*>(o_buf + off);
                            d[0] = make_float4(o8[0], o8[1], o8[2], o8[3]);
                            d[1] = make_float4(o8[4], o8[5], o8[6], o8[7]);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int it = 0; it < NE; ++it) {
                    const int r = (tid + NTHR * it) / (NC / 8);
                    if (tid + NTHR * it < NITEMS && r < n) {
                        const float* src = of + r * LDO + c8;
                        float4* d = reinterpret_cast<float4*>(o_buf + (row0 + r) * qkv + head_off + jv0 + c8);
                        d[0] = make_float4(src[0], src[1], src[2], src[3]);
                        d[1] = make_float4(src[4], src[5], src[6], src[7]);
                    }
                }
            }
        }

        KDA_LAUNDER_LANE();
        // ---- P7: S = diag(e^{G_last}) S + K_dec^T Ub (key block `wave`) ----
        {
            const int i = 16 * wave + l16;
            const float dec = sm.fn[GDN ? 0 : i];
            const float glast = gam_at<GDN>(sm.gam, CH - 1, i);
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                for (int r = 0; r < 4; ++r) accS[jb][r] *= dec;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 bkd;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int sr = 32 * kk + 8 * q4 + e;
                    bkd[e] = (__bf16)((float)sm.kh[sr][i] * exp_f(glast - gam_at<GDN>(sm.gam, sr, i)));
                }
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb)
                    accS[jb] = mfma_bf16(ld8(&sm.c.ubt[16 * jb + l16][32 * kk + 8 * q4]), bkd, accS[jb]);
            }
        }
        lds_barrier();
        if (c0 + CH < T) {
            store_raw<GDN, NC>(sm, raw, min(CH, T - c0 - CH), tid, lane);
            lds_barrier();
        }
    }

#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int jv = jv0 + jb * 16 + 4 * q4 + r, i = wave * 16 + l16;
            a.state_out[((size_t)bh * DK + jv) * DK + i] = accS[jb][r];
        }
}
#undef KDA_LAUNDER_LANE

// The ring roll of the chunked arm: new slot K-1-d = raw input at token T-d (the old
// ring for T-d < 0). Launched after the chunk kernel, which read the old ring.
template <bool BF>
__global__ __launch_bounds__(256) void ring_roll_kernel(MixerArgs a) {
    const size_t rows = (size_t)a.B * 3 * a.H * DK;
    const size_t row = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (row >= rows) return;
    const size_t qkv = (size_t)a.H * DK;
    const int b = (int)(row / (3 * qkv));
    const size_t cf = row % (3 * qkv);
    const int plane = (int)(cf / qkv);
    const size_t ch = cf % qkv;
    const void* x = plane == 0 ? a.q : (plane == 1 ? a.k : a.v);
    const int K = a.K, T = a.T;
    float* ring_row = a.ring + row * (K - 1);
    float nr[KMAX - 1];
#pragma unroll
    for (int d = 1; d < KMAX; ++d) {
        const int pos = T - d;
        nr[KMAX - 1 - d] = (d <= K - 1) ? (pos >= 0 ? ld_act<BF>(x, ((size_t)b * T + pos) * qkv + ch)
                                                     : ring_row[pos + K - 1])
                                        : 0.0f;
    }
#pragma unroll
    for (int d = 1; d < KMAX; ++d)
        if (d <= K - 1) ring_row[K - 1 - d] = nr[KMAX - 1 - d];
}

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
    const int nbh = a.B * a.H;
    const int grid = ((nbh + 7) / 8) * 8 * NCOL;
    if (a.K == 4)
        hipLaunchKernelGGL((chunk_kernel<BF, GDN, NC, 4>), dim3(grid), dim3(NTHR), 0, a.stream, a, o_buf);
    else
        hipLaunchKernelGGL((chunk_kernel<BF, GDN, NC, KMAX>), dim3(grid), dim3(NTHR), 0, a.stream, a, o_buf);
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
    const size_t rows = (size_t)a.B * 3 * a.H * DK;
    hipLaunchKernelGGL((ring_roll_kernel<BF>), dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                       a.stream, a);
    return hipGetLastError();
}

}  // namespace

size_t chunked_workspace_bytes(int B, int T, int H, int D, bool gdn) {
    (void)gdn;
    if (D != DK || chunk_ncol(B, H) == 1) return 0;
    return align256((size_t)B * T * H * D * 4);  // fp32 pre-norm output of the column splits
}

hipError_t launch_chunked(const MixerArgs& a) {
    if (a.D != DK) return hipErrorInvalidValue;
    if (a.bf16) return a.gdn ? chunk_launch<true, true>(a) : chunk_launch<true, false>(a);
    return a.gdn ? chunk_launch<false, true>(a) : chunk_launch<false, false>(a);
}

}  // namespace kda
