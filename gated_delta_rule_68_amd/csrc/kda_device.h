// Device helpers shared by every arm of the mixer. Each stage of the path is
// written once here and called by all kernels with the same lane mapping, so the
// fused decode kernel, the split prefill pipeline and the chunked prefill see
// bit-identical conv, l2 and norm results (the decode == verify identity of
// memra-engine kda.rs, ConvArm notes, and its scan-chain identity in stage 5).
//
// Build with -ffp-contract=off: every fused multiply-add below is explicit, so no
// arm can differ from another by a contraction the compiler chose on its own.
#pragma once

#include <hip/hip_runtime.h>

#include "kda_internal.h"

namespace kda {

// Widest conv kernel. The conv window lives in KMAX-1 registers per channel.
// (memra-engine kda.rs, KDA_MAX_CONV_KERNEL.)
constexpr int KMAX = 8;
// l2 epsilon, added to the sum of squares inside the square root (kda.rs,
// KDA_L2_EPS; aprender-serve gdn_ops.rs, gdn_per_head_l2_norm_into).
constexpr float L2_EPS = 1e-6f;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

using bf16_t = unsigned short;
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float((unsigned)b << 16); }

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ bf16_t f2bf(float f) {
    unsigned u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

template <bool BF>
__device__ __forceinline__ float ld_act(const void* p, size_t i) {
    if constexpr (BF)
        return bf2f(static_cast<const bf16_t*>(p)[i]);
    else
        return static_cast<const float*>(p)[i];
}

template <bool BF>
__device__ __forceinline__ void st_act(void* p, size_t i, float x) {
    if constexpr (BF)
        static_cast<bf16_t*>(p)[i] = f2bf(x);
    else
        static_cast<float*>(p)[i] = x;
}

// e^x through the hardware base-2 exponential.
__device__ __forceinline__ float exp_f(float x) { return __builtin_amdgcn_exp2f(x * LOG2E); }
// 1 / (1 + e^{-x}) through the hardware reciprocal (about 1 ulp; the IEEE division
// sequence costs several times more instructions on the conv's hot loop).
__device__ __forceinline__ float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.0f + exp_f(-x)); }
__device__ __forceinline__ float silu_f(float x) { return x * sigmoid_f(x); }
// ln(1 + e^x) through the hardware base-2 exponential and logarithm; x itself from 20
// on, where the two differ by less than e^-20.
__device__ __forceinline__ float softplus_f(float x) {
    return x > 20.0f ? x : __builtin_amdgcn_logf(1.0f + exp_f(x)) * LN2;
}

// Gate activations (memra-engine kda.rs, stage 4 and its per-channel gate kernel:
// g = lb * sigmoid(exp(A_log[h]) * (f + dt_bias[c])), beta = sigmoid(b_raw);
// aprender-serve gdn_ops.rs, the per-head gates: g = a[h] * softplus(alpha + dt_bias[h]),
// here also bounded below by lb). x is the pre-activation, c indexes the bias.
// m is the per-head factor of gate_head_factor.
__device__ __forceinline__ float gate_act_core(int form, float lb, float m, float bias, float x) {
    const float t = x + bias;
    return form == GATE_SIGMOID ? lb * sigmoid_f(m * t) : fmaxf(lb, m * softplus_f(t));
}
// The activated log gate times log2(e), for a form fixed at compile time, from the
// pre-activation x with per-column constants folded in (gate_log2_consts): sigmoid,
// lb2 / (1 + 2^{k1 x + k0}) with k1 = -m log2 e, k0 = k1 * bias; softplus,
// max(lb2, m * log2(1 + 2^u)) with u = x log2 e + k0, k0 = bias * log2 e, and u itself
// from x + bias = 20 on (as softplus_f). lb2 = lb * log2 e.
template <int FORM>
__device__ __forceinline__ float gate_act_log2(float lb2, float m, float k1, float k0, float x) {
    static_assert(FORM == GATE_SIGMOID || FORM == GATE_SOFTPLUS, "an activated form");
    const float u = fmaf(x, k1, k0);
    if constexpr (FORM == GATE_SIGMOID) return lb2 * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(u));
    else return fmaxf(lb2, m * (u > 20.0f * LOG2E ? u : __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(u))));
}
template <int FORM>
__device__ __forceinline__ void gate_log2_consts(float m, float bias, float* k1, float* k0) {
    *k1 = FORM == GATE_SIGMOID ? -m * LOG2E : LOG2E;
    *k0 = *k1 * bias;
}
// exp(A_log[h]) for the sigmoid form, a[h] for the softplus form.
__device__ __forceinline__ float gate_head_factor(const MixerArgs& a, int h) {
    return a.gate_form == GATE_SIGMOID ? exp_f(a.gate_a[h]) : a.gate_a[h];
}
// The beta a kernel uses for what it read from beta.
__device__ __forceinline__ float beta_in(const MixerArgs& a, float x) {
    return a.gate_form != GATE_GIVEN ? sigmoid_f(x) : x;
}
// Raw activation parameters of one gate column (head h, bias column c), for kernels
// whose threads keep one column: read before any large load is issued, so that using
// them waits for nothing else (vector-memory counters complete in order).
struct GateCol {
    float a, bias;
};
__device__ __forceinline__ GateCol gate_col(const MixerArgs& a, int h, size_t c) {
    GateCol p{0.0f, 0.0f};
    if (a.gate_form != GATE_GIVEN) {
        p.a = a.gate_a[h];
        p.bias = a.gate_bias[c];
    }
    return p;
}
// The log gate a kernel uses for what it read from g.
__device__ __forceinline__ float gate_in(const MixerArgs& a, const GateCol& p, float x) {
    if (a.gate_form == GATE_GIVEN) return x;
    const float m = a.gate_form == GATE_SIGMOID ? exp_f(p.a) : p.a;
    return gate_act_core(a.gate_form, a.gate_lb, m, p.bias, x);
}

// Butterfly sums. Every lane of the group ends with the same bits (each step adds
// the same two operands, only in swapped order).
// The 8-lane sum runs on DPP (no LDS crossbar traffic): quad_perm [1,0,3,2] and
// [2,3,0,1] pair lane bits 0 and 1, then row_half_mirror pairs lane l with 7 - l of
// its 8-lane group. After the first two steps every lane of a quad holds the same
// value, so the last step adds the two quads' values exactly as a partner across lane
// bit 2 would. The groups must be aligned to 8 lanes and the wavefront fully active.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float sum_lanes8(float v) {
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    v += dpp_mov<0x141>(v);
    return v;
}
// The same sum through the LDS crossbar (lane xor 1, 2, 4): identical bits. Kernels
// whose scan interleaves many column sums per thread (four columns in the grouped-head
// pair kernel) measured faster with it, the VALU pipe being the busier one there.
__device__ __forceinline__ float sum_lanes8_xbar(float v) {
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    v += __shfl_xor(v, 4, 64);
    return v;
}

// The 64-lane sum: the 8-lane steps, row_mirror (lane l with 15 - l: the two 8-lane
// halves of a row), then v_permlane16_swap and v_permlane32_swap (lane bits 4 and 5;
// each returns a lane's own value and its partner's, in an order that depends on the
// lane, which an addition does not see). As above, each step pairs groups whose lanes
// already hold one value, so the sum has the bits of the lane-xor butterfly.
__device__ __forceinline__ float sum_lanes64(float v) {
    v = sum_lanes8(v);
    v += dpp_mov<0x140>(v);
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// ---------------------------------------------------------------------------
// Causal depthwise conv, one channel per thread (memra-engine kda.rs, CONV FUSION
// notes and ConvArm; aprender-serve gdn_ops.rs, gdn_causal_conv1d_silu_into).
// win[KMAX-2] is the newest previous raw input, win[KMAX-1-d] the input d steps
// back; tap[d] = w[K-1-d] multiplies the input d steps back (tap[0] the current
// one); taps beyond K are zero, so the sum runs over the window in ascending time
// order (oldest first) exactly as for a K-wide window.
// ---------------------------------------------------------------------------
struct ConvChannel {
    float win[KMAX - 1];
    float tap[KMAX];
};

__device__ __forceinline__ void conv_load_taps(ConvChannel& c, const float* w_row, int K) {
#pragma unroll
    for (int d = 0; d < KMAX; ++d) c.tap[d] = (d < K) ? w_row[K - 1 - d] : 0.0f;
}

// Push the raw input x, return the pre-activation conv output for it.
__device__ __forceinline__ float conv_push(ConvChannel& c, float x) {
    float acc = 0.0f;
#pragma unroll
    for (int d = KMAX - 1; d >= 1; --d) acc = fmaf(c.tap[d], c.win[KMAX - 1 - d], acc);
    acc = fmaf(c.tap[0], x, acc);
#pragma unroll
    for (int e = 0; e < KMAX - 2; ++e) c.win[e] = c.win[e + 1];
    c.win[KMAX - 2] = x;
    return acc;
}

// Ring row of one channel: K-1 fp32 slots, slot 0 = oldest raw input.
__device__ __forceinline__ void conv_window_from_ring(ConvChannel& c, const float* ring_row, int K) {
#pragma unroll
    for (int d = 1; d < KMAX; ++d)
        c.win[KMAX - 1 - d] = (d <= K - 1) ? ring_row[K - 1 - d] : 0.0f;
}

__device__ __forceinline__ void conv_window_to_ring(const ConvChannel& c, float* ring_row, int K) {
#pragma unroll
    for (int d = 1; d < KMAX; ++d)
        if (d <= K - 1) ring_row[K - 1 - d] = c.win[KMAX - 1 - d];
}

// ---------------------------------------------------------------------------
// Per-row reductions, one wavefront per row of D <= 128 values held in LDS:
// lane l owns elements l and l + 64.
// ---------------------------------------------------------------------------

// l2-normalise the q and k rows of one (token, head) in place and return k.q of the
// normalised rows in *kq_out (memra-engine kda.rs, kda_core_gated stage 3).
template <int D>
__device__ __forceinline__ void l2_qk_row(float* qrow, float* krow, int lane, float* kq_out) {
    const bool h0 = lane < D, h1 = lane + 64 < D;
    float q0 = h0 ? qrow[lane] : 0.0f, q1 = h1 ? qrow[lane + 64] : 0.0f;
    float k0 = h0 ? krow[lane] : 0.0f, k1 = h1 ? krow[lane + 64] : 0.0f;
    const float iq = rsqrtf(sum_lanes64(fmaf(q1, q1, q0 * q0)) + L2_EPS);
    const float ik = rsqrtf(sum_lanes64(fmaf(k1, k1, k0 * k0)) + L2_EPS);
    q0 *= iq;
    q1 *= iq;
    k0 *= ik;
    k1 *= ik;
    if (h0) {
        qrow[lane] = q0;
        krow[lane] = k0;
    }
    if (h1) {
        qrow[lane + 64] = q1;
        krow[lane + 64] = k1;
    }
    const float kq = sum_lanes64(fmaf(k1, q1, k0 * q0));
    if (lane == 0) *kq_out = kq;
}

// Gated RMSNorm of one (token, head) row: o / sqrt(mean o^2 + eps) * w * gate(z),
// gate = sigmoid (KDA) or SiLU (GDN) (memra-engine kda.rs, kda_core_gated stage 6
// and kda_gated_rmsnorm; aprender-serve gdn_ops.rs, gdn_gated_rmsnorm_into).
// `off` is the element offset of the row in z / out; o_copy (may be null) receives
// the un-normalised row. The gate inputs are fetched separately (load_gate_row) so a
// kernel can issue that load long before the row is ready.
struct GateRow {
    float z0, z1;
};

template <int D, bool BF>
__device__ __forceinline__ GateRow load_gate_row(const MixerArgs& a, size_t off, int lane) {
    GateRow g;
    g.z0 = lane < D ? ld_act<BF>(a.z, off + lane) : 0.0f;
    g.z1 = lane + 64 < D ? ld_act<BF>(a.z, off + lane + 64) : 0.0f;
    return g;
}

template <int D, bool BF, bool GDN>
__device__ __forceinline__ void gated_rmsnorm_row(const float* orow, GateRow gz, const MixerArgs& a,
                                                  size_t off, int lane, float* o_copy) {
    const bool h0 = lane < D, h1 = lane + 64 < D;
    const float o0 = h0 ? orow[lane] : 0.0f, o1 = h1 ? orow[lane + 64] : 0.0f;
    const float ss = sum_lanes64(fmaf(o1, o1, o0 * o0));
    const float inv = rsqrtf(fmaf(ss, 1.0f / D, a.rms_eps));
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        if (!(half ? h1 : h0)) continue;
        const int j = lane + 64 * half;
        const float o = half ? o1 : o0;
        const float zz = half ? gz.z1 : gz.z0;
        const float gate = GDN ? silu_f(zz) : sigmoid_f(zz);
        st_act<BF>(a.out, off + j, ((o * inv) * a.norm_w[j]) * gate);
        if (o_copy) o_copy[off + j] = o;
    }
}

// ---------------------------------------------------------------------------
// The sequential scan on register-resident state (memra-engine kda.rs,
// kda_core_gated stage 5 and kda_scan; aprender-serve gdn_ops.rs,
// gdn_delta_rule_into). Value column j of a head's state is owned by 8
// consecutive lanes; sub-lane s (0..7) holds the D/8 keys
//   i = m*8*VEC + s*VEC + e   (m < D/(8*VEC), e < VEC, VEC = min(4, D/8)),
// so each 16-byte load of 8 sub-lanes covers 128 contiguous bytes of the row.
// ---------------------------------------------------------------------------
template <int D>
struct ColLayout {
    static constexpr int KPL = D / 8;
    static constexpr int VEC = KPL >= 4 ? 4 : KPL;
    static constexpr int M = KPL / VEC;
};

// Gather / scatter this sub-lane's keys of a D-long state row in HBM. The state is
// streamed once per call, so the 16-byte accesses are nontemporal (measured on the
// decode step: 5.6 TB/s with the hint against 4.8 TB/s without; the same hint on the
// conv ring and the activations, whose accesses are narrower, made it slower).
template <int D>
__device__ __forceinline__ void load_keys(float (&dst)[D / 8], const float* row, int s) {
    using L = ColLayout<D>;
#pragma unroll
    for (int m = 0; m < L::M; ++m) {
        const float* p = row + m * 8 * L::VEC + s * L::VEC;
        if constexpr (L::VEC == 4) {
            const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
            dst[4 * m + 0] = t[0];
            dst[4 * m + 1] = t[1];
            dst[4 * m + 2] = t[2];
            dst[4 * m + 3] = t[3];
        } else {
            static_assert(L::VEC == 2, "D must be 16 or a multiple of 32");
            const float2 t = *reinterpret_cast<const float2*>(p);
            dst[2 * m + 0] = t.x;
            dst[2 * m + 1] = t.y;
        }
    }
}

template <int D>
__device__ __forceinline__ void store_keys(float* row, const float (&src)[D / 8], int s) {
    using L = ColLayout<D>;
#pragma unroll
    for (int m = 0; m < L::M; ++m) {
        float* p = row + m * 8 * L::VEC + s * L::VEC;
        if constexpr (L::VEC == 4) {
            const f32x4 t = {src[4 * m], src[4 * m + 1], src[4 * m + 2], src[4 * m + 3]};
            __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(p));
        } else {
            *reinterpret_cast<float2*>(p) = make_float2(src[2 * m], src[2 * m + 1]);
        }
    }
}

// One token of the recurrence for CPT value columns of one head. Every column is
// owned by 8 consecutive lanes with the key mapping above; q, k are the
// l2-normalised rows, erow holds exp(g) (D values for KDA, one for GDN), vj the
// columns' v values, kq = k.q. The readout uses the post-update state, expanded as
// S'^T q + beta u (k.q) where S' is the decayed state, so both reductions run in one
// pass. The arithmetic of a column does not depend on CPT or XBAR (which lane path
// the column sums take): every arm produces the same bits for the same column.
template <int D, bool GDN, int CPT, bool XBAR = false>
__device__ __forceinline__ void scan_step_cols(float (&S)[CPT][D / 8], const float* qrow,
                                               const float* krow, const float* erow,
                                               const float (&vj)[CPT], float beta, float kq,
                                               float scale, int s, float (&o)[CPT]) {
    using L = ColLayout<D>;
    static_assert(L::VEC % 2 == 0, "keys per chunk must be even");
    float a0[CPT], a1[CPT], b0[CPT], b1[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) a0[c] = a1[c] = b0[c] = b1[c] = 0.0f;
    const float eh = GDN ? erow[0] : 0.0f;
#pragma unroll
    for (int m = 0; m < L::M; ++m) {
        const int base = m * 8 * L::VEC + s * L::VEC;
        float kv[L::VEC], qv[L::VEC], ev[L::VEC];
#pragma unroll
        for (int e = 0; e < L::VEC; ++e) {
            kv[e] = krow[base + e];
            qv[e] = qrow[base + e];
            ev[e] = GDN ? eh : erow[base + e];
        }
#pragma unroll
        for (int e = 0; e < L::VEC; ++e)
#pragma unroll
            for (int c = 0; c < CPT; ++c) S[c][m * L::VEC + e] *= ev[e];
#pragma unroll
        for (int e = 0; e < L::VEC; e += 2) {
            const int x = m * L::VEC + e;
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                a0[c] = fmaf(S[c][x], kv[e], a0[c]);
                a1[c] = fmaf(S[c][x + 1], kv[e + 1], a1[c]);
                b0[c] = fmaf(S[c][x], qv[e], b0[c]);
                b1[c] = fmaf(S[c][x + 1], qv[e + 1], b1[c]);
            }
        }
    }
    float bu[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const float sk = XBAR ? sum_lanes8_xbar(a0[c] + a1[c]) : sum_lanes8(a0[c] + a1[c]);
        const float sq = XBAR ? sum_lanes8_xbar(b0[c] + b1[c]) : sum_lanes8(b0[c] + b1[c]);
        bu[c] = beta * (vj[c] - sk);
        o[c] = scale * fmaf(bu[c], kq, sq);
    }
#pragma unroll
    for (int m = 0; m < L::M; ++m) {
        const int base = m * 8 * L::VEC + s * L::VEC;
#pragma unroll
        for (int e = 0; e < L::VEC; ++e) {
            const float kk = krow[base + e];
#pragma unroll
            for (int c = 0; c < CPT; ++c) S[c][m * L::VEC + e] = fmaf(kk, bu[c], S[c][m * L::VEC + e]);
        }
    }
}

}  // namespace kda
