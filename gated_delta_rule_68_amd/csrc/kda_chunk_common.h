// Device helpers shared by the two chunked prefill kernels (kda_chunk.hip: 64-row
// chunks, 8 wavefronts per workgroup; kda_c32.hip: 32-row chunks, 16 wavefronts in
// two specialised groups): MFMA and LDS primitives, cross-lane sums, conv taps, and the
// mapping of a segmented-arm workgroup to its run.
#pragma once

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int CHUNK_DK = 128;  // head dim of the chunked arms

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// MFMA 16x16x32 operand layout (lane l, q4 = l / 16, l16 = l % 16): an A fragment
// holds A[l16][8 q4 .. 8 q4 + 7] of a 16x32 tile, a B fragment B[8 q4 .. + 7][l16] of a
// 32x16 tile, and the 16x16 result D[4 q4 + r][l16] for r = 0..3. Only the pairing of
// the two fragments' slots matters: any k order shared by A and B gives the same sum.
__device__ __forceinline__ f32x4v mfma_bf16(bf16x8 a, bf16x8 b, f32x4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// 16x16x4 fp32: lane l gives A[l16][slot q4] and B[slot q4][l16]; result as above.
__device__ __forceinline__ f32x4v mfma_f32(float a, float b, f32x4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 ld8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void st8(__bf16* p, bf16x8 v) { *reinterpret_cast<bf16x8*>(p) = v; }
__device__ __forceinline__ bf16x2 ld2(const __bf16* p) { return *reinterpret_cast<const bf16x2*>(p); }
__device__ __forceinline__ void st2(__bf16* p, bf16x2 v) { *reinterpret_cast<bf16x2*>(p) = v; }
__device__ __forceinline__ f32x4v zero4() { return f32x4v{0.0f, 0.0f, 0.0f, 0.0f}; }
__device__ __forceinline__ f32x4v ld4f(const float* p) { return *reinterpret_cast<const f32x4v*>(p); }
// 2^x; gate sums in the chunked kernels are kept in log2 units (scaled by log2 e once).
__device__ __forceinline__ float exp2_f(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ bf16x8 zero8() {
    const __bf16 z = (__bf16)0.0f;
    return bf16x8{z, z, z, z, z, z, z, z};
}

// Raw buffer resource over `bytes` bytes from p (gfx9 word 3: 32-bit data format, no
// swizzle, no stride). Accesses at or past `bytes` do not touch memory: stores are
// dropped and loads return zero. Loads and stores through it take a wave-uniform scalar
// offset and a per-lane vector offset, so a row index that is the same across a
// wavefront costs scalar arithmetic only.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
constexpr uint32_t BUF_ALL = 0xffffffffu;  // no range limit (the caller keeps offsets in range)

// Workgroup barrier that orders LDS only: it waits for this wave's LDS operations and
// not for its outstanding global loads, so prefetched rows stay in flight across the
// phases of a chunk. (Every value crossing phases goes through LDS or registers;
// global stores are never read back.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// Orders this wave's own LDS writes before its later LDS reads (no other wave involved).
__device__ __forceinline__ void lds_wave_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// ---- cross-lane sums on the DPP / permlane paths (no LDS traffic) ----
// DPP controls: quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E, row_ror:8 = 0x128,
// row_mirror = 0x140, row_half_mirror = 0x141.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), CTRL, 0xf, 0xf, false));
}
// Sum over the 16 lanes of a DPP row (every lane of the row gets the sum).
__device__ __forceinline__ float sum_row16(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);  // lanes l and 7 - l: the two quads of each half row
    x += dpp<0x140>(x);  // lanes l and 15 - l: the two halves
    return x;
}
// Sixteen sums over the 64 lanes at once: lane l returns sum over all lanes of
// p[l >> 2]. Each step halves the values a lane keeps (it keeps the half selected by
// one lane bit and adds its partner's copy of that half): v_permlane32_swap pairs lane
// bit 5, v_permlane16_swap bit 4, DPP row_ror:8 bit 3, row_half_mirror bit 2, and the
// quad permutations finish the sum over bits 0 and 1.
__device__ __forceinline__ float sum16x64(float (&p)[16], int lane) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[i]), __float_as_uint(p[i + 8]), false, false);
        p[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);  // row i + 8 * bit5
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(p[i]), __float_as_uint(p[i + 4]), false, false);
        p[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);  // row i + 4 * bit4 + 8 * bit5
    }
    const bool b3 = lane & 8, b2 = lane & 4;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const float lo = p[i] + dpp<0x128>(p[i]), hi = p[i + 2] + dpp<0x128>(p[i + 2]);
        p[i] = b3 ? hi : lo;
    }
    const float lo = p[0] + dpp<0x141>(p[0]), hi = p[1] + dpp<0x141>(p[1]);
    float x = b2 ? hi : lo;
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    return x;
}

// Eight sums over the 64 lanes at once: lane l returns sum over all lanes of
// p[l >> 3]. The same halving steps as sum16x64 over lane bits 5, 4 and 3; the three
// remaining bits are then summed by row_half_mirror and the quad permutations.
__device__ __forceinline__ float sum8x64(float (&p)[8], int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[i]), __float_as_uint(p[i + 4]), false, false);
        p[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);  // row i + 4 * bit5
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(p[i]), __float_as_uint(p[i + 2]), false, false);
        p[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);  // row i + 2 * bit4 + 4 * bit5
    }
    const bool b3 = lane & 8;
    const float lo = p[0] + dpp<0x128>(p[0]), hi = p[1] + dpp<0x128>(p[1]);
    float x = b3 ? hi : lo;
    x += dpp<0x141>(x);
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    return x;
}

// Conv taps of N consecutive channels starting at fused conv row `row`, aligned so
// that w[e][KT-1] multiplies the current input (zero for the KT-K oldest slots).
template <int KT, int N>
__device__ __forceinline__ void load_taps(float (&w)[N][KT], const float* conv_w, size_t row, int K) {
#pragma unroll
    for (int e = 0; e < N; ++e)
#pragma unroll
        for (int j = 0; j < KT; ++j) {
            const int tap = j - (KT - K);  // index into the K-wide weight row (K <= KT)
            const float x = conv_w[(row + e) * K + max(tap, 0)];
            w[e][j] = tap >= 0 ? x : 0.0f;
        }
}

// The D x D fp32 state blocks of the segmented arm's workspace (seg_layout in
// kda_internal.h), in state layout [value][key]: the entry states S_s (s = 1 .. n-1)
// and the transitions M_s and offsets B_s (s = 1 .. n-2) of pair p.
struct SegSlots {
    float* base;
    int P, n;
    __device__ float* blk(size_t i, int p) const { return base + (i * P + p) * ((size_t)CHUNK_DK * CHUNK_DK); }
    __device__ float* S(int s, int p) const { return blk(s - 1, p); }
    __device__ float* M(int s, int p) const { return blk(n - 1 + s - 1, p); }
    __device__ float* B(int s, int p) const { return blk(2 * n - 3 + s - 1, p); }
};
__device__ __forceinline__ SegSlots seg_slots(const MixerArgs& a) {
    const int P = a.B * a.H;
    char* ws = reinterpret_cast<char*>(a.seg_ws);
    return SegSlots{reinterpret_cast<float*>(ws + seg_layout(P, a.H, CHUNK_DK, a.seg_n).slots), P, a.seg_n};
}

// The run of one workgroup of the segmented arm: its (b, h) pair, rows [ro, ro + len)
// of the sequence, where its state comes from and goes to, whether v is replaced by
// zeros (the M runs) and whether the outputs are written.
struct SegRun {
    int pair, ro, len;
    const float* s_in;
    float* s_out;
    bool zero_v, readout;
    int s_init;  // the entry state: 0 read from s_in, 1 zero, 2 identity (s_in holds it too)
};

// Pass 1: blocks [0, P) run segment 0 of pair b (dispatched first: they are the
// longest). Block P + 16 g + 8 kind + j runs the B (kind 0) or M (kind 1) run of slot
// 8 g + j = (s - 1) P + pair: the two runs of one slot are 8 blocks apart and so on
// the same XCD, whose L2 then serves both with the same rows. Pass 3: block
// (s - 1) P + pair runs segment s. Returns false for the padding blocks of the grid.
__device__ __forceinline__ bool seg_run(const MixerArgs& a, SegRun* r) {
    const int P = a.B * a.H, n = a.seg_n, L0 = a.seg_len0, L = a.seg_len;
    const size_t blk = (size_t)CHUNK_DK * CHUNK_DK;
    char* ws = reinterpret_cast<char*>(a.seg_ws);
    const SegLayout lay = seg_layout(P, a.H, CHUNK_DK, n);
    const SegSlots sl = seg_slots(a);
    const int d = blockIdx.x;
    r->zero_v = false;
    r->readout = true;
    r->s_init = 0;
    if (a.seg_pass == 1) {
        if (d < P) {
            r->pair = d;
            r->ro = 0;
            r->len = n == 1 ? a.T : L0;
            r->s_in = a.state_in + (size_t)d * blk;
            r->s_out = n == 1 ? a.state_out + (size_t)d * blk : sl.S(1, d);
            return true;
        }
        const int e = d - P, kind = (e % 16) / 8, slot = (e / 16) * 8 + e % 8;
        if (n < 3 || slot >= (n - 2) * P) return false;
        const int p = slot % P, sg = 1 + slot / P;
        r->pair = p;
        r->ro = L0 + (sg - 1) * L;
        r->len = L;
        r->readout = false;
        r->zero_v = kind == 1;
        r->s_init = kind ? 2 : 1;
        r->s_in = reinterpret_cast<const float*>(ws + (kind ? lay.ident : lay.zero));
        r->s_out = kind ? sl.M(sg, p) : sl.B(sg, p);
        return true;
    }
    if (d >= (n - 1) * P) return false;
    const int p = d % P, sg = 1 + d / P;
    r->pair = p;
    r->ro = L0 + (sg - 1) * L;
    r->len = sg == n - 1 ? a.T - r->ro : L;
    r->s_in = sl.S(sg, p);
    r->s_out = sg == n - 1 ? a.state_out + (size_t)p * blk : sl.B(sg, p);  // B_s is spent by then
    return true;
}

}  // namespace kda
