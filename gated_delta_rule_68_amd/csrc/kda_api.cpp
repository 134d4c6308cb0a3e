// Host side of the C ABI declared in include/kda.h: argument validation (all of
// it before any launch, so a rejected call writes nothing on the device), arm
// selection and dispatch to the HIP launchers.
//
// Status convention (memra-engine mla_ffi.rs, module header): 0 ok, 10000 + the
// runtime error of a failing launch, 40000 + a contract violation.
#include "kda.h"

#include <stdint.h>
#include <string.h>

#include "kda_internal.h"

namespace {

using kda::MixerArgs;

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
    bool writable;
    int id;
};

bool overlaps(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

bool head_dim_ok(int D) { return D == 16 || D == 128; }

// Shape checks shared by the entry points and the workspace / arm queries.
int check_shape(int B, int T, int H, int D, int K) {
    if (B < 1 || T < 1 || H < 1) return KDA_ERR_SHAPE;
    if (!head_dim_ok(D)) return KDA_ERR_HEAD_DIM;
    if (K < 2 || K > 8) return KDA_ERR_CONV_KERNEL;
    // Element counts are formed in 64-bit; keep every tensor below 2^40 elements and
    // the (b, h) grid inside a launch dimension.
    const double elems = (double)B * (double)T * (double)H * (double)D;
    const double state = (double)B * (double)H * (double)D * (double)D;
    if (elems > 1099511627776.0 || state > 1099511627776.0) return KDA_ERR_SHAPE;
    if ((double)B * (double)H * 8.0 > 2147483647.0) return KDA_ERR_SHAPE;
    return KDA_OK;
}

// Which arm runs. Sequential work needs many (b, h) pairs to fill the chip with one
// fused workgroup per pair; below that the column-split pipeline is used, except for
// very short prefills where its extra launches would dominate.
// The chunked arm (D = 128) computes its contractions with bf16 operands, so AUTO
// takes it only for bf16 activations, from 33 tokens on, or from 17 when there are
// fewer than 1024 (b, h) pairs (where the sequential arm would be the column-split
// pipeline): measured faster than either sequential arm there (e.g. B = 64, H = 64:
// 0.38 against 0.46 ms at T = 40, 0.40 against 0.75 ms at T = 64; B = 8, H = 64,
// T = 24: 53 against 89 us), and slower below (B = 64, H = 64: 0.38 against 0.35 ms
// at T = 32, against 0.27 ms at T = 24).
// Few (b, h) pairs leave most compute units idle in the chunked arm. AUTO takes the
// segmented arm (kda_internal.h, seg_plan) when its plan, with segments of at least
// kSegAutoChunks 64-row units, shortens the critical path to at most 85% of the
// chunked arm's (the margin covers the higher clock the chip holds with few units
// busy). The explicit mode plans by chunk counts alone and accepts segments of one
// unit, so it also cuts sequences too short for segments to pay.
constexpr int kSegAutoChunks = 8;
kda::SegPlan plan_for(int B, int T, int H, int mode) {
    return mode == KDA_MODE_SEGMENTED ? kda::seg_plan((long)B * H, T, 1, false)
                                      : kda::seg_plan((long)B * H, T, kSegAutoChunks, true);
}
bool segments_pay(int B, int T, int H) {
    const kda::SegPlan p = plan_for(B, T, H, KDA_MODE_AUTO);
    return p.n >= 3 && p.cost * 100 <= 85 * kda::seg_chunked_cost(T);
}

//
// The chunked and segmented arms take bf16 activations only: their contractions run
// on bf16 operands, which cannot meet the fp32 accuracy bar (rel L-inf <= 1e-3), so
// fp32 activations always take a sequential arm and the explicit modes reject them.
// Their decay factorisation needs g >= -5 (kda_chunk.hip). Given gates carry that
// as a precondition; activated gates are bounded by gate_lb, and a bound below -5
// (gates_ok false) sends AUTO to the fused sequential arm, which needs no workspace
// (so a workspace sized by the query for given gates still suffices), while the
// explicit chunked and segmented modes reject the call.
int pick_arm(int B, int T, int H, int D, bool bf16, int mode, bool gates_ok = true) {
    const bool chunk_ok = kda::kChunkedArmBuilt && D == 128 && bf16 && gates_ok;
    if (mode == KDA_MODE_CHUNKED) return chunk_ok ? kda::ARM_CHUNKED : -1;
    if (mode == KDA_MODE_SEGMENTED) return chunk_ok ? kda::ARM_SEGMENTED : -1;
    if (mode != KDA_MODE_AUTO && mode != KDA_MODE_SEQUENTIAL) return -1;
    const bool chunk_len = T > 32 || (T > 16 && (long)B * H < 1024);
    if (mode == KDA_MODE_AUTO && chunk_len && D == 128 && bf16) {
        if (!gates_ok) return kda::ARM_SEQ_FUSED;
        return segments_pay(B, T, H) ? kda::ARM_SEGMENTED : kda::ARM_CHUNKED;
    }
    if (T <= 16 || (long)B * H >= 1024) return kda::ARM_SEQ_FUSED;
    return kda::ARM_SEQ_SPLIT;
}

// Whether activated gates stay inside the chunked arm's range (g >= -5): gate_lb is
// their lower bound in both activation forms (NaN fails the test).
bool gates_in_chunk_range(int gate_form, float gate_lb) {
    return gate_form == kda::GATE_GIVEN || gate_lb >= -5.0f;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// Head of a packed batch's workspace: the longest-first order of its B sequences.
size_t order_bytes(int B) { return align256((size_t)B * 4); }

// Query / key heads: a divisor of the value heads H (grouped heads, GDN only).
int check_heads(int H, int Hk) { return Hk >= 1 && Hk <= H && H % Hk == 0 ? KDA_OK : KDA_ERR_SHAPE; }

// Arm of a packed variable-length batch: the fused sequential arm (one workgroup per
// (sequence, head), whatever the lengths) or the chunked arm; AUTO takes the chunked
// arm for bf16 activations at D = 128.
int pick_arm_varlen(int D, bool bf16, int mode, bool gates_ok = true) {
    const bool chunk_ok = kda::kChunkedArmBuilt && D == 128 && bf16 && gates_ok;
    if (mode == KDA_MODE_CHUNKED) return chunk_ok ? kda::ARM_CHUNKED : -1;
    if (mode == KDA_MODE_SEGMENTED) return -1;  // segments of equal-length sequences only
    if (mode == KDA_MODE_AUTO && chunk_ok) return kda::ARM_CHUNKED;
    if (mode != KDA_MODE_AUTO && mode != KDA_MODE_SEQUENTIAL) return -1;
    return kda::ARM_SEQ_FUSED;
}

// rows: activation rows of all sequences (B*T, or T for a packed batch).
size_t workspace_for(int B, int T, int H, int Hk, int D, bool gdn, int arm, size_t rows = 0,
                     int mode = KDA_MODE_AUTO) {
    if (rows == 0) rows = (size_t)B * T;
    switch (arm) {
        case kda::ARM_SEQ_SPLIT: return kda::split_workspace(B, T, H, Hk, D, gdn).total;
        case kda::ARM_CHUNKED: return kda::chunked_workspace_bytes(B, rows, H, D);
        case kda::ARM_SEGMENTED: return kda::segmented_workspace_bytes(B, H, D, plan_for(B, T, H, mode).n);
        default: return 0;
    }
}

// need_out (optional) receives the workspace bytes the call needs, once the shape,
// arm and pointer alignment have passed.
int validate(const MixerArgs& a, bool decode, int mode, int* arm_out, size_t* need_out = nullptr) {
    if (!a.q || !a.k || !a.v || !a.g || !a.beta || !a.conv_w || !a.ring || !a.state_in ||
        !a.state_out || !a.z || !a.norm_w || !a.out)
        return KDA_ERR_NULL;
    const bool packed = a.cu_seqlens != nullptr;
    // a packed batch: B sequences (the state / ring / grid dimension), T rows in all
    int rc = packed ? check_shape(1, a.T, a.H, a.D, a.K) : check_shape(a.B, a.T, a.H, a.D, a.K);
    if (!rc && packed) rc = check_shape(a.B, 1, a.H, a.D, a.K);
    if (rc) return rc;
    if (decode && a.T != 1) return KDA_ERR_DECODE_T;
    const bool gates_ok = gates_in_chunk_range(a.gate_form, a.gate_lb);
    const int arm = decode ? (int)kda::ARM_SEQ_FUSED
                           : (packed ? pick_arm_varlen(a.D, a.bf16, mode, gates_ok)
                                     : pick_arm(a.B, a.T, a.H, a.D, a.bf16, mode, gates_ok));
    if (arm < 0) return KDA_ERR_DTYPE_MODE;

    if (a.gate_form != kda::GATE_GIVEN && (!a.gate_a || !a.gate_bias)) return KDA_ERR_NULL;
    const void* ptrs[] = {a.q, a.k, a.v, a.g, a.beta, a.conv_w, a.ring, a.state_in,
                          a.state_out, a.z, a.norm_w, a.out, a.o_core, a.ws, a.gate_a, a.gate_bias};
    for (const void* p : ptrs)
        if (p && ((uintptr_t)p & 15u)) return KDA_ERR_ALIGN;
    if (packed && ((uintptr_t)a.cu_seqlens & 3u)) return KDA_ERR_ALIGN;

    const size_t es = a.bf16 ? 2 : 4;
    const size_t qkv = (size_t)a.H * a.D;
    const size_t rows = kda::total_rows(a);
    const size_t act = rows * qkv;
    const size_t kact = rows * a.Hk * a.D;  // q, k
    const size_t rrows = kda::ring_rows(a);
    const size_t gate_n = a.gdn ? rows * a.H : act;
    const size_t state_n = (size_t)a.B * a.H * a.D * a.D;
    const size_t need_ws = workspace_for(a.B, a.T, a.H, a.Hk, a.D, a.gdn, arm, rows, mode) +
                           (packed ? order_bytes(a.B) : 0);
    if (need_out) *need_out = need_ws;
    if (need_ws > 0 && (!a.ws || a.ws_bytes < need_ws)) return KDA_ERR_WORKSPACE;

    auto R = [](const void* p, size_t bytes, bool w, int id) {
        return Range{(uintptr_t)p, (uintptr_t)p + bytes, w, id};
    };
    Range rs[17];
    int n = 0;
    rs[n++] = R(a.q, kact * es, false, 0);
    rs[n++] = R(a.k, kact * es, false, 1);
    rs[n++] = R(a.v, act * es, false, 2);
    rs[n++] = R(a.g, gate_n * es, false, 3);
    rs[n++] = R(a.beta, rows * a.H * es, false, 4);
    rs[n++] = R(a.conv_w, rrows * a.K * 4, false, 5);
    rs[n++] = R(a.ring, (size_t)a.B * rrows * (a.K - 1) * 4, true, 6);
    rs[n++] = R(a.state_in, state_n * 4, false, 7);
    rs[n++] = R(a.state_out, state_n * 4, true, 8);
    rs[n++] = R(a.z, act * es, false, 9);
    rs[n++] = R(a.norm_w, (size_t)a.D * 4, false, 10);
    rs[n++] = R(a.out, act * es, true, 11);
    if (a.o_core) rs[n++] = R(a.o_core, act * 4, true, 12);
    if (need_ws > 0) rs[n++] = R(a.ws, need_ws, true, 13);
    if (a.gate_form != kda::GATE_GIVEN) {
        rs[n++] = R(a.gate_a, (size_t)a.H * 4, false, 14);
        rs[n++] = R(a.gate_bias, (a.gdn ? (size_t)a.H : qkv) * 4, false, 15);
    }
    if (packed) rs[n++] = R(a.cu_seqlens, ((size_t)a.B + 1) * 4, false, 16);
    for (int i = 0; i < n; ++i)
        for (int j = i + 1; j < n; ++j) {
            if (!(rs[i].writable || rs[j].writable) || !overlaps(rs[i], rs[j])) continue;
            const bool state_pair = (rs[i].id == 7 && rs[j].id == 8) && a.state_in == a.state_out;
            if (!state_pair) return KDA_ERR_ALIAS;
        }
    *arm_out = arm;
    return KDA_OK;
}

int run(MixerArgs a, int arm, int mode = KDA_MODE_AUTO) {
    hipError_t e;
    if (arm == kda::ARM_SEGMENTED) {
        const kda::SegPlan p = plan_for(a.B, a.T, a.H, mode);
        a.seg_n = p.n;
        a.seg_len0 = p.len0;
        a.seg_len = p.len;
    }
    switch (arm) {
        case kda::ARM_SEGMENTED: e = kda::launch_segmented(a); break;
        case kda::ARM_SEQ_FUSED: e = kda::launch_seq_fused(a); break;
        case kda::ARM_SEQ_SPLIT: e = kda::launch_seq_split(a); break;
        case kda::ARM_CHUNKED: e = kda::launch_chunked(a); break;
        default: return KDA_ERR_DTYPE_MODE;
    }
    return e == hipSuccess ? KDA_OK : KDA_ERR_RUNTIME_BASE + (int)e;
}

struct GateArgs {
    int form;
    const float* a;
    const float* bias;
    float lb;
};
constexpr GateArgs kGiven{kda::GATE_GIVEN, nullptr, nullptr, 0.0f};

int entry(bool gdn, bool decode, const void* q, const void* k, const void* v, const void* g,
          const void* beta, const float* conv_w, float* conv_ring, const float* state_in,
          float* state_out, const void* z, const float* norm_w, void* out, float* o_core,
          int B, int T, int H, int D, int K, float scale, float rms_eps, int dtype, int mode,
          void* workspace, size_t workspace_bytes, void* stream, GateArgs ga = kGiven, int Hk = 0,
          const int* cu_seqlens = nullptr, bool static_ws = false) {
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return KDA_ERR_DTYPE_MODE;
    if (ga.form != kda::GATE_GIVEN && ga.form != KDA_GATE_SIGMOID && ga.form != KDA_GATE_SOFTPLUS)
        return KDA_ERR_DTYPE_MODE;
    if (Hk == 0) Hk = H;
    if (check_heads(H, Hk) || (!gdn && Hk != H)) return KDA_ERR_SHAPE;
    MixerArgs a{q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z, norm_w, out,
                o_core, B, T, H, D, K, scale, rms_eps, dtype == KDA_DTYPE_BF16, gdn,
                workspace, workspace_bytes, (hipStream_t)stream, T, true,
                ga.form, ga.a, ga.bias, ga.lb, Hk, cu_seqlens, nullptr};
    if (ga.form == kda::GATE_GIVEN) {
        // Kernels read the gate parameters without a branch; point them at conv_w
        // (3*H*D*K >= H*D floats, allocated and 16-byte aligned), values unused.
        a.gate_a = conv_w;
        a.gate_bias = conv_w;
    }
    int arm = 0;
    size_t need = 0;
    int rc = validate(a, decode, mode, &arm, &need);
    if (static_ws && rc == KDA_ERR_WORKSPACE) {
        // The workspace comes from the library's static scratch: sized first, so a call
        // the contract refuses looks nothing up; then the contract is checked again with
        // the scratch in place (its range against every other buffer).
        if (need > kda::static_scratch_bytes()) return KDA_ERR_SCRATCH;
        void* p = nullptr;
        const hipError_t e = kda::static_scratch(a.stream, &p);
        if (e != hipSuccess) return KDA_ERR_RUNTIME_BASE + (int)e;
        a.ws = p;
        a.ws_bytes = kda::static_scratch_bytes();
        rc = validate(a, decode, mode, &arm);
    }
    if (rc) return rc;
    if (a.cu_seqlens) {  // rank the sequences first; the arm's own workspace follows
        int* order = static_cast<int*>(a.ws);
        a.ws = static_cast<char*>(a.ws) + order_bytes(a.B);
        a.ws_bytes -= order_bytes(a.B);
        a.seq_order = order;
        const hipError_t e = kda::launch_seq_order(a, order);
        if (e != hipSuccess) return KDA_ERR_RUNTIME_BASE + (int)e;
    }
    return run(a, arm, mode);
}

// Rollback of a verify round: ring <- ring_snap, then the sequential arm replays the
// first `keep` of the T_stash stored rows of every sequence from state_snap, with no
// readout. Validated in full before the copy or any launch.
int rollback(bool gdn, const void* q, const void* k, const void* v, const void* g,
             const void* beta, const float* conv_w, const float* ring_snap,
             const float* state_snap, float* conv_ring, float* state_out, int B, int T_stash,
             int keep, int H, int D, int K, int dtype, void* workspace, size_t workspace_bytes,
             void* stream, GateArgs ga = kGiven, int Hk = 0) {
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return KDA_ERR_DTYPE_MODE;
    if (ga.form != kda::GATE_GIVEN && ga.form != KDA_GATE_SIGMOID && ga.form != KDA_GATE_SOFTPLUS)
        return KDA_ERR_DTYPE_MODE;
    if (!q || !k || !v || !g || !beta || !conv_w || !ring_snap || !state_snap || !conv_ring ||
        !state_out)
        return KDA_ERR_NULL;
    if (ga.form != kda::GATE_GIVEN && (!ga.a || !ga.bias)) return KDA_ERR_NULL;
    int rc = check_shape(B, T_stash, H, D, K);
    if (rc) return rc;
    if (keep < 1 || keep > T_stash) return KDA_ERR_SHAPE;
    if (Hk == 0) Hk = H;
    if (check_heads(H, Hk) || (!gdn && Hk != H)) return KDA_ERR_SHAPE;
    const bool bf16 = dtype == KDA_DTYPE_BF16;
    const int arm = pick_arm(B, keep, H, D, bf16, KDA_MODE_SEQUENTIAL);
    const void* ptrs[] = {q, k, v, g, beta, conv_w, ring_snap, state_snap, conv_ring, state_out, workspace,
                          ga.a, ga.bias};
    for (const void* p : ptrs)
        if (p && ((uintptr_t)p & 15u)) return KDA_ERR_ALIGN;
    const size_t need_ws = workspace_for(B, keep, H, Hk, D, gdn, arm);
    if (need_ws > 0 && (!workspace || workspace_bytes < need_ws)) return KDA_ERR_WORKSPACE;

    const size_t es = bf16 ? 2 : 4;
    const size_t qkv = (size_t)H * D;
    const size_t act = (size_t)B * T_stash * qkv;
    const size_t kact = (size_t)B * T_stash * Hk * D;
    const size_t rrows = (size_t)(2 * Hk + H) * D;
    const size_t ring_bytes = (size_t)B * rrows * (K - 1) * 4;
    const size_t state_bytes = (size_t)B * H * D * D * 4;
    auto Rg = [](const void* p, size_t bytes, bool w, int id) {
        return Range{(uintptr_t)p, (uintptr_t)p + bytes, w, id};
    };
    Range rs[13];
    int n = 0;
    rs[n++] = Rg(q, kact * es, false, 0);
    rs[n++] = Rg(k, kact * es, false, 1);
    rs[n++] = Rg(v, act * es, false, 2);
    rs[n++] = Rg(g, (gdn ? (size_t)B * T_stash * H : act) * es, false, 3);
    rs[n++] = Rg(beta, (size_t)B * T_stash * H * es, false, 4);
    rs[n++] = Rg(conv_w, rrows * K * 4, false, 5);
    rs[n++] = Rg(ring_snap, ring_bytes, false, 6);
    rs[n++] = Rg(state_snap, state_bytes, false, 7);
    rs[n++] = Rg(conv_ring, ring_bytes, true, 8);
    rs[n++] = Rg(state_out, state_bytes, true, 9);
    if (need_ws > 0) rs[n++] = Rg(workspace, need_ws, true, 10);
    if (ga.form != kda::GATE_GIVEN) {
        rs[n++] = Rg(ga.a, (size_t)H * 4, false, 11);
        rs[n++] = Rg(ga.bias, (gdn ? (size_t)H : qkv) * 4, false, 12);
    }
    for (int i = 0; i < n; ++i)
        for (int j = i + 1; j < n; ++j) {
            if (!(rs[i].writable || rs[j].writable) || !overlaps(rs[i], rs[j])) continue;
            const bool same = rs[i].lo == rs[j].lo;
            const bool ring_pair = rs[i].id == 6 && rs[j].id == 8 && same;
            const bool state_pair = rs[i].id == 7 && rs[j].id == 9 && same;
            if (!ring_pair && !state_pair) return KDA_ERR_ALIAS;
        }

    if (conv_ring != ring_snap) {
        const hipError_t e = hipMemcpyAsync(conv_ring, ring_snap, ring_bytes, hipMemcpyDeviceToDevice,
                                            (hipStream_t)stream);
        if (e != hipSuccess) return KDA_ERR_RUNTIME_BASE + (int)e;
    }
    MixerArgs a{q, k, v, g, beta, conv_w, conv_ring, state_snap, state_out, nullptr, nullptr, nullptr,
                nullptr, B, keep, H, D, K, 1.0f, 0.0f, bf16, gdn, workspace, workspace_bytes,
                (hipStream_t)stream, T_stash, false, ga.form, conv_w, conv_w, ga.lb, Hk, nullptr, nullptr};
    if (ga.form != kda::GATE_GIVEN) {
        a.gate_a = ga.a;
        a.gate_bias = ga.bias;
    }
    return run(a, arm);
}

size_t ws_query(bool gdn, int B, int T, int H, int D, int dtype, int mode, int Hk = 0) {
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return (size_t)-1;
    if (check_shape(B, T, H, D, 4)) return (size_t)-1;
    if (Hk == 0) Hk = H;
    if (check_heads(H, Hk)) return (size_t)-1;
    const int arm = pick_arm(B, T, H, D, dtype == KDA_DTYPE_BF16, mode);
    if (arm < 0) return (size_t)-1;
    return workspace_for(B, T, H, Hk, D, gdn, arm, 0, mode);
}

int arm_query(int B, int T, int H, int D, int dtype, int mode) {
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return -1;
    if (check_shape(B, T, H, D, 4)) return -1;
    return pick_arm(B, T, H, D, dtype == KDA_DTYPE_BF16, mode);
}

}  // namespace

extern "C" {

int kda_prefill(const void* q, const void* k, const void* v, const void* g, const void* beta,
                const float* conv_w, float* conv_ring, const float* state_in, float* state_out,
                const void* z, const float* norm_w, void* out, float* o_core, int B, int T,
                int H, int D, int K, float scale, float rms_eps, int dtype, int mode,
                void* workspace, size_t workspace_bytes, void* stream) {
    return entry(false, false, q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z,
                 norm_w, out, o_core, B, T, H, D, K, scale, rms_eps, dtype, mode, workspace,
                 workspace_bytes, stream);
}

int gdn_prefill(const void* q, const void* k, const void* v, const void* g, const void* beta,
                const float* conv_w, float* conv_ring, const float* state_in, float* state_out,
                const void* z, const float* norm_w, void* out, float* o_core, int B, int T,
                int H, int D, int K, float scale, float rms_eps, int dtype, int mode,
                void* workspace, size_t workspace_bytes, void* stream) {
    return entry(true, false, q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z,
                 norm_w, out, o_core, B, T, H, D, K, scale, rms_eps, dtype, mode, workspace,
                 workspace_bytes, stream);
}

int kda_prefill_noalloc(const void* q, const void* k, const void* v, const void* g, const void* beta,
                        const float* conv_w, float* conv_ring, const float* state_in, float* state_out,
                        const void* z, const float* norm_w, void* out, float* o_core, int B, int T,
                        int H, int D, int K, float scale, float rms_eps, int dtype, int mode,
                        void* stream) {
    return entry(false, false, q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z,
                 norm_w, out, o_core, B, T, H, D, K, scale, rms_eps, dtype, mode, nullptr, 0,
                 stream, kGiven, 0, nullptr, true);
}

int kda_decode(const void* q, const void* k, const void* v, const void* g, const void* beta,
               const float* conv_w, float* conv_ring, const float* state_in, float* state_out,
               const void* z, const float* norm_w, void* out, float* o_core, int B, int T,
               int H, int D, int K, float scale, float rms_eps, int dtype, void* stream) {
    return entry(false, true, q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z,
                 norm_w, out, o_core, B, T, H, D, K, scale, rms_eps, dtype,
                 KDA_MODE_SEQUENTIAL, nullptr, 0, stream);
}

int gdn_decode(const void* q, const void* k, const void* v, const void* g, const void* beta,
               const float* conv_w, float* conv_ring, const float* state_in, float* state_out,
               const void* z, const float* norm_w, void* out, float* o_core, int B, int T,
               int H, int D, int K, float scale, float rms_eps, int dtype, void* stream) {
    return entry(true, true, q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z,
                 norm_w, out, o_core, B, T, H, D, K, scale, rms_eps, dtype,
                 KDA_MODE_SEQUENTIAL, nullptr, 0, stream);
}

#define KDA_GATED_PREFILL(NAME, GDN)                                                              \
    int NAME(const void* q, const void* k, const void* v, const void* gate_x, const void* beta_x,  \
             const float* gate_a, const float* gate_bias, float gate_lb, int gate_form,            \
             const float* conv_w, float* conv_ring, const float* state_in, float* state_out,       \
             const void* z, const float* norm_w, void* out, float* o_core, int B, int T, int H,    \
             int D, int K, float scale, float rms_eps, int dtype, int mode, void* workspace,       \
             size_t workspace_bytes, void* stream) {                                               \
        if (gate_form == 0) return KDA_ERR_DTYPE_MODE; /* 0: use the plain entry */               \
        return entry(GDN, false, q, k, v, gate_x, beta_x, conv_w, conv_ring, state_in, state_out,  \
                     z, norm_w, out, o_core, B, T, H, D, K, scale, rms_eps, dtype, mode,           \
                     workspace, workspace_bytes, stream,                                           \
                     GateArgs{gate_form, gate_a, gate_bias, gate_lb});                             \
    }
#define KDA_GATED_DECODE(NAME, GDN)                                                               \
    int NAME(const void* q, const void* k, const void* v, const void* gate_x, const void* beta_x,  \
             const float* gate_a, const float* gate_bias, float gate_lb, int gate_form,            \
             const float* conv_w, float* conv_ring, const float* state_in, float* state_out,       \
             const void* z, const float* norm_w, void* out, float* o_core, int B, int T, int H,    \
             int D, int K, float scale, float rms_eps, int dtype, void* stream) {                  \
        if (gate_form == 0) return KDA_ERR_DTYPE_MODE; /* 0: use the plain entry */               \
        return entry(GDN, true, q, k, v, gate_x, beta_x, conv_w, conv_ring, state_in, state_out,   \
                     z, norm_w, out, o_core, B, T, H, D, K, scale, rms_eps, dtype,                 \
                     KDA_MODE_SEQUENTIAL, nullptr, 0, stream,                                      \
                     GateArgs{gate_form, gate_a, gate_bias, gate_lb});                             \
    }
KDA_GATED_PREFILL(kda_prefill_gated, false)
KDA_GATED_PREFILL(gdn_prefill_gated, true)
KDA_GATED_DECODE(kda_decode_gated, false)
KDA_GATED_DECODE(gdn_decode_gated, true)
#undef KDA_GATED_PREFILL
#undef KDA_GATED_DECODE

int kda_rollback(const void* q, const void* k, const void* v, const void* g, const void* beta,
                 const float* conv_w, const float* ring_snap, const float* state_snap,
                 float* conv_ring, float* state_out, int B, int T_stash, int keep, int H, int D,
                 int K, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    return rollback(false, q, k, v, g, beta, conv_w, ring_snap, state_snap, conv_ring, state_out,
                    B, T_stash, keep, H, D, K, dtype, workspace, workspace_bytes, stream);
}

int gdn_rollback(const void* q, const void* k, const void* v, const void* g, const void* beta,
                 const float* conv_w, const float* ring_snap, const float* state_snap,
                 float* conv_ring, float* state_out, int B, int T_stash, int keep, int H, int D,
                 int K, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    return rollback(true, q, k, v, g, beta, conv_w, ring_snap, state_snap, conv_ring, state_out,
                    B, T_stash, keep, H, D, K, dtype, workspace, workspace_bytes, stream);
}

#define KDA_GATED_ROLLBACK(NAME, GDN)                                                             \
    int NAME(const void* q, const void* k, const void* v, const void* gate_x, const void* beta_x,  \
             const float* gate_a, const float* gate_bias, float gate_lb, int gate_form,            \
             const float* conv_w, const float* ring_snap, const float* state_snap,                 \
             float* conv_ring, float* state_out, int B, int T_stash, int keep, int H, int D,       \
             int K, int dtype, void* workspace, size_t workspace_bytes, void* stream) {            \
        if (gate_form == 0) return KDA_ERR_DTYPE_MODE; /* 0: use the plain entry */               \
        return rollback(GDN, q, k, v, gate_x, beta_x, conv_w, ring_snap, state_snap, conv_ring,    \
                        state_out, B, T_stash, keep, H, D, K, dtype, workspace, workspace_bytes,   \
                        stream, GateArgs{gate_form, gate_a, gate_bias, gate_lb});                  \
    }
KDA_GATED_ROLLBACK(kda_rollback_gated, false)
KDA_GATED_ROLLBACK(gdn_rollback_gated, true)
#undef KDA_GATED_ROLLBACK

int gdn_prefill_gqa(const void* q, const void* k, const void* v, const void* g, const void* beta,
                    const float* gate_a, const float* gate_bias, float gate_lb, int gate_form,
                    const float* conv_w, float* conv_ring, const float* state_in, float* state_out,
                    const void* z, const float* norm_w, void* out, float* o_core, int B, int T, int H,
                    int Hk, int D, int K, float scale, float rms_eps, int dtype, int mode,
                    void* workspace, size_t workspace_bytes, void* stream) {
    if (Hk < 1) return KDA_ERR_SHAPE;  // (0 is not a default here)
    return entry(true, false, q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z, norm_w,
                 out, o_core, B, T, H, D, K, scale, rms_eps, dtype, mode, workspace, workspace_bytes,
                 stream, GateArgs{gate_form, gate_a, gate_bias, gate_lb}, Hk);
}

int gdn_decode_gqa(const void* q, const void* k, const void* v, const void* g, const void* beta,
                   const float* gate_a, const float* gate_bias, float gate_lb, int gate_form,
                   const float* conv_w, float* conv_ring, const float* state_in, float* state_out,
                   const void* z, const float* norm_w, void* out, float* o_core, int B, int T, int H,
                   int Hk, int D, int K, float scale, float rms_eps, int dtype, void* stream) {
    if (Hk < 1) return KDA_ERR_SHAPE;  // (0 is not a default here)
    return entry(true, true, q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z, norm_w,
                 out, o_core, B, T, H, D, K, scale, rms_eps, dtype, KDA_MODE_SEQUENTIAL, nullptr, 0,
                 stream, GateArgs{gate_form, gate_a, gate_bias, gate_lb}, Hk);
}

int gdn_rollback_gqa(const void* q, const void* k, const void* v, const void* g, const void* beta,
                     const float* gate_a, const float* gate_bias, float gate_lb, int gate_form,
                     const float* conv_w, const float* ring_snap, const float* state_snap,
                     float* conv_ring, float* state_out, int B, int T_stash, int keep, int H, int Hk,
                     int D, int K, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    if (Hk < 1) return KDA_ERR_SHAPE;
    return rollback(true, q, k, v, g, beta, conv_w, ring_snap, state_snap, conv_ring, state_out, B,
                    T_stash, keep, H, D, K, dtype, workspace, workspace_bytes, stream,
                    GateArgs{gate_form, gate_a, gate_bias, gate_lb}, Hk);
}

int kda_prefill_varlen(const void* q, const void* k, const void* v, const void* g, const void* beta,
                       const float* gate_a, const float* gate_bias, float gate_lb, int gate_form,
                       const float* conv_w, float* conv_ring, const float* state_in, float* state_out,
                       const void* z, const float* norm_w, void* out, float* o_core, const int* cu_seqlens,
                       int N, int T_total, int H, int D, int K, float scale, float rms_eps, int dtype,
                       int mode, void* workspace, size_t workspace_bytes, void* stream) {
    if (!cu_seqlens) return KDA_ERR_NULL;
    return entry(false, false, q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z, norm_w, out,
                 o_core, N, T_total, H, D, K, scale, rms_eps, dtype, mode, workspace, workspace_bytes, stream,
                 GateArgs{gate_form, gate_a, gate_bias, gate_lb}, H, cu_seqlens);
}

int gdn_prefill_varlen(const void* q, const void* k, const void* v, const void* g, const void* beta,
                       const float* gate_a, const float* gate_bias, float gate_lb, int gate_form,
                       const float* conv_w, float* conv_ring, const float* state_in, float* state_out,
                       const void* z, const float* norm_w, void* out, float* o_core, const int* cu_seqlens,
                       int N, int T_total, int H, int Hk, int D, int K, float scale, float rms_eps,
                       int dtype, int mode, void* workspace, size_t workspace_bytes, void* stream) {
    if (!cu_seqlens) return KDA_ERR_NULL;
    if (Hk < 1) return KDA_ERR_SHAPE;
    return entry(true, false, q, k, v, g, beta, conv_w, conv_ring, state_in, state_out, z, norm_w, out,
                 o_core, N, T_total, H, D, K, scale, rms_eps, dtype, mode, workspace, workspace_bytes, stream,
                 GateArgs{gate_form, gate_a, gate_bias, gate_lb}, Hk, cu_seqlens);
}

size_t kda_prefill_varlen_workspace_bytes(int N, int T_total, int H, int D, int dtype, int mode) {
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return (size_t)-1;
    if (check_shape(1, T_total, H, D, 4) || check_shape(N, 1, H, D, 4)) return (size_t)-1;
    const int arm = pick_arm_varlen(D, dtype == KDA_DTYPE_BF16, mode);
    if (arm < 0) return (size_t)-1;
    return order_bytes(N) + workspace_for(N, T_total, H, H, D, false, arm, (size_t)T_total);
}

size_t gdn_prefill_varlen_workspace_bytes(int N, int T_total, int H, int Hk, int D, int dtype, int mode) {
    if (check_heads(H, Hk)) return (size_t)-1;
    return kda_prefill_varlen_workspace_bytes(N, T_total, H, D, dtype, mode);  // q / k not staged
}

size_t gdn_gqa_workspace_bytes(int B, int T, int H, int Hk, int D, int dtype, int mode) {
    if (Hk < 1) return (size_t)-1;
    return ws_query(true, B, T, H, D, dtype, mode, Hk);
}

size_t kda_rollback_workspace_bytes(int B, int keep, int H, int D, int dtype) {
    return ws_query(false, B, keep, H, D, dtype, KDA_MODE_SEQUENTIAL);
}
size_t gdn_rollback_workspace_bytes(int B, int keep, int H, int D, int dtype) {
    return ws_query(true, B, keep, H, D, dtype, KDA_MODE_SEQUENTIAL);
}

size_t kda_prefill_workspace_bytes(int B, int T, int H, int D, int dtype, int mode) {
    return ws_query(false, B, T, H, D, dtype, mode);
}
size_t gdn_prefill_workspace_bytes(int B, int T, int H, int D, int dtype, int mode) {
    return ws_query(true, B, T, H, D, dtype, mode);
}
int kda_prefill_arm(int B, int T, int H, int D, int dtype, int mode) {
    return arm_query(B, T, H, D, dtype, mode);
}
int gdn_prefill_arm(int B, int T, int H, int D, int dtype, int mode) {
    return arm_query(B, T, H, D, dtype, mode);
}

const char* kda_status_string(int rc) {
    switch (rc) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL: return "a required pointer is NULL";
        case KDA_ERR_HEAD_DIM: return "unsupported head dim: D must be 16 or 128";
        case KDA_ERR_CONV_KERNEL: return "conv kernel size K must be in 2..8";
        case KDA_ERR_SHAPE: return "B, T and H must be >= 1 and sizes must fit the launch limits";
        case KDA_ERR_DECODE_T: return "decode entry points take exactly one token (T == 1)";
        case KDA_ERR_WORKSPACE: return "workspace missing or smaller than the query returned";
        case KDA_ERR_ALIGN: return "every pointer must be 16-byte aligned";
        case KDA_ERR_DTYPE_MODE: return "unknown dtype or mode, or mode not valid for this shape";
        case KDA_ERR_SCRATCH:
            return "the call needs more workspace than the static scratch of kda_prefill_noalloc "
                   "(KDA_NOALLOC_SCRATCH_BYTES); use kda_prefill with a workspace";
        case KDA_ERR_ALIAS:
            return "buffers overlap (only state_in == state_out, or a rollback's snapshot and "
                   "live ring / state, may be the same buffer)";
        default: break;
    }
    if (rc >= KDA_ERR_RUNTIME_BASE && rc < 20000) return "HIP runtime error during launch";
    return "unknown status code";
}

}  // extern "C"
