/*
 * kda.h - C ABI of the MI355X (gfx950) KDA / GDN gated delta-rule mixer library.
 *
 * What the library computes (the mixer hot path, without its projections):
 *   memra-engine 0.125.0 kda.rs, module notes and kda_core_gated stages 2-6:
 *     2. per-plane causal depthwise conv (kernel K) + SiLU over q, k, v, reading
 *        the conv ring as the left pad, then the ring rolled to the last K-1 raw
 *        inputs (ConvArm; "CONV FUSION" notes);
 *     3. l2 normalisation of q and k over head_dim, eps 1e-6 inside the sqrt
 *        (KDA_L2_EPS);
 *     5. the gated delta rule per head: S <- diag(exp g_t) S (key axis),
 *        u = v_t - S^T k_t, S <- S + beta_t k_t u^T, o_t = scale * S^T q_t;
 *     6. gated RMSNorm over head_dim: o / sqrt(mean o^2 + rms_eps) * norm_w * gate(z),
 *        gate = sigmoid (KDA) or SiLU (GDN, aprender-serve gdn_ops.rs,
 *        gdn_gated_rmsnorm_into).
 *   The chunked prefill arm computes the same recurrence in chunks of 64 tokens
 *   (kda.rs module notes on the chunked twin: cumulative log gate per channel,
 *   UT/WY intra-chunk solve).
 *   Status codes follow memra-engine 0.124.0 mla_ffi.rs, module header:
 *   0 ok, 10000 + runtime error, 40000 + contract violation; the stream is
 *   passed as a void pointer.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers, caller-owned, 16-byte aligned.
 *    The library never allocates, frees or synchronises; it enqueues kernels on
 *    `stream` (a hipStream_t, NULL = the legacy default stream) and returns.
 *  - dtype (KDA_DTYPE_*) applies to q, k, v, g, beta, z and out. conv_w,
 *    conv_ring, state_in/state_out, norm_w and o_core are always fp32.
 *  - Shapes (row-major, batch outermost, channel c = h*D + i, token-major):
 *      q, k, v  [B][T][H*D]  raw (pre-conv) activations
 *      g        [B][T][H*D]  per-channel log gate (KDA)   | [B][T][H] (GDN)
 *               precondition g <= 0; the chunked arm also needs g >= -5
 *      beta     [B][T][H]    in [0, 1]
 *      conv_w   [3*H*D][K]   planes q, k, v; tap K-1 multiplies the newest input
 *      conv_ring[B][3*H*D][K-1]  in/out; slot 0 = oldest raw input
 *      state_in / state_out [B][H][D][D]: element [b][h][j][i] is S[i][j]
 *               (value column j major, key i fastest); may be the SAME pointer
 *               (updated in place), otherwise must not overlap
 *      z        [B][T][H*D]  output gate
 *      norm_w   [D]          shared by all heads
 *      out      [B][T][H*D]  gated, normalised output (dtype)
 *      o_core   [B][T][H*D]  fp32 scan output before the norm; may be NULL
 *    (The grouped-head entry points give q, k and the conv planes Hk heads, and the
 *    packed-batch entry points pack the rows of N sequences; see their sections.)
 *  - D must be 16 or 128, 2 <= K <= 8, B, T, H >= 1.
 *  - Contract violations are detected on the host BEFORE any launch: nothing is
 *    written on the device when a 4xxxx code is returned.
 *  - On 10000 + hipError_t the contents of every output are undefined.
 *  - The library keeps no state between calls. Calls on different streams with
 *    disjoint buffers may run concurrently.
 */
#ifndef KDA_MI355X_H
#define KDA_MI355X_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif
/* The library is built with hidden visibility: only what this header declares is exported. */
#if defined(__GNUC__) || defined(__clang__)
#pragma GCC visibility push(default)
#endif

/* ---- status codes ---- */
#define KDA_OK 0
#define KDA_ERR_RUNTIME_BASE 10000 /* + hipError_t of the failing launch */
#define KDA_ERR_NULL 40001         /* a required pointer is NULL */
#define KDA_ERR_HEAD_DIM 40002     /* D not in {16, 128} */
#define KDA_ERR_CONV_KERNEL 40003  /* K outside 2..8 */
#define KDA_ERR_SHAPE 40004        /* B, T or H < 1, keep outside 1..T_stash, or sizes overflow */
#define KDA_ERR_DECODE_T 40005     /* a decode entry point called with T != 1 */
#define KDA_ERR_WORKSPACE 40006    /* workspace NULL or smaller than required */
#define KDA_ERR_ALIGN 40007        /* a pointer is not 16-byte aligned */
#define KDA_ERR_DTYPE_MODE 40008   /* unknown dtype or mode, or mode not valid here */
#define KDA_ERR_ALIAS 40009        /* two buffers overlap (other than the allowed in-place pairs) */
#define KDA_ERR_SCRATCH 40010      /* kda_prefill_noalloc: the call needs more than the static scratch */

/* ---- dtype and prefill mode ---- */
#define KDA_DTYPE_F32 0
#define KDA_DTYPE_BF16 1
/* AUTO: for bf16 activations at D = 128, the sequential arm up to 32 tokens (up to 16
 * with fewer than 1024 (b, h) pairs), the chunked arm beyond, the segmented arm when its
 * plan shortens the critical path (few pairs, long sequences); fp32 activations and
 * D = 16 always take the sequential arm. *_prefill_arm reports the choice for given
 * gates. Gated calls (KDA_GATE_*) whose gate_lb is below -5 (or NaN) run on the fused
 * sequential arm wherever AUTO would take the chunked or segmented arm: that arm needs
 * no workspace, so a workspace sized by *_prefill_workspace_bytes still suffices.
 *
 * The chunked and segmented modes take bf16 activations only (their contractions use
 * bf16 operands, which cannot meet the fp32 accuracy bar): with KDA_DTYPE_F32 they
 * return KDA_ERR_DTYPE_MODE. Their decay factorisation needs every log gate >= -5:
 * for given gates that is a precondition (gates below it need KDA_MODE_SEQUENTIAL:
 * the library cannot see device values), and gated calls with gate_lb < -5 are refused with KDA_ERR_DTYPE_MODE. */
#define KDA_MODE_AUTO 0       /* library picks sequential, chunked or segmented from the shape */
#define KDA_MODE_SEQUENTIAL 1 /* token-by-token scan (bit-identical to chained decodes) */
#define KDA_MODE_CHUNKED 2    /* chunked WY form (32-row chunks for convs of up to 4 taps, 64-row
                               * beyond), bf16 MFMA operands, fp32 state (D = 128, bf16) */
/* The chunked form with every sequence cut into segments that run in parallel (D = 128,
 * equal-length sequences; not for packed batches). A run of tokens maps its entry state
 * affinely, S_out = M S_in + B: the decay and the delta-rule update of stage 5 above act
 * on the key index by left multiplication. The segments' M and B are computed in
 * parallel, a scan forms each segment's entry state, and the segments run again from
 * it with readout. AUTO takes it for few (b, h) pairs and long sequences, with
 * segment lengths from a timed cost model; this mode forces it, with segments as
 * short as 64 rows. Same accuracy contract as
 * KDA_MODE_CHUNKED. */
#define KDA_MODE_SEGMENTED 3

/* Gate activation of the *_gated entry points (the plain entry points take g and
 * beta already activated). x is the gate pre-activation read from `g`, b the beta
 * pre-activation read from `beta`; c = h*D + i (KDA) or h (GDN) indexes gate_bias:
 *   KDA_GATE_SIGMOID:  g = gate_lb * sigmoid(exp(gate_a[h]) * (x + gate_bias[c]))
 *                      (memra-engine kda.rs, stage 4: gate_a = A_log, gate_lb = the
 *                      forget-gate lower bound, e.g. -5)
 *   KDA_GATE_SOFTPLUS: g = max(gate_lb, gate_a[h] * softplus(x + gate_bias[c]))
 *                      (aprender-serve gdn_ops.rs, the per-head gates: gate_a = a,
 *                      usually -exp(A_log); gate_lb = -INFINITY for no bound)
 *   and in both forms beta = sigmoid(b). */
#define KDA_GATE_GIVEN 0 /* (grouped-head entries) g and beta already activated */
#define KDA_GATE_SIGMOID 1
#define KDA_GATE_SOFTPLUS 2

/* Which kernel arm a prefill with these arguments runs (for reporting). */
#define KDA_ARM_SEQ_FUSED 1   /* one kernel per (b, h): conv, l2, scan, norm and ring fused */
#define KDA_ARM_SEQ_SPLIT 2   /* pre-kernel, column-split scan, norm kernel */
#define KDA_ARM_CHUNKED 3     /* chunked prefill */
#define KDA_ARM_SEGMENTED 4   /* chunked prefill, segments of each sequence in parallel */

/*
 * kda_prefill - run the mixer over T tokens of B sequences.
 *   Reads q, k, v, g, beta, z, conv_w, norm_w, conv_ring (old), state_in.
 *   Writes out, o_core (if not NULL), conv_ring (rolled), state_out.
 *   scale multiplies the readout (head_dim^-1/2 in the source model);
 *   rms_eps is the RMSNorm epsilon.
 *   mode: KDA_MODE_*. The sequential mode gives results bit-identical to T
 *   successive kda_decode calls. The chunked and segmented modes agree with it to
 *   bf16-operand accuracy (rel L-inf <= 2e-2) and require D == 128 and bf16
 *   activations (else KDA_ERR_DTYPE_MODE).
 *   workspace: device buffer of at least kda_prefill_workspace_bytes(...) bytes
 *   (may be NULL when that is 0). Its contents on entry are ignored.
 * Returns KDA_OK or a status code above.
 */
int kda_prefill(const void* q, const void* k, const void* v, const void* g,
                const void* beta, const float* conv_w, float* conv_ring,
                const float* state_in, float* state_out, const void* z,
                const float* norm_w, void* out, float* o_core,
                int B, int T, int H, int D, int K, float scale, float rms_eps,
                int dtype, int mode, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * kda_decode - one new token per sequence (T must be 1, else KDA_ERR_DECODE_T).
 *   Same arguments and semantics as kda_prefill with T = 1 and the sequential
 *   arm; runs one fused kernel and needs no workspace. The ring is rolled and the
 *   state updated exactly as by kda_prefill(T = 1, KDA_MODE_SEQUENTIAL).
 */
int kda_decode(const void* q, const void* k, const void* v, const void* g,
               const void* beta, const float* conv_w, float* conv_ring,
               const float* state_in, float* state_out, const void* z,
               const float* norm_w, void* out, float* o_core,
               int B, int T, int H, int D, int K, float scale, float rms_eps,
               int dtype, void* stream);

/* GDN twins: g is [B][T][H] (one scalar log gate per token and head) and the
 * output gate is SiLU(z) = z * sigmoid(z) (aprender-serve gdn_ops.rs,
 * gdn_delta_rule_into and gdn_gated_rmsnorm_into). Everything else as above. */
int gdn_prefill(const void* q, const void* k, const void* v, const void* g,
                const void* beta, const float* conv_w, float* conv_ring,
                const float* state_in, float* state_out, const void* z,
                const float* norm_w, void* out, float* o_core,
                int B, int T, int H, int D, int K, float scale, float rms_eps,
                int dtype, int mode, void* workspace, size_t workspace_bytes,
                void* stream);
int gdn_decode(const void* q, const void* k, const void* v, const void* g,
               const void* beta, const float* conv_w, float* conv_ring,
               const float* state_in, float* state_out, const void* z,
               const float* norm_w, void* out, float* o_core,
               int B, int T, int H, int D, int K, float scale, float rms_eps,
               int dtype, void* stream);

/*
 * kda_prefill_noalloc - kda_prefill for callers that cannot allocate device memory
 *   (code under HIP graph capture, tight serving loops, harnesses that forbid
 *   hipMalloc): the same arguments without the workspace, which comes from a static
 *   device buffer of KDA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 *   runs on until the process ends. The call allocates nothing (no hipMalloc, no
 *   allocating library routine) and otherwise behaves as kda_prefill with a workspace:
 *   same arms, kernels and results.
 *   A call whose arm needs more workspace than the buffer (kda_prefill_workspace_bytes
 *   > KDA_NOALLOC_SCRATCH_BYTES) returns KDA_ERR_SCRATCH before any launch.
 *   Every call on one GPU shares that GPU's buffer: calls that overlap in time on one
 *   GPU (different host threads or streams with no ordering between them) race, so
 *   order them on one stream. The buffer keeps the last call's contents; the arms
 *   never read workspace contents they did not write in the same call.
 *   The buffer is on the device of `stream` (the current device for NULL).
 */
#define KDA_NOALLOC_SCRATCH_BYTES (64u << 20)
int kda_prefill_noalloc(const void* q, const void* k, const void* v, const void* g,
                        const void* beta, const float* conv_w, float* conv_ring,
                        const float* state_in, float* state_out, const void* z,
                        const float* norm_w, void* out, float* o_core,
                        int B, int T, int H, int D, int K, float scale, float rms_eps,
                        int dtype, int mode, void* stream);

/* Workspace bytes a prefill with these arguments needs (0 if none). Returns
 * (size_t)-1 for arguments the prefill would reject. */
size_t kda_prefill_workspace_bytes(int B, int T, int H, int D, int dtype, int mode);
size_t gdn_prefill_workspace_bytes(int B, int T, int H, int D, int dtype, int mode);

/* The arm (KDA_ARM_*) a prefill with these arguments runs, or -1 if rejected. */
int kda_prefill_arm(int B, int T, int H, int D, int dtype, int mode);
int gdn_prefill_arm(int B, int T, int H, int D, int dtype, int mode);

/*
 * Fused gate activation: the four mixer entry points with the gate and beta
 * pre-activations in place of g and beta (same shapes and dtype), activated inside
 * the kernels as they are read (see KDA_GATE_*). gate_a is [H] fp32, gate_bias is
 * [H*D] (KDA) or [H] (GDN) fp32, both 16-byte aligned. gate_form must be
 * KDA_GATE_SIGMOID or KDA_GATE_SOFTPLUS (else KDA_ERR_DTYPE_MODE). Everything else is
 * as for the plain entry points. The chunked arm needs activated gates >= -5, which
 * gate_lb >= -5 guarantees in both forms: with gate_lb < -5 (or NaN) AUTO runs the
 * sequential arm and the explicit chunked / segmented modes return KDA_ERR_DTYPE_MODE.
 */
int kda_prefill_gated(const void* q, const void* k, const void* v, const void* gate_x,
                      const void* beta_x, const float* gate_a, const float* gate_bias,
                      float gate_lb, int gate_form, const float* conv_w, float* conv_ring,
                      const float* state_in, float* state_out, const void* z,
                      const float* norm_w, void* out, float* o_core,
                      int B, int T, int H, int D, int K, float scale, float rms_eps,
                      int dtype, int mode, void* workspace, size_t workspace_bytes,
                      void* stream);
int gdn_prefill_gated(const void* q, const void* k, const void* v, const void* gate_x,
                      const void* beta_x, const float* gate_a, const float* gate_bias,
                      float gate_lb, int gate_form, const float* conv_w, float* conv_ring,
                      const float* state_in, float* state_out, const void* z,
                      const float* norm_w, void* out, float* o_core,
                      int B, int T, int H, int D, int K, float scale, float rms_eps,
                      int dtype, int mode, void* workspace, size_t workspace_bytes,
                      void* stream);
int kda_decode_gated(const void* q, const void* k, const void* v, const void* gate_x,
                     const void* beta_x, const float* gate_a, const float* gate_bias,
                     float gate_lb, int gate_form, const float* conv_w, float* conv_ring,
                     const float* state_in, float* state_out, const void* z,
                     const float* norm_w, void* out, float* o_core,
                     int B, int T, int H, int D, int K, float scale, float rms_eps,
                     int dtype, void* stream);
int gdn_decode_gated(const void* q, const void* k, const void* v, const void* gate_x,
                     const void* beta_x, const float* gate_a, const float* gate_bias,
                     float gate_lb, int gate_form, const float* conv_w, float* conv_ring,
                     const float* state_in, float* state_out, const void* z,
                     const float* norm_w, void* out, float* o_core,
                     int B, int T, int H, int D, int K, float scale, float rms_eps,
                     int dtype, void* stream);

/*
 * Speculative verify and exact rollback (memra-engine kda.rs: the batched verify-rows
 * call and the rollback of a verify round, which restores the pre-round conv ring,
 * re-rolls it over the kept raw rows, and replays the scan from the caller's
 * pre-round state snapshot).
 *
 * A verify round is kda_prefill over T_stash = K+1 draft rows with
 * mode = KDA_MODE_SEQUENTIAL: every output row, the rolled ring and the final
 * state are bit-identical to T_stash chained kda_decode calls. The caller keeps
 * copies of the conv ring and the state taken BEFORE that call (ring_snap,
 * state_snap) and the call's raw inputs q, k, v, g, beta ([B][T_stash][...]).
 *
 * kda_rollback - rebuild the ring and the state as they were after the first
 * `keep` rows of every sequence (1 <= keep <= T_stash): conv_ring <- ring_snap,
 * then the sequential arm replays rows 0 .. keep-1 of the stored inputs from
 * state_snap with no readout. The result is bit-identical to `keep` chained
 * kda_decode calls from the snapshots (same kernels, same per-step arithmetic).
 *   Reads q, k, v, g, beta (T_stash rows per sequence, only the first keep used),
 *   conv_w, ring_snap, state_snap. Writes conv_ring, state_out.
 *   ring_snap may be the same pointer as conv_ring (already restored: no copy) and
 *   state_snap the same pointer as state_out (replayed in place); any other overlap
 *   between a written buffer and another buffer is KDA_ERR_ALIAS.
 *   keep outside 1 .. T_stash is KDA_ERR_SHAPE. workspace: at least
 *   kda_rollback_workspace_bytes(B, keep, H, D, dtype) bytes (0 for keep <= 16 or
 *   B*H >= 1024). Other arguments and codes as for kda_prefill.
 */
int kda_rollback(const void* q, const void* k, const void* v, const void* g,
                 const void* beta, const float* conv_w, const float* ring_snap,
                 const float* state_snap, float* conv_ring, float* state_out,
                 int B, int T_stash, int keep, int H, int D, int K, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream);
int gdn_rollback(const void* q, const void* k, const void* v, const void* g,
                 const void* beta, const float* conv_w, const float* ring_snap,
                 const float* state_snap, float* conv_ring, float* state_out,
                 int B, int T_stash, int keep, int H, int D, int K, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream);
size_t kda_rollback_workspace_bytes(int B, int keep, int H, int D, int dtype);
size_t gdn_rollback_workspace_bytes(int B, int keep, int H, int D, int dtype);

/* Rollback of a round verified with kda_prefill_gated / gdn_prefill_gated
 * (mode = KDA_MODE_SEQUENTIAL): the same replay from the stored gate and beta
 * pre-activations, activated as the gated entry points activate them, so the result
 * is bit-identical to `keep` chained kda_decode_gated calls. gate_x, beta_x, gate_a,
 * gate_bias, gate_lb, gate_form as for kda_prefill_gated (gate_form 0 is
 * KDA_ERR_DTYPE_MODE, null gate_a / gate_bias KDA_ERR_NULL); everything else as for
 * kda_rollback, with the same workspace query. */
int kda_rollback_gated(const void* q, const void* k, const void* v, const void* gate_x,
                       const void* beta_x, const float* gate_a, const float* gate_bias,
                       float gate_lb, int gate_form, const float* conv_w,
                       const float* ring_snap, const float* state_snap, float* conv_ring,
                       float* state_out, int B, int T_stash, int keep, int H, int D, int K,
                       int dtype, void* workspace, size_t workspace_bytes, void* stream);
int gdn_rollback_gated(const void* q, const void* k, const void* v, const void* gate_x,
                       const void* beta_x, const float* gate_a, const float* gate_bias,
                       float gate_lb, int gate_form, const float* conv_w,
                       const float* ring_snap, const float* state_snap, float* conv_ring,
                       float* state_out, int B, int T_stash, int keep, int H, int D, int K,
                       int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grouped query / key heads for GDN (aprender-serve gdn_ops.rs, the delta-rule
 * recurrence wrapper: q and k have num_k_heads heads, v, beta and the gate
 * num_v_heads, and value head h reads query / key head h % num_k_heads, the tiled
 * order).
 *
 * gdn_prefill_gqa / gdn_decode_gqa / gdn_rollback_gqa - gdn_prefill, gdn_decode and
 * gdn_rollback with Hk query / key heads and H value heads (Hk >= 1 divides H, else
 * KDA_ERR_SHAPE; Hk == H is the plain layout). Shapes:
 *   q, k       [B][T][Hk*D]          (dtype)
 *   v, z, out  [B][T][H*D]           (dtype); o_core [B][T][H*D] fp32
 *   g, beta    [B][T][H]             (per value head)
 *   conv_w     [(2*Hk + H)*D][K]     planes q (Hk*D rows), k (Hk*D), v (H*D)
 *   conv_ring  [B][(2*Hk + H)*D][K-1] same plane order
 *   state      [B][H][D][D]          (per value head)
 * The conv, the ring roll and the l2 norm of q / k run once per key head channel; the
 * scan, the gated norm and the state are per value head.
 * gate_form 0 (KDA_GATE_GIVEN): g and beta hold the log gate and beta, gate_a and
 * gate_bias are unused and may be NULL; KDA_GATE_SIGMOID / KDA_GATE_SOFTPLUS: g and
 * beta hold pre-activations, gate_a [H] and gate_bias [H], as for gdn_prefill_gated.
 * workspace: at least gdn_gqa_workspace_bytes(B, T, H, Hk, D, dtype, mode) bytes
 * (rollback: T = keep, mode = KDA_MODE_SEQUENTIAL). Everything else, including the
 * arm choice (by B*H value heads) and the status codes, as for the plain entries.
 */
int gdn_prefill_gqa(const void* q, const void* k, const void* v, const void* g,
                    const void* beta, const float* gate_a, const float* gate_bias,
                    float gate_lb, int gate_form, const float* conv_w, float* conv_ring,
                    const float* state_in, float* state_out, const void* z,
                    const float* norm_w, void* out, float* o_core, int B, int T, int H,
                    int Hk, int D, int K, float scale, float rms_eps, int dtype, int mode,
                    void* workspace, size_t workspace_bytes, void* stream);
int gdn_decode_gqa(const void* q, const void* k, const void* v, const void* g,
                   const void* beta, const float* gate_a, const float* gate_bias,
                   float gate_lb, int gate_form, const float* conv_w, float* conv_ring,
                   const float* state_in, float* state_out, const void* z,
                   const float* norm_w, void* out, float* o_core, int B, int T, int H, int Hk,
                   int D, int K, float scale, float rms_eps, int dtype, void* stream);
int gdn_rollback_gqa(const void* q, const void* k, const void* v, const void* g,
                     const void* beta, const float* gate_a, const float* gate_bias,
                     float gate_lb, int gate_form, const float* conv_w,
                     const float* ring_snap, const float* state_snap, float* conv_ring,
                     float* state_out, int B, int T_stash, int keep, int H, int Hk, int D,
                     int K, int dtype, void* workspace, size_t workspace_bytes, void* stream);
size_t gdn_gqa_workspace_bytes(int B, int T, int H, int Hk, int D, int dtype, int mode);

/*
 * Packed variable-length prefill: N sequences of different lengths in one call, their
 * rows packed back to back (no padding). Sequence n holds activation rows
 * cu_seqlens[n] .. cu_seqlens[n+1]-1; its conv ring and state are slot n.
 *   cu_seqlens [N+1] int32 DEVICE array, non-decreasing from 0 to T_total (4-byte
 *              aligned; a sequence may be empty: its ring and state pass through).
 *              The kernels clamp every offset into [0, T_total], so a malformed table
 *              cannot make them read or write outside the buffers, but the results
 *              are then meaningless; the table is not checked on the host.
 *   q, k       [T_total][Hk*D]; v, z, out [T_total][H*D]; o_core [T_total][H*D] fp32
 *   g          [T_total][H*D] (KDA) or [T_total][H] (GDN); beta [T_total][H]
 *   conv_ring  [N][(2*Hk + H)*D][K-1]; state_in / state_out [N][H][D][D]
 * Hk: query / key heads (gdn_prefill_varlen; Hk divides H, Hk = H is the plain
 * layout; kda_prefill_varlen has Hk = H). gate_form / gate_a / gate_bias / gate_lb
 * as for gdn_prefill_gqa (0: g and beta given).
 * Arms: KDA_MODE_SEQUENTIAL runs the fused sequential arm (one workgroup per
 * (sequence, head)); KDA_MODE_CHUNKED the chunked arm (D = 128); KDA_MODE_SEGMENTED is
 * rejected (KDA_ERR_DTYPE_MODE); KDA_MODE_AUTO the
 * chunked arm for bf16 activations at D = 128, else the fused arm. Each sequence is
 * processed exactly as a call on that sequence alone would process it on the same arm
 * (the fused arm bit for bit). workspace: at least *_prefill_varlen_workspace_bytes
 * bytes, never 0: it holds the longest-first order in which the sequences are
 * dispatched (ranked on the device), and, for the chunked arm with N*H < 256, the
 * pre-norm rows. null cu_seqlens is KDA_ERR_NULL; everything else as for kda_prefill.
 */
int kda_prefill_varlen(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, const float* gate_a, const float* gate_bias,
                       float gate_lb, int gate_form, const float* conv_w, float* conv_ring,
                       const float* state_in, float* state_out, const void* z,
                       const float* norm_w, void* out, float* o_core, const int* cu_seqlens,
                       int N, int T_total, int H, int D, int K, float scale, float rms_eps,
                       int dtype, int mode, void* workspace, size_t workspace_bytes,
                       void* stream);
int gdn_prefill_varlen(const void* q, const void* k, const void* v, const void* g,
                       const void* beta, const float* gate_a, const float* gate_bias,
                       float gate_lb, int gate_form, const float* conv_w, float* conv_ring,
                       const float* state_in, float* state_out, const void* z,
                       const float* norm_w, void* out, float* o_core, const int* cu_seqlens,
                       int N, int T_total, int H, int Hk, int D, int K, float scale,
                       float rms_eps, int dtype, int mode, void* workspace,
                       size_t workspace_bytes, void* stream);
size_t kda_prefill_varlen_workspace_bytes(int N, int T_total, int H, int D, int dtype, int mode);
size_t gdn_prefill_varlen_workspace_bytes(int N, int T_total, int H, int Hk, int D, int dtype,
                                          int mode);

/* Static description of a status code (never NULL). */
const char* kda_status_string(int rc);

#if defined(__GNUC__) || defined(__clang__)
#pragma GCC visibility pop
#endif
#ifdef __cplusplus
}
#endif

#endif /* KDA_MI355X_H */
