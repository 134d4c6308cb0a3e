/*
 * fp64 CPU oracle for the KDA / GDN gated delta-rule mixer.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct
 * statement of what the mixer computes. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it. It shares no code, header, table or
 * helper with the HIP library, and the HIP library never calls it.
 *
 * Sources (docs.rs source pages):
 *   [kda.rs]     memra-engine 0.125.0, src/memra_engine/kda.rs: module notes
 *                (geometry, conv fusion, chunked twin), ConvArm, kda_core /
 *                kda_core_gated stages 2-6, and the launch wrappers
 *                kda_conv_silu / kda_conv_ring_roll / kda_scan / kda_gated_rmsnorm.
 *   [gdn_ops.rs] aprender-serve 0.70.2, src/cuda/executor/gdn_ops.rs: the
 *                wrappers gdn_causal_conv1d_silu_into, gdn_per_head_l2_norm_into,
 *                gdn_delta_rule_into, gdn_gated_rmsnorm_into.
 *
 * Layouts (all arrays fp64, row-major, batch outermost):
 *   activations q, k, v, z, o, out : [B][T][H*D], channel c = h*D + i
 *   g (KDA)                         : [B][T][H*D]   per-channel log gate
 *   g (GDN)                         : [B][T][H]     per-head log gate
 *   beta                            : [B][T][H]
 *   conv_w                          : [3*H*D][K]    planes q, k, v; tap K-1 = newest
 *   ring                            : [B][3*H*D][K-1], slot 0 = oldest raw input
 *   state                           : [B][H][D(value j)][D(key i)], i.e. S[i][j] is
 *                                     stored at state[b][h][j][i]
 *
 * Parity pins: every function here is pinned by tests that do not reuse its
 * code (a hand-derived three-token example, closed forms, invariants, a
 * transition-matrix restatement, and chunked == sequential by brute force).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#define IDX3(a, b, c, nb, nc) (((size_t)(a) * (nb) + (b)) * (nc) + (c))

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }
static double silu(double x) { return x * sigmoid(x); }

/*
 * Causal depthwise conv + SiLU for one plane, with the conv ring as the left pad,
 * and the rolled ring.
 *   [kda.rs] module notes "CONV FUSION" (fused [3*qkv, kernel] weight and fused
 *   ring, plane offset plane*qkv for both), kda_core_gated stage 2 (SiLU on every
 *   plane; the prefill conv reads the OLD ring for every token and the ring is
 *   rolled only afterwards), ConvArm (ascending tap order over the same window).
 *   [gdn_ops.rs] gdn_causal_conv1d_silu_into (window shifts left, the new sample
 *   is appended, weight channel-outer).
 * For channel c of the plane (fused row cf = plane*qkv + c):
 *   xt = [ring[b][cf][0..K-2], x[b][0..T-1][c]]            (length K-1+T)
 *   y[b][t][c] = SiLU( sum_{j=0}^{K-1} w[cf][j] * xt[t+j] )
 *   ring_out[b][cf][m] = xt[T+m],  m = 0..K-2               (last K-1 raw inputs)
 */
void orc_conv_silu_plane(int B, int T, int qkv, int K, int plane,
                         const double* x, const double* conv_w,
                         const double* ring_in, double* y, double* ring_out)
{
    const int pad = K - 1;
    const int rows = 3 * qkv;
    double* xt = (double*)malloc(sizeof(double) * (size_t)(pad + T));
    for (int b = 0; b < B; ++b) {
        for (int c = 0; c < qkv; ++c) {
            const int cf = plane * qkv + c;
            for (int m = 0; m < pad; ++m) xt[m] = ring_in[IDX3(b, cf, m, rows, pad)];
            for (int t = 0; t < T; ++t) xt[pad + t] = x[IDX3(b, t, c, T, qkv)];
            for (int t = 0; t < T; ++t) {
                double acc = 0.0;
                for (int j = 0; j < K; ++j) acc += conv_w[(size_t)cf * K + j] * xt[t + j];
                y[IDX3(b, t, c, T, qkv)] = silu(acc);
            }
            for (int m = 0; m < pad; ++m) ring_out[IDX3(b, cf, m, rows, pad)] = xt[T + m];
        }
    }
    free(xt);
}

/*
 * l2 normalisation of each length-D row: y = x / sqrt(sum x^2 + 1e-6).
 *   [kda.rs] KDA_L2_EPS (1e-6, inside the square root, independent of the rms
 *   eps) and kda_core_gated stage 3 (q and k only).
 *   [gdn_ops.rs] gdn_per_head_l2_norm_into (eps added to the SUM of squares).
 */
void orc_l2norm_rows(long rows, int D, const double* x, double* y)
{
    for (long r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int i = 0; i < D; ++i) ss += x[r * D + i] * x[r * D + i];
        const double inv = 1.0 / sqrt(ss + 1e-6);
        for (int i = 0; i < D; ++i) y[r * D + i] = x[r * D + i] * inv;
    }
}

/*
 * Sequential gated delta rule, the plain definition.
 *   [kda.rs] kda_core_gated stage 5 and the kda_scan wrapper (per-channel decay
 *   emitted as a raw log gate that the scan exponentiates; head_dim^-1/2 applied
 *   to the readout, passed here as `scale`; state in the transposed M[col][i]
 *   layout); module notes (per-channel decay on the key axis, which is the axis
 *   the chunked twin scales k and q by).
 *   [gdn_ops.rs] gdn_delta_rule_into (one scalar gate per head; state
 *   [v_heads][head_v_dim][head_k_dim], updated in place).
 * Per (b, h), with S[i][j] (i key, j value) and for t = 0..T-1:
 *   S[i][j] *= exp(g_t[i])            (GDN: exp(g_t[h]) for every i)
 *   u[j]     = v_t[j] - sum_i S[i][j] k_t[i]
 *   S[i][j] += beta_t * k_t[i] * u[j]
 *   o_t[j]   = scale * sum_i S[i][j] q_t[i]        (post-update state)
 */
void orc_scan(int B, int T, int H, int D, int gdn,
              const double* q, const double* k, const double* v,
              const double* g, const double* beta, double scale,
              const double* state_in, double* state_out, double* o)
{
    const int qkv = H * D;
    double* S = (double*)malloc(sizeof(double) * (size_t)D * D);
    double* u = (double*)malloc(sizeof(double) * (size_t)D);
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
            const double* sin = state_in + ((size_t)b * H + h) * D * D;
            for (int i = 0; i < D; ++i)
                for (int j = 0; j < D; ++j) S[i * D + j] = sin[(size_t)j * D + i];
            for (int t = 0; t < T; ++t) {
                const size_t row = IDX3(b, t, h * D, T, qkv);
                const double* qt = q + row;
                const double* kt = k + row;
                const double* vt = v + row;
                const double bt = beta[IDX3(b, t, h, T, H)];
                for (int i = 0; i < D; ++i) {
                    const double gi = gdn ? g[IDX3(b, t, h, T, H)] : g[row + i];
                    const double decay = exp(gi);
                    for (int j = 0; j < D; ++j) S[i * D + j] *= decay;
                }
                for (int j = 0; j < D; ++j) {
                    double sk = 0.0;
                    for (int i = 0; i < D; ++i) sk += S[i * D + j] * kt[i];
                    u[j] = vt[j] - sk;
                }
                for (int i = 0; i < D; ++i)
                    for (int j = 0; j < D; ++j) S[i * D + j] += bt * kt[i] * u[j];
                for (int j = 0; j < D; ++j) {
                    double sq = 0.0;
                    for (int i = 0; i < D; ++i) sq += S[i * D + j] * qt[i];
                    o[row + j] = scale * sq;
                }
            }
            double* sout = state_out + ((size_t)b * H + h) * D * D;
            for (int i = 0; i < D; ++i)
                for (int j = 0; j < D; ++j) sout[(size_t)j * D + i] = S[i * D + j];
        }
    }
    free(S);
    free(u);
}

/*
 * Chunked form of the same recurrence (used only to prove chunked == sequential).
 *   [kda.rs] module notes on the shelved chunked twin: a per-channel cumulative
 *   log gate Gcum[t][i], k scaled by exp(-Gcum) and q by exp(+Gcum), and the UT /
 *   WY intra-chunk solve; for GDN one scalar G per (token, head).
 * Per (b, h) and per chunk of n <= C rows with carried state S (rows r, s, j are
 * chunk-local token indices, i the key channel):
 *   G[r][i]   = sum_{s<=r} g_s[i]                          (inclusive cumulative gate)
 *   Kp = exp(G) * k,  Qp = exp(G) * q,  Kn = exp(-G) * k    (element-wise per row)
 *   L[s][j]   = Kp_s . Kn_j  for j < s      (strictly lower)
 *   P[s][j]   = Qp_s . Kn_j  for j <= s     (lower incl. diagonal)
 *   Tm        = (I + diag(beta) L)^{-1}                     (forward substitution)
 *   W = Tm diag(beta) Kp,   Ut = Tm diag(beta) V
 *   Ub = Ut - W S
 *   O  = scale * (Qp S + P Ub)
 *   S  = diag(exp(G[n-1])) S + Kd^T Ub,  Kd_s = exp(G[n-1] - G[s]) * k_s
 */
void orc_chunked_scan(int B, int T, int H, int D, int gdn, int C,
                      const double* q, const double* k, const double* v,
                      const double* g, const double* beta, double scale,
                      const double* state_in, double* state_out, double* o)
{
    const int qkv = H * D;
    const size_t CD = (size_t)C * D;
    double* S = (double*)malloc(sizeof(double) * (size_t)D * D);
    double* G = (double*)malloc(sizeof(double) * CD);
    double* Kp = (double*)malloc(sizeof(double) * CD);
    double* Qp = (double*)malloc(sizeof(double) * CD);
    double* Kn = (double*)malloc(sizeof(double) * CD);
    double* Kd = (double*)malloc(sizeof(double) * CD);
    double* L = (double*)malloc(sizeof(double) * (size_t)C * C);
    double* P = (double*)malloc(sizeof(double) * (size_t)C * C);
    double* Tm = (double*)malloc(sizeof(double) * (size_t)C * C);
    double* W = (double*)malloc(sizeof(double) * CD);
    double* Ut = (double*)malloc(sizeof(double) * CD);
    double* Ub = (double*)malloc(sizeof(double) * CD);
    double* bet = (double*)malloc(sizeof(double) * (size_t)C);
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
            const double* sin = state_in + ((size_t)b * H + h) * D * D;
            for (int i = 0; i < D; ++i)
                for (int j = 0; j < D; ++j) S[i * D + j] = sin[(size_t)j * D + i];
            for (int c0 = 0; c0 < T; c0 += C) {
                const int n = (T - c0 < C) ? (T - c0) : C;
                /* cumulative gate and the scaled k / q rows */
                for (int r = 0; r < n; ++r) {
                    const size_t row = IDX3(b, c0 + r, h * D, T, qkv);
                    bet[r] = beta[IDX3(b, c0 + r, h, T, H)];
                    for (int i = 0; i < D; ++i) {
                        const double gi = gdn ? g[IDX3(b, c0 + r, h, T, H)] : g[row + i];
                        G[r * D + i] = (r == 0 ? 0.0 : G[(r - 1) * D + i]) + gi;
                        Kp[r * D + i] = exp(G[r * D + i]) * k[row + i];
                        Qp[r * D + i] = exp(G[r * D + i]) * q[row + i];
                        Kn[r * D + i] = exp(-G[r * D + i]) * k[row + i];
                    }
                }
                for (int s = 0; s < n; ++s) {
                    const size_t row = IDX3(b, c0 + s, h * D, T, qkv);
                    for (int i = 0; i < D; ++i)
                        Kd[s * D + i] = exp(G[(n - 1) * D + i] - G[s * D + i]) * k[row + i];
                }
                /* intra-chunk L (strict lower) and P (lower incl. diagonal) */
                for (int s = 0; s < n; ++s) {
                    for (int j = 0; j < n; ++j) {
                        double l = 0.0, p = 0.0;
                        for (int i = 0; i < D; ++i) {
                            l += Kp[s * D + i] * Kn[j * D + i];
                            p += Qp[s * D + i] * Kn[j * D + i];
                        }
                        L[s * C + j] = (j < s) ? l : 0.0;
                        P[s * C + j] = (j <= s) ? p : 0.0;
                    }
                }
                /* Tm = (I + diag(beta) L)^{-1}: forward substitution, one column at a time */
                for (int col = 0; col < n; ++col) {
                    for (int s = 0; s < n; ++s) {
                        double acc = (s == col) ? 1.0 : 0.0;
                        for (int j = 0; j < s; ++j) acc -= bet[s] * L[s * C + j] * Tm[j * C + col];
                        Tm[s * C + col] = acc;
                    }
                }
                /* W = Tm diag(beta) Kp,  Ut = Tm diag(beta) V */
                for (int s = 0; s < n; ++s) {
                    for (int i = 0; i < D; ++i) {
                        double w = 0.0, ut = 0.0;
                        for (int j = 0; j < n; ++j) {
                            const size_t rowj = IDX3(b, c0 + j, h * D, T, qkv);
                            w += Tm[s * C + j] * bet[j] * Kp[j * D + i];
                            ut += Tm[s * C + j] * bet[j] * v[rowj + i];
                        }
                        W[s * D + i] = w;
                        Ut[s * D + i] = ut;
                    }
                }
                /* Ub = Ut - W S */
                for (int s = 0; s < n; ++s)
                    for (int jv = 0; jv < D; ++jv) {
                        double ws = 0.0;
                        for (int i = 0; i < D; ++i) ws += W[s * D + i] * S[i * D + jv];
                        Ub[s * D + jv] = Ut[s * D + jv] - ws;
                    }
                /* O = scale (Qp S + P Ub) */
                for (int s = 0; s < n; ++s) {
                    const size_t row = IDX3(b, c0 + s, h * D, T, qkv);
                    for (int jv = 0; jv < D; ++jv) {
                        double acc = 0.0;
                        for (int i = 0; i < D; ++i) acc += Qp[s * D + i] * S[i * D + jv];
                        for (int j = 0; j < n; ++j) acc += P[s * C + j] * Ub[j * D + jv];
                        o[row + jv] = scale * acc;
                    }
                }
                /* S = diag(exp(G[n-1])) S + Kd^T Ub */
                for (int i = 0; i < D; ++i) {
                    const double dec = exp(G[(n - 1) * D + i]);
                    for (int jv = 0; jv < D; ++jv) {
                        double acc = dec * S[i * D + jv];
                        for (int s = 0; s < n; ++s) acc += Kd[s * D + i] * Ub[s * D + jv];
                        S[i * D + jv] = acc;
                    }
                }
            }
            double* sout = state_out + ((size_t)b * H + h) * D * D;
            for (int i = 0; i < D; ++i)
                for (int j = 0; j < D; ++j) sout[(size_t)j * D + i] = S[i * D + j];
        }
    }
    free(S); free(G); free(Kp); free(Qp); free(Kn); free(Kd); free(L); free(P);
    free(Tm); free(W); free(Ut); free(Ub); free(bet);
}

/*
 * Gated RMSNorm over each length-D row:
 *   out[j] = o[j] / sqrt(mean_j o[j]^2 + eps) * w[j] * gate(z[j])
 * with gate = sigmoid for KDA and SiLU (z * sigmoid(z)) for GDN.
 *   [kda.rs] kda_core_gated stage 6 and the kda_gated_rmsnorm wrapper (fp32
 *   RMSNorm over head_dim with the layer rms eps, sigmoid gate; GDN gates with SiLU).
 *   [gdn_ops.rs] gdn_gated_rmsnorm_into (the input is normalised per head, the gate
 *   is not; weight [head_dim] shared across heads).
 */
void orc_gated_rmsnorm(long rows, int D, const double* o, const double* z,
                       const double* w, double eps, int gdn, double* out)
{
    for (long r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int j = 0; j < D; ++j) ss += o[r * D + j] * o[r * D + j];
        const double inv = 1.0 / sqrt(ss / D + eps);
        for (int j = 0; j < D; ++j) {
            const double zz = z[r * D + j];
            const double gate = gdn ? silu(zz) : sigmoid(zz);
            out[r * D + j] = o[r * D + j] * inv * w[j] * gate;
        }
    }
}

/*
 * The whole mixer hot path, stages 2-6 of [kda.rs] kda_core_gated without the
 * projections: conv + SiLU on q, k, v (ring rolled), l2 on q and k, the
 * sequential scan, and the gated RMSNorm. Argument order follows the library's
 * prefill entry point. o_core (pre-norm scan output) may be NULL.
 */
void orc_mixer(int gdn, int B, int T, int H, int D, int K,
               const double* q_raw, const double* k_raw, const double* v_raw,
               const double* g, const double* beta, const double* conv_w,
               const double* ring_in, double* ring_out,
               const double* state_in, double* state_out,
               const double* z, const double* norm_w,
               double* out, double* o_core, double scale, double rms_eps)
{
    const int qkv = H * D;
    const size_t n = (size_t)B * T * qkv;
    double* qc = (double*)malloc(sizeof(double) * n);
    double* kc = (double*)malloc(sizeof(double) * n);
    double* vc = (double*)malloc(sizeof(double) * n);
    double* o = (double*)malloc(sizeof(double) * n);
    orc_conv_silu_plane(B, T, qkv, K, 0, q_raw, conv_w, ring_in, qc, ring_out);
    orc_conv_silu_plane(B, T, qkv, K, 1, k_raw, conv_w, ring_in, kc, ring_out);
    orc_conv_silu_plane(B, T, qkv, K, 2, v_raw, conv_w, ring_in, vc, ring_out);
    orc_l2norm_rows((long)B * T * H, D, qc, qc);
    orc_l2norm_rows((long)B * T * H, D, kc, kc);
    orc_scan(B, T, H, D, gdn, qc, kc, vc, g, beta, scale, state_in, state_out, o);
    orc_gated_rmsnorm((long)B * T * H, D, o, z, norm_w, rms_eps, gdn, out);
    if (o_core) memcpy(o_core, o, sizeof(double) * n);
    free(qc); free(kc); free(vc); free(o);
}
