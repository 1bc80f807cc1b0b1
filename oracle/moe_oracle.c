/*
 * moe_oracle.c -- CPU oracle for the MoE block-verify layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The HIP product path never
 * links, loads or calls it, and it shares no source with the HIP path (its
 * decode tables, bf16 handling and selection are written here from the
 * definitions).
 *
 * Plain single-threaded C, double precision throughout.  It computes the
 * plain definition of one MoE layer per routed *slot*: no cross-row expert
 * deduplication, no blocking, no fusion.  The canonical dedup lists that the
 * GPU uses to stream each expert once are produced separately from their set
 * definition (orc_dedup) so the GPU's deduplicated gather is checked against a
 * computation that never deduplicates.
 *
 * Sources (web pages):
 *  [PR844]  "Validate submission ... Porting the retired serial track's
 *           compiled fusions onto the DFlash scored target", mlxfast-challenge
 *           PR #844: section 2 (byte budget, NVFP4 on switch_mlp / shared
 *           expert only), section 4 (router tail: f32 cast, sigmoid, bias add;
 *           argPartition + takeAlong; normalised expert combine), section 5
 *           (combine expression order: weighted sum, * 2.5, + shared,
 *           + residual), section 8 (gather without cross-row dedup).
 *  [README] "mlxfast -- Poolside Laguna XS 2.1 (DFlash)" README, section
 *           "Why this challenge exists" (256 routed + 1 shared expert, top-8,
 *           MoE intermediate 512, NVFP4 4-bit group-16, bf16 routers).
 *  E2M1 / E4M3FN bit layouts follow the OCP Microscaling (MX) v1.0 and OCP
 *  8-bit floating point specifications (NVFP4 = E2M1 values, one E4M3 scale
 *  per 16 elements, one fp32 tensor scale).
 *
 * Pins: every function here is checked against something other than itself
 * in tests/test_oracle_pins.py (library decode routines, brute force, closed
 * forms, page byte counts).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_SCORE_SOFTMAX 0
#define ORC_SCORE_SIGMOID_BIAS 1

/* ------------------------------------------------------------------------ */
/* O-1 decode                                                                */
/* ------------------------------------------------------------------------ */

/* E2M1: sign bit 3, exponent bits 2..1 with bias 1, mantissa bit 0.
 * Exponent field 0 is subnormal: value = mantissa * 0.5. */
double orc_e2m1(int code) {
    int sign = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -mag : mag;
}

/* E4M3FN: sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0.
 * No infinities; exponent 15 with mantissa 7 is NaN; exponent 0 is subnormal
 * (m/8 * 2^-6). */
double orc_e4m3fn(int byte) {
    int sign = (byte >> 7) & 1;
    int e = (byte >> 3) & 15;
    int m = byte & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* bf16 is the top half of an IEEE binary32. */
double orc_bf16(int bits) {
    uint32_t u = ((uint32_t)(bits & 0xFFFF)) << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* binary32 -> bf16, round to nearest, ties to even (NaN stays quiet NaN). */
uint16_t orc_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
    {
        uint32_t lsb = (u >> 16) & 1u;
        u += 0x7FFFu + lsb;
    }
    return (uint16_t)(u >> 16);
}

/* n doubles -> binary32 -> bf16 (round to nearest even each time): the bf16
 * output of a layer next to its fp32 result. */
void orc_bf16_round(const double* y, int n, uint16_t* out) {
    int i;
    for (i = 0; i < n; ++i) out[i] = orc_f32_to_bf16((float)y[i]);
}

static double g_e2m1[16];
static double g_e4m3[256];
static int g_tables_ready = 0;

static void tables(void) {
    int i;
    if (g_tables_ready) return;
    for (i = 0; i < 16; ++i) g_e2m1[i] = orc_e2m1(i);
    for (i = 0; i < 256; ++i) g_e4m3[i] = orc_e4m3fn(i);
    g_tables_ready = 1;
}

/* One dequantised weight of expert matrix e:
 *   W[n][c] = e2m1(code of column c in row n) * e4m3(scale of block c/16) * ts[e]
 * q: [E][rows][cols/2] (even column in the low nibble), s: [E][rows][cols/16]. */
double orc_nvfp4_weight(const uint8_t* q, const uint8_t* s, const float* ts,
                        int rows, int cols, int e, int n, int c) {
    size_t qrow = (size_t)e * rows * (cols / 2) + (size_t)n * (cols / 2);
    size_t srow = (size_t)e * rows * (cols / 16) + (size_t)n * (cols / 16);
    uint8_t byte = q[qrow + c / 2];
    int code = (c & 1) ? (byte >> 4) : (byte & 15);
    tables();
    return g_e2m1[code] * g_e4m3[s[srow + c / 16]] * (double)ts[e];
}

/* Whole matrix e dequantised into out[rows][cols] (double). */
void orc_nvfp4_dequant(const uint8_t* q, const uint8_t* s, const float* ts,
                       int rows, int cols, int e, double* out) {
    int n, c;
    for (n = 0; n < rows; ++n)
        for (c = 0; c < cols; ++c)
            out[(size_t)n * cols + c] = orc_nvfp4_weight(q, s, ts, rows, cols, e, n, c);
}

/* ------------------------------------------------------------------------ */
/* O-2 router GEMV: bf16 router weights (README "Why this challenge exists") */
/* ------------------------------------------------------------------------ */

void orc_router(const uint16_t* x, const uint16_t* wr, int K, int E, int H, float* logits) {
    int r, e, h;
    for (r = 0; r < K; ++r)
        for (e = 0; e < E; ++e) {
            double acc = 0.0;
            for (h = 0; h < H; ++h)
                acc += orc_bf16(x[(size_t)r * H + h]) * orc_bf16(wr[(size_t)e * H + h]);
            logits[(size_t)r * E + e] = (float)acc;
        }
}

/* ------------------------------------------------------------------------ */
/* O-3 key, O-4 top-k, O-5 weights                                           */
/* ------------------------------------------------------------------------ */

/* Selection key.  Softmax scoring selects on the logit itself (monotone in
 * the softmax probability).  Sigmoid scoring follows PR844 section 4's router
 * tail: f32 sigmoid, then the per-expert bias is added (selection only). */
float orc_key(float logit, const float* bias, int e, int score_fn) {
    if (score_fn == ORC_SCORE_SOFTMAX) return logit;
    {
        float sig = (float)(1.0 / (1.0 + exp(-(double)logit)));
        return sig + bias[e];
    }
}

typedef struct { float key; int idx; } orc_kv;

static int cmp_desc(const void* a, const void* b) {
    const orc_kv* x = (const orc_kv*)a;
    const orc_kv* y = (const orc_kv*)b;
    if (x->key > y->key) return -1;
    if (x->key < y->key) return 1;
    return (x->idx < y->idx) ? -1 : (x->idx > y->idx);
}

/* Per row: sort all E experts by (key descending, expert index ascending) and
 * keep the first k in that order (argPartition + takeAlong, PR844 section 4;
 * ties to the lower index).  Mixture weights over the selected set:
 *   softmax:  w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0)  (= full softmax
 *             renormalised over the selection);
 *   sigmoid:  w_j = sig(l_j), divided by their sum when norm_topk.
 * The routed scale is NOT folded in here; it multiplies the weighted sum
 * (PR844 section 5 expression order). */
void orc_topk(const float* logits, const float* bias, int K, int E, int k,
              int score_fn, int norm_topk, int32_t* ids, double* w) {
    int r, j, e;
    orc_kv* kv = (orc_kv*)malloc(sizeof(orc_kv) * (size_t)E);
    for (r = 0; r < K; ++r) {
        const float* l = logits + (size_t)r * E;
        double sum = 0.0;
        for (e = 0; e < E; ++e) {
            kv[e].key = orc_key(l[e], bias, e, score_fn);
            kv[e].idx = e;
        }
        qsort(kv, (size_t)E, sizeof(orc_kv), cmp_desc);
        for (j = 0; j < k; ++j) ids[(size_t)r * k + j] = kv[j].idx;
        if (score_fn == ORC_SCORE_SOFTMAX) {
            double lmax = -INFINITY;
            for (j = 0; j < k; ++j) {
                double v = (double)l[ids[(size_t)r * k + j]];
                if (v > lmax) lmax = v;
            }
            for (j = 0; j < k; ++j) {
                double v = exp((double)l[ids[(size_t)r * k + j]] - lmax);
                w[(size_t)r * k + j] = v;
                sum += v;
            }
            for (j = 0; j < k; ++j) w[(size_t)r * k + j] /= sum;
        } else {
            for (j = 0; j < k; ++j) {
                double v = 1.0 / (1.0 + exp(-(double)l[ids[(size_t)r * k + j]]));
                w[(size_t)r * k + j] = v;
                sum += v;
            }
            if (norm_topk)
                for (j = 0; j < k; ++j) w[(size_t)r * k + j] /= sum;
        }
    }
    free(kv);
}

/* ------------------------------------------------------------------------ */
/* O-6 canonical dedup (not on the pages: PR844 section 8 notes the gather   */
/* reads a repeated expert once per slot; this is the set that removes it)   */
/* ------------------------------------------------------------------------ */

/* ids: n flat slots (slot = r*k + j).  Outputs:
 *   uniq[0..U)   distinct expert ids, ascending;
 *   off[0..U]    exclusive prefix sum of per-expert slot counts (off[U] = n);
 *   asg[off[u]+t] the t-th smallest flat slot whose id is uniq[u];
 *   inv[slot]    position of the slot inside asg.
 * Returns U. */
int orc_dedup(const int32_t* ids, int n, int n_experts, int32_t* uniq, int32_t* off,
              int32_t* asg, int32_t* inv) {
    int U = 0, e, s, pos = 0;
    int* count = (int*)calloc((size_t)n_experts, sizeof(int));
    for (s = 0; s < n; ++s) count[ids[s]]++;
    off[0] = 0;
    for (e = 0; e < n_experts; ++e) {
        if (!count[e]) continue;
        uniq[U] = e;
        for (s = 0; s < n; ++s)
            if (ids[s] == e) {
                asg[pos] = s;
                inv[s] = pos;
                pos++;
            }
        U++;
        off[U] = pos;
    }
    free(count);
    return U;
}

/* ------------------------------------------------------------------------ */
/* O-7 SwiGLU expert FFN (PR844 section 4: silu(gate) * up, then down)        */
/* ------------------------------------------------------------------------ */

static double silu(double g) { return g / (1.0 + exp(-g)); }

/* out[H] = W_down[e] * (silu(W_gate[e] x) .* (W_up[e] x)), all in double.
 * gate/up: [E][I][H] packed; down: [E][H][I] packed. */
void orc_expert_ffn(const uint16_t* xrow, int H, int I,
                    const uint8_t* gq, const uint8_t* gs, const float* gts,
                    const uint8_t* uq, const uint8_t* us, const float* uts,
                    const uint8_t* dq, const uint8_t* ds, const float* dts,
                    int e, double* out) {
    int i, c, n;
    double* hbuf = (double*)malloc(sizeof(double) * (size_t)I);
    double* xd = (double*)malloc(sizeof(double) * (size_t)H);
    for (c = 0; c < H; ++c) xd[c] = orc_bf16(xrow[c]);
    for (i = 0; i < I; ++i) {
        double g = 0.0, v = 0.0;
        for (c = 0; c < H; ++c) {
            g += xd[c] * orc_nvfp4_weight(gq, gs, gts, I, H, e, i, c);
            v += xd[c] * orc_nvfp4_weight(uq, us, uts, I, H, e, i, c);
        }
        hbuf[i] = silu(g) * v;
    }
    for (n = 0; n < H; ++n) {
        double acc = 0.0;
        for (i = 0; i < I; ++i) acc += hbuf[i] * orc_nvfp4_weight(dq, ds, dts, H, I, e, n, i);
        out[n] = acc;
    }
    free(hbuf);
    free(xd);
}

/* ------------------------------------------------------------------------ */
/* O-8 one MoE layer, per slot, no dedup                                     */
/* ------------------------------------------------------------------------ */

/* y[r] = rs * sum_{j<k} w[r][j] * FFN_{ids[r][j]}(x_r)  + FFN_shared(x_r)
 *        (+ residual[r])
 * in that order (PR844 section 5: weighted sum, * routed scale, + shared,
 * + residual).  The shared expert is ungated (weight 1).
 * Outputs: logits fp32 [K][E], ids [K][k], w [K][k] (without rs), y [K][H].
 * sh_* may be NULL (no shared expert); residual may be NULL. */
void orc_moe_layer(int K, int H, int E, int k, int I, int Is,
                   int score_fn, int norm_topk, double rs,
                   const uint16_t* x, const uint16_t* router_w, const float* bias,
                   const uint8_t* gq, const uint8_t* gs, const float* gts,
                   const uint8_t* uq, const uint8_t* us, const float* uts,
                   const uint8_t* dq, const uint8_t* ds, const float* dts,
                   const uint8_t* sgq, const uint8_t* sgs, const float* sgts,
                   const uint8_t* suq, const uint8_t* sus, const float* suts,
                   const uint8_t* sdq, const uint8_t* sds, const float* sdts,
                   const uint16_t* residual,
                   float* logits, int32_t* ids, double* w, double* y) {
    int r, j, n;
    double* o = (double*)malloc(sizeof(double) * (size_t)H);
    double* acc = (double*)malloc(sizeof(double) * (size_t)H);
    orc_router(x, router_w, K, E, H, logits);
    orc_topk(logits, bias, K, E, k, score_fn, norm_topk, ids, w);
    for (r = 0; r < K; ++r) {
        const uint16_t* xr = x + (size_t)r * H;
        double* yr = y + (size_t)r * H;
        for (n = 0; n < H; ++n) acc[n] = 0.0;
        for (j = 0; j < k; ++j) {
            int e = ids[(size_t)r * k + j];
            double wj = w[(size_t)r * k + j];
            orc_expert_ffn(xr, H, I, gq, gs, gts, uq, us, uts, dq, ds, dts, e, o);
            for (n = 0; n < H; ++n) acc[n] += wj * o[n];
        }
        for (n = 0; n < H; ++n) yr[n] = rs * acc[n];
        if (Is > 0 && sgq) {
            orc_expert_ffn(xr, H, Is, sgq, sgs, sgts, suq, sus, suts, sdq, sds, sdts, 0, o);
            for (n = 0; n < H; ++n) yr[n] += o[n];
        }
        if (residual)
            for (n = 0; n < H; ++n) yr[n] += orc_bf16(residual[(size_t)r * H + n]);
    }
    free(o);
    free(acc);
}

/* ------------------------------------------------------------------------ */
/* Dense first layer (README "Why this challenge exists": the target's layer */
/* 0 has a dense SwiGLU MLP of intermediate 8192 instead of the MoE block)   */
/* ------------------------------------------------------------------------ */

/* y[t] = W_down (silu(W_gate x_t) .* (W_up x_t)) (+ residual[t]), every
 * weight bf16: gate/up [I][H], down [H][I]; double throughout.  The
 * residual, when given (bf16 [T][H]), is added last, as in the MoE layer. */
void orc_dense_mlp(const uint16_t* x, int T, int H, int I, const uint16_t* wg, const uint16_t* wu,
                   const uint16_t* wd, const uint16_t* residual, double* y) {
    int t, i, c, n;
    double* xd = (double*)malloc(sizeof(double) * (size_t)H);
    double* hbuf = (double*)malloc(sizeof(double) * (size_t)I);
    for (t = 0; t < T; ++t) {
        for (c = 0; c < H; ++c) xd[c] = orc_bf16(x[(size_t)t * H + c]);
        for (i = 0; i < I; ++i) {
            double g = 0.0, v = 0.0;
            for (c = 0; c < H; ++c) {
                g += xd[c] * orc_bf16(wg[(size_t)i * H + c]);
                v += xd[c] * orc_bf16(wu[(size_t)i * H + c]);
            }
            hbuf[i] = silu(g) * v;
        }
        for (n = 0; n < H; ++n) {
            double acc = 0.0;
            for (i = 0; i < I; ++i) acc += hbuf[i] * orc_bf16(wd[(size_t)n * I + i]);
            if (residual) acc += orc_bf16(residual[(size_t)t * H + n]);
            y[(size_t)t * H + n] = acc;
        }
    }
    free(xd);
    free(hbuf);
}

/* ------------------------------------------------------------------------ */
/* O-9 stack glue: x_next = bf16(fp32(gamma * y / sqrt(mean(y^2) + eps)))    */
/* ------------------------------------------------------------------------ */

/* RMSNorm of each row of y (double), times the per-column weight gamma
 * (bf16 [H]; NULL = all ones), rounded once to binary32 and then to bf16.
 * The mean of squares runs over the row itself, before gamma: gamma scales
 * the normalised row, it does not enter the norm. */
void orc_rmsnorm_bf16(const double* y, int K, int H, double eps, const uint16_t* gamma, uint16_t* xout) {
    int r, n;
    for (r = 0; r < K; ++r) {
        const double* yr = y + (size_t)r * H;
        double ss = 0.0, inv;
        for (n = 0; n < H; ++n) ss += yr[n] * yr[n];
        inv = 1.0 / sqrt(ss / H + eps);
        for (n = 0; n < H; ++n) {
            double v = yr[n] * inv;
            if (gamma) v *= orc_bf16(gamma[n]);
            xout[(size_t)r * H + n] = orc_f32_to_bf16((float)v);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Verify-row lm_head and greedy acceptance (the step after the MoE stack)   */
/* ------------------------------------------------------------------------ */

/* lm_head over every verify row: logits[r][v] = sum_h x[r][h] * W[v][h],
 * bf16 inputs, double accumulation.  W: bf16 [V][H] (100,352 x 2048 on the
 * pages: 0.41 GB, PR #844 section 2).  Every row gets its logits (PR #844
 * section 5, trap 1: the verifier needs one greedy token per verify row). */
void orc_lm_head(const uint16_t* x, const uint16_t* w, int K, int V, int H, double* logits) {
    int r, v, h;
    double* xd = (double*)malloc(sizeof(double) * (size_t)K * H);
    for (r = 0; r < K; ++r)
        for (h = 0; h < H; ++h) xd[(size_t)r * H + h] = orc_bf16(x[(size_t)r * H + h]);
    for (v = 0; v < V; ++v) {
        const uint16_t* wv = w + (size_t)v * H;
        for (r = 0; r < K; ++r) {
            const double* xr = xd + (size_t)r * H;
            double acc = 0.0;
            for (h = 0; h < H; ++h) acc += xr[h] * orc_bf16(wv[h]);
            logits[(size_t)r * V + v] = acc;
        }
    }
    free(xd);
}

/* Greedy verification of one block of K rows.  Row r's greedy token is the
 * argmax of its logits (ties to the lower token id).  Row r's input token is
 * the draft token draft[r-1] for r >= 1 (row 0 holds the last token already
 * emitted), so draft[j-1] is checked against row j-1's prediction: it is
 * accepted when it equals that greedy token or when its logit ties the row's
 * maximum within tie_tol (the mlxfast README, "Correctness fixtures", accepts
 * a token on an exact match and on a tie of the top logit within a 1e-6
 * tolerance; tie_tol = 0 is plain greedy).  Per the README's description of
 * the DFlash track, a step keeps the accepted prefix; it then adds the
 * target's own greedy token at the first row that prefix does not cover.
 * Outputs: target[K] greedy tokens; emitted[0..n) = the accepted draft
 * tokens then that greedy token; *n_emitted = accepted + 1.  Returns the
 * number of accepted draft tokens. */
int orc_greedy_accept(const double* logits, int K, int V, const int32_t* draft, double tie_tol,
                      int32_t* target, int32_t* emitted, int32_t* n_emitted) {
    int r, v, a = 0;
    for (r = 0; r < K; ++r) {
        const double* l = logits + (size_t)r * V;
        int best = 0;
        for (v = 1; v < V; ++v)
            if (l[v] > l[best]) best = v;
        target[r] = best;
    }
    while (a < K - 1) {
        const double* l = logits + (size_t)a * V;
        int d = draft[a];
        if (d == target[a] || (d >= 0 && d < V && l[d] >= l[target[a]] - tie_tol)) {
            emitted[a] = d;
            ++a;
        } else {
            break;
        }
    }
    emitted[a] = target[a];
    *n_emitted = a + 1;
    return a;
}
