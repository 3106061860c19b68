/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for the forward pass of one
 * expert-specialised MoE layer (top-k softmax gate, padding-free token buffers,
 * dispatch, SwiGLU experts, weighted combine) and its backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load this
 * file: only the test suite, the package smoke check and the benchmark's CPU-baseline
 * leg use it.  It shares no code, header, table or helper with the HIP library; the
 * two are compared on identical host inputs.
 *
 * Sources (web pages, cited by title and section):
 *   [XMOE]  "X-MoE: 在HPC平台上实现新兴混合专家架构的可扩展训练" (xllm-io paper review
 *           of arXiv:2508.13337).  Section 三 (技术架构): 核心公式 / PFT复杂度分析,
 *           模型组件 table, 训练流程 steps 1-7.  Section 五: 模型配置 table.
 *   [FSMOE] "FSMoE: A Flexible and Scalable Training System for Sparse Mixture-of-Experts
 *           Models" (fmread report).  第三部分 item 1: Gating / Order / Dispatch /
 *           Combine / Expert modules.
 *   [FDMOE] "FlashDMoE：分布式 MoE 执行范式的变革" (yjmstr blog).  Section 1.1 (DMoE
 *           算子定义); section 5, 载荷高效的数据处理.
 *
 * Arithmetic: every accumulation is in IEEE double; values are rounded only where the
 * layer stores them (logits and routing weights as fp32; h, y and the layer output in
 * the layer's storage type, round-to-nearest-even).  bf16 values travel as uint16_t
 * bit patterns and are decoded exactly to double.
 *
 * Readings of points the pages leave open (each also listed in the design notes):
 *   - gate = softmax over all E logits (logit = x.Wg + bias), keep the k largest,
 *     renormalise the kept probabilities to sum 1;
 *   - selection compares the fp32 logits, larger first, equal logits -> lower expert id
 *     first; slot j of a token holds its j-th pick in that order;
 *   - the buffer order is a stable sort of the flattened (token, slot) list by expert;
 *   - SwiGLU expert: h = silu(x.W1^T) * (x.W3^T), y = h.W2^T, silu(a) = a / (1 + e^-a),
 *     W1, W3 stored [E][F][H] and W2 stored [E][H][F] (row = output feature);
 *   - no capacity and no token dropping; the combine applies the routing weights.
 *
 * Pins (tests marked "not gpu"): brute-force rank selection, exact-tie and exact-logit
 * inputs, closed-form weights, brute-force buffer positions and the buffer invariants,
 * dispatch+combine round trip, the dense capacity-padded (GShard-style) formulation,
 * the E=1/k=1 dense SwiGLU FFN, identical experts, pure-Python per-row loops, and the
 * bf16 rounding of a library conversion; for the backward, central finite differences
 * of the forward, an independent float64 autograd of the same mixture, the zero-sum of
 * softmax-routing logit gradients and linearity in dout.  Every function below is pinned
 * by at least one.
 */
#define _POSIX_C_SOURCE 200809L
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

#define OR_F32 0
#define OR_BF16 1

#define OR_OK 0
#define OR_EINVAL 1
#define OR_ERANGE 2
#define OR_ENOMEM 3

/* ---------------------------------------------------------------- storage types -- */

static double bf16_bits_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double straight to the nearest bf16 (8 significant bits, fp32 exponent
 * range, subnormals down to 2^-133), ties to even, without passing through fp32. */
static uint16_t double_to_bf16_bits(double v) {
    float f;
    uint32_t u;
    if (isnan(v)) return 0x7fc0;
    if (v == 0.0 || isinf(v)) {
        f = (float)v;
        memcpy(&u, &f, sizeof u);
        return (uint16_t)(u >> 16);
    }
    double a = fabs(v), q;
    int ex;
    frexp(a, &ex);               /* a = m * 2^ex, m in [0.5, 1) */
    int lsb_exp = ex - 8;        /* 8 significant bits */
    if (lsb_exp < -133) lsb_exp = -133;   /* subnormal quantum */
    q = ldexp(nearbyint(ldexp(a, -lsb_exp)), lsb_exp);   /* default mode: ties to even */
    if (q > 0x1.fep127) q = INFINITY;     /* largest finite bf16 is (2 - 2^-7) * 2^127 */
    f = (float)(v < 0 ? -q : q);          /* exact: q has <= 8 significant bits */
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static double load_elem(int dt, const void *p, size_t i) {
    if (dt == OR_F32) return (double)((const float *)p)[i];
    return bf16_bits_to_double(((const uint16_t *)p)[i]);
}

static void store_elem(int dt, void *p, size_t i, double v) {
    if (dt == OR_F32) ((float *)p)[i] = (float)v;      /* C conversion: nearest, ties even */
    else ((uint16_t *)p)[i] = double_to_bf16_bits(v);
}

static size_t elem_size(int dt) { return dt == OR_F32 ? 4 : 2; }

static int valid_dtype(int dt) { return dt == OR_F32 || dt == OR_BF16; }

/* Exported for the pins: bf16 rounding of n doubles. */
void oracle_round_bf16(const double *in, uint16_t *out, long n) {
    for (long i = 0; i < n; ++i) out[i] = double_to_bf16_bits(in[i]);
}

/* ------------------------------------------------------------------------ gate -- */
/*
 * Gating ([XMOE] 训练流程 step 2, gating computed directly in buffer form; [FSMOE]
 * Gating Function module; [FDMOE] 1.1, each token picks a few experts).
 *   logit[t][e] = fp32( sum_h x[t][h] * Wg[e][h] + bias[e] )       (double sum)
 *   picks       = the k experts first in the order (logit desc, expert id asc)
 *   routing 0 (softmax top-k, [FSMOE] 第六部分 routing functions, the X-MoE configs):
 *     weight[t][j] = p(pick j) / sum_{i<k} p(pick i),  p = softmax over all E logits
 *   routing 1 (sigmoid top-k, [FSMOE] 第六部分 lists Sigmoid routing; the pages give no
 *   formula, read here as the plainest form): each expert scores sigmoid(logit), the
 *   picks are the same (sigmoid is increasing), and their scores are renormalised:
 *     weight[t][j] = s(pick j) / sum_{i<k} s(pick i),  s = 1 / (1 + exp(-logit))
 * Outputs top_experts[T][k] (int32), top_weights[T][k] (fp32); optionally the fp32
 * logits [T][E] and the unrounded double logits [T][E].
 */
int oracle_gate_topk(int dt, int T, int H, int E, int k, int routing, const void *x, const void *wg,
                     const float *bias, int32_t *top_experts, float *top_weights,
                     float *logits_out, double *logits64_out) {
    if (!valid_dtype(dt) || T < 0 || H <= 0 || E <= 0 || k < 1 || k > E) return OR_EINVAL;
    if (routing != 0 && routing != 1) return OR_EINVAL;
    int err = OR_OK;
#pragma omp parallel for schedule(dynamic, 4)
    for (int t = 0; t < T; ++t) {
        float *l = (float *)malloc(sizeof(float) * (size_t)E);
        int *order = (int *)malloc(sizeof(int) * (size_t)E);
        double *p = (double *)malloc(sizeof(double) * (size_t)E);
        if (!l || !order || !p) {
            err = OR_ENOMEM;
            free(l); free(order); free(p);
            continue;
        }
        for (int e = 0; e < E; ++e) {
            double s = 0.0;
            for (int h = 0; h < H; ++h)
                s += load_elem(dt, x, (size_t)t * H + h) * load_elem(dt, wg, (size_t)e * H + h);
            if (bias) s += (double)bias[e];
            l[e] = (float)s;
            if (logits_out) logits_out[(size_t)t * E + e] = l[e];
            if (logits64_out) logits64_out[(size_t)t * E + e] = s;
        }
        /* Selection: insertion sort of expert ids under (logit desc, id asc). */
        for (int e = 0; e < E; ++e) {
            int j = e;
            while (j > 0 && (l[order[j - 1]] < l[e] || (l[order[j - 1]] == l[e] && order[j - 1] > e))) {
                order[j] = order[j - 1];
                --j;
            }
            order[j] = e;
        }
        if (routing == 0) {
            /* Softmax over all E, then renormalise over the k picks. */
            double m = (double)l[order[0]], z = 0.0;
            for (int e = 0; e < E; ++e) z += exp((double)l[e] - m);
            for (int e = 0; e < E; ++e) p[e] = exp((double)l[e] - m) / z;
        } else {
            /* Sigmoid score of every expert. */
            for (int e = 0; e < E; ++e) p[e] = 1.0 / (1.0 + exp(-(double)l[e]));
        }
        double zsel = 0.0;
        for (int j = 0; j < k; ++j) zsel += p[order[j]];
        for (int j = 0; j < k; ++j) {
            top_experts[(size_t)t * k + j] = order[j];
            top_weights[(size_t)t * k + j] = (float)(p[order[j]] / zsel);
        }
        free(l); free(order); free(p);
    }
    return err;
}

/* ------------------------------------------------------------ padding-free buffers -- */
/*
 * PFT construction ([XMOE] 训练流程 step 1: flatten top_experts and sort it to form
 * token_ids and expert_ids; 模型组件: token_ids / expert_ids / num_ids; PFT复杂度分析:
 * the buffer holds only the routed rows, O(B*H) with no E*C capacity).
 * Flat index i = t*k + j.  The sort is by expert and stable in i:
 *   counts[e]   = #{ i : top_experts[i] == e }              ("num_ids")
 *   offsets[e]  = sum_{e' < e} counts[e'],  offsets[E] = N = T*k
 *   position(i) = offsets[e] + #{ i' < i : top_experts[i'] == e },  e = top_experts[i]
 *   token_ids[position(i)] = i / k,  expert_ids[position(i)] = e,  dest_pos[i] = position(i)
 * Returns OR_ERANGE (and writes nothing past the counts) if an id lies outside [0, E).
 */
int oracle_pft_build(int T, int k, int E, const int32_t *top_experts, int32_t *counts,
                     int32_t *offsets, int32_t *token_ids, int32_t *expert_ids,
                     int32_t *dest_pos) {
    if (T < 0 || k < 1 || E < 1) return OR_EINVAL;
    long N = (long)T * k;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (long i = 0; i < N; ++i) {
        int e = top_experts[i];
        if (e < 0 || e >= E) return OR_ERANGE;
        counts[e] += 1;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *cursor = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    if (!cursor) return OR_ENOMEM;
    for (long i = 0; i < N; ++i) {          /* ascending i: this is what makes it stable */
        int e = top_experts[i];
        int32_t p = offsets[e] + cursor[e]++;
        token_ids[p] = (int32_t)(i / k);
        expert_ids[p] = e;
        dest_pos[i] = p;
    }
    free(cursor);
    return OR_OK;
}

/* ------------------------------------------------------------------- dispatch -- */
/*
 * Padding-free dispatch ([XMOE] 训练流程 step 3; [FDMOE] 5, only the routed tokens are
 * moved, no zero-filled rows): the row of token t goes to buffer row dest_pos[t][j] for
 * each of its k slots.  A bit copy; every one of the N buffer rows is written once.
 */
int oracle_dispatch(int dt, int T, int k, int H, const void *x, const int32_t *dest_pos,
                    void *xd) {
    if (!valid_dtype(dt) || T < 0 || k < 1 || H <= 0) return OR_EINVAL;
    size_t row = (size_t)H * elem_size(dt);
    long N = (long)T * k;
    for (long i = 0; i < N; ++i) {
        long p = dest_pos[i];
        if (p < 0 || p >= N) return OR_ERANGE;
        memcpy((char *)xd + (size_t)p * row, (const char *)x + (size_t)(i / k) * row, row);
    }
    return OR_OK;
}

/* ------------------------------------------------------------------- experts -- */
/*
 * Expert computation over the uneven per-expert segments ([XMOE] 训练流程 step 5: one
 * GEMM per expert over its own rows, no padding to a capacity).  Rows
 * p in [offsets[e], offsets[e+1]) belong to expert e:
 *   a[f] = sum_h xd[p][h] * W1[e][f][h],   g[f] = sum_h xd[p][h] * W3[e][f][h]
 *   h[p][f] = store( a[f] / (1 + exp(-a[f])) * g[f] )
 *   y[p][c] = store( sum_f h[p][f] * W2[e][c][f] )      (the stored h is what is used)
 * h may be NULL (a private row buffer is used then).
 */
int oracle_grouped_gemm_swiglu(int dt, int N, int E, int H, int F, const void *xd,
                               const int32_t *offsets, const void *w1, const void *w3,
                               const void *w2, void *h, void *y) {
    if (!valid_dtype(dt) || N < 0 || E < 1 || H <= 0 || F <= 0) return OR_EINVAL;
    if (offsets[0] != 0 || offsets[E] != N) return OR_EINVAL;
    for (int e = 0; e < E; ++e)
        if (offsets[e + 1] < offsets[e]) return OR_EINVAL;
    int err = OR_OK;
    for (int e = 0; e < E; ++e) {
        size_t wbase1 = (size_t)e * F * H;   /* W1[e], W3[e]: [F][H] */
        size_t wbase2 = (size_t)e * H * F;   /* W2[e]: [H][F] */
#pragma omp parallel for schedule(dynamic, 1)
        for (int p = offsets[e]; p < offsets[e + 1]; ++p) {
            char *hrow_own = NULL;
            void *hrow;
            size_t hoff;
            if (h) {
                hrow = h;
                hoff = (size_t)p * F;
            } else {
                hrow_own = (char *)malloc((size_t)F * elem_size(dt));
                if (!hrow_own) { err = OR_ENOMEM; continue; }
                hrow = hrow_own;
                hoff = 0;
            }
            for (int f = 0; f < F; ++f) {
                double a = 0.0, g = 0.0;
                for (int c = 0; c < H; ++c) {
                    double xv = load_elem(dt, xd, (size_t)p * H + c);
                    a += xv * load_elem(dt, w1, wbase1 + (size_t)f * H + c);
                    g += xv * load_elem(dt, w3, wbase1 + (size_t)f * H + c);
                }
                store_elem(dt, hrow, hoff + f, a / (1.0 + exp(-a)) * g);
            }
            for (int c = 0; c < H; ++c) {
                double s = 0.0;
                for (int f = 0; f < F; ++f)
                    s += load_elem(dt, hrow, hoff + f) * load_elem(dt, w2, wbase2 + (size_t)c * F + f);
                store_elem(dt, y, (size_t)p * H + c, s);
            }
            free(hrow_own);
        }
    }
    return err;
}

/* -------------------------------------------------------------------- combine -- */
/*
 * Padding-free combine ([XMOE] 训练流程 step 6; [FDMOE] 1.1, results are merged back
 * with the gate weights):
 *   out[t][c] = store( sum_{j=0}^{k-1} top_weights[t][j] * y[dest_pos[t][j]][c] )
 * summed over j in ascending order.
 */
int oracle_combine(int dt, int T, int k, int H, const void *y, const int32_t *dest_pos,
                   const float *top_weights, void *out) {
    if (!valid_dtype(dt) || T < 0 || k < 1 || H <= 0) return OR_EINVAL;
    long N = (long)T * k;
    for (long i = 0; i < N; ++i)
        if (dest_pos[i] < 0 || dest_pos[i] >= N) return OR_ERANGE;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int c = 0; c < H; ++c) {
            double s = 0.0;
            for (int j = 0; j < k; ++j) {
                size_t p = (size_t)dest_pos[(size_t)t * k + j];
                s += (double)top_weights[(size_t)t * k + j] * load_elem(dt, y, p * H + c);
            }
            store_elem(dt, out, (size_t)t * H + c, s);
        }
    }
    return OR_OK;
}

/* --------------------------------------------------------------- whole layer -- */
/*
 * The five steps in order ([XMOE] 训练流程 steps 1-3, 5, 6; [FDMOE] 1.1 with the
 * all-to-all exchanges absent on one device).  Intermediates are allocated here.
 * Per-stage wall times (seconds, monotonic clock) go to stage_seconds[5] when it is
 * not NULL: gate, buffers, dispatch, experts, combine.
 */
static double wall_seconds(void) {
    struct timespec ts;
    clock_gettime(CLOCK_MONOTONIC, &ts);
    return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

int oracle_layer_forward(int dt, int T, int H, int E, int F, int k, int routing, const void *x,
                         const void *wg, const float *bias, const void *w1, const void *w3,
                         const void *w2, void *out, double *stage_seconds) {
    if (!valid_dtype(dt) || T < 0 || H <= 0 || E < 1 || F <= 0 || k < 1 || k > E)
        return OR_EINVAL;
    if (routing != 0 && routing != 1) return OR_EINVAL;
    long N = (long)T * k;
    size_t es = elem_size(dt);
    int32_t *te = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N ? N : 1));
    float *tw = (float *)malloc(sizeof(float) * (size_t)(N ? N : 1));
    int32_t *counts = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    int32_t *offsets = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *tok = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N ? N : 1));
    int32_t *eid = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N ? N : 1));
    int32_t *dpos = (int32_t *)malloc(sizeof(int32_t) * (size_t)(N ? N : 1));
    void *xd = malloc((size_t)(N ? N : 1) * H * es);
    void *y = malloc((size_t)(N ? N : 1) * H * es);
    int rc = OR_ENOMEM;
    double t0 = 0, t1 = 0;
    if (!te || !tw || !counts || !offsets || !tok || !eid || !dpos || !xd || !y) goto done;
#define STAGE_BEGIN() do { t0 = wall_seconds(); } while (0)
#define STAGE_END(i) do { t1 = wall_seconds(); if (stage_seconds) stage_seconds[i] = t1 - t0; } while (0)
    STAGE_BEGIN();
    rc = oracle_gate_topk(dt, T, H, E, k, routing, x, wg, bias, te, tw, NULL, NULL);
    STAGE_END(0);
    if (rc) goto done;
    STAGE_BEGIN();
    rc = oracle_pft_build(T, k, E, te, counts, offsets, tok, eid, dpos);
    STAGE_END(1);
    if (rc) goto done;
    STAGE_BEGIN();
    rc = oracle_dispatch(dt, T, k, H, x, dpos, xd);
    STAGE_END(2);
    if (rc) goto done;
    STAGE_BEGIN();
    rc = oracle_grouped_gemm_swiglu(dt, (int)N, E, H, F, xd, offsets, w1, w3, w2, NULL, y);
    STAGE_END(3);
    if (rc) goto done;
    STAGE_BEGIN();
    rc = oracle_combine(dt, T, k, H, y, dpos, tw, out);
    STAGE_END(4);
#undef STAGE_BEGIN
#undef STAGE_END
done:
    free(te); free(tw); free(counts); free(offsets); free(tok); free(eid); free(dpos);
    free(xd); free(y);
    return rc;
}

/* ------------------------------------------------------------------- backward -- */
/*
 * Gradients of the layer above for a loss L with dL/dout = dout, the expert picks held
 * fixed (top-k selection is piecewise constant in the logits).  The pages name training
 * as the purpose of the layer ([XMOE] 训练流程 steps 4-7 follow the forward with the
 * backward and the weight update; [FDMOE] section 10 lists training as future work) but
 * give no backward formulas; these are the derivatives of the forward as defined above,
 * with the reading that a value rounded to storage (h, y, the fp32 routing weights) is
 * used as stored where the forward uses it, and differentiated as if unrounded.  All
 * gradient arithmetic is in double; gradients are returned as double arrays.
 */

/*
 * Combine backward: out[t] = sum_j w[t][j] * y[p] with p = dest_pos[t][j], so
 *   dy[p][c]   = w[t][j] * dout[t][c]
 *   dw[t][j]   = sum_c dout[t][c] * y[p][c]
 * dy [N][H] and dw [T][k] are written (double).
 */
int oracle_combine_backward(int dt, int T, int k, int H, const void *dout, const void *y,
                            const int32_t *dest_pos, const float *top_weights, double *dy,
                            double *dw) {
    if (!valid_dtype(dt) || T < 0 || k < 1 || H <= 0) return OR_EINVAL;
    long N = (long)T * k;
    for (long i = 0; i < N; ++i)
        if (dest_pos[i] < 0 || dest_pos[i] >= N) return OR_ERANGE;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int j = 0; j < k; ++j) {
            size_t i = (size_t)t * k + j, p = (size_t)dest_pos[i];
            double w = (double)top_weights[i], d = 0.0;
            for (int c = 0; c < H; ++c) {
                double g = load_elem(dt, dout, (size_t)t * H + c);
                dy[p * H + c] = w * g;
                d += g * load_elem(dt, y, p * H + c);
            }
            dw[i] = d;
        }
    }
    return OR_OK;
}

/*
 * Expert backward for rows p of expert e (segments as in the forward), with
 * a = xd.W1[e]^T, g = xd.W3[e]^T (unrounded), h the forward's stored h:
 *   dh[f]        = sum_c dy[p][c] * W2[e][c][f]
 *   da[f]        = dh[f] * g[f] * silu'(a[f]),  silu'(a) = s * (1 + a * (1 - s)),  s = 1/(1+e^-a)
 *   dg[f]        = dh[f] * silu(a[f])
 *   dxd[p][c]    = sum_f da[f] * W1[e][f][c] + dg[f] * W3[e][f][c]
 *   dW2[e][c][f] = sum_p dy[p][c] * h[p][f]
 *   dW1[e][f][c] = sum_p da[f] * xd[p][c],   dW3[e][f][c] = sum_p dg[f] * xd[p][c]
 * h may be NULL: it is then recomputed and rounded to storage as the forward does.
 * dxd [N][H], dw1 and dw3 [E][F][H], dw2 [E][H][F] are written (double).
 */
int oracle_expert_backward(int dt, int N, int E, int H, int F, const void *xd,
                           const int32_t *offsets, const void *w1, const void *w3,
                           const void *w2, const void *h, const double *dy, double *dxd,
                           double *dw1, double *dw3, double *dw2) {
    if (!valid_dtype(dt) || N < 0 || E < 1 || H <= 0 || F <= 0) return OR_EINVAL;
    if (offsets[0] != 0 || offsets[E] != N) return OR_EINVAL;
    for (int e = 0; e < E; ++e)
        if (offsets[e + 1] < offsets[e]) return OR_EINVAL;
    size_t es = elem_size(dt);
    memset(dw1, 0, sizeof(double) * (size_t)E * F * H);
    memset(dw3, 0, sizeof(double) * (size_t)E * F * H);
    memset(dw2, 0, sizeof(double) * (size_t)E * H * F);
    double *da = (double *)malloc(sizeof(double) * (size_t)(N ? N : 1) * F);
    double *dg = (double *)malloc(sizeof(double) * (size_t)(N ? N : 1) * F);
    char *hs = (char *)malloc((size_t)(N ? N : 1) * F * es);   /* stored h, [N][F] */
    if (!da || !dg || !hs) { free(da); free(dg); free(hs); return OR_ENOMEM; }
    for (int e = 0; e < E; ++e) {
        size_t wb1 = (size_t)e * F * H, wb2 = (size_t)e * H * F;
#pragma omp parallel for schedule(dynamic, 1)
        for (int p = offsets[e]; p < offsets[e + 1]; ++p) {
            for (int f = 0; f < F; ++f) {
                double a = 0.0, g = 0.0, dh = 0.0;
                for (int c = 0; c < H; ++c) {
                    double xv = load_elem(dt, xd, (size_t)p * H + c);
                    a += xv * load_elem(dt, w1, wb1 + (size_t)f * H + c);
                    g += xv * load_elem(dt, w3, wb1 + (size_t)f * H + c);
                    dh += dy[(size_t)p * H + c] * load_elem(dt, w2, wb2 + (size_t)c * F + f);
                }
                double sg = 1.0 / (1.0 + exp(-a));
                da[(size_t)p * F + f] = dh * g * sg * (1.0 + a * (1.0 - sg));
                dg[(size_t)p * F + f] = dh * a * sg;
                if (h) memcpy(hs + ((size_t)p * F + f) * es, (const char *)h + ((size_t)p * F + f) * es, es);
                else store_elem(dt, hs, (size_t)p * F + f, a * sg * g);
            }
            for (int c = 0; c < H; ++c) {
                double s = 0.0;
                for (int f = 0; f < F; ++f)
                    s += da[(size_t)p * F + f] * load_elem(dt, w1, wb1 + (size_t)f * H + c) +
                         dg[(size_t)p * F + f] * load_elem(dt, w3, wb1 + (size_t)f * H + c);
                dxd[(size_t)p * H + c] = s;
            }
        }
        /* weight gradients: sums over the expert's rows in ascending p */
#pragma omp parallel for schedule(static)
        for (int f = 0; f < F; ++f) {
            for (int p = offsets[e]; p < offsets[e + 1]; ++p) {
                double a_ = da[(size_t)p * F + f], g_ = dg[(size_t)p * F + f];
                double hv = load_elem(dt, hs, (size_t)p * F + f);
                for (int c = 0; c < H; ++c) {
                    double xv = load_elem(dt, xd, (size_t)p * H + c);
                    dw1[wb1 + (size_t)f * H + c] += a_ * xv;
                    dw3[wb1 + (size_t)f * H + c] += g_ * xv;
                    dw2[wb2 + (size_t)c * F + f] += dy[(size_t)p * H + c] * hv;
                }
            }
        }
    }
    free(da); free(dg); free(hs);
    return OR_OK;
}

/* Dispatch backward: xd[p] = x[t] for every slot, so dx[t][c] = sum_j dxd[dest_pos[t][j]][c]. */
int oracle_dispatch_backward(int T, int k, int H, const double *dxd, const int32_t *dest_pos,
                             double *dx) {
    if (T < 0 || k < 1 || H <= 0) return OR_EINVAL;
    long N = (long)T * k;
    for (long i = 0; i < N; ++i)
        if (dest_pos[i] < 0 || dest_pos[i] >= N) return OR_ERANGE;
    for (int t = 0; t < T; ++t)
        for (int c = 0; c < H; ++c) {
            double s = 0.0;
            for (int j = 0; j < k; ++j) s += dxd[(size_t)dest_pos[(size_t)t * k + j] * H + c];
            dx[(size_t)t * H + c] = s;
        }
    return OR_OK;
}

/*
 * Gate backward.  The picks are held fixed and the weights of token t depend only on its
 * picked logits l_j (the fp32 logits of the forward, differentiated as exact):
 *   routing 0: w_j = exp(l_j) / sum_i exp(l_i)  (the all-expert softmax normaliser cancels)
 *              dl_j = w_j * (dw_j - sum_i w_i dw_i)
 *   routing 1: w_j = s_j / S, s = sigmoid(l), S = sum_i s_i
 *              dl_j = (dw_j - sum_i w_i dw_i) / S * s_j * (1 - s_j)
 * with w in double before its fp32 rounding.  Unpicked logits get no gradient.  Then, as
 * logit = x.Wg^T + bias:
 *   dx[t][h] += sum_j dl_j Wg[e_j][h],  dWg[e][h] = sum_t dl_te x[t][h],  dbias[e] = sum_t dl_te
 * dx is accumulated into (the caller initialises it); dwg [E][H] and dbias [E] are written.
 * dl [T][k] (double) is written when not NULL.
 */
int oracle_gate_backward(int dt, int T, int H, int E, int k, int routing, const void *x,
                         const void *wg, const float *bias, const int32_t *top_experts,
                         const double *dw, double *dx, double *dwg, double *dbias, double *dl) {
    if (!valid_dtype(dt) || T < 0 || H <= 0 || E <= 0 || k < 1 || k > E) return OR_EINVAL;
    if (routing != 0 && routing != 1) return OR_EINVAL;
    for (long i = 0; i < (long)T * k; ++i)
        if (top_experts[i] < 0 || top_experts[i] >= E) return OR_ERANGE;
    memset(dwg, 0, sizeof(double) * (size_t)E * H);
    memset(dbias, 0, sizeof(double) * (size_t)E);
    double *dlt = (double *)malloc(sizeof(double) * (size_t)(T ? T : 1) * k);
    if (!dlt) return OR_ENOMEM;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        double l[64], w[64], z = 0.0, S = 0.0, m = -INFINITY;   /* k <= 64 */
        for (int j = 0; j < k; ++j) {
            int e = top_experts[(size_t)t * k + j];
            double s = 0.0;
            for (int h = 0; h < H; ++h)
                s += load_elem(dt, x, (size_t)t * H + h) * load_elem(dt, wg, (size_t)e * H + h);
            if (bias) s += (double)bias[e];
            l[j] = (double)(float)s;
            if (l[j] > m) m = l[j];
        }
        for (int j = 0; j < k; ++j) {
            w[j] = routing == 0 ? exp(l[j] - m) : 1.0 / (1.0 + exp(-l[j]));
            z += w[j];
        }
        S = z;
        double wdw = 0.0;
        for (int j = 0; j < k; ++j) {
            w[j] /= z;
            wdw += w[j] * dw[(size_t)t * k + j];
        }
        for (int j = 0; j < k; ++j) {
            double r = dw[(size_t)t * k + j] - wdw;
            if (routing == 0) {
                dlt[(size_t)t * k + j] = w[j] * r;
            } else {
                double sj = w[j] * S;              /* sigmoid(l_j) */
                dlt[(size_t)t * k + j] = r / S * sj * (1.0 - sj);
            }
        }
        for (int h = 0; h < H; ++h) {
            double s = 0.0;
            for (int j = 0; j < k; ++j)
                s += dlt[(size_t)t * k + j] * load_elem(dt, wg, (size_t)top_experts[(size_t)t * k + j] * H + h);
            dx[(size_t)t * H + h] += s;
        }
    }
    /* dWg and dbias: sums over tokens in ascending t */
#pragma omp parallel for schedule(static)
    for (int e = 0; e < E; ++e) {
        for (int t = 0; t < T; ++t)
            for (int j = 0; j < k; ++j) {
                if (top_experts[(size_t)t * k + j] != e) continue;
                double d = dlt[(size_t)t * k + j];
                dbias[e] += d;
                for (int h = 0; h < H; ++h) dwg[(size_t)e * H + h] += d * load_elem(dt, x, (size_t)t * H + h);
            }
    }
    if (dl) memcpy(dl, dlt, sizeof(double) * (size_t)T * k);
    free(dlt);
    return OR_OK;
}

/*
 * The whole backward: the forward's gate, buffers, dispatch and experts are run again
 * (h and y as the forward stores them), then combine, expert, dispatch and gate
 * backward in that order.  dx [T][H], dwg [E][H], dbias [E], dw1 and dw3 [E][F][H],
 * dw2 [E][H][F] are written (double); dtw [T][k] (the routing-weight gradient) too when
 * not NULL.
 */
int oracle_layer_backward(int dt, int T, int H, int E, int F, int k, int routing, const void *x,
                          const void *wg, const float *bias, const void *w1, const void *w3,
                          const void *w2, const void *dout, double *dx, double *dwg,
                          double *dbias, double *dw1, double *dw3, double *dw2, double *dtw) {
    if (!valid_dtype(dt) || T < 0 || H <= 0 || E < 1 || F <= 0 || k < 1 || k > E)
        return OR_EINVAL;
    if (routing != 0 && routing != 1) return OR_EINVAL;
    long N = (long)T * k;
    size_t es = elem_size(dt), n1 = (size_t)(N ? N : 1);
    int32_t *te = (int32_t *)malloc(sizeof(int32_t) * n1);
    float *tw = (float *)malloc(sizeof(float) * n1);
    int32_t *counts = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
    int32_t *offsets = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *tok = (int32_t *)malloc(sizeof(int32_t) * n1);
    int32_t *eid = (int32_t *)malloc(sizeof(int32_t) * n1);
    int32_t *dpos = (int32_t *)malloc(sizeof(int32_t) * n1);
    void *xd = malloc(n1 * H * es), *h = malloc(n1 * F * es), *y = malloc(n1 * H * es);
    double *dy = (double *)malloc(sizeof(double) * n1 * H);
    double *dxd = (double *)malloc(sizeof(double) * n1 * H);
    double *dwt = (double *)malloc(sizeof(double) * n1);
    int rc = OR_ENOMEM;
    if (!te || !tw || !counts || !offsets || !tok || !eid || !dpos || !xd || !h || !y || !dy ||
        !dxd || !dwt)
        goto done;
    rc = oracle_gate_topk(dt, T, H, E, k, routing, x, wg, bias, te, tw, NULL, NULL);
    if (rc) goto done;
    rc = oracle_pft_build(T, k, E, te, counts, offsets, tok, eid, dpos);
    if (rc) goto done;
    rc = oracle_dispatch(dt, T, k, H, x, dpos, xd);
    if (rc) goto done;
    rc = oracle_grouped_gemm_swiglu(dt, (int)N, E, H, F, xd, offsets, w1, w3, w2, h, y);
    if (rc) goto done;
    rc = oracle_combine_backward(dt, T, k, H, dout, y, dpos, tw, dy, dwt);
    if (rc) goto done;
    rc = oracle_expert_backward(dt, (int)N, E, H, F, xd, offsets, w1, w3, w2, h, dy, dxd, dw1,
                                dw3, dw2);
    if (rc) goto done;
    rc = oracle_dispatch_backward(T, k, H, dxd, dpos, dx);
    if (rc) goto done;
    rc = oracle_gate_backward(dt, T, H, E, k, routing, x, wg, bias, te, dwt, dx, dwg, dbias, NULL);
    if (rc) goto done;
    if (dtw) memcpy(dtw, dwt, sizeof(double) * (size_t)N);
done:
    free(te); free(tw); free(counts); free(offsets); free(tok); free(eid); free(dpos);
    free(xd); free(h); free(y); free(dy); free(dxd); free(dwt);
    return rc;
}

/* Threads the OpenMP runtime will use (1 when built without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
