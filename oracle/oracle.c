/*
 * oracle.c -- plain, slow CPU reference of the speculative-decoding drafter block.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path links, loads or calls
 * this file: only the tests, the smoke entry point and the CPU-baseline leg of
 * the benchmark do. It shares no code, header, table or constant generator with
 * the HIP library.
 *
 * Arithmetic: IEEE F64 throughout (inputs are F32 or BF16 and widen exactly).
 * BF16 values are decoded by moving their 16 bits into the high half of an F32
 * word, as the hf2q 0.1.1 page `spec_decode/dflash/tensors.rs` describes for
 * `decode_bf16_bytes_to_f32`. No fast-math, no FMA contraction (build with
 * -ffp-contract=off). OpenMP splits only independent outputs (features, rows,
 * heads); every sum runs in plain index order.
 *
 * Sources (hf2q 0.1.1 source pages on docs.rs):
 *   [MTP]   src/inference/models/qwen35/mtp.rs
 *   [TENS]  src/inference/spec_decode/dflash/tensors.rs
 *   [ORCH]  src/inference/spec_decode/dflash/qwen35_orchestrator.rs
 * Where the pages leave a step open, the reading taken is named at the step.
 *
 * Parity pins: every exported function here is pinned by the CPU tests against
 * closed forms, invariants, brute force and the bit facts the [TENS] page prints;
 * the composed block forward has no printed worked example on the pages and is
 * "parity unpinned" beyond the composition of its pinned parts.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_EINVAL -1
#define ORC_ERANGE -4
#define ORC_ENAN -7

/* ------------------------------------------------------------------------ */
/* BF16                                                                      */
/* ------------------------------------------------------------------------ */

/* [TENS] `decode_bf16_bytes_to_f32`: little-endian BF16 bytes -> F32 by
 * shifting the 16 bits into the top half of the word; an odd byte count is
 * rejected. Returns the element count, or ORC_EINVAL for odd lengths. */
long orc_decode_bf16_bytes(const uint8_t *bytes, long nbytes, float *out) {
    if (nbytes < 0 || (nbytes % 2) != 0) return ORC_EINVAL;
    long n = nbytes / 2;
    for (long i = 0; i < n; i++) {
        uint32_t bits = ((uint32_t)bytes[2 * i] | ((uint32_t)bytes[2 * i + 1] << 8)) << 16;
        float f;
        memcpy(&f, &bits, 4);
        out[i] = f;
    }
    return n;
}

static inline double bf(uint16_t b) {
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

/* F32 -> BF16 with round-to-nearest-even (ties to the even 16-bit pattern).
 * Used for storing K/V rows into a BF16 cache. Finite inputs only. */
uint16_t orc_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* ------------------------------------------------------------------------ */
/* Building blocks                                                           */
/* ------------------------------------------------------------------------ */

/* [MTP] `rms_norm_with_weight` (kernel params [eps, hidden_size]):
 * y_i = x_i / sqrt(mean_j x_j^2 + eps) * w_i. The weight multiplies as stored
 * (no 1+w offset): the page passes the weight buffer straight to the kernel. */
void orc_rmsnorm(const double *x, const float *w, int n, double eps, double *y) {
    double ss = 0.0;
    for (int i = 0; i < n; i++) ss += x[i] * x[i];
    double r = 1.0 / sqrt(ss / (double)n + eps);
    for (int i = 0; i < n; i++) y[i] = x[i] * r * (double)w[i];
}

/* [TENS] `DFlashLayerTensors`, DType policy: projection weights are row-major
 * BF16 [out, in] consumed against F32 activations: Y[m,o] = sum_k X[m,k] W[o,k]. */
void orc_linear(const double *X, int M, int K, const uint16_t *W, int N, double *Y) {
    #pragma omp parallel
    {
        double *wrow = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        #pragma omp for schedule(static)
        for (int o = 0; o < N; o++) {
            const uint16_t *wr = W + (size_t)o * K;
            for (int k = 0; k < K; k++) wrow[k] = bf(wr[k]);
            for (int m = 0; m < M; m++) {
                const double *xr = X + (size_t)m * K;
                double acc = 0.0;
                for (int k = 0; k < K; k++) acc += xr[k] * wrow[k];
                Y[(size_t)m * N + o] = acc;
            }
        }
        free(wrow);
    }
}

/* [MTP] `forward_full_attention`, the IMROPE step. For text tokens all four
 * IMROPE position ids are equal, so every rotary section sees the same position
 * and the rotation is plain rotate-half RoPE over the first `rotary_dim` lanes:
 * pair (j, j + d/2) for j < d/2 turns by pos * theta^(-2j/d); lanes >= d pass
 * through. Angles are formed in F64. */
void orc_rope(double *v, int head_dim, int rotary_dim, double pos, double theta) {
    int half = rotary_dim / 2;
    for (int j = 0; j < half; j++) {
        double inv = pow(theta, -2.0 * (double)j / (double)rotary_dim);
        double a = pos * inv;
        double c = cos(a), s = sin(a);
        double x0 = v[j], x1 = v[j + half];
        v[j] = x0 * c - x1 * s;
        v[j + half] = x0 * s + x1 * c;
    }
    (void)head_dim;
}

static inline double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }
static inline double silu(double z) { return z / (1.0 + exp(-z)); }

/* Softmax attention of one query over n keys (scale 1/sqrt(hd)), subtracting
 * the maximum before exponentiating. [MTP] `forward_full_attention` passes no
 * scale override to `apply_sdpa_with_kv_cache`, read as the default 1/sqrt(hd). */
void orc_sdpa_one(const double *q, const double *keys, const double *vals, int n, int hd,
                  double *o) {
    double *s = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double scale = 1.0 / sqrt((double)hd);
    double mx = -INFINITY;
    for (int j = 0; j < n; j++) {
        double acc = 0.0;
        for (int d = 0; d < hd; d++) acc += q[d] * keys[(size_t)j * hd + d];
        s[j] = acc * scale;
        if (s[j] > mx) mx = s[j];
    }
    double den = 0.0;
    for (int j = 0; j < n; j++) {
        s[j] = exp(s[j] - mx);
        den += s[j];
    }
    for (int d = 0; d < hd; d++) o[d] = 0.0;
    for (int j = 0; j < n; j++) {
        double p = s[j] / den;
        for (int d = 0; d < hd; d++) o[d] += p * vals[(size_t)j * hd + d];
    }
    free(s);
}

/* ------------------------------------------------------------------------ */
/* Block forward                                                             */
/* ------------------------------------------------------------------------ */

typedef struct {
    int32_t kind; /* 0 = DFlash drafter, 1 = MTP block */
    int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, rotary_dim;
    int32_t intermediate, n_target_hidden, vocab;
    int32_t ffn_moe, n_experts, top_k, expert_intermediate, shared_intermediate;
    int32_t has_gate;
    int32_t kv_bf16;
    int32_t block_bidir; /* 1: every block row attends to all M block rows */
    double eps, theta;
} orc_cfg;

typedef struct {
    const float *in_norm, *post_norm;
    const uint16_t *wq, *wk, *wv, *wgate, *wo;
    const float *q_norm, *k_norm;
    const uint16_t *ffn_gate, *ffn_up, *ffn_down;
    const uint16_t *router, *exp_gate, *exp_up, *exp_down;
    const uint16_t *sh_gate, *sh_up, *sh_down, *sh_gate_inp;
} orc_layer;

typedef struct {
    const uint16_t *fc;
    const float *hidden_norm;
    const float *enorm, *hnorm;
    const uint16_t *eh_embed, *eh_hidden;
    const orc_layer *layers;
    const float *final_norm;
    const uint16_t *embed;
} orc_weights;

typedef struct {
    void *k, *v; /* [L][n_kv][capacity][hd], F32 or BF16 bits */
    int64_t capacity;
    int64_t seq_len;
} orc_cache;

typedef struct {
    const int32_t *tokens; /* [M] or NULL */
    const float *x0;       /* [M,H] if tokens == NULL */
    const float *ctx;      /* DFlash: [R, n_t*H]; MTP: prev_hidden [M,H] */
    int32_t M, R;
    double *layer_hidden;  /* [L][M][H] or NULL: x after each layer */
    double *hidden_out;    /* [M][H] or NULL: pre-norm hidden */
    double *h_final;       /* [M][H] required */
    int32_t *moe_sel;      /* [L][M][top_k] or NULL */
    double *moe_gap;       /* [L][M] or NULL: router logit gap rank top_k vs top_k+1 */
    double *attn_out;      /* [L][M][q_total] or NULL: gated attention output */
} orc_io;

static void cache_store(const orc_cfg *c, const orc_cache *kv, int is_v, int layer, int head,
                        int64_t pos, const double *row) {
    size_t off = (((size_t)layer * c->n_kv_heads + head) * (size_t)kv->capacity + (size_t)pos) *
                 (size_t)c->head_dim;
    void *base = is_v ? kv->v : kv->k;
    for (int d = 0; d < c->head_dim; d++) {
        float f = (float)row[d]; /* kernel precision is F32: round there first */
        if (c->kv_bf16)
            ((uint16_t *)base)[off + d] = orc_f32_to_bf16(f);
        else
            ((float *)base)[off + d] = f;
    }
}

static double cache_load(const orc_cfg *c, const orc_cache *kv, int is_v, int layer, int head,
                         int64_t pos, int d) {
    size_t off = (((size_t)layer * c->n_kv_heads + head) * (size_t)kv->capacity + (size_t)pos) *
                     (size_t)c->head_dim + (size_t)d;
    const void *base = is_v ? kv->v : kv->k;
    return c->kv_bf16 ? bf(((const uint16_t *)base)[off]) : (double)((const float *)base)[off];
}

/* Per-head RMSNorm over head_dim slices: [MTP] `forward_full_attention`
 * (`apply_q_or_k_per_head_rms_norm`), weights [head_dim] in F32 ([TENS]). */
static void per_head_norm(double *v, int n_heads, int hd, const float *w, double eps) {
    double *tmp = (double *)malloc(sizeof(double) * (size_t)hd);
    for (int h = 0; h < n_heads; h++) {
        orc_rmsnorm(v + (size_t)h * hd, w, hd, eps, tmp);
        memcpy(v + (size_t)h * hd, tmp, sizeof(double) * (size_t)hd);
    }
    free(tmp);
}

/* SwiGLU: down( silu(gate x) * up(x) ). [MTP] `forward_ffn_residual` (dense
 * branch) and [TENS] `DFlashLayerTensors` (mlp_gate / mlp_up / mlp_down). */
static void swiglu(const double *x, int M, int H, const uint16_t *wg, const uint16_t *wu,
                   const uint16_t *wd, int I, double *y) {
    double *g = (double *)malloc(sizeof(double) * (size_t)M * I);
    double *u = (double *)malloc(sizeof(double) * (size_t)M * I);
    orc_linear(x, M, H, wg, I, g);
    orc_linear(x, M, H, wu, I, u);
    for (size_t i = 0; i < (size_t)M * I; i++) g[i] = silu(g[i]) * u[i];
    orc_linear(g, M, I, wd, H, y);
    free(g);
    free(u);
}

/* Router selection for one row: softmax over all experts, keep the top_k
 * largest (ties to the lower index), renormalise the kept probabilities to sum
 * to one. Writes sel[top_k] (descending probability), wsel[top_k] and returns
 * the logit gap between rank top_k and rank top_k+1 (INFINITY if top_k == E). */
double orc_moe_route(const double *logits, int E, int top_k, int32_t *sel, double *wsel) {
    double mx = -INFINITY;
    for (int e = 0; e < E; e++)
        if (logits[e] > mx) mx = logits[e];
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    char *taken = (char *)calloc((size_t)E, 1);
    double den = 0.0;
    for (int e = 0; e < E; e++) {
        p[e] = exp(logits[e] - mx);
        den += p[e];
    }
    for (int e = 0; e < E; e++) p[e] /= den;
    double kept = 0.0;
    for (int t = 0; t < top_k; t++) {
        int best = -1;
        for (int e = 0; e < E; e++)
            if (!taken[e] && (best < 0 || p[e] > p[best])) best = e;
        taken[best] = 1;
        sel[t] = best;
        wsel[t] = p[best];
        kept += p[best];
    }
    for (int t = 0; t < top_k; t++) wsel[t] /= kept;
    double gap = INFINITY;
    if (top_k < E) {
        double next = -INFINITY;
        for (int e = 0; e < E; e++)
            if (!taken[e] && logits[e] > next) next = logits[e];
        gap = logits[sel[top_k - 1]] - next;
    }
    free(p);
    free(taken);
    return gap;
}

/* MoE FFN with a shared expert ([MTP] `MtpFfnWeightsGpu::Moe`; the page's
 * quantized expert blocks are replaced by BF16 [out,in] experts):
 * y = sum_{e in top_k} w_e * SwiGLU_e(x) + sigmoid(x . w_sg) * SwiGLU_shared(x). */
static void moe_ffn(const orc_cfg *c, const orc_layer *lw, const double *x, int M, double *y,
                    int32_t *sel_out, double *gap_out) {
    int H = c->hidden, E = c->n_experts, K = c->top_k;
    int Ie = c->expert_intermediate, Is = c->shared_intermediate;
    double *logit = (double *)malloc(sizeof(double) * (size_t)M * E);
    orc_linear(x, M, H, lw->router, E, logit);
    double *ye = (double *)malloc(sizeof(double) * (size_t)H);
    double *ysh = (double *)malloc(sizeof(double) * (size_t)M * H);
    double *sg = (double *)malloc(sizeof(double) * (size_t)M);
    int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
    double *ws = (double *)malloc(sizeof(double) * (size_t)K);
    swiglu(x, M, H, lw->sh_gate, lw->sh_up, lw->sh_down, Is, ysh);
    orc_linear(x, M, H, lw->sh_gate_inp, 1, sg);
    for (int m = 0; m < M; m++) {
        double gap = orc_moe_route(logit + (size_t)m * E, E, K, sel, ws);
        if (sel_out)
            for (int t = 0; t < K; t++) sel_out[(size_t)m * K + t] = sel[t];
        if (gap_out) gap_out[m] = gap;
        double *yr = y + (size_t)m * H;
        for (int h = 0; h < H; h++) yr[h] = 0.0;
        for (int t = 0; t < K; t++) {
            size_t e = (size_t)sel[t];
            swiglu(x + (size_t)m * H, 1, H, lw->exp_gate + e * Ie * H, lw->exp_up + e * Ie * H,
                   lw->exp_down + e * H * Ie, Ie, ye);
            for (int h = 0; h < H; h++) yr[h] += ws[t] * ye[h];
        }
        double s = sigmoid(sg[m]);
        for (int h = 0; h < H; h++) yr[h] += s * ysh[(size_t)m * H + h];
    }
    free(logit);
    free(ye);
    free(ysh);
    free(sg);
    free(sel);
    free(ws);
}

/* One pass of the drafter block over M block rows (and, for DFlash, R new
 * context rows). Steps, in the pages' order:
 *
 *  input   DFlash: x = embed[tokens] (or the given x0); h_ctx = RMSNorm(T fc^T,
 *          hidden_norm) over the R new context rows ([TENS] `DFlashModelTensors`:
 *          fc and hidden_norm; [ORCH] per-round loop, steps 1-4, new rows only).
 *          MTP: x = RMSNorm(e, enorm, 1e-6) ehE^T + RMSNorm(h, hnorm, 1e-6) ehH^T
 *          ([MTP] `project_embedding_and_hidden`; eps fixed at 1e-6 there), e the
 *          given embed_t or, for a chained step, embed[token].
 *  layer   ([MTP] `forward_full_attention`, `forward_ffn_residual`)
 *          xh = RMSNorm(x, in_norm); q = xh Wq^T, k = xh Wk^T, v = xh Wv^T,
 *          g = xh Wg^T (if gated); per-head RMSNorm of q and k; RoPE at each
 *          row's position; K/V stored in the cache at those positions; SDPA over
 *          the cache; o *= sigmoid(g); x1 = x + o Wo^T; x = x1 + FFN(RMSNorm(x1,
 *          post_norm)).
 *          Readings where the pages are silent (DFlash forward math is not on the
 *          pages): the context rows h_ctx go through each layer's Wk/Wv, k_norm and
 *          RoPE with no input norm and sit at positions P0..P0+R-1; block row i
 *          sits at P0+R+i and attends causally to cache rows [0, P0+R+i].
 *          With block_bidir (the block-diffusion reading of the in-block mask)
 *          every block row attends to cache rows [0, P0+R+M): all M block rows.
 *  output  hidden_out = x; h_final = RMSNorm(x, final_norm) ([MTP]
 *          `forward_shared_head`; [TENS] final `norm`).
 *
 * On success seq_len advances by R + M (the block rows stay in the cache; a
 * DFlash drafter drops them again with a rollback of M). */
int orc_block_forward(const orc_cfg *c, const orc_weights *w, orc_cache *kv, const orc_io *io) {
    const int H = c->hidden, M = io->M, R = io->R, L = c->n_layers;
    const int nq = c->n_q_heads, nkv = c->n_kv_heads, hd = c->head_dim;
    const int qt = nq * hd, kt = nkv * hd;
    const int64_t P0 = kv->seq_len;
    if (M < 1 || R < 0 || !io->h_final) return ORC_EINVAL;
    if (c->kind == 1 && R != 0) return ORC_EINVAL;
    if (P0 + R + M > kv->capacity) return ORC_ERANGE;
    const double eps = c->eps;

    double *x = (double *)calloc((size_t)M * H, sizeof(double));
    double *hctx = NULL;
    if (c->kind == 0) {
        for (int m = 0; m < M; m++)
            for (int h = 0; h < H; h++)
                x[(size_t)m * H + h] = io->tokens ? bf(w->embed[(size_t)io->tokens[m] * H + h])
                                                  : (double)io->x0[(size_t)m * H + h];
        if (R > 0) {
            int Kin = c->n_target_hidden * H;
            double *T = (double *)malloc(sizeof(double) * (size_t)R * Kin);
            for (size_t i = 0; i < (size_t)R * Kin; i++) T[i] = (double)io->ctx[i];
            double *proj = (double *)malloc(sizeof(double) * (size_t)R * H);
            orc_linear(T, R, Kin, w->fc, H, proj);
            hctx = (double *)malloc(sizeof(double) * (size_t)R * H);
            for (int r = 0; r < R; r++)
                orc_rmsnorm(proj + (size_t)r * H, w->hidden_norm, H, eps, hctx + (size_t)r * H);
            free(T);
            free(proj);
        }
    } else {
        double *e = (double *)malloc(sizeof(double) * (size_t)M * H);
        double *hp = (double *)malloc(sizeof(double) * (size_t)M * H);
        double *en = (double *)malloc(sizeof(double) * (size_t)M * H);
        double *hn = (double *)malloc(sizeof(double) * (size_t)M * H);
        double *pe = (double *)malloc(sizeof(double) * (size_t)M * H);
        double *ph = (double *)malloc(sizeof(double) * (size_t)M * H);
        /* embed_t: given, or the embedding row of the token a chained step drafts
         * from (the target's shared embedding, as for DFlash block rows) */
        for (int m = 0; m < M; m++)
            for (int h = 0; h < H; h++) {
                const size_t i = (size_t)m * H + h;
                e[i] = io->tokens ? bf(w->embed[(size_t)io->tokens[m] * H + h]) : (double)io->x0[i];
                hp[i] = (double)io->ctx[i];
            }
        for (int m = 0; m < M; m++) {
            orc_rmsnorm(e + (size_t)m * H, w->enorm, H, 1e-6, en + (size_t)m * H);
            orc_rmsnorm(hp + (size_t)m * H, w->hnorm, H, 1e-6, hn + (size_t)m * H);
        }
        orc_linear(en, M, H, w->eh_embed, H, pe);
        orc_linear(hn, M, H, w->eh_hidden, H, ph);
        for (size_t i = 0; i < (size_t)M * H; i++) x[i] = pe[i] + ph[i];
        free(e); free(hp); free(en); free(hn); free(pe); free(ph);
    }

    double *xh = (double *)malloc(sizeof(double) * (size_t)M * H);
    double *q = (double *)malloc(sizeof(double) * (size_t)M * qt);
    double *kb = (double *)malloc(sizeof(double) * (size_t)M * kt);
    double *vb = (double *)malloc(sizeof(double) * (size_t)M * kt);
    double *g = c->has_gate ? (double *)malloc(sizeof(double) * (size_t)M * qt) : NULL;
    double *o = (double *)malloc(sizeof(double) * (size_t)M * qt);
    double *a = (double *)malloc(sizeof(double) * (size_t)M * H);
    double *x1 = (double *)malloc(sizeof(double) * (size_t)M * H);
    double *f = (double *)malloc(sizeof(double) * (size_t)M * H);
    double *kc = R > 0 ? (double *)malloc(sizeof(double) * (size_t)R * kt) : NULL;
    double *vc = R > 0 ? (double *)malloc(sizeof(double) * (size_t)R * kt) : NULL;
    int64_t nkeys_max = P0 + R + M;
    int rc = ORC_OK;

    for (int l = 0; l < L; l++) {
        const orc_layer *lw = &w->layers[l];
        for (int m = 0; m < M; m++)
            orc_rmsnorm(x + (size_t)m * H, lw->in_norm, H, eps, xh + (size_t)m * H);
        orc_linear(xh, M, H, lw->wq, qt, q);
        orc_linear(xh, M, H, lw->wk, kt, kb);
        orc_linear(xh, M, H, lw->wv, kt, vb);
        if (g) orc_linear(xh, M, H, lw->wgate, qt, g);
        for (int m = 0; m < M; m++) {
            double pos = (double)(P0 + R + m);
            per_head_norm(q + (size_t)m * qt, nq, hd, lw->q_norm, eps);
            per_head_norm(kb + (size_t)m * kt, nkv, hd, lw->k_norm, eps);
            for (int h = 0; h < nq; h++)
                orc_rope(q + (size_t)m * qt + (size_t)h * hd, hd, c->rotary_dim, pos, c->theta);
            for (int h = 0; h < nkv; h++)
                orc_rope(kb + (size_t)m * kt + (size_t)h * hd, hd, c->rotary_dim, pos, c->theta);
        }
        if (R > 0) {
            orc_linear(hctx, R, H, lw->wk, kt, kc);
            orc_linear(hctx, R, H, lw->wv, kt, vc);
            for (int r = 0; r < R; r++) {
                per_head_norm(kc + (size_t)r * kt, nkv, hd, lw->k_norm, eps);
                for (int h = 0; h < nkv; h++)
                    orc_rope(kc + (size_t)r * kt + (size_t)h * hd, hd, c->rotary_dim,
                             (double)(P0 + r), c->theta);
            }
            for (int r = 0; r < R; r++)
                for (int h = 0; h < nkv; h++) {
                    cache_store(c, kv, 0, l, h, P0 + r, kc + (size_t)r * kt + (size_t)h * hd);
                    cache_store(c, kv, 1, l, h, P0 + r, vc + (size_t)r * kt + (size_t)h * hd);
                }
        }
        for (int m = 0; m < M; m++)
            for (int h = 0; h < nkv; h++) {
                cache_store(c, kv, 0, l, h, P0 + R + m, kb + (size_t)m * kt + (size_t)h * hd);
                cache_store(c, kv, 1, l, h, P0 + R + m, vb + (size_t)m * kt + (size_t)h * hd);
            }
        /* SDPA per (row, q head); GQA maps q head h to kv head floor(h*nkv/nq). */
        #pragma omp parallel
        {
            double *keys = (double *)malloc(sizeof(double) * (size_t)nkeys_max * hd);
            double *vals = (double *)malloc(sizeof(double) * (size_t)nkeys_max * hd);
            #pragma omp for schedule(dynamic)
            for (int t = 0; t < M * nq; t++) {
                int m = t / nq, h = t % nq;
                int kvh = (int)(((int64_t)h * nkv) / nq);
                int64_t n = c->block_bidir ? P0 + R + M : P0 + R + m + 1;
                for (int64_t j = 0; j < n; j++)
                    for (int d = 0; d < hd; d++) {
                        keys[(size_t)j * hd + d] = cache_load(c, kv, 0, l, kvh, j, d);
                        vals[(size_t)j * hd + d] = cache_load(c, kv, 1, l, kvh, j, d);
                    }
                orc_sdpa_one(q + (size_t)m * qt + (size_t)h * hd, keys, vals, (int)n, hd,
                             o + (size_t)m * qt + (size_t)h * hd);
            }
            free(keys);
            free(vals);
        }
        if (g)
            for (size_t i = 0; i < (size_t)M * qt; i++) o[i] *= sigmoid(g[i]);
        if (io->attn_out) memcpy(io->attn_out + (size_t)l * M * qt, o, sizeof(double) * (size_t)M * qt);
        orc_linear(o, M, qt, lw->wo, H, a);
        for (size_t i = 0; i < (size_t)M * H; i++) x1[i] = x[i] + a[i];
        for (int m = 0; m < M; m++)
            orc_rmsnorm(x1 + (size_t)m * H, lw->post_norm, H, eps, xh + (size_t)m * H);
        if (c->ffn_moe)
            moe_ffn(c, lw, xh, M, f, io->moe_sel ? io->moe_sel + (size_t)l * M * c->top_k : NULL,
                    io->moe_gap ? io->moe_gap + (size_t)l * M : NULL);
        else
            swiglu(xh, M, H, lw->ffn_gate, lw->ffn_up, lw->ffn_down, c->intermediate, f);
        for (size_t i = 0; i < (size_t)M * H; i++) x[i] = x1[i] + f[i];
        if (io->layer_hidden) memcpy(io->layer_hidden + (size_t)l * M * H, x, sizeof(double) * (size_t)M * H);
    }
    if (io->hidden_out) memcpy(io->hidden_out, x, sizeof(double) * (size_t)M * H);
    for (int m = 0; m < M; m++)
        orc_rmsnorm(x + (size_t)m * H, w->final_norm, H, eps, io->h_final + (size_t)m * H);
    for (size_t i = 0; i < (size_t)M * H; i++)
        if (!isfinite(io->h_final[i])) rc = ORC_ENAN;
    if (rc == ORC_OK) kv->seq_len = P0 + R + M;

    free(x); free(hctx); free(xh); free(q); free(kb); free(vb); free(g); free(o);
    free(a); free(x1); free(f); free(kc); free(vc);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Head, accept walk, rollback                                               */
/* ------------------------------------------------------------------------ */

/* [MTP] `forward_shared_head` / [ORCH] per-position argmax over the normed
 * hidden: z = h W^T; argmax takes the lowest index among equal maxima; the
 * margin is z(1) - z(2), the gap to the best other entry. logits may be NULL. */
int orc_lm_head(const double *h, int M, int H, const uint16_t *W, int V, double *logits,
                int32_t *argmax, double *margin) {
    double *z = logits ? logits : (double *)malloc(sizeof(double) * (size_t)M * V);
    orc_linear(h, M, H, W, V, z);
    int rc = ORC_OK;
    for (int m = 0; m < M; m++) {
        const double *zr = z + (size_t)m * V;
        int best = 0;
        for (int v = 1; v < V; v++)
            if (zr[v] > zr[best]) best = v;
        double second = -INFINITY;
        for (int v = 0; v < V; v++)
            if (v != best && zr[v] > second) second = zr[v];
        for (int v = 0; v < V; v++)
            if (zr[v] != zr[v]) rc = ORC_ENAN;
        if (argmax) argmax[m] = best;
        if (margin) margin[m] = zr[best] - second;
    }
    if (!logits) free(z);
    return rc;
}

/* Greedy accept-prefix walk ([ORCH] module doc, greedy accept-walk invariant,
 * and per-round steps 7-8): a draft is accepted only while it equals the target
 * argmax at its position; accept_count a is the length of that prefix; the
 * free token is the target argmax at a; the committed tokens are targets
 * 0..a inclusive (the accepted drafts and the free token); rollback = K - a.
 * EOS (the rule is not on the page): committed stops after the first EOS,
 * inclusive, and hit_eos is set; accept_count and rollback ignore EOS.
 * result = {accept_count, free_token, rollback, hit_eos, n_committed}. */
int orc_accept_prefix(const int32_t *drafts, const int32_t *target, int K, const int32_t *eos,
                      int n_eos, int32_t *result, int32_t *committed) {
    if (K < 1 || !drafts || !target || !result || n_eos < 0 || (n_eos > 0 && !eos))
        return ORC_EINVAL;
    int a = 0;
    while (a < K && drafts[a] == target[a]) a++;
    int n = 0, hit = 0;
    for (int i = 0; i <= a; i++) {
        if (committed) committed[n] = target[i];
        n++;
        for (int e = 0; e < n_eos; e++)
            if (target[i] == eos[e]) hit = 1;
        if (hit) break;
    }
    result[0] = a;
    result[1] = target[a];
    result[2] = K - a;
    result[3] = hit;
    result[4] = n;
    return ORC_OK;
}

/* Sampling from softmax(z / T) by inverse CDF. p_i = exp(z_i/T - max)/sum, in
 * F64; the draw is the smallest index whose running sum of p (index order)
 * exceeds u, u in [0, 1) given by the caller (the random numbers are inputs).
 * Where rounding leaves u at or past the last running sum, the draw is the last
 * index of nonzero probability. */
static void orc_softmax_t(const float *z, int V, double T, double *p) {
    double m = -INFINITY;
    for (int i = 0; i < V; i++) {
        const double y = (double)z[i] / T;
        if (y > m) m = y;
    }
    double s = 0.0;
    for (int i = 0; i < V; i++) {
        p[i] = exp((double)z[i] / T - m);
        s += p[i];
    }
    for (int i = 0; i < V; i++) p[i] /= s;
}

static int orc_icdf(const double *w, int V, double u) {
    double tot = 0.0;
    for (int i = 0; i < V; i++) tot += w[i];
    const double tgt = u * tot;
    double c = 0.0;
    int last = 0;
    for (int i = 0; i < V; i++) {
        if (w[i] > 0.0) last = i;
        c += w[i];
        if (w[i] > 0.0 && c > tgt) return i;
    }
    return last;
}

/* One draw per row: token[m] ~ softmax(z[m] / T) with uniform u[m]; prob[m] (if
 * not NULL) is the token's probability. */
int orc_sample_tokens(const float *z, int M, int V, double T, const double *u, int32_t *token,
                      double *prob) {
    if (!z || !u || !token || M < 1 || V < 1 || !(T > 0.0) || !isfinite(T)) return ORC_EINVAL;
    double *p = (double *)malloc((size_t)V * sizeof(double));
    if (!p) return ORC_EINVAL;
    for (int m = 0; m < M; m++) {
        orc_softmax_t(z + (size_t)m * V, V, T, p);
        const int t = orc_icdf(p, V, u[m]);
        token[m] = t;
        if (prob) prob[m] = p[t];
    }
    free(p);
    return ORC_OK;
}

/* Sampled acceptance of one drafted token, MTP K = 1 ([ORCH] module doc,
 * "Non-greedy (Metropolis-Hastings)": the page names stochastic acceptance on
 * the MTP K = 1 path and gives no rule). The reading taken is the standard
 * speculative-sampling rule, under which the next emitted token is distributed
 * exactly as the target's softmax:
 *   q = softmax(zq / T)        the drafter's distribution the draft d came from
 *   p0 = softmax(zt[0] / T)    the target's distribution at the draft's position
 *   p1 = softmax(zt[1] / T)    the target's distribution one position later
 *   accept iff u0 * q(d) < p0(d), i.e. with probability min(1, p0(d) / q(d));
 *   accepted: free token drawn from p1 with u1 (the bonus token);
 *   rejected: free token drawn from max(0, p0 - q) / sum with u1 (from p0 when
 *   that residual is all zero).
 * result = {a (0 or 1), free_token, rollback = 1 - a, hit_eos, n_committed} as in
 * the greedy walk; committed = [d, free] when accepted, [free] otherwise, cut
 * after the first EOS (inclusive). info (if not NULL) = {q(d), p0(d), residual
 * sum}. */
int orc_accept_sampled(const float *zq, const float *zt, int V, double T, int32_t d, double u0,
                       double u1, const int32_t *eos, int n_eos, int32_t *result, int32_t *committed,
                       double *info) {
    if (!zq || !zt || !result || V < 1 || d < 0 || d >= V || !(T > 0.0) || !isfinite(T) ||
        n_eos < 0 || (n_eos > 0 && !eos))
        return ORC_EINVAL;
    double *q = (double *)malloc((size_t)V * sizeof(double));
    double *p0 = (double *)malloc((size_t)V * sizeof(double));
    double *p1 = (double *)malloc((size_t)V * sizeof(double));
    if (!q || !p0 || !p1) {
        free(q);
        free(p0);
        free(p1);
        return ORC_EINVAL;
    }
    orc_softmax_t(zq, V, T, q);
    orc_softmax_t(zt, V, T, p0);
    orc_softmax_t(zt + V, V, T, p1);
    const double qd = q[d], pd = p0[d];
    const int a = u0 * qd < pd;
    int free_tok;
    double rsum = 0.0;
    if (a) {
        free_tok = orc_icdf(p1, V, u1);
    } else {
        for (int i = 0; i < V; i++) {
            const double r = p0[i] - q[i];
            q[i] = r > 0.0 ? r : 0.0;  /* q now holds the residual */
            rsum += q[i];
        }
        free_tok = orc_icdf(rsum > 0.0 ? q : p0, V, u1);
    }
    if (info) {
        info[0] = qd;
        info[1] = pd;
        info[2] = rsum;
    }
    const int32_t seq[2] = {d, free_tok};
    const int32_t *c = a ? seq : seq + 1;
    const int nc = a ? 2 : 1;
    int n = 0, hit = 0;
    for (int i = 0; i < nc; i++) {
        if (committed) committed[n] = c[i];
        n++;
        for (int e = 0; e < n_eos; e++)
            if (c[i] == eos[e]) hit = 1;
        if (hit) break;
    }
    result[0] = a;
    result[1] = free_tok;
    result[2] = 1 - a;
    result[3] = hit;
    result[4] = n;
    free(q);
    free(p0);
    free(p1);
    return ORC_OK;
}

/* [ORCH] step 8: the rollback length saturates at zero on the page; removing
 * more rows than the cache holds is an error here. */
int orc_kv_rollback(orc_cache *kv, int n) {
    if (n < 0 || (int64_t)n > kv->seq_len) return ORC_ERANGE;
    kv->seq_len -= n;
    return ORC_OK;
}

int orc_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
