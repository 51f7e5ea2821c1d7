// api.hip -- the C ABI of libdbf (include/dbf.h): argument validation, workspace
// planning and the launch sequence of the drafter block.
//
// Everything is validated before the first enqueue, so an error leaves the stream
// and the cache untouched. No C++ exception crosses the ABI.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/dbf.h"
#include "internal.hpp"
#include "kernels.hpp"

using namespace dbf;

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

const char *dtname(int dt) {
    return dt == DBF_F32 ? "F32" : dt == DBF_BF16 ? "BF16" : dt == DBF_I32 ? "I32" : dt == DBF_BF16_T16 ? "BF16_T16" : "?";
}

int check_t(const dbf_tensor &t, const char *name, int dtype, int ndim, int64_t s0, int64_t s1 = -1,
            int64_t s2 = -1) {
    if (!t.data) return fail(DBF_EINVAL, "%s: null data pointer", name);
    // projections (requested as BF16) may be row-major BF16 or tiled BF16_T16
    const bool ok = t.dtype == dtype || (dtype == DBF_BF16 && t.dtype == DBF_BF16_T16);
    if (!ok)
        return fail(DBF_EDTYPE, "%s: dtype %s, expected %s", name, dtname(t.dtype), dtname(dtype));
    const int64_t want[3] = {s0, s1, s2};
    if (t.ndim != ndim) return fail(DBF_ESHAPE, "%s: ndim %d, expected %d", name, t.ndim, ndim);
    for (int i = 0; i < ndim; i++)
        if (t.shape[i] != want[i])
            return fail(DBF_ESHAPE, "%s: shape[%d] = %lld, expected %lld", name, i,
                        (long long)t.shape[i], (long long)want[i]);
    return DBF_OK;
}

#define CHECK(expr)                \
    do {                           \
        int rc_ = (expr);          \
        if (rc_ != DBF_OK) return rc_; \
    } while (0)

constexpr int TARGET_UNITS = 2048;  // wave units per projection launch (256 CUs x 8)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---------------------------------------------------------------------------
// workspace plan
// ---------------------------------------------------------------------------
struct Plan {
    int H, qt, kt, I, Kin, rd;
    GemmPlan in, q, k, v, g, gate, up, down;
    size_t xres, x1, xs_blk, xs_hctx, xs_o, xs_ff, qbuf, gbuf, attn;
    size_t ssp_x, ssp_x1, ssp_ctx, ssp_e, ssp_h;
    int ncb, ncb16;  // row-scale partials per row: 64-column (row kernels) and 16-column (O epilogue)
    size_t p_in0, p_in1, p_q, p_k, p_v, p_g, p_gate, p_up, p_down;
    // MoE
    int max_slots;
    GemmPlan router, sgi, shg, eg, ed, shd;
    size_t p_router, p_sgi, p_shg, p_shu, p_eg, p_eu, p_ed, p_shd, xs_e, xs_sh;
    size_t moe_n, moe_slot, moe_coef, moe_sscale, moe_sel;
    size_t head_part;  // fused head: per-workgroup top-2 records
    size_t total;
};

Plan make_plan(const dbf_config &c, int M, int R) {
    Plan p{};
    p.H = c.hidden;
    p.qt = c.n_q_heads * c.head_dim;
    p.kt = c.n_kv_heads * c.head_dim;
    p.I = c.intermediate;
    p.Kin = c.kind == DBF_KIND_DFLASH ? c.n_target_hidden * c.hidden : c.hidden;
    p.rd = c.rotary_dim > 0 ? c.rotary_dim : c.head_dim;
    // Launch shapes measured on MI355X at the benchmark sizes: the wide projections
    // of the normalized hidden rows (Q/K/V/gate in one launch, FFN gate+up in one),
    // the input projections (MTP eh halves; DFlash fc, which stages its F32 context
    // rows itself) and the 16-row down projection stream faster with the activation
    // slice in LDS; the one-row MTP down projections with the plain split-K kernel,
    // O whole-K.
    p.in = gemm_plan_lds(p.H, p.Kin, TARGET_UNITS / 4, 1);
    const int nbq = R > 0 ? 2 : 1;  // K/V also project the context rows
    p.q = gemm_plan_lds(p.qt, p.H, TARGET_UNITS / 4, nbq);
    p.k = gemm_plan_lds(p.kt, p.H, TARGET_UNITS / 4, nbq);
    p.v = p.k;
    p.g = p.q;
    if (c.ffn_kind == DBF_FFN_DENSE) {
        p.gate = gemm_plan_lds(p.I, p.H, TARGET_UNITS / 4, 1);
        p.up = p.gate;
        // With one to a few block rows (MTP) the partials are small, so the long down
        // projection takes about twice the waves, capped at 23 slices: its consumer
        // then still sums them in one batch of loads. The DFlash down projection is
        // LDS-staged with the full target (at H 2816, I 8448: 22 slices of 12 steps,
        // 484 workgroups; 14 slices of 20 steps were slower than split-K).
        p.down = c.kind == DBF_KIND_MTP ? gemm_plan(p.H, p.I, 23 * ((p.H + 31) / 32))
                                        : gemm_plan_lds(p.H, p.I, TARGET_UNITS, 1);
    }
    const int rows_kv = R > 0 ? 32 : 16;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off += align256(bytes);
        return at;
    };
    const size_t f = sizeof(float);
    p.xres = take((size_t)DBF_MAX_M * p.H * f);
    p.x1 = take((size_t)DBF_MAX_M * p.H * f);
    p.xs_blk = take(split_tile_bytes(p.H));
    p.xs_hctx = take(split_tile_bytes(p.H));
    p.xs_o = take(split_tile_bytes(p.qt));
    p.xs_ff = take(split_tile_bytes(p.I > 0 ? p.I : 32));
    p.ncb = (p.H + 63) / 64;
    p.ncb16 = (p.H + FULL_SSP_COLS - 1) / FULL_SSP_COLS;
    p.ssp_x = take((size_t)16 * p.ncb * f);
    p.ssp_x1 = take((size_t)16 * p.ncb16 * f);
    p.ssp_ctx = take((size_t)16 * p.ncb * f);
    // MTP: per-k-slice sums of squares of the e and h rows, written by the eh launch
    const int n_ssq = p.ncb > p.in.ksplit ? p.ncb : p.in.ksplit;
    p.ssp_e = take((size_t)16 * n_ssq * f);
    p.ssp_h = take((size_t)16 * n_ssq * f);
    p.qbuf = take((size_t)DBF_MAX_M * p.qt * f);
    p.gbuf = take((size_t)DBF_MAX_M * p.qt * f);
    p.attn = take((size_t)ATT_CHUNKS_MAX * DBF_MAX_M * c.n_q_heads * (c.head_dim + ATT_PART_EXTRA) * f);
    p.p_in0 = take((size_t)p.in.ksplit * 16 * p.H * f);
    p.p_in1 = take((size_t)p.in.ksplit * 16 * p.H * f);
    p.p_q = take((size_t)p.q.ksplit * 16 * p.qt * f);
    p.p_k = take((size_t)p.k.ksplit * rows_kv * p.kt * f);
    p.p_v = take((size_t)p.v.ksplit * rows_kv * p.kt * f);
    p.p_g = take((size_t)p.g.ksplit * 16 * p.qt * f);
    if (c.ffn_kind == DBF_FFN_DENSE) {
        p.p_gate = take((size_t)p.gate.ksplit * 16 * p.I * f);
        p.p_up = take((size_t)p.up.ksplit * 16 * p.I * f);
        p.p_down = take((size_t)p.down.ksplit * 16 * p.H * f);
    }
    if (c.ffn_kind == DBF_FFN_MOE) {
        const int E = c.n_experts, Ie = c.expert_intermediate, Is = c.shared_intermediate;
        p.max_slots = E < M * c.top_k ? E : M * c.top_k;  // >= 1: M >= 1, top_k >= 1
        // the router, shared-expert gate input and shared gate/up share one launch,
        // LDS-staged (0.3-2.0 us per step faster than split-K in six A/B pairs)
        p.router = gemm_plan_lds(E, p.H, TARGET_UNITS / 4, 1);
        p.sgi = gemm_plan_lds(1, p.H, 64, 1);
        p.shg = gemm_plan_lds(Is, p.H, TARGET_UNITS / 8, 1);
        int per_slot = TARGET_UNITS / (2 * p.max_slots);
        p.eg = gemm_plan(Ie, p.H, per_slot < 1 ? 1 : per_slot);
        per_slot = TARGET_UNITS / p.max_slots;
        // the expert and shared-expert down projections (one launch) are LDS-staged:
        // the MoE draft block at H 2048 with 256 experts, top 8, one or four rows,
        // steps 1.5-1.8 us faster than with split-K; the expert gate/up stay split-K
        // (LDS-staged was slower there)
        p.ed = gemm_plan_lds(p.H, Ie, per_slot < 1 ? 1 : per_slot, 1);
        p.shd = gemm_plan_lds(p.H, Is, TARGET_UNITS / 8, 1);
        p.p_router = take((size_t)p.router.ksplit * 16 * E * f);
        p.p_sgi = take((size_t)p.sgi.ksplit * 16 * 1 * f);
        p.p_shg = take((size_t)p.shg.ksplit * 16 * Is * f);
        p.p_shu = take((size_t)p.shg.ksplit * 16 * Is * f);
        p.p_eg = take((size_t)p.max_slots * p.eg.ksplit * 16 * Ie * f);
        p.p_eu = take((size_t)p.max_slots * p.eg.ksplit * 16 * Ie * f);
        p.p_ed = take((size_t)p.max_slots * p.ed.ksplit * 16 * p.H * f);
        p.p_shd = take((size_t)p.shd.ksplit * 16 * p.H * f);
        p.xs_e = take((size_t)p.max_slots * split_tile_bytes(Ie));
        p.xs_sh = take(split_tile_bytes(Is));
        p.moe_n = take(sizeof(int32_t));
        p.moe_slot = take((size_t)p.max_slots * sizeof(int32_t));
        p.moe_coef = take((size_t)p.max_slots * 16 * f);
        p.moe_sscale = take(16 * f);
        p.moe_sel = take((size_t)16 * c.top_k * sizeof(int32_t));
    }
    p.head_part = take((size_t)head_blocks(c.vocab) * 16 * sizeof(float4));
    p.total = off;
    return p;
}

// One projection launch: segments planned with the same lds flag (the first
// segment's plan fixes the kernel). rows: activation rows that hold data (M block
// rows, or R context rows), the default for every split tile added.
struct SegList {
    GemmArgs a{};
    int nbmax = 1, rows;
    const char *bad = nullptr;  // why the launch cannot run (checked before launching)
    explicit SegList(int rows_) : rows(rows_) {}
    void add(const dbf_tensor &t, int N, int K, const GemmPlan &pl, float *out, const uint16_t *xs0,
             const uint16_t *xs1 = nullptr, int rows0 = 0, int rows1 = 0) {
        if (a.nseg == GEMM_MAXSEG) {
            bad = "more segments than one projection launch holds";
            return;
        }
        if (a.nseg == 0) a.lds_x = pl.lds;
        else if (pl.lds != a.lds_x) bad = "LDS-staged and split-K plans mixed in one launch";  // units miscounted
        GemmSeg &s = a.seg[a.nseg++];
        s.W = (const uint16_t *)t.data;
        s.tiled = t.dtype == DBF_BF16_T16;
        s.out = out;
        s.xs0 = xs0;
        s.xs1 = xs1;
        s.N = N;
        s.K = K;
        s.nb = xs1 ? 2 : 1;
        s.ksplit = pl.ksplit;
        s.kslice_steps = pl.kslice_steps;
        s.tiles = pl.tiles;
        s.mrows[0] = rows0 > 0 ? rows0 : rows;
        s.mrows[1] = rows1 > 0 ? rows1 : rows;
        s.unit_begin = a.total_units;
        a.total_units += plan_units(pl);
        if (s.nb > nbmax) nbmax = s.nb;
    }
    // grouped (MoE experts): `slots` matrices selected on the device
    void add_grouped(const dbf_tensor &t, int N, int K, const GemmPlan &pl, float *out,
                     const uint16_t *xs0, long long xs_stride, int slots, const int32_t *slot_expert,
                     const int32_t *nslots) {
        add(t, N, K, pl, out, xs0);
        if (bad) return;
        GemmSeg &s = a.seg[a.nseg - 1];
        s.slots = slots;
        s.slot_expert = slot_expert;
        s.nslots = nslots;
        s.w_stride = s.tiled ? (long long)tiled_elems(N, K) : (long long)N * K;
        s.xs_stride = xs_stride;
        s.out_stride = (long long)pl.ksplit * 16 * N;
        a.total_units += (slots - 1) * plan_units(pl);
    }
    // segment seg (0 or 1) reads F32 rows instead of its split tile
    void f32_source(int seg, const GemmF32Src &s) {
        a.xf[seg] = s;
        a.xf_on = 1;
    }
    int launch(hipStream_t st) {
        if (bad) return fail(DBF_EINVAL, "internal: projection launch: %s", bad);
        if (!launch_gemm(a, nbmax, st))
            return fail(DBF_EINVAL, "internal: a projection launch its kernels do not take (two split tiles "
                                    "or an F32 source on anything but one plain LDS-staged segment)");
        return DBF_OK;
    }
};

int validate_config(const dbf_config *c) {
    if (!c) return fail(DBF_EINVAL, "config is null");
    if (c->kind != DBF_KIND_DFLASH && c->kind != DBF_KIND_MTP)
        return fail(DBF_EINVAL, "config.kind %d unknown", c->kind);
    if (c->n_layers < 1 || c->hidden < 8 || c->n_q_heads < 1 || c->n_kv_heads < 1 ||
        c->head_dim < 2 || c->vocab < 1)
        return fail(DBF_EINVAL, "config: non-positive dimension");
    if (c->hidden % 8) return fail(DBF_ESHAPE, "config.hidden %d not a multiple of 8", c->hidden);
    if (c->n_q_heads % c->n_kv_heads)
        return fail(DBF_ESHAPE, "n_q_heads %d not a multiple of n_kv_heads %d", c->n_q_heads,
                    c->n_kv_heads);
    if (!attn_supported(c->head_dim))
        return fail(DBF_ESHAPE, "head_dim %d unsupported (64, 128 or 256)", c->head_dim);
    const int rd = c->rotary_dim > 0 ? c->rotary_dim : c->head_dim;
    if (rd % 2 || rd > c->head_dim) return fail(DBF_ESHAPE, "rotary_dim %d invalid", rd);
    if (c->kind == DBF_KIND_DFLASH && c->n_target_hidden < 1)
        return fail(DBF_EINVAL, "DFlash config needs n_target_hidden >= 1");
    if (c->block_mask != DBF_MASK_CAUSAL && c->block_mask != DBF_MASK_BIDIR)
        return fail(DBF_EINVAL, "block_mask %d unknown", c->block_mask);
    if (c->ffn_kind == DBF_FFN_DENSE) {
        if (c->intermediate < 8 || c->intermediate % 8)
            return fail(DBF_ESHAPE, "intermediate %d must be a positive multiple of 8", c->intermediate);
    } else if (c->ffn_kind == DBF_FFN_MOE) {
        if (c->n_experts < 1 || c->n_experts > 1024)
            return fail(DBF_EINVAL, "n_experts %d outside [1, 1024]", c->n_experts);
        if (c->top_k < 1 || c->top_k > c->n_experts || c->top_k > DBF_MAX_TOPK)
            return fail(DBF_EINVAL, "top_k %d outside [1, min(E, %d)]", c->top_k, DBF_MAX_TOPK);
        if (c->expert_intermediate < 8 || c->expert_intermediate % 8 || c->shared_intermediate < 8 ||
            c->shared_intermediate % 8)
            return fail(DBF_ESHAPE, "expert/shared intermediate sizes must be positive multiples of 8");
    } else {
        return fail(DBF_EINVAL, "ffn_kind %d unknown", c->ffn_kind);
    }
    if (!(c->rms_eps >= 0.0) || !(c->rope_theta > 0.0))
        return fail(DBF_EINVAL, "rms_eps must be >= 0 and rope_theta > 0");
    return DBF_OK;
}

int validate_weights(const dbf_config &c, const dbf_weights *w, bool need_embed) {
    if (!w) return fail(DBF_EINVAL, "weights are null");
    const int H = c.hidden, qt = c.n_q_heads * c.head_dim, kt = c.n_kv_heads * c.head_dim;
    const int hd = c.head_dim;
    if (need_embed) {
        CHECK(check_t(w->embed, "embed", DBF_BF16, 2, c.vocab, H));
        if (w->embed.dtype != DBF_BF16) return fail(DBF_EDTYPE, "embed must be row-major BF16");
    }
    if (c.kind == DBF_KIND_DFLASH) {
        CHECK(check_t(w->fc, "fc", DBF_BF16, 2, H, (int64_t)c.n_target_hidden * H));
        CHECK(check_t(w->hidden_norm, "hidden_norm", DBF_F32, 1, H));
    } else {
        CHECK(check_t(w->enorm, "enorm", DBF_F32, 1, H));
        CHECK(check_t(w->hnorm, "hnorm", DBF_F32, 1, H));
        CHECK(check_t(w->eh_embed, "eh_embed", DBF_BF16, 2, H, H));
        CHECK(check_t(w->eh_hidden, "eh_hidden", DBF_BF16, 2, H, H));
    }
    CHECK(check_t(w->final_norm, "final_norm", DBF_F32, 1, H));
    if (!w->layers) return fail(DBF_EINVAL, "weights.layers is null");
    for (int l = 0; l < c.n_layers; l++) {
        const dbf_layer_weights &L = w->layers[l];
        char nm[64];
#define T(field, ...)                                              \
    snprintf(nm, sizeof nm, "layers[%d]." #field, l);              \
    CHECK(check_t(L.field, nm, __VA_ARGS__));
        T(in_norm, DBF_F32, 1, H);
        T(post_norm, DBF_F32, 1, H);
        T(wq, DBF_BF16, 2, qt, H);
        T(wk, DBF_BF16, 2, kt, H);
        T(wv, DBF_BF16, 2, kt, H);
        T(wo, DBF_BF16, 2, H, qt);
        T(q_norm, DBF_F32, 1, hd);
        T(k_norm, DBF_F32, 1, hd);
        if (c.has_attn_gate) { T(attn_gate, DBF_BF16, 2, qt, H); }
        if (c.ffn_kind == DBF_FFN_DENSE) {
            T(ffn_gate, DBF_BF16, 2, c.intermediate, H);
            T(ffn_up, DBF_BF16, 2, c.intermediate, H);
            T(ffn_down, DBF_BF16, 2, H, c.intermediate);
        } else {
            const int E = c.n_experts, Ie = c.expert_intermediate, Is = c.shared_intermediate;
            T(router, DBF_BF16, 2, E, H);
            T(exp_gate, DBF_BF16, 3, E, Ie, H);
            T(exp_up, DBF_BF16, 3, E, Ie, H);
            T(exp_down, DBF_BF16, 3, E, H, Ie);
            T(sh_gate, DBF_BF16, 2, Is, H);
            T(sh_up, DBF_BF16, 2, Is, H);
            T(sh_down, DBF_BF16, 2, H, Is);
            T(sh_gate_inp, DBF_BF16, 2, 1, H);
        }
#undef T
    }
    return DBF_OK;
}

int hip_check(const char *what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DBF_EHIP, "%s: %s", what, hipGetErrorString(e));
    return DBF_OK;
}

template <typename T>
T *at(void *ws, size_t off) {
    return (T *)((char *)ws + off);
}

}  // namespace

extern "C" {

int dbf_abi_version(void) { return DBF_ABI_VERSION; }

const char *dbf_last_error(void) { return g_err.c_str(); }

size_t draft_block_workspace_bytes(const dbf_config *cfg, int32_t M, int32_t R) {
    if (validate_config(cfg) != DBF_OK) return 0;
    if (M < 1 || M > DBF_MAX_M || R < 0 || R > DBF_MAX_R) return 0;
    if (cfg->kind == DBF_KIND_MTP) R = 0;
    return make_plan(*cfg, M, R).total;
}

int draft_block_forward(const dbf_config *cfg, const dbf_weights *w, dbf_kv_cache *cache,
                        const dbf_block_io *io, void *ws, size_t ws_bytes, void *stream) {
    g_err.clear();
    CHECK(validate_config(cfg));
    const dbf_config &c = *cfg;
    if (!io) return fail(DBF_EINVAL, "io is null");
    const int M = io->M, R = io->R;
    if (M < 1 || M > DBF_MAX_M) return fail(DBF_EINVAL, "M = %d outside [1, %d]", M, DBF_MAX_M);
    if (R < 0 || R > DBF_MAX_R) return fail(DBF_EINVAL, "R = %d outside [0, %d]", R, DBF_MAX_R);
    if (c.kind == DBF_KIND_MTP && R != 0) return fail(DBF_EINVAL, "MTP block takes no context rows (R = %d)", R);
    if (!io->h_final) return fail(DBF_EINVAL, "io.h_final is null");
    if (c.kind == DBF_KIND_DFLASH) {
        if (!io->tokens && !io->x0) return fail(DBF_EINVAL, "io: neither tokens nor x0 given");
        if (R > 0 && !io->ctx && !io->ctx_layers)
            return fail(DBF_EINVAL, "io: neither ctx nor ctx_layers given with R = %d", R);
        if (R > 0 && !io->ctx && io->ctx_layers) {
            if (c.n_target_hidden > DBF_MAX_CTX_LAYERS)
                return fail(DBF_EINVAL, "ctx_layers: n_target_hidden %d > %d", c.n_target_hidden,
                            DBF_MAX_CTX_LAYERS);
            for (int t = 0; t < c.n_target_hidden; t++)
                if (!io->ctx_layers[t]) return fail(DBF_EINVAL, "ctx_layers[%d] is null", t);
            if (io->ctx_ld < c.hidden || io->ctx_row0 < 0)
                return fail(DBF_EINVAL, "ctx_ld %lld (>= H) or ctx_row0 %lld (>= 0) invalid",
                            (long long)io->ctx_ld, (long long)io->ctx_row0);
        }
    } else {
        if (!io->tokens && !io->x0) return fail(DBF_EINVAL, "io: neither tokens nor x0 (embed_t) given");
        if (!io->ctx) return fail(DBF_EINVAL, "io.ctx (prev_hidden) is null");
    }
    CHECK(validate_weights(c, w, io->tokens != nullptr));
    int K_acc = 0;
    if (io->lm_head) {
        const dbf_tensor &lm = *io->lm_head;
        CHECK(check_t(lm, "io.lm_head", DBF_BF16, 2, c.vocab, c.hidden));
        if (!io->argmax) return fail(DBF_EINVAL, "io.argmax is required with io.lm_head");
    }
    if (io->target) {
        if (!io->lm_head) return fail(DBF_EINVAL, "io.target needs io.lm_head (the drafts are its argmaxes)");
        K_acc = c.kind == DBF_KIND_DFLASH ? M - 1 : 1;
        if (K_acc < 1) return fail(DBF_EINVAL, "accept walk of a DFlash block needs M >= 2 (M = %d)", M);
        if (!io->accept_result) return fail(DBF_EINVAL, "io.accept_result is required with io.target");
        if (io->n_eos < 0 || io->n_eos > 1024 || (io->n_eos > 0 && !io->eos))
            return fail(DBF_EINVAL, "io eos list invalid (n_eos = %d)", io->n_eos);
    } else if (io->accept_result || io->committed || io->n_eos) {
        return fail(DBF_EINVAL, "io.accept_result, io.committed and io.n_eos need io.target");
    }
    if (!io->lm_head && (io->argmax || io->top2_margin))
        return fail(DBF_EINVAL, "io.argmax and io.top2_margin need io.lm_head");
    if (!cache || !cache->k || !cache->v) return fail(DBF_EINVAL, "cache or its buffers are null");
    if (cache->dtype != DBF_F32 && cache->dtype != DBF_BF16)
        return fail(DBF_EDTYPE, "cache dtype %s (F32 or BF16)", dtname(cache->dtype));
    if (cache->n_layers != c.n_layers || cache->n_kv_heads != c.n_kv_heads ||
        cache->head_dim != c.head_dim)
        return fail(DBF_ESHAPE, "cache shape [%d, %d, *, %d] does not match the config",
                    cache->n_layers, cache->n_kv_heads, cache->head_dim);
    if (cache->seq_len < 0 || cache->capacity < 0)
        return fail(DBF_ERANGE, "cache seq_len/capacity negative");
    if (cache->seq_len + R + M > cache->capacity)
        return fail(DBF_ERANGE, "cache overflow: seq_len %lld + R %d + M %d > capacity %lld",
                    (long long)cache->seq_len, R, M, (long long)cache->capacity);
    const Plan p = make_plan(c, M, R);
    if (!ws) return fail(DBF_EWORKSPACE, "workspace is null");
    if ((uintptr_t)ws % 256) return fail(DBF_EWORKSPACE, "workspace not 256-byte aligned");
    if (ws_bytes < p.total)
        return fail(DBF_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, p.total);

    hipStream_t st = (hipStream_t)stream;
    (void)hipGetLastError();
    const int H = p.H, qt = p.qt, kt = p.kt, hd = c.head_dim;
    const float eps = (float)c.rms_eps;
    const long long P0 = cache->seq_len;
    float *xres = at<float>(ws, p.xres), *x1 = at<float>(ws, p.x1);
    uint16_t *xs_blk = at<uint16_t>(ws, p.xs_blk);
    uint16_t *xs_hctx = at<uint16_t>(ws, p.xs_hctx);
    uint16_t *xs_o = at<uint16_t>(ws, p.xs_o), *xs_ff = at<uint16_t>(ws, p.xs_ff);
    float *qbuf = at<float>(ws, p.qbuf), *gbuf = at<float>(ws, p.gbuf);
    float *attn_part = at<float>(ws, p.attn);
    const dbf_layer_weights *Ls = w->layers;

    float *ssp_x = at<float>(ws, p.ssp_x), *ssp_x1 = at<float>(ws, p.ssp_x1);
    float *ssp_ctx = at<float>(ws, p.ssp_ctx);
    const int ncb = p.ncb;
    auto col = [&]() {
        ColArgs a{};
        a.H = H;
        a.ncb_in = ncb;
        a.ncb_out = ncb;
        return a;
    };

    // ---- input projection
    if (c.kind == DBF_KIND_DFLASH) {
        // x = embed[tokens] (or x0); split(x (.) in_norm_0) for the first layer
        ColArgs a = col();
        a.M = M;
        a.tokens = io->tokens;
        a.embed = (const uint16_t *)w->embed.data;
        a.V = c.vocab;
        a.base = io->x0;
        a.ldb = H;
        a.out = xres;
        a.w = (const float *)Ls[0].in_norm.data;
        a.xs = xs_blk;
        a.ssp_out = ssp_x;
        if (R == 0) launch_colsum(a, st);
        if (R > 0) {
            // h_ctx = RMSNorm(T fc^T, hidden_norm): the projection reads the F32 rows
            // of T (or gathers the captured target layers) and splits them as it
            // goes; then the block rows and split(proj (.) hidden_norm) in one launch
            SegList sl(R);
            sl.add(w->fc, H, p.Kin, p.in, at<float>(ws, p.p_in0), nullptr);
            GemmF32Src src{};
            if (io->ctx) {
                src.xf = io->ctx;
                src.xf_ld = p.Kin;
            } else {
                for (int i = 0; i < c.n_target_hidden; i++) src.xg[i] = io->ctx_layers[i];
                src.xg_cols = H;
                src.xg_ld = io->ctx_ld;
                src.xg_row0 = io->ctx_row0;
            }
            sl.f32_source(0, src);
            CHECK(sl.launch(st));
            ColArgs h = col();
            h.M = R;
            h.p0 = at<float>(ws, p.p_in0);
            h.ks0 = p.in.ksplit;
            h.rows0 = 16;
            h.w = (const float *)w->hidden_norm.data;
            h.xs = xs_hctx;
            h.ssp_out = ssp_ctx;
            launch_colsum2(a, h, st);
        }
    } else {
        // x = RMSNorm(e, enorm) eh_embed^T + RMSNorm(h, hnorm) eh_hidden^T (eps 1e-6)
        float *ssp_e = at<float>(ws, p.ssp_e), *ssp_h = at<float>(ws, p.ssp_h);
        // The eh launch stages e (embed[token] for chained steps, else x0) and h
        // (prev_hidden) itself, enorm / hnorm applied, and writes each k-slice's
        // sums of squares of the raw rows; the pass after it forms the row scales.
        SegList sl(M);
        sl.add(w->eh_embed, H, H, p.in, at<float>(ws, p.p_in0), nullptr);
        sl.add(w->eh_hidden, H, H, p.in, at<float>(ws, p.p_in1), nullptr);
        GemmF32Src se{}, sh{};
        se.xf = io->x0;
        se.xf_ld = H;
        se.tokens = io->tokens;
        se.embed = (const uint16_t *)w->embed.data;
        se.V = c.vocab;
        se.w = (const float *)w->enorm.data;
        se.ssq = ssp_e;
        se.ssq_ld = p.in.ksplit;
        sh.xf = io->ctx;  // prev_hidden rows are given, never gathered
        sh.xf_ld = H;
        sh.w = (const float *)w->hnorm.data;
        sh.ssq = ssp_h;
        sh.ssq_ld = p.in.ksplit;
        sl.f32_source(0, se);
        sl.f32_source(1, sh);
        CHECK(sl.launch(st));
        ColArgs x = col();
        x.ncb_in = p.in.ksplit;  // the row-scale partials are per k-slice
        x.M = M;
        x.p0 = at<float>(ws, p.p_in0);
        x.ks0 = p.in.ksplit;
        x.rows0 = 16;
        x.ssp0 = ssp_e;
        x.eps0 = 1e-6f;
        x.p1 = at<float>(ws, p.p_in1);
        x.ks1 = p.in.ksplit;
        x.rows1 = 16;
        x.ssp1 = ssp_h;
        x.eps1 = 1e-6f;
        x.out = xres;
        x.w = (const float *)Ls[0].in_norm.data;
        x.xs = xs_blk;
        x.ssp_out = ssp_x;
        launch_colsum(x, st);
    }

    int chunk = 0, n_chunks = 0;
    {
        const int nq_group = (c.n_q_heads / c.n_kv_heads) * M;
        const int qt = attn_qtiles(hd, nq_group, cache->dtype == DBF_BF16);
        const int qgroups = (nq_group + 16 * qt - 1) / (16 * qt);
        attn_plan(P0 + R + M, c.n_kv_heads * qgroups, &chunk, &n_chunks);
    }
    // RoPE inverse frequencies theta^(-2j/rotary_dim), in F64, shared by every layer
    double inv_freq[ROPE_MAX_PAIRS];
    for (int j = 0; j < p.rd / 2 && j < ROPE_MAX_PAIRS; j++)
        inv_freq[j] = pow(c.rope_theta, -2.0 * (double)j / (double)p.rd);
    const size_t elt = cache->dtype == DBF_BF16 ? 2 : 4;
    const size_t layer_stride = (size_t)c.n_kv_heads * cache->capacity * hd * elt;

    for (int l = 0; l < c.n_layers; l++) {
        const dbf_layer_weights &L = Ls[l];
        const bool last = l == c.n_layers - 1;
        float *pq = at<float>(ws, p.p_q), *pk = at<float>(ws, p.p_k), *pv = at<float>(ws, p.p_v);
        float *pg = at<float>(ws, p.p_g);
        {
            SegList sl(M);
            sl.add(L.wq, qt, H, p.q, pq, xs_blk);
            if (R > 0) {
                sl.add(L.wk, kt, H, p.k, pk, xs_hctx, xs_blk, R, M);
                sl.add(L.wv, kt, H, p.v, pv, xs_hctx, xs_blk, R, M);
            } else {
                sl.add(L.wk, kt, H, p.k, pk, xs_blk);
                sl.add(L.wv, kt, H, p.v, pv, xs_blk);
            }
            if (c.has_attn_gate) sl.add(L.attn_gate, qt, H, p.g, pg, xs_blk);
            CHECK(sl.launch(st));
        }
        void *ck = (char *)cache->k + l * layer_stride;
        void *cv = (char *)cache->v + l * layer_stride;
        {
            QkvPostArgs qa{};
            qa.pq = pq;
            qa.pk = pk;
            qa.pv = pv;
            qa.pg = c.has_attn_gate ? pg : nullptr;
            qa.ksq = p.q.ksplit;
            qa.ksk = p.k.ksplit;
            qa.ksv = p.v.ksplit;
            qa.ksg = p.g.ksplit;
            qa.rows_kv = R > 0 ? 32 : 16;
            qa.kv_block_row0 = R > 0 ? 16 : 0;
            qa.ssp_x = ssp_x;
            qa.ssp_ctx = ssp_ctx;
            qa.ncb = ncb;
            qa.ncb_ctx = ncb;
            qa.H = H;
            qa.q_norm = (const float *)L.q_norm.data;
            qa.k_norm = (const float *)L.k_norm.data;
            qa.eps = eps;
            memcpy(qa.inv_freq, inv_freq, sizeof(double) * (size_t)(p.rd / 2));
            qa.rotary_dim = p.rd;
            qa.M = M;
            qa.R = R;
            qa.nq = c.n_q_heads;
            qa.nkv = c.n_kv_heads;
            qa.hd = hd;
            qa.P0 = P0;
            qa.q_out = qbuf;
            qa.g_out = c.has_attn_gate ? gbuf : nullptr;
            qa.cache_k = ck;
            qa.cache_v = cv;
            qa.kv_bf16 = cache->dtype == DBF_BF16;
            qa.capacity = cache->capacity;
            launch_qkv_post(qa, st);
        }
        {
            AttnArgs aa{};
            aa.q = qbuf;
            aa.cache_k = ck;
            aa.cache_v = cv;
            aa.kv_bf16 = cache->dtype == DBF_BF16;
            aa.capacity = cache->capacity;
            aa.n_ctx = P0 + R;
            aa.M = M;
            aa.nq = c.n_q_heads;
            aa.nkv = c.n_kv_heads;
            aa.hd = hd;
            aa.chunk = chunk;
            aa.n_chunks = n_chunks;
            aa.bidir = c.block_mask == DBF_MASK_BIDIR;
            aa.part = attn_part;
            launch_attn(aa, st);
            CombineArgs ca{};
            ca.part = attn_part;
            ca.n_chunks = n_chunks;
            ca.M = M;
            ca.nq = c.n_q_heads;
            ca.hd = hd;
            ca.g = c.has_attn_gate ? gbuf : nullptr;
            ca.xs = xs_o;
            launch_attn_combine(ca, st);
        }
        {
            // x1 = x + o Wo^T; split(x1 (.) post_norm) and its sums of squares for the FFN
            FullArgs fa{};
            fa.W = (const uint16_t *)L.wo.data;
            fa.tiled = L.wo.dtype == DBF_BF16_T16;
            fa.xs = xs_o;
            fa.N = H;
            fa.K = qt;
            fa.M = M;
            fa.base = xres;
            fa.out = x1;
            fa.w = (const float *)L.post_norm.data;
            fa.ssp_out = ssp_x1;
            fa.xs_out = xs_blk;
            launch_gemm_full(fa, st);
        }
        if (c.ffn_kind == DBF_FFN_DENSE) {
            {
                SegList sl(M);
                sl.add(L.ffn_gate, p.I, H, p.gate, at<float>(ws, p.p_gate), xs_blk);
                sl.add(L.ffn_up, p.I, H, p.up, at<float>(ws, p.p_up), xs_blk);
                CHECK(sl.launch(st));
                SwigluArgs sa{};
                sa.pg = at<float>(ws, p.p_gate);
                sa.pu = at<float>(ws, p.p_up);
                sa.ksg = p.gate.ksplit;
                sa.ksu = p.up.ksplit;
                sa.ssp = ssp_x1;
                sa.ncb = p.ncb16;
                sa.H = H;
                sa.eps = eps;
                sa.M = M;
                sa.I = p.I;
                sa.xs = xs_ff;
                launch_swiglu(sa, st);
                SegList sd(M);
                sd.add(L.ffn_down, H, p.I, p.down, at<float>(ws, p.p_down), xs_ff);
                CHECK(sd.launch(st));
            }
        } else {
            // MoE: router + shared-expert projections, routing, grouped experts, combine
            const int E = c.n_experts, Ie = c.expert_intermediate, Is = c.shared_intermediate;
            int32_t *nsl = at<int32_t>(ws, p.moe_n), *slot_e = at<int32_t>(ws, p.moe_slot);
            float *coef = at<float>(ws, p.moe_coef), *sscale = at<float>(ws, p.moe_sscale);
            {
                SegList sl(M);
                sl.add(L.router, E, H, p.router, at<float>(ws, p.p_router), xs_blk);
                sl.add(L.sh_gate_inp, 1, H, p.sgi, at<float>(ws, p.p_sgi), xs_blk);
                sl.add(L.sh_gate, Is, H, p.shg, at<float>(ws, p.p_shg), xs_blk);
                sl.add(L.sh_up, Is, H, p.shg, at<float>(ws, p.p_shu), xs_blk);
                CHECK(sl.launch(st));
            }
            {
                MoeRouteArgs ra{};
                ra.p_router = at<float>(ws, p.p_router);
                ra.ks_router = p.router.ksplit;
                ra.p_sgi = at<float>(ws, p.p_sgi);
                ra.ks_sgi = p.sgi.ksplit;
                ra.ssp = ssp_x1;
                ra.ncb = p.ncb16;
                ra.H = H;
                ra.eps = eps;
                ra.M = M;
                ra.E = E;
                ra.top_k = c.top_k;
                ra.max_slots = p.max_slots;
                ra.nslots = nsl;
                ra.slot_expert = slot_e;
                ra.coef = coef;
                ra.shared_scale = sscale;
                ra.sel = at<int32_t>(ws, p.moe_sel);
                ra.touched_out = io->moe_experts ? io->moe_experts + l : nullptr;
                launch_moe_route(ra, st);
            }
            {
                SegList sl(M);
                sl.add_grouped(L.exp_gate, Ie, H, p.eg, at<float>(ws, p.p_eg), xs_blk, 0, p.max_slots,
                               slot_e, nsl);
                sl.add_grouped(L.exp_up, Ie, H, p.eg, at<float>(ws, p.p_eu), xs_blk, 0, p.max_slots,
                               slot_e, nsl);
                CHECK(sl.launch(st));
            }
            {
                MoeSwigluArgs sa{};
                sa.pg = at<float>(ws, p.p_eg);
                sa.pu = at<float>(ws, p.p_eu);
                sa.ks = p.eg.ksplit;
                sa.psg = at<float>(ws, p.p_shg);
                sa.psu = at<float>(ws, p.p_shu);
                sa.ks_sh = p.shg.ksplit;
                sa.ssp = ssp_x1;
                sa.ncb = p.ncb16;
                sa.H = H;
                sa.eps = eps;
                sa.M = M;
                sa.Ie = Ie;
                sa.Is = Is;
                sa.max_slots = p.max_slots;
                sa.nslots = nsl;
                sa.xs_e = at<uint16_t>(ws, p.xs_e);
                sa.xs_sh = at<uint16_t>(ws, p.xs_sh);
                launch_moe_swiglu(sa, st);
            }
            {
                SegList sl(M);
                sl.add_grouped(L.exp_down, H, Ie, p.ed, at<float>(ws, p.p_ed), at<uint16_t>(ws, p.xs_e),
                               (long long)(split_tile_bytes(Ie) / 2), p.max_slots, slot_e, nsl);
                sl.add(L.sh_down, H, Is, p.shd, at<float>(ws, p.p_shd), at<uint16_t>(ws, p.xs_sh));
                CHECK(sl.launch(st));
            }
        }
        {
            // x = x1 + FFN; split(x (.) next in_norm), or the final norm after the last layer
            float *lh = io->layer_hidden ? io->layer_hidden + (size_t)l * M * H : nullptr;
            const float *wn = last ? nullptr : (const float *)Ls[l + 1].in_norm.data;
            if (c.ffn_kind == DBF_FFN_DENSE) {
                ColArgs a = col();
                a.M = M;
                a.base = x1;
                a.ldb = H;
                a.p0 = at<float>(ws, p.p_down);
                a.ks0 = p.down.ksplit;
                a.rows0 = 16;
                a.out = xres;
                a.copy0 = lh;
                a.copy1 = last ? io->hidden_out : nullptr;
                a.w = wn;
                a.xs = last ? nullptr : xs_blk;
                a.ssp_out = ssp_x;
                launch_colsum(a, st);
            } else {
                MoeCombineArgs a{};
                a.base = x1;
                a.pd = at<float>(ws, p.p_ed);
                a.ks = p.ed.ksplit;
                a.psd = at<float>(ws, p.p_shd);
                a.ks_sh = p.shd.ksplit;
                a.nslots = at<int32_t>(ws, p.moe_n);
                a.coef = at<float>(ws, p.moe_coef);
                a.shared_scale = at<float>(ws, p.moe_sscale);
                a.M = M;
                a.H = H;
                a.max_slots = p.max_slots;
                a.out = xres;
                a.copy0 = lh;
                a.copy1 = last ? io->hidden_out : nullptr;
                a.w = wn;
                a.xs = last ? nullptr : xs_blk;
                a.ssp_out = ssp_x;
                a.ncb = ncb;
                launch_moe_combine(a, st);
            }
            if (last && io->lm_head) {
                // shared head: final norm folded into the lm_head staging, then the
                // argmax reduction and the accept walk in one workgroup
                HeadNorm nrm{(const float *)w->final_norm.data, ssp_x, ncb, eps, io->h_final};
                float4 *part = at<float4>(ws, p.head_part);
                launch_head((const uint16_t *)io->lm_head->data, io->lm_head->dtype == DBF_BF16_T16, xres,
                            c.vocab, H, M, nullptr, part, &nrm, st);
                AcceptArgs acc{io->target, K_acc, c.kind == DBF_KIND_DFLASH ? 1 : 0, io->eos, io->n_eos,
                               io->accept_result, io->committed};
                launch_head_finish(part, head_blocks(c.vocab), M, io->argmax, io->top2_margin, acc, st);
            } else if (last) {
                launch_final_norm(xres, ssp_x, ncb, M, H, (const float *)w->final_norm.data, eps,
                                  io->h_final, st);
            }
        }
    }
    CHECK(hip_check("draft_block_forward launch"));
    cache->seq_len = P0 + R + M;
    return DBF_OK;
}

size_t lm_head_argmax_workspace_bytes(int32_t M, int32_t H, int32_t V) {
    if (M < 1 || M > DBF_MAX_M || H < 8 || V < 1) return 0;
    return align256((size_t)head_blocks(V) * 16 * sizeof(float4));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// lm_head + argmax. The checks and the launches are shared by the entry point
// that takes the caller's workspace and the one that uses the library's static
// device scratch (for callers that cannot allocate).
namespace {

int head_check(const float *h, int32_t M, int32_t H, const dbf_tensor *lm_head, const int32_t *argmax,
               int *V_out) {
    if (!h || !lm_head || !argmax) return fail(DBF_EINVAL, "h, lm_head and argmax are required");
    if (M < 1 || M > DBF_MAX_M) return fail(DBF_EINVAL, "M = %d outside [1, %d]", M, DBF_MAX_M);
    if (H < 8 || H % 8) return fail(DBF_ESHAPE, "H = %d must be a positive multiple of 8", H);
    if (lm_head->ndim != 2 || lm_head->shape[1] != H || lm_head->shape[0] < 1)
        return fail(DBF_ESHAPE, "lm_head must be [V, %d]", H);
    if (lm_head->dtype != DBF_BF16 && lm_head->dtype != DBF_BF16_T16)
        return fail(DBF_EDTYPE, "lm_head dtype %s, expected BF16 or BF16_T16", dtname(lm_head->dtype));
    if (!lm_head->data) return fail(DBF_EINVAL, "lm_head data is null");
    if (lm_head->shape[0] > 0x7fffffffLL) return fail(DBF_ESHAPE, "vocabulary too large");
    *V_out = (int)lm_head->shape[0];
    return DBF_OK;
}

int head_launch(const float *h, int32_t M, int32_t H, const dbf_tensor *lm_head, int V, int32_t *argmax,
                float *logits, float *top2_margin, void *ws, void *stream) {
    hipStream_t st = (hipStream_t)stream;
    (void)hipGetLastError();
    float4 *part = (float4 *)ws;
    launch_head((const uint16_t *)lm_head->data, lm_head->dtype == DBF_BF16_T16, h, V, H, M, logits,
                part, nullptr, st);
    launch_head_reduce(part, head_blocks(V), M, argmax, top2_margin, st);
    return hip_check("lm_head_argmax launch");
}

}  // namespace

// Static device scratch of lm_head_argmax_noalloc: the per-workgroup top-2 records
// (V/1024 workgroups x 16 rows x 16 bytes). Each device the library runs on holds
// its own copy for the life of the process. Host code never uses this name as an
// address: the device address is taken once per device with hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[DBF_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[SCRATCH_MAX_DEVICES];

// device address of `scratch` on the current device (looked up on the first call)
int scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DBF_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= SCRATCH_MAX_DEVICES)
        return fail(DBF_EHIP, "device %d outside the %d the static scratch supports", dev, SCRATCH_MAX_DEVICES);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(DBF_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return DBF_OK;
}

}  // namespace

extern "C" {

int lm_head_argmax(const float *h, int32_t M, int32_t H, const dbf_tensor *lm_head, int32_t *argmax,
                   float *logits, float *top2_margin, void *ws, size_t ws_bytes, void *stream) {
    g_err.clear();
    int V = 0;
    CHECK(head_check(h, M, H, lm_head, argmax, &V));
    const size_t need = lm_head_argmax_workspace_bytes(M, H, V);
    if (!ws) return fail(DBF_EWORKSPACE, "workspace is null");
    if ((uintptr_t)ws % 256) return fail(DBF_EWORKSPACE, "workspace not 256-byte aligned");
    if (ws_bytes < need) return fail(DBF_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    return head_launch(h, M, H, lm_head, V, argmax, logits, top2_margin, ws, stream);
}

int lm_head_argmax_noalloc(const float *h, int32_t M, int32_t H, const dbf_tensor *lm_head, int32_t *argmax,
                           float *logits, float *top2_margin, void *stream) {
    g_err.clear();
    int V = 0;
    CHECK(head_check(h, M, H, lm_head, argmax, &V));
    const size_t need = lm_head_argmax_workspace_bytes(M, H, V);
    if (need > DBF_NOALLOC_SCRATCH_BYTES)
        return fail(DBF_ERANGE, "vocabulary %d needs %zu bytes of scratch, more than the static %d "
                                "(lm_head_argmax_noalloc takes V <= %d)",
                    V, need, DBF_NOALLOC_SCRATCH_BYTES, DBF_NOALLOC_MAX_VOCAB);
    void *ptr = nullptr;
    CHECK(scratch_address(&ptr));
    return head_launch(h, M, H, lm_head, V, argmax, logits, top2_margin, ptr, stream);
}

int accept_prefix(const int32_t *drafts, const int32_t *target, int32_t K, const int32_t *eos,
                  int32_t n_eos, int32_t *result, int32_t *committed, void *stream) {
    g_err.clear();
    if (!drafts || !target || !result) return fail(DBF_EINVAL, "drafts, target and result are required");
    if (K < 1 || K > 1024) return fail(DBF_EINVAL, "K = %d outside [1, 1024]", K);
    if (n_eos < 0 || (n_eos > 0 && !eos)) return fail(DBF_EINVAL, "eos list invalid (n_eos = %d)", n_eos);
    (void)hipGetLastError();
    launch_accept(drafts, target, K, eos, n_eos, result, committed, (hipStream_t)stream);
    return hip_check("accept_prefix launch");
}

// ---------------------------------------------------------------------------
// Sampling from softmax(logits / T) and sampled acceptance of one draft
static constexpr double LOG2E = 1.4426950408889634;

static int check_temperature(float T) {
    if (!(T >= 1e-3f && T <= 1e3f)) return fail(DBF_EINVAL, "temperature %g outside [1e-3, 1e3]", (double)T);
    return DBF_OK;
}

static int check_ws(const void *ws, size_t ws_bytes, size_t need) {
    if (!ws) return fail(DBF_EWORKSPACE, "workspace is null");
    if ((uintptr_t)ws % 256) return fail(DBF_EWORKSPACE, "workspace not 256-byte aligned");
    if (ws_bytes < need) return fail(DBF_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    return DBF_OK;
}

size_t sample_tokens_workspace_bytes(int32_t M, int32_t V) {
    if (M < 1 || M > DBF_MAX_SAMPLE_ROWS || V < 1 || V > DBF_MAX_VOCAB) return 0;
    return align256((size_t)M * smp_blocks(V) * sizeof(float2));
}

int sample_tokens(const float *logits, int32_t M, int32_t V, float temperature, const float *u,
                  int32_t *token, float *prob, void *ws, size_t ws_bytes, void *stream) {
    g_err.clear();
    if (!logits || !u || !token) return fail(DBF_EINVAL, "logits, u and token are required");
    if (M < 1 || M > DBF_MAX_SAMPLE_ROWS) return fail(DBF_EINVAL, "M = %d outside [1, %d]", M, DBF_MAX_SAMPLE_ROWS);
    if (V < 1 || V > DBF_MAX_VOCAB) return fail(DBF_ESHAPE, "V = %d outside [1, %d]", V, DBF_MAX_VOCAB);
    int rc = check_temperature(temperature);
    if (rc) return rc;
    if ((rc = check_ws(ws, ws_bytes, sample_tokens_workspace_bytes(M, V)))) return rc;
    const int nb = smp_blocks(V);
    const float c = (float)(LOG2E / (double)temperature);
    float2 *stats = (float2 *)ws;
    (void)hipGetLastError();
    SmpStatArgs sa{};
    sa.z[0] = logits;
    sa.nptr = 1;
    sa.ld = V;
    sa.V = V;
    sa.nb = nb;
    sa.c = c;
    sa.stats = stats;
    launch_smp_stats(sa, M, (hipStream_t)stream);
    SmpDrawArgs da{};
    da.z = logits;
    da.stats = stats;
    da.u = u;
    da.V = V;
    da.nb = nb;
    da.c = c;
    da.token = token;
    da.prob = prob;
    launch_smp_draw(da, M, (hipStream_t)stream);
    return hip_check("sample_tokens launch");
}

size_t accept_sampled_workspace_bytes(int32_t V) {
    if (V < 1 || V > DBF_MAX_VOCAB) return 0;
    const size_t nb = (size_t)smp_blocks(V);
    return align256(3 * nb * sizeof(float2)) + align256(nb * sizeof(float));
}

int accept_sampled(const float *draft_logits, const float *target_logits, int32_t V, float temperature,
                   const int32_t *draft, const float *u, const int32_t *eos, int32_t n_eos,
                   int32_t *result, int32_t *committed, void *ws, size_t ws_bytes, void *stream) {
    g_err.clear();
    if (!draft_logits || !target_logits || !draft || !u || !result)
        return fail(DBF_EINVAL, "draft_logits, target_logits, draft, u and result are required");
    if (V < 1 || V > DBF_MAX_VOCAB) return fail(DBF_ESHAPE, "V = %d outside [1, %d]", V, DBF_MAX_VOCAB);
    if (n_eos < 0 || n_eos > 1024 || (n_eos > 0 && !eos))
        return fail(DBF_EINVAL, "eos list invalid (n_eos = %d)", n_eos);
    int rc = check_temperature(temperature);
    if (rc) return rc;
    if ((rc = check_ws(ws, ws_bytes, accept_sampled_workspace_bytes(V)))) return rc;
    const int nb = smp_blocks(V);
    const float c = (float)(LOG2E / (double)temperature);
    float2 *stats = (float2 *)ws;
    float *rsum = (float *)((char *)ws + align256(3 * (size_t)nb * sizeof(float2)));
    const float *zp0 = target_logits, *zp1 = target_logits + V;
    (void)hipGetLastError();
    SmpStatArgs sa{};
    sa.z[0] = draft_logits;
    sa.z[1] = zp0;
    sa.z[2] = zp1;
    sa.nptr = 3;
    sa.V = V;
    sa.nb = nb;
    sa.c = c;
    sa.stats = stats;
    launch_smp_stats(sa, 3, (hipStream_t)stream);
    SmpResidualArgs ra{};
    ra.zq = draft_logits;
    ra.zp = zp0;
    ra.stats = stats;
    ra.V = V;
    ra.nb = nb;
    ra.c = c;
    ra.rsum = rsum;
    launch_smp_residual(ra, (hipStream_t)stream);
    SmpAcceptArgs aa{};
    aa.zq = draft_logits;
    aa.zp0 = zp0;
    aa.zp1 = zp1;
    aa.stats = stats;
    aa.rsum = rsum;
    aa.draft = draft;
    aa.u = u;
    aa.eos = eos;
    aa.n_eos = n_eos;
    aa.V = V;
    aa.nb = nb;
    aa.c = c;
    aa.result = result;
    aa.committed = committed;
    launch_smp_accept(aa, (hipStream_t)stream);
    return hip_check("accept_sampled launch");
}

size_t dbf_tiled_bytes(int64_t N, int64_t K) {
    if (N < 1 || K < 1) return 0;
    return tiled_elems(N, K) * sizeof(uint16_t);
}

int dbf_tile_weight(const dbf_tensor *src, void *dst, void *stream) {
    g_err.clear();
    if (!src || !src->data || !dst) return fail(DBF_EINVAL, "src, src->data and dst are required");
    if (src->dtype != DBF_BF16) return fail(DBF_EDTYPE, "tiling takes a row-major BF16 weight");
    if (src->ndim != 2 && src->ndim != 3) return fail(DBF_ESHAPE, "tiling takes [N, K] or [B, N, K]");
    const int64_t B = src->ndim == 3 ? src->shape[0] : 1;
    const int64_t N = src->shape[src->ndim - 2], K = src->shape[src->ndim - 1];
    if (B < 1 || N < 1 || K < 8 || K % 8 || N > 0x7fffffff || K > 0x7fffffff)
        return fail(DBF_ESHAPE, "tiling shape invalid (K must be a positive multiple of 8)");
    const char *s0 = (const char *)src->data, *d0 = (const char *)dst;
    const size_t sb = (size_t)B * N * K * 2, db = (size_t)B * tiled_elems(N, K) * 2;
    if (d0 < s0 + sb && s0 < d0 + db) return fail(DBF_EINVAL, "dst overlaps src");
    (void)hipGetLastError();
    launch_tile((const uint16_t *)src->data, (uint16_t *)dst, B, (int)N, (int)K, (hipStream_t)stream);
    return hip_check("dbf_tile_weight launch");
}

int kv_rollback(dbf_kv_cache *cache, int32_t n) {
    g_err.clear();
    if (!cache) return fail(DBF_EINVAL, "cache is null");
    if (n < 0 || (int64_t)n > cache->seq_len)
        return fail(DBF_ERANGE, "rollback of %d rows from seq_len %lld", n, (long long)cache->seq_len);
    cache->seq_len -= n;
    return DBF_OK;
}

}  // extern "C"
