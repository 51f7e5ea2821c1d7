/*
 * dbf.h -- C ABI of the MI355X (gfx950) drafter block forward library (libdbf.so).
 *
 * The library runs the speculative-decoding drafter hot path in hand-written HIP
 * kernels: the drafter block forward over M = K+1 token rows, the lm_head with a
 * per-row argmax, the greedy accept-prefix walk, and KV-cache rollback.
 *
 * Sources (hf2q 0.1.1 source pages on docs.rs):
 *   [MTP]  src/inference/models/qwen35/mtp.rs
 *   [TENS] src/inference/spec_decode/dflash/tensors.rs
 *   [ORCH] src/inference/spec_decode/dflash/qwen35_orchestrator.rs
 *
 * Conventions
 *   - Every pointer named "device" is HIP device memory (or memory the device can
 *     read); the caller allocates and owns every buffer. The library allocates no
 *     device memory and keeps no pointer after a call returns; buffers must stay
 *     alive until the stream has executed the enqueued work.
 *   - `stream` is a hipStream_t passed as void*. Entry points enqueue on it and
 *     never synchronize, so a caller may capture them into a HIP graph.
 *   - All arguments are validated on the host before anything is enqueued: on an
 *     error nothing runs and the KV cache (including seq_len) is unchanged. The
 *     return value is 0 or a negative DBF_E* code; dbf_last_error() describes it.
 *   - Tensors are row-major and contiguous. Projection weights are BF16 [out, in]
 *     with no transpose ([TENS] module doc and `DFlashLayerTensors`); every RMSNorm
 *     weight is F32 ([TENS] `DFlashLayerTensors`, "DType policy": a BF16 buffer
 *     read by an F32 norm kernel silently corrupts and reads out of bounds, so a
 *     norm weight of any other dtype is rejected with DBF_EDTYPE).
 *   - Inner (input) dimensions of every projection must be multiples of 8 (the
 *     kernels stream weights in 16-byte vectors); DBF_ESHAPE otherwise.
 *   - Every projection weight (and lm_head, embed excepted) may instead be given in
 *     the tiled layout DBF_BF16_T16 produced once at upload time by
 *     dbf_tile_weight: same logical shape, stored in the order the gfx950 matrix
 *     cores consume it, which streams ~1.35x faster than row-major. Layouts may be
 *     mixed freely across tensors.
 */
#ifndef DBF_H
#define DBF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DBF_ABI_VERSION 4

/* status codes */
#define DBF_OK 0
#define DBF_EINVAL -1    /* null pointer, or a count outside its range (M, R, K, ...) */
#define DBF_ESHAPE -2    /* a tensor's ndim/shape disagrees with the config */
#define DBF_EDTYPE -3    /* a tensor or cache has the wrong dtype */
#define DBF_ERANGE -4    /* KV capacity exceeded, or a rollback larger than seq_len */
#define DBF_EWORKSPACE -5 /* workspace missing, too small or not 256-byte aligned */
#define DBF_EHIP -6      /* a HIP runtime call failed (message in dbf_last_error) */

/* dtypes */
#define DBF_F32 0
#define DBF_BF16 1
#define DBF_I32 2
#define DBF_BF16_T16 3 /* BF16 weight tiled for the matrix cores (dbf_tile_weight) */

/* block kinds */
#define DBF_KIND_DFLASH 0 /* DFlash drafter ([TENS] `DFlashModelTensors`) */
#define DBF_KIND_MTP 1    /* Qwen3.5 MTP block ([MTP] `MtpWeights`) */

/* FFN kinds ([MTP] `MtpFfnWeightsGpu`) */
#define DBF_FFN_DENSE 0
#define DBF_FFN_MOE 1

/* block attention masks */
#define DBF_MASK_CAUSAL 0 /* block row i sees block rows <= i (causal within the block; the default) */
#define DBF_MASK_BIDIR 1  /* every block row sees all M block rows (block-diffusion reading) */

#define DBF_MAX_M 16   /* block rows per call (K+1 <= 16) */
#define DBF_MAX_CTX_LAYERS 8 /* captured target layers gathered on the device */
#define DBF_MAX_R 16   /* new context rows per call */
#define DBF_MAX_TOPK 16
#define DBF_MAX_SAMPLE_ROWS 1024  /* rows per sample_tokens call */
#define DBF_MAX_VOCAB (1 << 24)   /* logits per row for the sampling calls */

/* Non-owning view of a device tensor: row-major, contiguous. */
typedef struct {
    void *data;
    int32_t dtype; /* DBF_F32 | DBF_BF16 | DBF_I32 */
    int32_t ndim;
    int64_t shape[4];
} dbf_tensor;

/* Model shape. ([MTP] `Qwen35Config` fields used by `forward_full_attention`;
 * [TENS] `DFlashLayerTensors` shapes.) */
typedef struct {
    int32_t kind;            /* DBF_KIND_DFLASH | DBF_KIND_MTP */
    int32_t n_layers;        /* decoder layers in the block (>= 1) */
    int32_t hidden;          /* H */
    int32_t n_q_heads;       /* nq */
    int32_t n_kv_heads;      /* nkv, divides nq (GQA groups are contiguous) */
    int32_t head_dim;        /* hd, even, <= 256 */
    int32_t rotary_dim;      /* rotated lanes per head, even, <= hd; 0 means hd */
    int32_t intermediate;    /* dense SwiGLU width I */
    int32_t n_target_hidden; /* DFlash: target hidden states concatenated into fc */
    int32_t vocab;           /* V (embedding rows for the token gather) */
    int32_t ffn_kind;        /* DBF_FFN_DENSE | DBF_FFN_MOE */
    int32_t n_experts;       /* MoE: E */
    int32_t top_k;           /* MoE: experts kept per row, <= min(E, DBF_MAX_TOPK) */
    int32_t expert_intermediate; /* MoE: per-expert SwiGLU width */
    int32_t shared_intermediate; /* MoE: shared-expert SwiGLU width */
    int32_t has_attn_gate;   /* 1: o *= sigmoid(x Wg^T) before O ([MTP] `w_gate`) */
    int32_t block_mask;      /* DBF_MASK_CAUSAL (default) | DBF_MASK_BIDIR */
    int32_t reserved_;       /* zero */
    double rms_eps;          /* RMSNorm eps of every norm except MTP enorm/hnorm (fixed 1e-6) */
    double rope_theta;       /* RoPE base */
} dbf_config;

/* Per-layer weights. Unused members (by kind/ffn_kind/has_attn_gate) are ignored
 * and may be zero. Shapes: in_norm, post_norm [H] F32; wq [nq*hd, H];
 * wk, wv [nkv*hd, H]; attn_gate [nq*hd, H]; wo [H, nq*hd]; q_norm, k_norm [hd] F32;
 * dense: ffn_gate, ffn_up [I, H], ffn_down [H, I];
 * MoE: router [E, H], exp_gate, exp_up [E, Ie, H], exp_down [E, H, Ie],
 *      sh_gate, sh_up [Is, H], sh_down [H, Is], sh_gate_inp [1, H].
 * All projections BF16. */
typedef struct {
    dbf_tensor in_norm, post_norm;
    dbf_tensor wq, wk, wv, attn_gate, wo;
    dbf_tensor q_norm, k_norm;
    dbf_tensor ffn_gate, ffn_up, ffn_down;
    dbf_tensor router, exp_gate, exp_up, exp_down;
    dbf_tensor sh_gate, sh_up, sh_down, sh_gate_inp;
} dbf_layer_weights;

/* Block weights. DFlash: fc [H, n_t*H] BF16, hidden_norm [H] F32.
 * MTP: enorm, hnorm [H] F32, eh_embed, eh_hidden [H, H] BF16.
 * final_norm [H] F32 (DFlash `norm`; MTP `shared_head_norm`).
 * embed [V, H] BF16: only read when block tokens are given (shared with the
 * target, [TENS] module doc). `layers` is a HOST array of n_layers entries. */
typedef struct {
    dbf_tensor fc, hidden_norm;
    dbf_tensor enorm, hnorm, eh_embed, eh_hidden;
    const dbf_layer_weights *layers;
    dbf_tensor final_norm;
    dbf_tensor embed;
} dbf_weights;

/* KV cache, caller-owned: k and v are device arrays [n_layers][n_kv_heads]
 * [capacity][head_dim] of dtype F32 or BF16. Row p of a head holds the key/value
 * of position p. seq_len (host metadata) is the number of valid positions. */
typedef struct {
    void *k;
    void *v;
    int32_t dtype;
    int32_t n_layers, n_kv_heads, head_dim;
    int64_t capacity;
    int64_t seq_len;
} dbf_kv_cache;

/* Block inputs/outputs (device pointers).
 *   tokens      [M] int32 or NULL. Rows are embed[tokens[i]]: DFlash block
 *               rows ([ORCH] per-round steps 1-2: [last_token, mask x K]); MTP
 *               embed_t, the embedding of the token a chained step drafts from
 *               (the previous step's argmax, read on the device). Ids are
 *               clamped into [0, V).
 *   x0          [M, H] F32 block rows when tokens == NULL (MTP: embed_t).
 *   ctx         DFlash: [R, n_t*H] F32 concatenated target hidden states of the R
 *               new context rows (may be NULL when R == 0, or when ctx_layers is
 *               given). MTP: prev_hidden [M, H] F32 (required).
 *   ctx_layers  DFlash, optional: HOST array of n_t device pointers, the target's
 *               captured hidden rows of each drafter target layer, [*, ctx_ld] F32
 *               indexed by position. The R context rows are gathered on the
 *               device: row r = concat_t ctx_layers[t][(ctx_row0 + r) * ctx_ld ..
 *               + H) ([ORCH] per-round step 3, `extract_drafter_concat`, new rows
 *               only, without its host copy). With buffers indexed by position,
 *               accepted verify positions need no append: the next round gathers
 *               them where the target wrote them. n_t <= DBF_MAX_CTX_LAYERS.
 *   ctx_ld      row stride of every ctx_layers buffer, elements (>= H).
 *   ctx_row0    position of the first new context row in ctx_layers.
 *   M           block rows, 1..DBF_MAX_M.  R: new context rows, 0..DBF_MAX_R
 *               (MTP: must be 0).
 *   hidden_out  [M, H] F32 pre-norm hidden of the last layer, or NULL.
 *   h_final     [M, H] F32 final-normed hidden (required).
 *   layer_hidden [n_layers, M, H] F32 hidden after each layer, or NULL.
 *   moe_experts [n_layers] int32 out, or NULL (MoE FFN only): the number of
 *               distinct experts the layer's M rows were routed to, i.e. the
 *               experts whose weights the layer read ([MTP] `MtpFfnWeightsGpu::Moe`).
 * Optional fused shared head and accept walk, in the same call ([MTP]
 * `forward_shared_head`: the final norm, lm_head and argmax submitted together;
 * [ORCH] per-round steps 5-8). All NULL (and n_eos 0) when not wanted.
 *   lm_head     BF16 or BF16_T16 [V, H] with V = cfg.vocab, or NULL. When given,
 *               the call also computes the lm_head argmax of the M normed rows (the
 *               final RMSNorm is folded into the head's staging, h_final is still
 *               written, with the same bits as without the head) and writes
 *   argmax      [M] int32 (required with lm_head) and
 *   top2_margin [M] F32 or NULL, as lm_head_argmax would.
 *   target      [K+1] int32 or NULL (needs lm_head): the target's argmax at each
 *               drafted position; the greedy accept walk of the block's drafts then
 *               runs as accept_prefix would, with drafts = argmax rows 1..M-1 and
 *               K = M - 1 for DFlash, argmax row 0 and K = 1 for MTP ([ORCH]
 *               per-round step 5; reading of the MTP M > 1 workload: row 0 drafts).
 *   eos, n_eos  EOS ids (n_eos in 0..1024; eos may be NULL when n_eos is 0).
 *   accept_result [5] int32 out (required with target), committed [K+1] out or NULL. */
typedef struct {
    const int32_t *tokens;
    const float *x0;
    const float *ctx;
    int32_t M, R;
    float *hidden_out;
    float *h_final;
    float *layer_hidden;
    const float *const *ctx_layers;
    int64_t ctx_ld;
    int64_t ctx_row0;
    int32_t *moe_experts;
    const dbf_tensor *lm_head;
    int32_t *argmax;
    float *top2_margin;
    const int32_t *target;
    const int32_t *eos;
    int32_t n_eos;
    int32_t *accept_result;
    int32_t *committed;
} dbf_block_io;

/* Drafter block forward ([MTP] `forward_draft_with_hidden` and its helpers
 * `project_embedding_and_hidden`, `forward_full_attention`,
 * `forward_ffn_residual`, `forward_shared_head` up to the norm; [TENS]
 * `DFlashModelTensors` for the DFlash input projection and per-layer tensors;
 * [ORCH] per-round step 4 for the block call with new context rows).
 *
 * Input: DFlash x = embed[tokens] (or x0), h_ctx = RMSNorm(ctx fc^T, hidden_norm);
 * MTP x = RMSNorm(x0, enorm) eh_embed^T + RMSNorm(ctx, hnorm) eh_hidden^T.
 * Each layer: RMSNorm, Q/K/V (+gate) projections, per-head RMSNorm of q and k,
 * RoPE, K/V stored in the cache, GQA attention (q head h uses kv head
 * h*nkv/nq) over cache rows [0, P0+R+i] for block row i (causal within the
 * block; with cfg.block_mask == DBF_MASK_BIDIR over [0, P0+R+M), every block
 * row), optional sigmoid gate, O projection + residual, RMSNorm, SwiGLU or
 * MoE FFN + residual. Then h_final = RMSNorm(x, final_norm).
 * DFlash context rows go through each layer's wk/wv, k_norm and RoPE (no input
 * norm) and are stored at positions P0..P0+R-1; block rows at P0+R+i, where P0 =
 * cache->seq_len on entry. On success cache->seq_len += R + M (a DFlash drafter
 * that keeps only context rows calls kv_rollback(cache, M) afterwards).
 *
 * ws: device workspace of at least draft_block_workspace_bytes(cfg, M, R) bytes,
 * 256-byte aligned, contents irrelevant on entry. Calls sharing a workspace must
 * be ordered on one stream. */
int draft_block_forward(const dbf_config *cfg, const dbf_weights *w, dbf_kv_cache *cache,
                        const dbf_block_io *io, void *ws, size_t ws_bytes, void *stream);

size_t draft_block_workspace_bytes(const dbf_config *cfg, int32_t M, int32_t R);

/* lm_head + per-row argmax ([ORCH] per-round step 5, per-position argmax over the
 * drafter's normed hidden through the target lm_head; [MTP] `forward_shared_head`).
 *   h          [M, H] F32 device, already normed; M in 1..DBF_MAX_M.
 *   lm_head    BF16 [V, H].
 *   argmax     [M] int32 device out: index of the largest logit of each row, the
 *              lowest index among equal maxima.
 *   logits     [M, V] F32 device out, or NULL (written only on request).
 *   top2_margin [M] F32 device out, or NULL: largest logit minus the largest
 *              logit at any other index (0 on a tie).
 * Non-finite logits give an unspecified argmax.
 * ws: at least lm_head_argmax_workspace_bytes(M, H, V) bytes, 256-byte aligned. */
int lm_head_argmax(const float *h, int32_t M, int32_t H, const dbf_tensor *lm_head,
                   int32_t *argmax, float *logits, float *top2_margin, void *ws,
                   size_t ws_bytes, void *stream);

size_t lm_head_argmax_workspace_bytes(int32_t M, int32_t H, int32_t V);

/* lm_head_argmax without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments, results and errors as lm_head_argmax, whose
 * kernels it runs; the records between its two kernels live in a static device
 * array of DBF_NOALLOC_SCRATCH_BYTES bytes that the library holds on each device it
 * runs on until the process ends. The call allocates nothing.
 *   V must be <= DBF_NOALLOC_MAX_VOCAB: a larger vocabulary is refused with
 *   DBF_ERANGE before anything is enqueued.
 *   Every call on one device shares that device's array: calls that may overlap on
 *   one device (different streams, different threads) race and must be ordered by
 *   the caller. Each call writes every record it reads, so nothing has to be cleared
 *   between calls. The first call on a device looks the array's address up
 *   (hipGetSymbolAddress) with that device current. */
#define DBF_NOALLOC_MAX_VOCAB (1 << 20)
#define DBF_NOALLOC_SCRATCH_BYTES 262144 /* = lm_head_argmax_workspace_bytes(16, H, DBF_NOALLOC_MAX_VOCAB) */
int lm_head_argmax_noalloc(const float *h, int32_t M, int32_t H, const dbf_tensor *lm_head,
                           int32_t *argmax, float *logits, float *top2_margin, void *stream);

/* Greedy accept-prefix walk ([ORCH] module doc, "Greedy accept-walk consistency
 * invariant", and per-round steps 7-8). Device pointers:
 *   drafts [K] int32, target [K+1] int32 (the target's argmax at each position),
 *   eos [n_eos] int32 or NULL when n_eos == 0.
 *   result [5] int32 out: {accept_count a, free_token = target[a],
 *          rollback = K - a, hit_eos, n_committed}.
 *   committed [K+1] int32 out or NULL: target[0..a] (the accepted drafts then the
 *          free token), cut after the first EOS (inclusive; hit_eos = 1 then); the
 *          first n_committed entries are written, the rest are left as they were.
 * a is the length of the longest prefix with drafts[i] == target[i]; EOS does not
 * change a or rollback. K in 1..1024. One wavefront; enqueued only. */
int accept_prefix(const int32_t *drafts, const int32_t *target, int32_t K, const int32_t *eos,
                  int32_t n_eos, int32_t *result, int32_t *committed, void *stream);

/* KV rollback ([ORCH] per-round step 8: drop the rejected positions). Host-side
 * metadata only: cache->seq_len -= n. DBF_ERANGE when n < 0 or n > seq_len. */
int kv_rollback(dbf_kv_cache *cache, int32_t n);

/* One draw per row from softmax(logits[m] / T) by inverse CDF (the drafter's
 * sampled draft for the stochastic MTP K = 1 round named in the [ORCH] module
 * doc, "Non-greedy (Metropolis-Hastings)"; its rule is not on the pages, see
 * accept_sampled). Device pointers:
 *   logits [M][V] F32 (e.g. lm_head_argmax's logits), u [M] F32 uniforms in [0, 1)
 *   supplied by the caller (the library draws no random numbers);
 *   token [M] int32 out: the smallest index whose running sum of probability, in
 *   index order, exceeds u[m] (the last index of nonzero probability where
 *   rounding leaves u[m] at the end);
 *   prob [M] F32 out or NULL: the drawn token's probability.
 * M in 1..DBF_MAX_SAMPLE_ROWS, V in 1..DBF_MAX_VOCAB, temperature in [1e-3, 1e3].
 * Probabilities are formed in F32 (sums over fixed trees, so a draw is
 * reproducible); a u within rounding of a cumulative boundary may land on either
 * side of it. Non-finite logits give an unspecified token in [0, V).
 * ws: at least sample_tokens_workspace_bytes(M, V) bytes, 256-byte aligned.
 * Enqueued only (two kernels). */
int sample_tokens(const float *logits, int32_t M, int32_t V, float temperature, const float *u,
                  int32_t *token, float *prob, void *ws, size_t ws_bytes, void *stream);

size_t sample_tokens_workspace_bytes(int32_t M, int32_t V);

/* Sampled acceptance of one drafted token, MTP K = 1 ([ORCH] module doc,
 * "Non-greedy (Metropolis-Hastings)": stochastic acceptance is named for this path
 * without its rule; the rule taken is standard speculative sampling, under which
 * the emitted token is distributed exactly as the target's softmax):
 *   q = softmax(draft_logits / T), p0 = softmax(target_logits[0] / T),
 *   p1 = softmax(target_logits[1] / T);
 *   accepted iff u[0] * q(d) < p0(d), i.e. with probability min(1, p0(d)/q(d));
 *   accepted: free token drawn from p1 with u[1] (the bonus token);
 *   rejected: free token drawn from max(0, p0 - q), normalised, with u[1] (from p0
 *   when that residual is empty).
 * Draws are by inverse CDF as in sample_tokens. Device pointers:
 *   draft_logits [V] F32 (the drafter's logits at the drafted position);
 *   target_logits [2][V] F32 (the target's logits at the draft's position and the
 *   next); draft [1] int32 (d, e.g. from sample_tokens); u [2] F32 uniforms;
 *   eos [n_eos] int32 or NULL when n_eos == 0 (n_eos <= 1024);
 *   result [5] int32 out: {accept_count a (0 or 1), free_token, rollback = 1 - a,
 *          hit_eos, n_committed}, as accept_prefix;
 *   committed [2] int32 out or NULL: [d, free_token] when accepted, [free_token]
 *          otherwise, cut after the first EOS (inclusive).
 * A draft outside [0, V) is not read: result = {-1, -1, -1, 0, 0}.
 * V in 1..DBF_MAX_VOCAB, temperature in [1e-3, 1e3]; the acceptance test and the
 * draws are formed in F32 (a u within rounding of a boundary may go either way).
 * ws: at least accept_sampled_workspace_bytes(V) bytes, 256-byte aligned.
 * Enqueued only (three kernels); no host synchronisation. */
int accept_sampled(const float *draft_logits, const float *target_logits, int32_t V, float temperature,
                   const int32_t *draft, const float *u, const int32_t *eos, int32_t n_eos,
                   int32_t *result, int32_t *committed, void *ws, size_t ws_bytes, void *stream);

size_t accept_sampled_workspace_bytes(int32_t V);

/* Tiled weight layout. For a row-major BF16 weight [N, K] (or a batch [B, N, K] of
 * them, e.g. MoE experts), the tiled copy holds ceil(N/16) x ceil(K/32) blocks of
 * 1 KiB; element (n, k) sits at BF16 offset
 *   ((n/16 * ceil(K/32) + k/32) * 64 + ((k % 32) / 8) * 16 + n % 16) * 8 + k % 8
 * and padding rows/columns are zero. Matrices of a batch follow one another.
 * dbf_tiled_bytes: bytes of one tiled [N, K] matrix.
 * dbf_tile_weight: enqueue the repack of src (BF16, ndim 2 or 3, device) into dst
 * (device, batch * dbf_tiled_bytes bytes, caller-owned; must not overlap src).
 * Pass the result as a dbf_tensor {dst, DBF_BF16_T16, same ndim and shape}. */
size_t dbf_tiled_bytes(int64_t N, int64_t K);
int dbf_tile_weight(const dbf_tensor *src, void *dst, void *stream);

/* Kernel timing, for measurement only ([MTP] `forward_draft_with_hidden`: the
 * per-sub-step profile the page takes with HF2Q_MTP_PROFILE). While profiling is
 * on, every kernel the library launches, from any thread, carries a pair of HIP
 * events bound to its dispatch (hipExtLaunchKernel), so its recorded duration is
 * the kernel's own execution, without host or marker overhead. Calls made while
 * profiling is on must not be captured into a HIP graph.
 *   dbf_profile_start(max_records): clear the record list and time the next
 *     max_records launches (1..DBF_PROF_MAX_RECORDS); later launches run untimed.
 *   dbf_profile_stop(out, max_out, n_out): stop, wait for the timed kernels to
 *     finish, copy up to max_out records (host array) in launch order and set
 *     *n_out to the number of timed launches. */
#define DBF_PROF_MAX_RECORDS 65536
#define DBF_PROF_PROJ 0   /* skinny projections: fc/eh, Q/K/V/gate, O, FFN, router, experts */
#define DBF_PROF_ATTN 1   /* attention over the KV cache and its chunk combine */
#define DBF_PROF_ROWS 2   /* row kernels: residual sums, norms, RoPE + KV append, SwiGLU, MoE routing */
#define DBF_PROF_HEAD 3   /* lm_head and its argmax reduction */
#define DBF_PROF_ACCEPT 4 /* greedy accept walk */
#define DBF_PROF_SAMPLE 5 /* sampling and sampled acceptance */
#define DBF_PROF_OTHER 6  /* weight tiling */
typedef struct {
    int32_t cls;        /* DBF_PROF_* */
    int32_t reserved_;
    const char *kernel; /* static name of the kernel */
    double us;          /* execution time, microseconds */
} dbf_prof_record;

int dbf_profile_start(int32_t max_records);
int dbf_profile_stop(dbf_prof_record *out, int32_t max_out, int32_t *n_out);

/* Description of the last error on the calling thread ("" when none). */
const char *dbf_last_error(void);

int dbf_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DBF_H */
