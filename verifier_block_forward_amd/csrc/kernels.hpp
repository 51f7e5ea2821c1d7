// kernels.hpp -- host-side launch interface of the libdbf kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dbf {

// ---------------------------------------------------------------------------
// Skinny projection Y[m, o] = sum_k X[m, k] W[o, k] for up to 32 activation rows
// (two split tiles), BF16 W [N, K] row-major, split-K partial sums in F32:
// out[ks][16*nb][N] (row m of tile b at 16*b + m). Consumers add the ks partials
// in increasing ks order.
// ---------------------------------------------------------------------------
constexpr int GEMM_MAXSEG = 8;

struct GemmSeg {
    const uint16_t *W;
    float *out;
    const uint16_t *xs0;  // split tile 0
    const uint16_t *xs1;  // split tile 1 (nb == 2)
    int N, K, nb, ksplit, kslice_steps, tiles, unit_begin, pad_;
};

struct GemmArgs {
    GemmSeg seg[GEMM_MAXSEG];
    int nseg;
    int total_units;
};

// Work decomposition of one segment: rows per wave unit = 16 * na.
struct GemmPlan {
    int tiles, ksplit, kslice_steps;
};
GemmPlan gemm_plan(int N, int K, int na, int target_units);

void launch_gemm(const GemmArgs &a, int na, int nbmax, hipStream_t s);

// ---------------------------------------------------------------------------
// lm_head: logits = h W^T over V rows, with per-unit top-2 records for the
// argmax, then a per-row reduction.
// ---------------------------------------------------------------------------
constexpr int HEAD_NA = 4;  // 64 vocabulary rows per wave unit
int head_units(int V);
void launch_head(const uint16_t *W, const uint16_t *xs, int V, int K, int M, float *logits,
                 float4 *part, hipStream_t s);
void launch_head_reduce(const float4 *part, int units, int M, int32_t *argmax, float *margin,
                        hipStream_t s);

// ---------------------------------------------------------------------------
// row kernels (elementwise / norms / splits)
// ---------------------------------------------------------------------------
void launch_split_rows(const float *X, int rows, int K, int ldx, uint16_t *tile, hipStream_t s);

void launch_input_dflash(const int32_t *tokens, const float *x0, const uint16_t *embed, int V,
                         int M, int H, const float *norm_w, float eps, float *xres,
                         uint16_t *xs, hipStream_t s);

void launch_mtp_input(const float *e, const float *hp, int M, int H, const float *enorm,
                      const float *hnorm, uint16_t *xs_e, uint16_t *xs_h, hipStream_t s);

// out = base + sum_{set} sum_{ks} P_set[ks][prow0_set + m][:]; optional copies;
// norm_out = RMSNorm(out, w); split into xs (tile rows 0..15, zero for m >= M).
struct SumNormArgs {
    const float *base;     // [M][H] or null
    const float *p0;       // partial set 0: [ks0][rows0][H]
    int ks0, rows0;
    const float *p1;       // partial set 1 or null
    int ks1, rows1;
    float *out;            // [M][H] (may alias base)
    float *copy0, *copy1;  // optional extra copies of out
    const float *w;        // norm weight [H]
    float eps;
    float *normed;         // optional f32 normed rows [M][H]
    uint16_t *xs;          // split tile (K = H), required
    int M, H;
};
void launch_sum_norm_split(const SumNormArgs &a, hipStream_t s);

void launch_hctx(const float *p, int ks, int R, int H, const float *w, float eps, uint16_t *xs,
                 hipStream_t s);

struct QkvPostArgs {
    const float *pq;   // [ksq][16][qt]
    const float *pk;   // [ksk][rows_kv][kt]
    const float *pv;   // [ksv][rows_kv][kt]
    const float *pg;   // [ksg][16][qt] or null
    int ksq, ksk, ksv, ksg, rows_kv, kv_block_row0;
    const float *q_norm, *k_norm;
    float eps;
    double theta;
    int rotary_dim;
    int M, R, nq, nkv, hd;
    long long P0;
    float *q_out;      // [M][qt]
    float *g_out;      // [M][qt] or null
    void *cache_k, *cache_v;  // this layer's [nkv][cap][hd]
    int kv_bf16;
    long long capacity;
};
void launch_qkv_post(const QkvPostArgs &a, hipStream_t s);

struct AttnArgs {
    const float *q;        // [M][nq*hd], normed + rotated
    const void *cache_k, *cache_v;  // this layer's [nkv][cap][hd]
    int kv_bf16;
    long long capacity;
    long long n_ctx;       // keys visible to block row 0 minus one: P0 + R
    int M, nq, nkv, hd;
    int chunk, n_chunks;
    float *part;           // [n_chunks][M*nq][hd + 2]
};
void attn_plan(long long n_keys, int *chunk, int *n_chunks);
bool attn_supported(int hd);
void launch_attn(const AttnArgs &a, hipStream_t s);

struct CombineArgs {
    const float *part;
    int n_chunks, M, nq, hd;
    const float *g;        // [M][nq*hd] raw gate or null
    uint16_t *xs;          // split tile (K = nq*hd)
};
void launch_attn_combine(const CombineArgs &a, hipStream_t s);

void launch_swiglu_split(const float *pg, int ksg, const float *pu, int ksu, int M, int I,
                         uint16_t *xs, hipStream_t s);

void launch_accept(const int32_t *drafts, const int32_t *target, int K, const int32_t *eos,
                   int n_eos, int32_t *result, int32_t *committed, hipStream_t s);

}  // namespace dbf
