// kernels.hpp -- host-side launch interface of the libdbf kernels (internal).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dbf {

// ---------------------------------------------------------------------------
// Launches. Every kernel goes through launch_k, which times it when profiling is
// on (prof.hip): the start/stop events are then bound to the dispatch.
// ---------------------------------------------------------------------------
enum ProfClass { PROF_PROJ = 0, PROF_ATTN = 1, PROF_ROWS = 2, PROF_HEAD = 3, PROF_ACCEPT = 4,
                 PROF_SAMPLE = 5, PROF_OTHER = 6 };
bool prof_take(int cls, const char *name, hipEvent_t *e0, hipEvent_t *e1);

template <typename... KArgs, typename... Args>
inline void launch_k(int cls, const char *name, void (*k)(KArgs...), dim3 grid, dim3 block,
                     size_t shmem, hipStream_t s, Args... args) {
    hipEvent_t e0, e1;
    if (prof_take(cls, name, &e0, &e1))
        hipExtLaunchKernelGGL(k, grid, block, (uint32_t)shmem, s, e0, e1, 0u, args...);
    else
        hipLaunchKernelGGL(k, grid, block, shmem, s, args...);
}

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
    int N, K, nb, ksplit, kslice_steps, tiles, unit_begin, tiled;  // tiled: DBF_BF16_T16 layout
    // grouped (MoE) segments: `slots` independent matrices W + slot_expert[s] * w_stride,
    // each with its own split tile xs0 + s * xs_stride and output out + s * out_stride;
    // slots >= *nslots (known only on the device) exit at once. slots == 0: plain.
    const int32_t *slot_expert;
    const int32_t *nslots;
    long long w_stride, xs_stride, out_stride;
    int slots;
    // activation rows that hold data in xs0 / xs1: partial rows at or past them are
    // not written (consumers read rows below them only)
    int mrows[2];
    int pad_;
};

// F32 activation rows read by an LDS-staged launch in place of a split tile, split
// hi/lo as they are staged: row m, column k is xf[m * xf_ld + k], or, with xf
// null (the captured target layers gathered), xg[k / xg_cols][(xg_row0 + m) *
// xg_ld + k % xg_cols]. xg_cols is a multiple of 8, so a lane's 8-column run lies
// in one source.
// With tokens set, row m is instead the BF16 row embed[clamp(tokens[m], 0, V-1)]
// (xf_ld columns). With w set, column k is multiplied by w[k] after it is read.
// With ssq set, the workgroups of the segment's first row-tile group write, for
// each row m and k-slice ks, the sum of squares of the row's values over the slice
// (before w) to ssq[m * ssq_ld + ks].
struct GemmF32Src {
    const float *xf;
    long long xf_ld;
    const float *xg[8];
    long long xg_ld;
    int xg_cols, xg_row0;
    const int32_t *tokens;
    const uint16_t *embed;
    int V;
    const float *w;
    float *ssq;
    int ssq_ld;
};

struct GemmArgs {
    GemmSeg seg[GEMM_MAXSEG];
    int nseg;
    int total_units;  // wave units (lds_x = 0) or workgroup units (lds_x = 1)
    int lds_x;        // 1: k_gemm_lds (activation slice staged in LDS)
    int xf_on;        // 1: the plain LDS-staged segments read xf[segment], not xs0
    GemmF32Src xf[2];
};

// Work decomposition of one segment: rows per wave unit = 16 * GEMM_NA; lds selects
// the kernel with the activation slice staged in LDS (units are then workgroups of
// four row tiles). Segments of one launch share lds.
// Row tiles (16 weight rows each) per wave in every projection launch: two measured
// best in both the split-K and the LDS-staged kernels (four, with twice the bytes
// in flight per wave, were slower in each).
constexpr int GEMM_NA = 2;
struct GemmPlan {
    int tiles, ksplit, kslice_steps, lds;
};
// target_units: wave units (tiles x ksplit) to aim for; max_steps > 0 caps the
// k-slice length (steps of 32 columns)
GemmPlan gemm_plan(int N, int K, int target_units, int max_steps = 0);
constexpr int LDS_X_STEPS_NB1 = 20;  // 40 KiB of split activations per workgroup
constexpr int LDS_X_STEPS_NB2 = 10;
// LDS-staged plan for a launch whose segments have up to nbmax split tiles
GemmPlan gemm_plan_lds(int N, int K, int target_units, int nbmax);
// units (waves, or workgroups for lds plans) of one matrix of the segment
inline int plan_units(const GemmPlan &p) {
    return p.lds ? ((p.tiles + 3) / 4) * p.ksplit : p.tiles * p.ksplit;
}

// false (nothing launched) for a split-K launch with two split tiles per segment,
// or F32 activation sources on anything but one or two plain LDS-staged segments
bool launch_gemm(const GemmArgs &a, int nbmax, hipStream_t s);

// ---------------------------------------------------------------------------
// Whole-K projection with the residual epilogue: one workgroup owns 16 or 32 output
// columns and all of K, its waves split K and reduce through LDS in a fixed order,
// so the workgroup holds complete outputs and finishes the row work itself:
//   out = base + X W^T (the residual add); xs_out <- split(out (.) w) for the next
//   projection; ssp_out[m][n / 16] <- sum of out^2 over each 16-column block (the
//   row-scale partials of the next RMSNorm); copies of out on request.
// xs_out is a split tile of K = N (padding columns and rows >= M written as zeros).
// ---------------------------------------------------------------------------
struct FullArgs {
    const uint16_t *W;       // [N, K]
    int tiled;               // DBF_BF16_T16 layout
    const uint16_t *xs;      // split tile of the input, K columns, 16 rows
    int N, K, M;
    const float *base;       // [M][N] rows added to the product, or null
    float *out, *copy0, *copy1;  // [M][N] (copies optional)
    const float *w;          // norm weight [N] applied before the split, or null (1)
    float *ssp_out;          // [16][ceil(N/16)], or null
    uint16_t *xs_out;        // split tile, K = N
};
constexpr int FULL_SSP_COLS = 16;  // columns per sum-of-squares partial
void launch_gemm_full(const FullArgs &a, hipStream_t s);

// ---------------------------------------------------------------------------
// lm_head: logits = h W^T over V rows, with per-workgroup top-2 records for the
// argmax, then a per-row reduction.
// ---------------------------------------------------------------------------
constexpr int HEAD_NA = 8;  // 16*HEAD_NA vocabulary rows per wave unit
int head_units(int V);
int head_blocks(int V);  // workgroups of the head launch (8 wave units each)
// Final RMSNorm folded into the head's staging: h then holds the pre-norm rows x,
// the head forms x * s_m * w (s_m from the rows' sum-of-squares partials ssp
// [16][ncb]) and workgroup 0 writes those rows to h_out.
struct HeadNorm {
    const float *w;    // final norm weight [K]
    const float *ssp;  // [16][ncb]
    int ncb;
    float eps;
    float *h_out;      // [M][K]
};
// h: F32 [M][K] hidden rows (normed, or pre-norm with nrm); part: [16][head_blocks(V)]
// top-2 records
void launch_head(const uint16_t *W, int tiled, const float *h, int V, int K, int M,
                 float *logits, float4 *part, const HeadNorm *nrm, hipStream_t s);
// greedy accept walk after the argmax reduction (k_head_finish)
struct AcceptArgs {
    const int32_t *target;  // [K+1], or null: no walk
    int K, first;           // drafts are the argmaxes of rows first .. first+K-1
    const int32_t *eos;
    int n_eos;
    int32_t *result;        // [5]
    int32_t *committed;     // [K+1] or null
};
void launch_head_finish(const float4 *part, int blocks, int M, int32_t *argmax, float *margin,
                        const AcceptArgs &acc, hipStream_t s);

// weight tiling (MFMA operand order, see gemm.hip)
size_t tiled_elems(long long N, long long K);
void launch_tile(const uint16_t *src, uint16_t *dst, long long batch, int N, int K, hipStream_t s);
void launch_head_reduce(const float4 *part, int blocks, int M, int32_t *argmax, float *margin,
                        hipStream_t s);

// ---------------------------------------------------------------------------
// row kernels (column-parallel; see rows.hip for the split-RMSNorm convention)
// ---------------------------------------------------------------------------
struct ColArgs {
    int M, H;                 // valid rows, columns
    const int32_t *tokens;    // gather embed[tokens[m]] (BF16) as the base, or null
    const uint16_t *embed;
    int V;
    const float *base;        // [M][ldb] base rows, or null
    int ldb;
    const float *p0;          // split-K partials [ks0][rows0][H], or null
    int ks0, rows0;
    const float *ssp0;        // row-scale source for set 0 ([16][ncb_in]) or null (scale 1)
    float eps0;
    const float *p1;
    int ks1, rows1;
    const float *ssp1;
    float eps1;
    int ncb_in;
    float *out, *copy0, *copy1;  // [M][H] copies of the summed rows, each optional
    const float *w;           // multiply before the split (norm weight) or null
    uint16_t *xs;             // split tile (K = H) or null
    float *ssp_out;           // [16][ncb_out] partial sums of squares, or null
    int ncb_out;
};
void launch_colsum(const ColArgs &a, hipStream_t s);
void launch_colsum2(const ColArgs &a0, const ColArgs &a1, hipStream_t s);  // independent jobs
// ssp: [16][ncb] row-scale partials of x (ncb per row: 64- or 16-column partials)
void launch_final_norm(const float *x, const float *ssp, int ncb, int M, int H, const float *w, float eps,
                       float *out, hipStream_t s);

constexpr int ROPE_MAX_PAIRS = 128;  // rotary_dim <= 256

struct QkvPostArgs {
    const float *pq;   // [ksq][16][qt]
    const float *pk;   // [ksk][rows_kv][kt]
    const float *pv;   // [ksv][rows_kv][kt]
    const float *pg;   // [ksg][16][qt] or null
    int ksq, ksk, ksv, ksg, rows_kv, kv_block_row0;
    const float *ssp_x;    // block rows' norm partials [16][ncb]
    const float *ssp_ctx;  // context rows' norm partials [16][ncb_ctx]
    int ncb, ncb_ctx, H;
    const float *q_norm, *k_norm;
    float eps;
    double inv_freq[ROPE_MAX_PAIRS];  // theta^(-2j/rotary_dim), j < rotary_dim/2, in F64
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


struct SwigluArgs {
    const float *pg, *pu;
    int ksg, ksu;
    const float *ssp;  // FFN input rows' norm partials [16][ncb]
    int ncb, H;
    float eps;
    int M, I;
    uint16_t *xs;
};
void launch_swiglu(const SwigluArgs &a, hipStream_t s);

struct AttnArgs {
    const float *q;        // [M][nq*hd], normed + rotated
    const void *cache_k, *cache_v;  // this layer's [nkv][cap][hd]
    int kv_bf16;
    long long capacity;
    long long n_ctx;       // keys visible to block row 0 minus one: P0 + R
    int M, nq, nkv, hd;
    int chunk, n_chunks;
    int bidir;             // 1: every block row sees all M block rows
    float *part;           // [n_chunks][M*nq][hd + 4]
};
constexpr int ATT_PART_EXTRA = 4;  // partial record: acc[hd], m, l, 2 pad floats
constexpr int ATT_CHUNKS_MAX = 256;
// groups: workgroups per chunk (kv heads x query tiles)
void attn_plan(long long n_keys, int groups, int *chunk, int *n_chunks);
void attn_plan_keys(long long n_keys, int keys_per_wave, int *chunk, int *n_chunks);
int attn_qtiles(int hd, int nq_group, bool kv_bf16);
bool attn_supported(int hd);
void launch_attn(const AttnArgs &a, hipStream_t s);

struct CombineArgs {
    const float *part;
    int n_chunks, M, nq, hd;
    const float *g;        // [M][nq*hd] raw gate or null
    uint16_t *xs;          // split tile (K = nq*hd)
};
void launch_attn_combine(const CombineArgs &a, hipStream_t s);

void launch_accept(const int32_t *drafts, const int32_t *target, int K, const int32_t *eos,
                   int n_eos, int32_t *result, int32_t *committed, hipStream_t s);

// ---------------------------------------------------------------------------
// Sampling from softmax(logits / T) and sampled acceptance (sample.hip)
int smp_blocks(int V);  // segments per logits row

struct SmpStatArgs {
    const float *z[3];  // row r: z[r] (nptr == 3), or z[0] + r * ld (nptr == 1)
    int nptr;
    long long ld;
    int V, nb;
    float c;            // log2(e) / T
    float2 *stats;      // out: [rows][nb] (max y, sum 2^(y - max)) per segment
};
void launch_smp_stats(const SmpStatArgs &a, int rows, hipStream_t s);

struct SmpResidualArgs {
    const float *zq, *zp;  // draft logits, target logits at the draft's position
    const float2 *stats;   // [2][nb]: q's rows then p0's
    int V, nb;
    float c;
    float *rsum;           // out: [nb] segment sums of max(0, p0 - q)
};
void launch_smp_residual(const SmpResidualArgs &a, hipStream_t s);

struct SmpDrawArgs {
    const float *z;        // [M][V]
    const float2 *stats;   // [M][nb]
    const float *u;        // [M]
    int V, nb;
    float c;
    int32_t *token;        // out [M]
    float *prob;           // out [M] or null
};
void launch_smp_draw(const SmpDrawArgs &a, int M, hipStream_t s);

struct SmpAcceptArgs {
    const float *zq, *zp0, *zp1;
    const float2 *stats;   // [3][nb]: q, p0, p1
    const float *rsum;     // [nb]
    const int32_t *draft;  // [1]
    const float *u;        // [2]
    const int32_t *eos;
    int n_eos;
    int V, nb;
    float c;
    int32_t *result;       // out [5]
    int32_t *committed;    // out [2] or null
};
void launch_smp_accept(const SmpAcceptArgs &a, hipStream_t s);

// ---------------------------------------------------------------------------
// MoE FFN (moe.hip)
// ---------------------------------------------------------------------------
struct MoeRouteArgs {
    const float *p_router;  // [ks][16][E] router partials (unscaled by the row norm)
    int ks_router;
    const float *p_sgi;     // [ks][16][1] shared-expert gate-input partials
    int ks_sgi;
    const float *ssp;       // FFN input rows' norm partials [16][ncb]
    int ncb, H;
    float eps;
    int M, E, top_k, max_slots;
    int32_t *nslots;        // out: number of distinct experts touched
    int32_t *slot_expert;   // out: [max_slots] expert ids, ascending
    float *coef;            // out: [max_slots][16] routing weight of each row (0: not routed)
    float *shared_scale;    // out: [16] sigmoid(x . w_sg) per row
    int32_t *sel;           // out: [16][top_k] selected experts per row (descending weight)
    int32_t *touched_out;   // out (nullable): copy of the distinct-expert count
};
void launch_moe_route(const MoeRouteArgs &a, hipStream_t s);

struct MoeSwigluArgs {
    const float *pg, *pu;   // expert partials [slot][ks][16][Ie]
    int ks;
    const float *psg, *psu; // shared-expert partials [ks_sh][16][Is]
    int ks_sh;
    const float *ssp;
    int ncb, H;
    float eps;
    int M, Ie, Is, max_slots;
    const int32_t *nslots;
    uint16_t *xs_e;         // [max_slots] split tiles (K = Ie)
    uint16_t *xs_sh;        // split tile (K = Is)
};
void launch_moe_swiglu(const MoeSwigluArgs &a, hipStream_t s);

struct MoeCombineArgs {
    const float *base;      // x1 [M][H]
    const float *pd;        // expert down partials [slot][ks][16][H]
    int ks;
    const float *psd;       // shared down partials [ks_sh][16][H]
    int ks_sh;
    const int32_t *nslots;
    const float *coef;      // [max_slots][16]
    const float *shared_scale;
    int M, H, max_slots;
    float *out, *copy0, *copy1;
    const float *w;         // next norm weight or null
    uint16_t *xs;           // split tile or null
    float *ssp_out;
    int ncb;
};
void launch_moe_combine(const MoeCombineArgs &a, hipStream_t s);

}  // namespace dbf
