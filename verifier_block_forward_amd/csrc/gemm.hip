// gemm.hip -- skinny BF16-weight projections on the gfx950 matrix cores.
//
// Y[m, o] = sum_k X[m, k] W[o, k]: BF16 weights [out, in] times F32 activations
// with F32 accumulation (the weight/activation dtype policy of the hf2q 0.1.1
// page spec_decode/dflash/tensors.rs, `DFlashLayerTensors`). The block has at most
// 16 (or 32, with context rows) activation rows, so every projection is a weight
// stream: bytes, not flops, set its speed.
//
// Weight layouts. Row-major [out, in] (as stored on disk): per 32-column k-step a
// lane reads 16 bytes of row (l % 16) at columns 8*(l/16)..+7, i.e. 64-byte runs
// per row per load instruction, which streams at ~4.6 TB/s on MI355X. Tiled
// (DBF_BF16_T16, written once by dbf_tile_weight): rows in tiles of 16, each
// (tile, k-step) block stored as the 64 lanes' 16-byte A operands back to back,
// so every load instruction reads one contiguous 1 KiB (~6.2 TB/s, the read
// ceiling measured with a plain streaming kernel). Element (n, k) of a tiled
// [N, K] weight sits at ((n/16 * S + k/32) * 64 + ((k%32)/8) * 16 + n%16) * 8 + k%8,
// S = ceil(K/32); padding rows and columns are zero.
//
// Mapping: a wavefront owns 16*NA consecutive weight rows and a slice of the
// input dimension. Per k-step of 32 columns, lane l loads 16 bytes of row
// (l % 16) at columns 8*(l/16)..+7 of each of its NA row tiles (each row gets 64
// contiguous bytes per step, 128 per pair of steps), plus the pre-split
// activation hi/lo halves (two coalesced 1 KiB reads shared by all NA tiles), and
// issues 2*NA*NB v_mfma_f32_16x16x32_bf16. MFMA A = weights (16 rows x 32 k),
// B = activations (32 k x 16 rows), D[4*(l/16)+j][l%16] = Y[row, m].
#include "internal.hpp"
#include "kernels.hpp"

namespace dbf {

__device__ __forceinline__ bf16x8 ld16(const uint16_t *p) {
    return __builtin_bit_cast(bf16x8, *(const uint4 *)p);
}

// Weights are read exactly once per launch: nontemporal loads. A plain streaming
// read tops out near 6.2 TB/s on MI355X; the same read with nontemporal loads
// reaches ~7.0 TB/s (probe over a 4 GiB buffer).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 ldw16(const uint16_t *p) {
    return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load((const u32x4_t *)p));
}

__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

// Workgroup order across the XCDs. Workgroups are handed to the 8 XCDs round-robin
// (hardware index b runs on XCD b % 8), and each XCD has its own L2. With the remap,
// the logical index of b is its rank within its XCD plus the count of workgroups on
// lower XCDs, so consecutive logical indices -- which share a k-slice of the
// activations -- sit on one XCD and its L2. A bijection on [0, n) for any n.
constexpr int N_XCD = 8;
__device__ __forceinline__ int xcd_logical(int b, int n) {
    const int q = n / N_XCD, r = n % N_XCD;
    const int x = b % N_XCD, i = b / N_XCD;
    return x * q + (x < r ? x : r) + i;
}

#define MFMA(a, b, c) __builtin_amdgcn_mfma_f32_16x16x32_bf16((a), (b), (c), 0, 0, 0)

// Write a wave's NA x NB accumulator tiles into a [rows][N] F32 partial: lane l
// holds output columns row0 + 16 a + 4 (l / 16) + 0..3 of activation row l % 16 of
// split tile b, stored as one float4 (N % 4 == 0; scalar stores at a ragged edge).
// Rows at or past mr0 (tile 0) / mr1 (tile 1) hold no activation and are skipped:
// with few rows most of the partial's bytes are never written.
template <int NA, int NB>
__device__ __forceinline__ void store_partials(float *out, int N, int nb, int row0, int lane, int mr0,
                                               int mr1, const f32x4 (&acc)[NA][NB]) {
    const int r = lane & 15, g = lane >> 4;
    const bool vec = (N & 3) == 0;
#pragma unroll
    for (int b = 0; b < NB; b++) {
        if (b >= nb || r >= (b == 0 ? mr0 : mr1)) continue;
        float *orow = out + (size_t)(16 * b + r) * N;
#pragma unroll
        for (int a = 0; a < NA; a++) {
            const int o = row0 + 16 * a + 4 * g;
            if (vec && o + 3 < N) {
                *(f32x4 *)(orow + o) = acc[a][b];
            } else {
#pragma unroll
                for (int j = 0; j < 4; j++)
                    if (o + j < N) orow[o + j] = acc[a][b][j];
            }
        }
    }
}

// Accumulate the NA x NB tile product over k-steps [s0, s1), software-pipelined:
// a ring of PIPE register stages holds the loads of k-steps s+1..s+PIPE while
// step s feeds the matrix cores, so every wave keeps PIPE*(NA + 2*NB) 16-byte
// loads in flight. Stages past s1 (or columns past K) re-read a valid address and
// are zeroed or ignored, so the loop has no control flow around its loads. Lanes
// whose activation row r = lane % 16 holds no data (r >= mr[b]) take zeros
// instead of loading: the matrix cores' output columns are independent, so those
// rows' products, which nobody stores, are all that changes.
template <int NA, int NB, int PIPE>
__device__ __forceinline__ void skinny_mainloop(const uint16_t *const wrow[NA], int wstep,
                                                bool tiled, const uint16_t *const xs[NB], const int mr[NB],
                                                int K, int s0, int s1, int lane, f32x4 acc[NA][NB]) {
    const int g = lane >> 4, r16 = lane & 15;
    bf16x8 wb[PIPE][NA], xh[PIPE][NB], xl[PIPE][NB];
    const int n = s1 - s0;
#define DBF_LOAD_STAGE(u, step)                                                 \
    do {                                                                        \
        const int sc_ = (step) < s1 ? (step) : s1 - 1;                          \
        const bool in_ = tiled || 32 * sc_ + 8 * g < K;                         \
        const int col_ = in_ ? wstep * sc_ : 0;                                 \
        _Pragma("unroll") for (int a = 0; a < NA; a++) {                        \
            const bf16x8 v_ = ldw16(wrow[a] + col_);                            \
            wb[u][a] = in_ ? v_ : zero8();                                      \
        }                                                                       \
        _Pragma("unroll") for (int b = 0; b < NB; b++) {                        \
            const uint16_t *x_ = xs[b] + ((size_t)sc_ * 2 * 64 + lane) * 8;     \
            if (r16 < mr[b]) {                                                  \
                xh[u][b] = ld16(x_);                                            \
                xl[u][b] = ld16(x_ + 64 * 8);                                   \
            } else {                                                            \
                xh[u][b] = zero8();                                             \
                xl[u][b] = zero8();                                             \
            }                                                                   \
        }                                                                       \
    } while (0)
#pragma unroll
    for (int u = 0; u < PIPE; u++) DBF_LOAD_STAGE(u, s0 + u);
    for (int base = 0; base < n; base += PIPE) {
#pragma unroll
        for (int u = 0; u < PIPE; u++) {
            if (base + u < n) {
#pragma unroll
                for (int a = 0; a < NA; a++)
#pragma unroll
                    for (int b = 0; b < NB; b++) {
                        acc[a][b] = MFMA(wb[u][a], xh[u][b], acc[a][b]);
                        acc[a][b] = MFMA(wb[u][a], xl[u][b], acc[a][b]);
                    }
            }
            DBF_LOAD_STAGE(u, s0 + base + u + PIPE);
        }
    }
#undef DBF_LOAD_STAGE
}

// Column k of activation row m of an F32 source (see GemmF32Src).
__device__ __forceinline__ const float *f32_src_at(const GemmF32Src &s, int m, int k) {
    if (s.xf) return s.xf + (size_t)m * s.xf_ld + k;
    const int t = k / s.xg_cols;
    const float *b = s.xg[0];
#pragma unroll
    for (int i = 1; i < 8; i++)  // a select chain: no indexed copy of the argument array
        if (t == i) b = s.xg[i];
    return b + (size_t)(s.xg_row0 + m) * s.xg_ld + (k - t * s.xg_cols);
}

// Stages in flight per wave, chosen per launch from its longest k-slice: 3 for
// slices of up to 24 steps (the 16-row down and input projections: 12 and 20 steps;
// the one-row 17408-deep down: 24; 2 and 4 were slower), 2 for slices of
// GEMM_LONG_SLICE steps or more (e.g. 32-step MoE expert slices), where the steady
// state dominates and a shorter queue of requests wins.
constexpr int GEMM_PIPE = 3;
constexpr int GEMM_PIPE_LONG = 2;
constexpr int GEMM_LONG_SLICE = 25;

// W waves per workgroup take W consecutive units; with the tile index fastest they
// share one k-slice of the activations, which the CU's vector cache then serves once.
// Plain launches with slices of SPLITK_W_LONG_STEPS steps or more (the long down and
// input projections) use 8 (the 16-row DFlash and one-row dense MTP steps -0.3% each
// against 4), launches with expert slots 2 (the four-row MoE MTP step -0.5%; 8 was
// +1.9% there), other plain launches 4.
constexpr int SPLITK_W_LONG = 8;
constexpr int SPLITK_W_LONG_STEPS = 8;
constexpr int SPLITK_W_SLOTS = 2;
constexpr int SPLITK_W = 4;
static_assert(SPLITK_W_LONG_STEPS <= GEMM_LONG_SLICE, "long slices always take SPLITK_W_LONG waves");

// One split tile per segment: the launches that also project the context rows (a
// second split tile) are LDS-staged.
template <int NA, int PIPE, int W>
__global__ __launch_bounds__(64 * W) void k_gemm_splitk(GemmArgs args) {
    const int lane = threadIdx.x & 63;
    // scalar wave index: the unit, the segment lookup and the segment's fields are
    // then scalar (kernel-argument loads, not vector loads)
    const int wv = wave_id();
    int ub[GEMM_MAXSEG];  // every segment boundary, loaded with the grid size
#pragma unroll
    for (int i = 0; i < GEMM_MAXSEG; i++) ub[i] = args.seg[i].unit_begin;
    const int nblk = gridDim.x, nseg = args.nseg, total = args.total_units;
    __builtin_amdgcn_sched_barrier(0);  // keep those loads ahead of their first use: one trip
    const int unit = xcd_logical(blockIdx.x, nblk) * W + wv;
    int si = 0;
#pragma unroll
    for (int i = 1; i < GEMM_MAXSEG; i++)
        if (i < nseg && unit >= ub[i]) si = i;
    // segment chosen before the exit test, so the boundary loads are not sunk below
    // it into a second round trip
    asm volatile("" : "+s"(si));
    if (unit >= total) return;
    const GemmSeg &sg = args.seg[si];
    int local = unit - sg.unit_begin;
    const uint16_t *Wbase = sg.W;
    const uint16_t *xsb0 = sg.xs0;
    float *outb = sg.out;
    if (sg.slots > 0) {  // grouped: this unit's matrix is the slot's expert
        const int per = sg.tiles * sg.ksplit;
        const int slot = local / per;
        // the slot count and the slot's expert load together (slot < slots, so the
        // entry is in bounds; it is used only for a slot below the count)
        const int ns = *sg.nslots, ex = sg.slot_expert[slot];
        asm volatile("" ::"s"(ns), "s"(ex));
        if (slot >= ns) return;
        local -= slot * per;
        Wbase += (size_t)ex * (size_t)sg.w_stride;
        xsb0 += (size_t)slot * (size_t)sg.xs_stride;
        outb += (size_t)slot * (size_t)sg.out_stride;
    }
    const int tile = local % sg.tiles;
    const int ks = local / sg.tiles;
    const int N = sg.N, K = sg.K, mr0 = sg.mrows[0];
    const int S = (K + 31) >> 5;
    const int s0 = ks * sg.kslice_steps;
    int s1 = s0 + sg.kslice_steps;
    if (s1 > S) s1 = S;
    const int r = lane & 15, g = lane >> 4;
    const int row0 = tile * 16 * NA;

    const uint16_t *wrow[NA];
    const int wstep = sg.tiled ? 512 : 32;
#pragma unroll
    for (int a = 0; a < NA; a++) {
        if (sg.tiled) {
            int t = tile * NA + a;
            const int T = (N + 15) >> 4;
            if (t > T - 1) t = T - 1;  // tile past the padded rows: re-read, result dropped
            wrow[a] = Wbase + ((size_t)t * S * 64 + lane) * 8;
        } else {
            int row = row0 + 16 * a + r;
            if (row > N - 1) row = N - 1;  // ragged last tile: re-read a valid row, result dropped
            wrow[a] = Wbase + (size_t)row * K + 8 * g;
        }
    }
    f32x4 acc[NA][1];
#pragma unroll
    for (int a = 0; a < NA; a++) acc[a][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t *xs[1] = {xsb0};
    const int mrs[1] = {mr0};
    skinny_mainloop<NA, 1, PIPE>(wrow, wstep, sg.tiled, xs, mrs, K, s0, s1, lane, acc);
    store_partials<NA, 1>(outb + (size_t)ks * 16 * N, N, 1, row0, lane, mr0, mr0, acc);
}

// ---------------------------------------------------------------------------
// Variant with the activation slice staged in LDS: the four waves of a workgroup
// share (segment, k-slice) and own consecutive row tiles, so the slice's split
// activations are read once per workgroup (not once per wave) and each wave's
// registers hold only weights, in a ring of LP stages. A launch of these kernels
// asks for tens of MB at once; for long slices the ring is kept short (2 stages
// measured best on the 18-20-step slices, against 1, 3, 4 and 6) because more
// requests in flight only lengthen the queue that the activation loads, which gate
// the first product, wait in. Slices of at most LPIPE_SHORT_MAX steps take a ring
// of LPIPE_SHORT stages. Ring loads past the slice end are not issued.
constexpr int LPIPE = 2;
constexpr int LPIPE_SHORT = 6;
constexpr int LPIPE_SHORT_MAX = 10;
constexpr int LDS_X_BYTES = 40 * 1024;  // per workgroup: NB * slice_steps * 2 KiB

template <int NA, int NB, int LP, bool F32X = false>
__global__ __launch_bounds__(256) void k_gemm_lds(GemmArgs args) {
    extern __shared__ __align__(16) uint4 xl[];  // NB * kslice_steps * 2 KiB (<= LDS_X_BYTES)
    const int lane = threadIdx.x & 63, wv = wave_id();
    int ub[GEMM_MAXSEG];  // every segment boundary, loaded with the grid size
#pragma unroll
    for (int i = 0; i < GEMM_MAXSEG; i++) ub[i] = args.seg[i].unit_begin;
    const int nblk = gridDim.x, nseg = args.nseg;
    __builtin_amdgcn_sched_barrier(0);  // keep those loads ahead of their first use: one trip
    const int wg = xcd_logical(blockIdx.x, nblk);
    int si = 0;
#pragma unroll
    for (int i = 1; i < GEMM_MAXSEG; i++)
        if (i < nseg && wg >= ub[i]) si = i;
    const GemmSeg &sg = args.seg[si];
    int local = wg - sg.unit_begin;  // workgroup units: (tile group, ks) per slot
    const int groups = (sg.tiles + 3) / 4;
    const uint16_t *Wbase = sg.W;
    const uint16_t *xsb0 = sg.xs0;
    float *outb = sg.out;
    if (sg.slots > 0) {
        const int per = groups * sg.ksplit;
        const int slot = local / per;
        // the slot count and the slot's expert load together (slot < slots, so the
        // entry is in bounds; it is used only for a slot below the count)
        const int ns = *sg.nslots, ex = sg.slot_expert[slot];
        asm volatile("" ::"s"(ns), "s"(ex));
        if (slot >= ns) return;  // whole workgroup leaves together
        local -= slot * per;
        Wbase += (size_t)ex * (size_t)sg.w_stride;
        xsb0 += (size_t)slot * (size_t)sg.xs_stride;
        outb += (size_t)slot * (size_t)sg.out_stride;
    }
    const int grp = local % groups, ks = local / groups;
    const int tile = grp * 4 + wv;
    const int N = sg.N, K = sg.K, mr0 = sg.mrows[0], mr1 = sg.mrows[1];
    const int S = (K + 31) >> 5;
    const int s0 = ks * sg.kslice_steps;
    int s1 = s0 + sg.kslice_steps;
    if (s1 > S) s1 = S;
    const int n = s1 - s0;
    const int nb = NB == 1 ? 1 : sg.nb;
    const int r = lane & 15, g = lane >> 4;
    const int row0 = tile * 16 * NA;
    const uint16_t *wrow[NA];
    const int wstep = sg.tiled ? 512 : 32;
#pragma unroll
    for (int a = 0; a < NA; a++) {
        if (sg.tiled) {
            int t = tile * NA + a;
            const int T = (N + 15) >> 4;
            if (t > T - 1) t = T - 1;  // also for waves past the last tile: valid, unused
            wrow[a] = Wbase + ((size_t)t * S * 64 + lane) * 8;
        } else {
            int row = row0 + 16 * a + r;
            if (row > N - 1) row = N - 1;
            wrow[a] = Wbase + (size_t)row * K + 8 * g;
        }
    }
    f32x4 acc[NA][NB];
#pragma unroll
    for (int a = 0; a < NA; a++)
#pragma unroll
        for (int b = 0; b < NB; b++) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    bf16x8 wb[LP][NA];
    const bool tiled = sg.tiled;
    // Loads only: columns past K (row-major weights) re-read column 0 here and are
    // zeroed where the stage is consumed. A select right after the load made the
    // compiler wait for every load in flight at the end of each ring pass. Steps
    // past the slice are skipped by a wave-uniform branch.
#define DBF_LOAD_W(u, step)                                                     \
    do {                                                                        \
        const int sc_ = (step);                                                 \
        if (sc_ < s1) {                                                         \
            const bool in_ = tiled || 32 * sc_ + 8 * g < K;                     \
            const int col_ = in_ ? wstep * sc_ : 0;                             \
            _Pragma("unroll") for (int a = 0; a < NA; a++) wb[u][a] = ldw16(wrow[a] + col_); \
        }                                                                       \
    } while (0)
    // Stage the activation slice (per tile, steps [s0, s1) are contiguous, 2 KiB each):
    // this thread's share is loaded first, the weight ring is issued behind it, and
    // only then is the share stored, so the store waits for the activation loads
    // alone (loads complete in issue order) while the weight loads are in flight.
    constexpr int XPT = LDS_X_BYTES / 16 / 256;  // uint4 per thread at most
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // register-friendly
    u32x4 xr[F32X ? 1 : XPT];
    const int per = n * 128;  // uint4 per tile
    const int xtot = (NB > 1 && nb > 1) ? 2 * per : per;
    // F32X: the slice comes from args.xf's F32 rows: run i (step i / 64, lane i % 64
    // of the split layout) is 8 values of row (i % 16), split hi/lo (split8, the
    // values a split pass would store) on their way into LDS. The runs are read
    // element by element, so the rows need only 4-byte alignment (the compiler
    // issues 16-byte loads, which gfx950 serves at any 4-byte address).
    constexpr int RPT = LDS_X_BYTES / 32 / 256;  // runs per thread at most
    float xv[F32X ? RPT : 1][8];
    const int runs = n * 64;
    // every run of this thread is of row threadIdx.x % 16 (256 q + i keeps i % 16)
    float ssq_part = 0.f;
    if constexpr (F32X) {
        const GemmF32Src &xs_ = args.xf[si];
#pragma unroll
        for (int q = 0; q < RPT; q++) {
            if (256 * q < runs) {
                const int i = threadIdx.x + 256 * q;
                const int ic = i < runs ? i : runs - 1;
                const int l = ic & 63, row = l & 15, col = 32 * (s0 + (ic >> 6)) + 8 * (l >> 4);
                if (row < mr0 && col < K && i < runs) {
                    if (xs_.tokens) {
                        int t = xs_.tokens[row];
                        t = t < 0 ? 0 : (t >= xs_.V ? xs_.V - 1 : t);
                        const uint16_t *e_ = xs_.embed + (size_t)t * xs_.xf_ld + col;
#pragma unroll
                        for (int j = 0; j < 8; j++) xv[q][j] = bf16_to_f32(e_[j]);
                    } else {
                        const float *x_ = f32_src_at(xs_, row, col);
#pragma unroll
                        for (int j = 0; j < 8; j++) xv[q][j] = x_[j];
                    }
#pragma unroll
                    for (int j = 0; j < 8; j++) ssq_part += xv[q][j] * xv[q][j];
                    if (xs_.w) {
#pragma unroll
                        for (int j = 0; j < 8; j++) xv[q][j] *= xs_.w[col + j];
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 8; j++) xv[q][j] = 0.f;
                }
            }
        }
    } else {
        const uint4 *src0 = (const uint4 *)(xsb0 + (size_t)s0 * 2 * 64 * 8);
        const uint4 *src1 = (const uint4 *)(sg.xs1 + (size_t)s0 * 2 * 64 * 8);
        // element i of a split tile belongs to activation row i % 16 (= threadIdx.x % 16
        // here); rows that hold no data are staged as zeros without a load
        const int xrow = threadIdx.x & 15;
#pragma unroll
        for (int q = 0; q < XPT; q++) {
            if (256 * q < xtot) {  // uniform: rounds wholly past the slice are skipped
                const int i = threadIdx.x + 256 * q;
                const int ic = i < xtot ? i : xtot - 1;  // always a valid address
                const bool t0 = ic < per;
                const uint4 *sp = t0 ? src0 + ic : src1 + (ic - per);  // pointer select
                if (xrow < (t0 ? mr0 : mr1))
                    xr[q] = *(const u32x4 *)sp;
                else
                    xr[q] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
#pragma unroll
    for (int u = 0; u < LP; u++) DBF_LOAD_W(u, s0 + u);
    if constexpr (F32X) {
#pragma unroll
        for (int q = 0; q < RPT; q++) {
            const int i = threadIdx.x + 256 * q;
            if (i < runs) {
                bf16x8 hi, lo;
                split8(xv[q], hi, lo);
                const int sl = i >> 6, l = i & 63;
                xl[(sl * 2 + 0) * 64 + l] = __builtin_bit_cast(uint4, hi);
                xl[(sl * 2 + 1) * 64 + l] = __builtin_bit_cast(uint4, lo);
            }
        }
        const GemmF32Src &xs_ = args.xf[si];
        if (xs_.ssq && grp == 0) {  // the slice's sum of squares per row, in a fixed order
            __shared__ float ssq_w[4][16];
            float v = ssq_part;
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            if ((threadIdx.x & 63) < 16) ssq_w[wv][threadIdx.x & 15] = v;
            __syncthreads();
            if (threadIdx.x < 16 && (int)threadIdx.x < mr0)
                xs_.ssq[(size_t)threadIdx.x * xs_.ssq_ld + ks] =
                    (ssq_w[0][threadIdx.x] + ssq_w[1][threadIdx.x]) + (ssq_w[2][threadIdx.x] + ssq_w[3][threadIdx.x]);
        }
    } else {
#pragma unroll
        for (int q = 0; q < XPT; q++) {
            const int i = threadIdx.x + 256 * q;
            if (i < xtot) *(u32x4 *)&xl[i] = xr[q];
        }
    }
    __syncthreads();
    if (tile >= sg.tiles) return;

    for (int base = 0; base < n; base += LP) {
#pragma unroll
        for (int u = 0; u < LP; u++) {
            const int j = base + u;
            if (j < n) {
                const bool in_ = tiled || 32 * (s0 + j) + 8 * g < K;
                bf16x8 w[NA];
#pragma unroll
                for (int a = 0; a < NA; a++) w[a] = in_ ? wb[u][a] : zero8();
#pragma unroll
                for (int b = 0; b < NB; b++) {
                    if (b >= nb) continue;
                    const bf16x8 xh = __builtin_bit_cast(bf16x8, xl[b * per + (j * 2 + 0) * 64 + lane]);
                    const bf16x8 xlo = __builtin_bit_cast(bf16x8, xl[b * per + (j * 2 + 1) * 64 + lane]);
#pragma unroll
                    for (int a = 0; a < NA; a++) {
                        acc[a][b] = MFMA(w[a], xh, acc[a][b]);
                        acc[a][b] = MFMA(w[a], xlo, acc[a][b]);
                    }
                }
            }
            DBF_LOAD_W(u, s0 + base + u + LP);
        }
    }
#undef DBF_LOAD_W
    store_partials<NA, NB>(outb + (size_t)ks * 16 * nb * N, N, nb, row0, lane, mr0, mr1, acc);
}

// ---------------------------------------------------------------------------
// Whole-K projection with the residual epilogue (FullArgs in kernels.hpp). A
// workgroup of FULL_W waves owns NT output tiles of 16 columns over all of K: wave w
// streams k-steps [S w / FULL_W, S (w + 1) / FULL_W) of every tile with its own
// activation slice (skinny_mainloop), the accumulators are summed through LDS in
// wave order, and the workgroup finishes its complete outputs: the residual add, the
// split of out (.) w for the next projection and the sums of squares of out. The
// residual rows and norm weights the epilogue needs are loaded before the main loop.
// NT = 1 when a wave has at most FULL_SHORT k-steps (more workgroups for short K),
// else 2 (each wave's activation slice then feeds two weight tiles).
constexpr int FULL_SHORT = 16;  // k-steps per wave up to which one tile per workgroup is used

template <int FULL_W, int NT>
__global__ __launch_bounds__(64 * FULL_W) void k_gemm_full(FullArgs a) {
    static_assert(256 * NT <= 64 * FULL_W, "one epilogue element per thread");
    // the arguments into scalar registers in one round trip
    asm volatile("" ::"s"(a.W), "s"(a.tiled), "s"(a.xs), "s"(a.N), "s"(a.K), "s"(a.M), "s"(a.base),
                 "s"(a.out), "s"(a.copy0), "s"(a.copy1), "s"(a.w), "s"(a.ssp_out), "s"(a.xs_out));
    __shared__ float4 red[FULL_W][NT][64];
    __shared__ float res[NT * 16][17];  // [output column of the workgroup][activation row], padded
    __shared__ float sspp[FULL_W][16];  // per-wave sums of squares
    const int lane = threadIdx.x & 63, wv = wave_id(), tid = threadIdx.x;
    const int N = a.N, K = a.K, S = (K + 31) >> 5;
    const int n0 = blockIdx.x * 16 * NT;
    const int r = lane & 15, g = lane >> 4;

    // epilogue element of this thread: activation row m, output column n
    const int m = tid & 15, nl = tid >> 4, n = n0 + nl;
    const bool has_e = tid < 256 * NT;
    const bool in_e = has_e && m < a.M && n < N;
    float bv = 0.f, wn = 1.f;
    if (in_e) {
        if (a.base) bv = a.base[(size_t)m * N + n];
        if (a.w) wn = a.w[n];
    }

    const uint16_t *wrow[NT];
    const int wstep = a.tiled ? 512 : 32;
    const int T = (N + 15) >> 4;
#pragma unroll
    for (int t = 0; t < NT; t++) {
        const int tt = n0 / 16 + t;
        if (a.tiled) {
            const int tc = tt > T - 1 ? T - 1 : tt;  // tiles past N: re-read, result dropped
            wrow[t] = a.W + ((size_t)tc * S * 64 + lane) * 8;
        } else {
            int row = tt * 16 + r;
            if (row > N - 1) row = N - 1;
            wrow[t] = a.W + (size_t)row * K + 8 * g;
        }
    }
    f32x4 acc[NT][1];
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int s0 = (S * wv) / FULL_W, s1 = (S * (wv + 1)) / FULL_W;
    if (s1 > s0) {
        const uint16_t *xs[1] = {a.xs};
        const int mrs[1] = {a.M};
        skinny_mainloop<NT, 1, GEMM_PIPE>(wrow, wstep, a.tiled != 0, xs, mrs, K, s0, s1, lane, acc);
    }
#pragma unroll
    for (int t = 0; t < NT; t++)
        red[wv][t][lane] = make_float4(acc[t][0][0], acc[t][0][1], acc[t][0][2], acc[t][0][3]);
    __syncthreads();
    // sum the waves' accumulators in wave order: element (tile t, lane l, j) is output
    // column 16 t + 4 (l / 16) + j of the workgroup for activation row l % 16
    for (int e = tid; e < NT * 256; e += 64 * FULL_W) {
        const int t = e >> 8, l = (e >> 2) & 63, j = e & 3;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < FULL_W; w++) sum += ((const float *)&red[w][t][l])[j];
        res[t * 16 + 4 * (l >> 4) + j][l & 15] = sum;
    }
    __syncthreads();

    float v = 0.f;
    if (in_e) {
        v = bv + res[nl][m];
        a.out[(size_t)m * N + n] = v;
        if (a.copy0) a.copy0[(size_t)m * N + n] = v;
        if (a.copy1) a.copy1[(size_t)m * N + n] = v;
    }
    const int Np = (N + 31) & ~31;
    if (has_e && n < Np) split_store(a.xs_out, m, n, v * wn);
    if (a.ssp_out) {
        // sum of squares over each 16-column tile: a wave's lanes hold 4 columns x 16
        // rows; the four waves of a tile are then added in order
        float ss = v * v;
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        if (lane < 16) sspp[wv][lane] = ss;
        __syncthreads();
        if (tid < 16 * NT) {
            const int t = tid >> 4, mm = tid & 15;
            const float q = (sspp[4 * t][mm] + sspp[4 * t + 1][mm]) + (sspp[4 * t + 2][mm] + sspp[4 * t + 3][mm]);
            const int blk = n0 / 16 + t, nblk = (N + 15) / 16;
            if (blk < nblk) a.ssp_out[(size_t)mm * nblk + blk] = q;
        }
    }
}

void launch_gemm_full(const FullArgs &a, hipStream_t s) {
    constexpr int W = 8;
    const int S = (a.K + 31) / 32, Np = (a.N + 31) & ~31;
    if ((S + W - 1) / W <= FULL_SHORT)
        launch_k(PROF_PROJ, "k_gemm_full", k_gemm_full<W, 1>, dim3((Np + 15) / 16), dim3(64 * W), 0, s, a);
    else
        launch_k(PROF_PROJ, "k_gemm_full", k_gemm_full<W, 2>, dim3((Np + 31) / 32), dim3(64 * W), 0, s, a);
}

GemmPlan gemm_plan(int N, int K, int target_units, int max_steps) {
    GemmPlan p{0, 0, 0, 0};
    if (N < 1 || K < 1) return p;  // empty projection: no units
    p.tiles = (N + 16 * GEMM_NA - 1) / (16 * GEMM_NA);
    const int S = (K + 31) / 32;
    int ks = (target_units + p.tiles - 1) / p.tiles;
    const int ks_min = max_steps > 0 ? (S + max_steps - 1) / max_steps : 1;
    if (ks < ks_min) ks = ks_min;
    int max_ks = S / 4;  // keep at least 4 k-steps (128 columns) per slice
    if (max_ks < ks_min) max_ks = ks_min;
    if (max_ks < 1) max_ks = 1;
    if (ks > max_ks) ks = max_ks;
    if (ks < 1) ks = 1;
    int steps = (S + ks - 1) / ks;
    steps = (steps + 1) & ~1;  // even: slices start on 128-byte boundaries
    if (max_steps > 0 && steps > max_steps) steps = max_steps & ~1;
    p.kslice_steps = steps;
    p.ksplit = (S + steps - 1) / steps;
    return p;
}

GemmPlan gemm_plan_lds(int N, int K, int target_units, int nbmax) {
    GemmPlan p = gemm_plan(N, K, target_units, nbmax > 1 ? LDS_X_STEPS_NB2 : LDS_X_STEPS_NB1);
    p.lds = 1;
    return p;
}

template <int PIPE, int W>
static void go_splitk(const GemmArgs &a, hipStream_t s) {
    const dim3 grid((a.total_units + W - 1) / W), block(64 * W);
    launch_k(PROF_PROJ, PIPE == GEMM_PIPE_LONG ? "k_gemm_splitk(long)" : "k_gemm_splitk",
             (k_gemm_splitk<GEMM_NA, PIPE, W>), grid, block, 0, s, a);
}

// NB split tiles per segment at most. With two, slices are at most LDS_X_STEPS_NB2
// steps, so those launches always take the short-slice ring.
template <int NB, bool F32X = false>
static void go_lds(const GemmArgs &a, hipStream_t s) {
    static_assert(NB == 1 || LDS_X_STEPS_NB2 <= LPIPE_SHORT_MAX, "two-tile slices take the short ring");
    size_t lds = 0;
    int steps = 0;
    for (int i = 0; i < a.nseg; i++) {
        const size_t b = (size_t)(NB > 1 ? a.seg[i].nb : 1) * a.seg[i].kslice_steps * 2048;
        if (b > lds) lds = b;
        if (a.seg[i].kslice_steps > steps) steps = a.seg[i].kslice_steps;
    }
    const dim3 grid(a.total_units);  // total_units counts workgroups
    if (NB == 2 || steps <= LPIPE_SHORT_MAX)
        launch_k(PROF_PROJ, "k_gemm_lds", (k_gemm_lds<GEMM_NA, NB, LPIPE_SHORT, F32X>), grid, dim3(256), lds, s, a);
    else
        launch_k(PROF_PROJ, "k_gemm_lds", (k_gemm_lds<GEMM_NA, 1, LPIPE, F32X>), grid, dim3(256), lds, s, a);
}

bool launch_gemm(const GemmArgs &a, int nbmax, hipStream_t s) {
    if (a.total_units <= 0) return true;
    if (a.xf_on) {  // one or two plain LDS-staged segments reading F32 rows
        if (!a.lds_x || nbmax > 1 || a.nseg > 2) return false;
        for (int i = 0; i < a.nseg; i++)
            if (a.seg[i].slots > 0) return false;
        go_lds<1, true>(a, s);
        return true;
    }
    if (a.lds_x) {
        if (nbmax == 1)
            go_lds<1>(a, s);
        else
            go_lds<2>(a, s);
        return true;
    }
    if (nbmax > 1) return false;  // the split-K kernel reads one split tile per segment
    int steps = 0;
    bool slots = false;
    for (int i = 0; i < a.nseg; i++) {
        if (a.seg[i].kslice_steps > steps) steps = a.seg[i].kslice_steps;
        slots |= a.seg[i].slots > 0;
    }
    const bool lg = steps >= GEMM_LONG_SLICE;
    if (slots) {
        if (lg)
            go_splitk<GEMM_PIPE_LONG, SPLITK_W_SLOTS>(a, s);
        else
            go_splitk<GEMM_PIPE, SPLITK_W_SLOTS>(a, s);
    } else if (lg) {
        go_splitk<GEMM_PIPE_LONG, SPLITK_W_LONG>(a, s);
    } else if (steps >= SPLITK_W_LONG_STEPS) {
        go_splitk<GEMM_PIPE, SPLITK_W_LONG>(a, s);
    } else {
        go_splitk<GEMM_PIPE, SPLITK_W>(a, s);
    }
    return true;
}

// ---------------------------------------------------------------------------
// lm_head with a top-2 epilogue. Each wave unit covers 64 vocabulary rows over the
// full hidden dimension and emits, for each of the 16 activation rows, the best
// (value, index) and the second-best value among its rows. Ties keep the lower
// index. Optional logits are written row-major [M][V].
// ---------------------------------------------------------------------------
struct Top2 {
    float v1;
    int i1;
    float v2;
};

__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

__device__ __forceinline__ Top2 merge(Top2 a, Top2 b) {
    Top2 r;
    if (better(a.v1, a.i1, b.v1, b.i1)) {
        r.v1 = a.v1;
        r.i1 = a.i1;
        r.v2 = fmaxf(a.v2, b.v1);
    } else {
        r.v1 = b.v1;
        r.i1 = b.i1;
        r.v2 = fmaxf(b.v2, a.v1);
    }
    return r;
}

__device__ __forceinline__ Top2 shfl_top2(Top2 t, int mask) {
    Top2 o;
    o.v1 = __shfl_xor(t.v1, mask, 64);
    o.i1 = __shfl_xor(t.i1, mask, 64);
    o.v2 = __shfl_xor(t.v2, mask, 64);
    return o;
}

// The hidden rows come in as F32 [M][K]. The workgroup stages them through LDS in
// chunks of HEAD_XCH k-steps: its threads load a chunk once (16 rows x 64
// contiguous bytes per load instruction), split every value into the BF16 hi/lo
// pair and store the chunk in the split-tile order, double-buffered; the waves
// then read their B operands from LDS as contiguous 1 KiB lines. The next
// chunk's loads are in flight while the current one feeds the matrix cores, and
// the weight ring runs across chunk boundaries. Rows r >= M and columns past K
// are zeros. The waves merge their records in LDS, so the workgroup writes one
// record per activation row, stored [16][workgroups].
// One workgroup of HEAD_WAVES = 8 waves fills a CU (two waves per SIMD): its waves
// advance through K together, held by the per-chunk barrier. With two 4-wave
// workgroups per CU instead, the one whose loads were served first finished
// about 45 us (a fifth of the launch) before the other, which then ran alone at
// half occupancy.
// weight stages in flight per wave, and k-steps per staged chunk of the hidden
// rows: 2 and 4 measured best with 8-wave workgroups (A/B in the 5-layer, 16-row
// DFlash step with its 262144 x 2816 head, against
// 4/8, 1/8, 2/8, 2/16, 4/16, 4/4 and 3/12)
constexpr int HEAD_PIPE = 2;
constexpr int HEAD_XCH = 4;  // k-steps per staged chunk (a multiple of HEAD_PIPE)
static_assert(HEAD_XCH % HEAD_PIPE == 0, "chunk must hold whole pipeline rounds");
constexpr int HEAD_WAVES = 8;  // waves per workgroup, one 16*HEAD_NA-row unit each
constexpr int HEAD_THREADS = 64 * HEAD_WAVES;

// this thread's share of chunk c: HEAD_XPT float4 (row tid % 16, float4 columns
// tid/16 + (HEAD_THREADS/16)*i); a chunk is 16 rows x HEAD_XCH*32 columns =
// HEAD_XCH*128 float4
constexpr int HEAD_XPT = HEAD_XCH * 128 / HEAD_THREADS;
static_assert(HEAD_XCH * 128 % HEAD_THREADS == 0, "a chunk splits evenly over the threads");
// With the final RMSNorm folded in (PRE), h holds the pre-norm rows x: the load
// also fetches the norm weight w of the same columns (wr), and head_x_apply then
// forms x * s_m * w (the row scale s_m from rsc) in the order k_final_norm forms it,
// so the hidden rows are the same bits; workgroup 0 also writes them out as h_final.
// The first chunk is loaded before the row scales are formed, so the two round
// trips overlap.
template <bool PRE>
__device__ __forceinline__ void head_x_load(float4 (&xr)[HEAD_XPT], float4 (&wr)[HEAD_XPT], const float *h,
                                            int M, int K, int c, const HeadNorm &nrm) {
    const int r = threadIdx.x & 15, q = threadIdx.x >> 4;
    const bool rok = r < M;
    const float *row = h + (size_t)(rok ? r : 0) * K;
#pragma unroll
    for (int i = 0; i < HEAD_XPT; i++) {
        const int col = c * HEAD_XCH * 32 + 4 * (q + (HEAD_THREADS / 16) * i);
        const bool ok = rok && col < K;  // K % 8 == 0: a float4 is all in or all out
        const float4 v = *(const float4 *)(row + (ok ? col : 0));
        if constexpr (PRE) wr[i] = *(const float4 *)(nrm.w + (ok ? col : 0));
        xr[i].x = ok ? v.x : 0.f;
        xr[i].y = ok ? v.y : 0.f;
        xr[i].z = ok ? v.z : 0.f;
        xr[i].w = ok ? v.w : 0.f;
    }
}

template <bool PRE>
__device__ __forceinline__ void head_x_apply(float4 (&xr)[HEAD_XPT], const float4 (&wr)[HEAD_XPT], int M, int K,
                                             int c, const HeadNorm &nrm, const float *rsc) {
    if constexpr (PRE) {
        const int r = threadIdx.x & 15, q = threadIdx.x >> 4;
        const float sc = rsc[r];
#pragma unroll
        for (int i = 0; i < HEAD_XPT; i++) {
            const int col = c * HEAD_XCH * 32 + 4 * (q + (HEAD_THREADS / 16) * i);
            float4 v = xr[i];
            v.x = v.x * sc * wr[i].x;
            v.y = v.y * sc * wr[i].y;
            v.z = v.z * sc * wr[i].z;
            v.w = v.w * sc * wr[i].w;
            xr[i] = v;  // rows >= M and columns >= K stay 0
            if (r < M && col < K && blockIdx.x == 0) *(float4 *)(nrm.h_out + (size_t)r * K + col) = v;
        }
    }
}

// split the thread's share and store it in split-tile order (element offset
// ((s*2 + half)*64 + g*16 + r)*8 + j for local step s, column 8g + j)
__device__ __forceinline__ void head_x_store(uint16_t *buf, const float4 (&xr)[HEAD_XPT]) {
    const int r = threadIdx.x & 15, q = threadIdx.x >> 4;
#pragma unroll
    for (int i = 0; i < HEAD_XPT; i++) {
        const int k = 4 * (q + (HEAD_THREADS / 16) * i);  // local column
        const int s = k >> 5, g = (k & 31) >> 3, j = k & 7;
        const float f[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
        uint32_t hw[2], lw[2];
#pragma unroll
        for (int e = 0; e < 2; e++) {
            const __bf16 h0 = (__bf16)f[2 * e], h1 = (__bf16)f[2 * e + 1];
            const __bf16 l0 = (__bf16)(f[2 * e] - (float)h0), l1 = (__bf16)(f[2 * e + 1] - (float)h1);
            hw[e] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
            lw[e] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
        }
        *(uint2 *)(buf + ((s * 2 + 0) * 64 + g * 16 + r) * 8 + j) = make_uint2(hw[0], hw[1]);
        *(uint2 *)(buf + ((s * 2 + 1) * 64 + g * 16 + r) * 8 + j) = make_uint2(lw[0], lw[1]);
    }
}

template <bool PRE>
__global__ __launch_bounds__(HEAD_THREADS) __attribute__((amdgpu_waves_per_eu(2))) void k_head(
    const uint16_t *__restrict__ W, int tiled, const float *__restrict__ h, int V, int K, int M,
    float *__restrict__ logits, float4 *__restrict__ part, int units, HeadNorm nrm) {
    // the arguments into scalar registers in one round trip
    asm volatile("" ::"s"(W), "s"(tiled), "s"(h), "s"(V), "s"(K), "s"(M), "s"(logits), "s"(part), "s"(units),
                 "s"(nrm.w), "s"(nrm.ssp), "s"(nrm.ncb), "s"(nrm.eps), "s"(nrm.h_out));
    constexpr int NA = HEAD_NA, PIPE = HEAD_PIPE;
    constexpr int CHE = HEAD_XCH * 2 * 64 * 8;  // elements of one staged chunk
    __shared__ __align__(16) uint16_t xbuf[2][CHE];
    __shared__ Top2 wrec[HEAD_WAVES][16];
    __shared__ float rsc[16];  // PRE: row scales of the final RMSNorm
    const int lane = threadIdx.x & 63, wv = wave_id();
    const int unit = blockIdx.x * HEAD_WAVES + wv;
    const bool active = unit < units;
    const int r = lane & 15, g = lane >> 4;
    const int row0 = unit * 16 * NA;
    const int S = (K + 31) >> 5;
    const int nch = (S + HEAD_XCH - 1) / HEAD_XCH;

    const uint16_t *wrow[NA];
#pragma unroll
    for (int a = 0; a < NA; a++) {
        if (tiled) {
            int tt = unit * NA + a;
            const int T = (V + 15) >> 4;
            if (tt > T - 1) tt = T - 1;
            wrow[a] = W + ((size_t)tt * S * 64 + lane) * 8;
        } else {
            int row = row0 + 16 * a + r;
            if (row > V - 1) row = V - 1;
            wrow[a] = W + (size_t)row * K + 8 * g;
        }
    }
    const int wstep = tiled ? 512 : 32;
    f32x4 acc[NA];
#pragma unroll
    for (int a = 0; a < NA; a++) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 wb[PIPE][NA];
#define DBF_HEAD_STAGE(u, step)                                                 \
    do {                                                                        \
        const int sc_ = (step) < S ? (step) : S - 1;                            \
        const bool in_ = tiled || 32 * sc_ + 8 * g < K;                         \
        const int col_ = in_ ? wstep * sc_ : 0;                                 \
        _Pragma("unroll") for (int a = 0; a < NA; a++) {                        \
            const bf16x8 v_ = ldw16(wrow[a] + col_);                            \
            wb[u][a] = in_ ? v_ : zero8();                                      \
        }                                                                       \
    } while (0)
    if (active) {
#pragma unroll
        for (int u = 0; u < PIPE; u++) DBF_HEAD_STAGE(u, u);
    }
    float4 xr[HEAD_XPT], wr[HEAD_XPT];
    head_x_load<PRE>(xr, wr, h, M, K, 0, nrm);
    if constexpr (PRE) {
        // row scale of the final RMSNorm, from the rows' sum-of-squares partials:
        // wave w forms rows w and w + HEAD_WAVES (whole waves, as k_final_norm)
        for (int mm = wv; mm < 16; mm += HEAD_WAVES) {
            const float *sr = nrm.ssp + (size_t)(mm < M ? mm : 0) * nrm.ncb;
            const float f = row_scale_first(sr, nrm.ncb);
            const float sc = row_scale_finish(f, sr, nrm.ncb, K, nrm.eps);
            if (lane == 0) rsc[mm] = sc;
        }
        __syncthreads();
    }
    head_x_apply<PRE>(xr, wr, M, K, 0, nrm, rsc);
    head_x_store(xbuf[0], xr);
    if (nch > 1) head_x_load<PRE>(xr, wr, h, M, K, 1, nrm);
    __syncthreads();
    for (int c = 0; c < nch; c++) {
        if (active) {
            const uint4 *xb = (const uint4 *)xbuf[c & 1];
#pragma unroll
            for (int base = 0; base < HEAD_XCH; base += PIPE) {
#pragma unroll
                for (int u = 0; u < PIPE; u++) {
                    const int sl = base + u, step = c * HEAD_XCH + sl;
                    if (step < S) {
                        const bf16x8 xh = __builtin_bit_cast(bf16x8, xb[(sl * 2 + 0) * 64 + lane]);
                        const bf16x8 xl = __builtin_bit_cast(bf16x8, xb[(sl * 2 + 1) * 64 + lane]);
#pragma unroll
                        for (int a = 0; a < NA; a++) {
                            acc[a] = MFMA(wb[u][a], xh, acc[a]);
                            acc[a] = MFMA(wb[u][a], xl, acc[a]);
                        }
                    }
                    DBF_HEAD_STAGE(u, step + PIPE);
                }
            }
        }
        if (c + 1 < nch) {
            head_x_apply<PRE>(xr, wr, M, K, c + 1, nrm, rsc);
            head_x_store(xbuf[(c + 1) & 1], xr);
            if (c + 2 < nch) head_x_load<PRE>(xr, wr, h, M, K, c + 2, nrm);
        }
        __syncthreads();
    }
#undef DBF_HEAD_STAGE

    Top2 t{-INFINITY, 0x7fffffff, -INFINITY};
    if (active) {
        // lane holds rows o = row0 + 16a + 4g + j for activation row m = r
#pragma unroll
        for (int a = 0; a < NA; a++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int o = row0 + 16 * a + 4 * g + j;
                if (o < V) {
                    Top2 cnd{acc[a][j], o, -INFINITY};
                    t = merge(t, cnd);
                }
            }
        if (logits && r < M) {
#pragma unroll
            for (int a = 0; a < NA; a++)
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int o = row0 + 16 * a + 4 * g + j;
                    if (o < V) logits[(size_t)r * V + o] = acc[a][j];
                }
        }
        t = merge(t, shfl_top2(t, 16));
        t = merge(t, shfl_top2(t, 32));
    }
    if (g == 0) wrec[wv][r] = t;
    __syncthreads();
    if (threadIdx.x < 16) {
        const int m = threadIdx.x;
        Top2 q = wrec[0][m];
#pragma unroll
        for (int w = 1; w < HEAD_WAVES; w++) q = merge(q, wrec[w][m]);
        part[(size_t)m * gridDim.x + blockIdx.x] = make_float4(q.v1, __int_as_float(q.i1), q.v2, 0.f);
    }
}

int head_units(int V) { return (V + 16 * HEAD_NA - 1) / (16 * HEAD_NA); }
int head_blocks(int V) { return (head_units(V) + HEAD_WAVES - 1) / HEAD_WAVES; }

void launch_head(const uint16_t *W, int tiled, const float *h, int V, int K, int M, float *logits,
                 float4 *part, const HeadNorm *nrm, hipStream_t s) {
    const int units = head_units(V);
    if (nrm)
        launch_k(PROF_HEAD, "k_head", k_head<true>, dim3(head_blocks(V)), dim3(HEAD_THREADS), 0, s, W, tiled, h, V,
                 K, M, logits, part, units, *nrm);
    else
        launch_k(PROF_HEAD, "k_head", k_head<false>, dim3(head_blocks(V)), dim3(HEAD_THREADS), 0, s, W, tiled, h,
                 V, K, M, logits, part, units, HeadNorm{});
}

// ---------------------------------------------------------------------------
// Tiling of a row-major BF16 weight [batch][N][K] into the MFMA-operand order
// described at the top of this file. One wave writes one 1 KiB (tile, k-step)
// block; padding rows/columns are written as zeros.
__global__ __launch_bounds__(256) void k_tile(const uint16_t *__restrict__ src,
                                              uint16_t *__restrict__ dst, int N, int K,
                                              long long blocks_per_mat, long long total) {
    const long long blk = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blk >= total) return;
    const int lane = threadIdx.x & 63;
    const int S = (K + 31) >> 5;
    const long long mat = blk / blocks_per_mat;
    const long long b = blk - mat * blocks_per_mat;
    const int t = (int)(b / S), st = (int)(b - (long long)t * S);
    const int row = t * 16 + (lane & 15), col = st * 32 + 8 * (lane >> 4);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < N && col < K) v = *(const uint4 *)(src + (size_t)mat * N * K + (size_t)row * K + col);
    *(uint4 *)(dst + ((size_t)mat * blocks_per_mat * 64 + (size_t)b * 64 + lane) * 8) = v;
}

size_t tiled_elems(long long N, long long K) {
    return (size_t)((N + 15) / 16) * (size_t)((K + 31) / 32) * 512;
}

void launch_tile(const uint16_t *src, uint16_t *dst, long long batch, int N, int K, hipStream_t s) {
    const long long per = (long long)((N + 15) / 16) * ((K + 31) / 32);
    const long long total = per * batch;
    launch_k(PROF_OTHER, "k_tile", k_tile, dim3((unsigned)((total + 3) / 4)), dim3(256), 0, s, src, dst, N, K,
                       per, total);
}

// one block per activation row: fold the workgroups' top-2 records of that row
// (contiguous), in a fixed order
__global__ __launch_bounds__(256) void k_head_reduce(const float4 *__restrict__ part, int blocks,
                                                     int32_t *__restrict__ argmax,
                                                     float *__restrict__ margin) {
    // the arguments into scalar registers in one round trip
    asm volatile("" ::"s"(part), "s"(blocks), "s"(argmax), "s"(margin));
    const int m = blockIdx.x;
    Top2 t{-INFINITY, 0x7fffffff, -INFINITY};
    const float4 *pm = part + (size_t)m * blocks;
    for (int u = threadIdx.x; u < blocks; u += 256) {
        const float4 p = pm[u];
        Top2 c{p.x, __float_as_int(p.y), p.z};
        t = merge(t, c);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) t = merge(t, shfl_top2(t, o));
    __shared__ Top2 sh[4];
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = t;
    __syncthreads();
    if (threadIdx.x == 0) {
        Top2 r = merge(merge(sh[0], sh[1]), merge(sh[2], sh[3]));
        argmax[m] = r.i1;
        if (margin) margin[m] = r.v1 - r.v2;
    }
}

// One workgroup: wave m folds row m's records (as k_head_reduce, same total order),
// then wave 0 runs the greedy accept walk of the drafts among those argmaxes
// against the target's argmaxes (drafts: rows 1..M-1 when draft_row0 is 1, with
// K = M - 1; row 0 with K = 1 otherwise).
__global__ __launch_bounds__(1024) void k_head_finish(const float4 *__restrict__ part, int blocks, int M,
                                                      int32_t *__restrict__ argmax, float *__restrict__ margin,
                                                      AcceptArgs acc) {
    // the arguments into scalar registers in one round trip
    asm volatile("" ::"s"(part), "s"(blocks), "s"(M), "s"(argmax), "s"(margin), "s"(acc.target), "s"(acc.K),
                 "s"(acc.first), "s"(acc.eos), "s"(acc.n_eos), "s"(acc.result), "s"(acc.committed));
    __shared__ int32_t am[16];
    const int lane = threadIdx.x & 63, m = wave_id();
    if (m < M) {
        Top2 t{-INFINITY, 0x7fffffff, -INFINITY};
        const float4 *pm = part + (size_t)m * blocks;
        for (int u = lane; u < blocks; u += 64) {
            const float4 p = pm[u];
            Top2 c{p.x, __float_as_int(p.y), p.z};
            t = merge(t, c);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) t = merge(t, shfl_top2(t, o));
        if (lane == 0) {
            argmax[m] = t.i1;
            am[m] = t.i1;
            if (margin) margin[m] = t.v1 - t.v2;
        }
    }
    __syncthreads();
    if (m == 0 && acc.target)
        accept_walk(am + acc.first, acc.target, acc.K, acc.eos, acc.n_eos, acc.result, acc.committed);
}

void launch_head_finish(const float4 *part, int blocks, int M, int32_t *argmax, float *margin,
                        const AcceptArgs &acc, hipStream_t s) {
    launch_k(PROF_HEAD, "k_head_finish", k_head_finish, dim3(1), dim3(1024), 0, s, part, blocks, M, argmax, margin,
             acc);
}

void launch_head_reduce(const float4 *part, int blocks, int M, int32_t *argmax, float *margin,
                        hipStream_t s) {
    launch_k(PROF_HEAD, "k_head_reduce", k_head_reduce, dim3(M), dim3(256), 0, s, part, blocks, argmax, margin);
}

}  // namespace dbf
