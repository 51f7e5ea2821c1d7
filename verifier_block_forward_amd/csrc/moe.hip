// moe.hip -- MoE FFN of the MTP block: routing, expert SwiGLU and the combine.
//
// (hf2q qwen35/mtp.rs: `MtpFfnWeightsGpu::Moe`, run by `forward_ffn_residual`;
// router `ffn_gate_inp`, experts `ffn_{gate,up,down}_exps`, and a shared expert
// with its own sigmoid gate. The page's experts are quantized GGML blocks; here
// they are BF16.)
//   y = sum_{e in top_k(softmax(x Wr^T))} w_e SwiGLU_e(x) + sigmoid(x . w_sg) SwiGLU_sh(x)
// with the top_k probabilities renormalised to sum to one. Because that
// renormalisation divides by the kept probabilities only, w_t = exp(z_t - z_max) /
// sum_{s in top_k} exp(z_s - z_max): the full softmax denominator cancels.
// Selection orders by logit, ties to the lower expert index.
//
// The experts a block touches are known only on the device, so routing writes a
// de-duplicated, ascending slot list (slot -> expert) plus each row's weight per
// slot; the grouped projections run over a fixed grid sized for min(E, M*top_k)
// slots and surplus slots exit immediately. Every touched expert is applied to all
// M rows (rows that did not pick it get weight 0), which costs matrix-core work
// but no extra weight bytes.
#include "internal.hpp"
#include "kernels.hpp"

namespace dbf {

// (value, index) with ties to the lower index
__device__ __forceinline__ void better_pair(float &v, int &i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

// Routing in one block of 1024 threads. Rows go in passes of up to 16 (and
// rows * E <= ROUTE_Z logits): every thread sums the router partials of its
// (row, expert) entries into LDS, then wave w picks the top_k of the pass's row w
// with cross-lane shuffles only, one pick per round and no block barrier between
// picks. The touched experts are compacted in ascending order with a ballot
// prefix, and each (slot, row) coefficient is written exactly once. A NaN logit
// ranks as -inf, so every pick is an in-range expert.
constexpr int ROUTE_THREADS = 1024;         // one thread per expert at E = 1024
constexpr int ROUTE_WAVES = ROUTE_THREADS / 64;
constexpr int ROUTE_Z = 8192;               // router logits held in LDS per pass
constexpr int ROUTE_EPL = 1024 / 64;        // experts per lane at E = 1024

__global__ __launch_bounds__(ROUTE_THREADS) void k_moe_route(MoeRouteArgs a) {
    // the arguments into scalar registers in one round trip
    asm volatile("" ::"s"(a.p_router), "s"(a.ks_router), "s"(a.p_sgi), "s"(a.ks_sgi), "s"(a.ssp), "s"(a.ncb),
                 "s"(a.H), "s"(a.eps), "s"(a.M), "s"(a.E), "s"(a.top_k), "s"(a.max_slots), "s"(a.nslots),
                 "s"(a.slot_expert), "s"(a.coef), "s"(a.shared_scale), "s"(a.sel));
    __shared__ float z[ROUTE_Z];            // unscaled router sums, [pass row][E]
    __shared__ float rscale[16];
    __shared__ unsigned char used[1024];
    __shared__ int esel[16 * DBF_MAX_TOPK_DEV];
    __shared__ float wsel[16 * DBF_MAX_TOPK_DEV];
    __shared__ int sexp[1024];
    __shared__ int wtot[ROUTE_WAVES];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int E = a.E, K = a.top_k, M = a.M;
    const int rg = ROUTE_Z / E < ROUTE_WAVES ? ROUTE_Z / E : ROUTE_WAVES;  // >= 8
    for (int e = tid; e < E; e += ROUTE_THREADS) used[e] = 0;
    // row scale and shared-expert gate, one wave per row: the norm partials and the
    // gate's split-K partials load together; the scale is finished after the first
    // pass's router sums (rows <= 16 = ROUTE_WAVES, so one wave per row)
    const float *sr = a.ssp + (size_t)(wv < M ? wv : 0) * a.ncb;
    float f = 0.f, gsum = 0.f;
    if (wv < M) {
        f = row_scale_first(sr, a.ncb);
        gsum = sum_partials(a.p_sgi, a.ks_sgi, 16, 1, wv, 0);
    }
    for (int m0 = 0; m0 < M; m0 += rg) {
        const int rows = M - m0 < rg ? M - m0 : rg;
        for (int i = tid; i < rows * E; i += ROUTE_THREADS) {
            const int r = i / E;
            z[i] = sum_partials(a.p_router, a.ks_router, 16, E, m0 + r, i - r * E);
        }
        if (m0 == 0 && wv < M) {
            const float s = row_scale_finish(f, sr, a.ncb, a.H, a.eps);
            if (lane == 0) {
                rscale[wv] = s;
                a.shared_scale[wv] = sigmoidf_(s * gsum);
            }
        }
        __syncthreads();
        if (wv < rows) {
            const int m = m0 + wv;
            const float s = rscale[m];
            float zr[ROUTE_EPL];
            unsigned taken = 0;  // bit j: expert lane + 64 j is out of range or already picked
#pragma unroll
            for (int j = 0; j < ROUTE_EPL; j++) {
                const int e = lane + 64 * j;
                float v = e < E ? s * z[wv * E + e] : 0.f;
                zr[j] = v != v ? -INFINITY : v;
                if (e >= E) taken |= 1u << j;
            }
            float myv = 0.f;  // lane t keeps pick t
            int myi = 0;
            for (int t = 0; t < K; t++) {
                float bv = -INFINITY;
                int bi = 0x7fffffff;
#pragma unroll
                for (int j = 0; j < ROUTE_EPL; j++)
                    if (!((taken >> j) & 1u)) better_pair(bv, bi, zr[j], lane + 64 * j);
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) {
                    const float v2 = __shfl_xor(bv, o, 64);
                    const int i2 = __shfl_xor(bi, o, 64);
                    better_pair(bv, bi, v2, i2);
                }
                // all lanes agree on (bv, bi); bi < E because K <= E untaken entries existed
                if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
                if (lane == t) {
                    myv = bv;
                    myi = bi;
                }
            }
            // renormalised top-k weights: softmax over the kept logits, summed in pick order
            const float zmax = __shfl(myv, 0, 64);
            const float ex = lane < K ? expf(myv - zmax) : 0.f;
            float den = 0.f;
            for (int t = 0; t < K; t++) den += __shfl(ex, t, 64);
            if (lane < K) {
                esel[m * DBF_MAX_TOPK_DEV + lane] = myi;
                wsel[m * DBF_MAX_TOPK_DEV + lane] = ex / den;
                a.sel[m * K + lane] = myi;
                used[myi] = 1;
            }
        }
        __syncthreads();
    }
    // ascending slot list: ballot prefix over expert e = tid
    const bool u = tid < E && used[tid];
    const unsigned long long bal = __ballot(u);
    const int below = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wtot[wv] = __popcll(bal);
    __syncthreads();
    int off = 0, total = 0;
#pragma unroll
    for (int w = 0; w < ROUTE_WAVES; w++) {
        const int c = wtot[w];
        off += w < wv ? c : 0;
        total += c;
    }
    if (u) {
        a.slot_expert[off + below] = tid;
        sexp[off + below] = tid;
    }
    if (tid == 0) {
        *a.nslots = total;
        if (a.touched_out) *a.touched_out = total;
    }
    __syncthreads();
    // coefficient of (slot, row): the row's weight for the slot's expert, else 0;
    // slots past the touched ones get 0, so a reader needs no slot count
    for (int i = tid; i < a.max_slots * 16; i += ROUTE_THREADS) {
        const int sl = i >> 4, m = i & 15;
        float c = 0.f;
        if (sl < total && m < M) {
            const int e = sexp[sl];
            for (int t = 0; t < K; t++)
                if (esel[m * DBF_MAX_TOPK_DEV + t] == e) c = wsel[m * DBF_MAX_TOPK_DEV + t];
        }
        a.coef[i] = c;
    }
}

void launch_moe_route(const MoeRouteArgs &a, hipStream_t s) {
    launch_k(PROF_ROWS, "k_moe_route", k_moe_route, dim3(1), dim3(ROUTE_THREADS), 0, s, a);
}

// Expert (and shared-expert) SwiGLU: h = silu(s_m * sum P_gate) * (s_m * sum P_up),
// split for the down projections. Grid (cols/64, 4 row groups, max_slots + 1); the
// last z-slice is the shared expert.
__global__ __launch_bounds__(256) void k_moe_swiglu(MoeSwigluArgs a) {
    // the arguments into scalar registers in one round trip
    asm volatile("" ::"s"(a.pg), "s"(a.pu), "s"(a.ks), "s"(a.psg), "s"(a.psu), "s"(a.ks_sh), "s"(a.ssp),
                 "s"(a.ncb), "s"(a.H), "s"(a.eps), "s"(a.M), "s"(a.Ie), "s"(a.Is), "s"(a.max_slots),
                 "s"(a.nslots), "s"(a.xs_e), "s"(a.xs_sh));
    const int slot = blockIdx.z;
    const bool shared = slot == a.max_slots;
    // the slot count, the row-scale share and the partials load together: a slot
    // past the count reads its (allocated, unused) partials and leaves afterwards
    const int ns = shared ? 0 : *a.nslots;
    const int I = shared ? a.Is : a.Ie;
    const int m = blockIdx.y * 4 + wave_id();
    const int k = blockIdx.x * 64 + (threadIdx.x & 63);
    const int Ip = (I + 31) & ~31;
    float h = 0.f;
    const float *sr = a.ssp + (size_t)(m < a.M ? m : 0) * a.ncb;
    const float f = m < a.M ? row_scale_first(sr, a.ncb) : 0.f;
    if (m < a.M) {
        float g = 0.f, u = 0.f;
        if (k < I) {
            const float *pg = shared ? a.psg : a.pg + (size_t)slot * a.ks * 16 * I;
            const float *pu = shared ? a.psu : a.pu + (size_t)slot * a.ks * 16 * I;
            const size_t off = (size_t)m * I + k;
            const float *b[2] = {pg + off, pu + off};
            float o[2];
            sum_partials_n<2>(b, shared ? a.ks_sh : a.ks, (size_t)16 * I, o);
            g = o[0];
            u = o[1];
        }
        // whole wave (wave-uniform m) forms the row scale: no lane has left yet
        const float s = row_scale_finish(f, sr, a.ncb, a.H, a.eps);
        if (k < I) {
            g *= s;
            u *= s;
            h = g / (1.0f + expf(-g)) * u;
        }
    }
    if (!shared && slot >= ns) return;  // whole block: slot is uniform
    uint16_t *xs = shared ? a.xs_sh : a.xs_e + (size_t)slot * (split_tile_bytes(a.Ie) / 2);
    if (k < Ip) split_store(xs, m, k, h);
}

void launch_moe_swiglu(const MoeSwigluArgs &a, hipStream_t s) {
    const int I = a.Ie > a.Is ? a.Ie : a.Is;
    launch_k(PROF_ROWS, "k_moe_swiglu", k_moe_swiglu, dim3((I + 63) / 64, 4, a.max_slots + 1), dim3(256), 0, s, a);
}

// x = x1 + sum_slots coef[slot][m] * down_slot + shared_scale[m] * down_shared; then the
// same outputs as the column kernel (copies, split of x * w, norm partials).
// The routed sum reads each selected slot's down partials. The row's selected
// slots come from one wave-wide load of the coefficients per 64 slots and a
// ballot, and up to MOE_CB slots have their partials loaded together, so a row
// pays about one memory round trip per MOE_CB experts (and per slice) instead of
// one per expert. Additions keep the order slot ascending, slice ascending.
constexpr int MOE_CB = 8;

__global__ __launch_bounds__(256) void k_moe_combine(MoeCombineArgs a) {
    // the arguments into scalar registers in one round trip
    asm volatile("" ::"s"(a.base), "s"(a.pd), "s"(a.ks), "s"(a.psd), "s"(a.ks_sh), "s"(a.coef),
                 "s"(a.shared_scale), "s"(a.M), "s"(a.H), "s"(a.max_slots), "s"(a.out), "s"(a.copy0),
                 "s"(a.copy1), "s"(a.w), "s"(a.xs), "s"(a.ssp_out), "s"(a.ncb));
    const int m = blockIdx.y * 4 + wave_id();
    const int lane = threadIdx.x & 63;
    const int k = blockIdx.x * 64 + lane;
    const bool row_ok = m < a.M;  // wave-uniform
    const bool ok = row_ok && k < a.H;
    const int kc = k < a.H ? k : a.H - 1;  // lanes past H load a valid column, unused
    float v = 0.f;
    // the base value and the norm weight go out with the first loads
    const float bv = ok ? a.base[(size_t)m * a.H + k] : 0.f;
    const float wk = ok && a.xs && a.w ? a.w[k] : 1.f;
    if (row_ok) {
        const int ns = a.max_slots;  // coefficients past the touched slots are 0
        const size_t col = (size_t)m * a.H + kc;
        const size_t pstride = (size_t)16 * a.H;  // between slices
        // shared expert first: its loads go out with the routed ones
        const float ysh = a.shared_scale[m] * sum_partials(a.psd, a.ks_sh, 16, a.H, m, kc);
        float y = 0.f;
        for (int s0 = 0; s0 < ns; s0 += 64) {
            const int sl = s0 + lane;
            const float c = sl < ns ? a.coef[(size_t)sl * 16 + m] : 0.f;
            unsigned long long bal = __ballot(c != 0.f);
            while (bal) {
                int js[MOE_CB];
                float cs[MOE_CB];
                int nb = 0;
#pragma unroll
                for (int j = 0; j < MOE_CB; j++) {
                    js[j] = s0;
                    cs[j] = 0.f;
                    if (bal) {
                        const int b = __ffsll((long long)bal) - 1;
                        bal &= bal - 1;
                        js[j] = s0 + b;
                        cs[j] = __shfl(c, b, 64);
                        nb = j + 1;
                    }
                }
                float acc[MOE_CB];
#pragma unroll
                for (int j = 0; j < MOE_CB; j++) acc[j] = 0.f;
                for (int t = 0; t < a.ks; t++) {
                    float x[MOE_CB];
#pragma unroll
                    for (int j = 0; j < MOE_CB; j++)
                        x[j] = a.pd[((size_t)js[j] * a.ks + t) * pstride + col];
#pragma unroll
                    for (int j = 0; j < MOE_CB; j++) acc[j] += j < nb ? x[j] : 0.f;
                }
#pragma unroll
                for (int j = 0; j < MOE_CB; j++)
                    if (j < nb) y += cs[j] * acc[j];
            }
        }
        y += ysh;
        if (ok) {
            v = bv + y;
            if (a.out) a.out[(size_t)m * a.H + k] = v;
            if (a.copy0) a.copy0[(size_t)m * a.H + k] = v;
            if (a.copy1) a.copy1[(size_t)m * a.H + k] = v;
        }
    }
    if (row_ok && a.ssp_out) {
        const float ss = wave_sum(v * v);
        if (lane == 0) a.ssp_out[(size_t)m * a.ncb + blockIdx.x] = ss;
    }
    if (a.xs && k < ((a.H + 31) & ~31)) split_store(a.xs, m, k, ok ? v * wk : 0.f);
}

void launch_moe_combine(const MoeCombineArgs &a, hipStream_t s) {
    const int ncb = (a.H + 63) / 64;
    launch_k(PROF_ROWS, "k_moe_combine", k_moe_combine, dim3(ncb, a.xs ? 4 : (a.M + 3) / 4), dim3(256), 0, s, a);
}

}  // namespace dbf
