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

// Selection keys: (value, index) as one 64-bit unsigned integer whose order is the
// pick order -- the high word maps a float (NaN excluded, -0 folded into +0
// beforehand) to an unsigned integer of the same order, the low word is ~index so
// that equal values rank the lower index first. Key 0 is below every expert's key:
// it marks an expert that is out of range or already picked.
__device__ __forceinline__ unsigned order_key(float v) {
    const unsigned u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(unsigned k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ void key_max(unsigned &h, unsigned &l, unsigned h2, unsigned l2) {
    const unsigned long long a = ((unsigned long long)h << 32) | l;
    const unsigned long long b = ((unsigned long long)h2 << 32) | l2;
    const bool t = b > a;
    h = t ? h2 : h;
    l = t ? l2 : l;
}

// one DPP exchange step of the key maximum; lanes in rows ROWMASK leaves out keep
// their own key
template <int CTRL, int ROWMASK>
__device__ __forceinline__ void dpp_key_step(unsigned &h, unsigned &l) {
    const unsigned h2 = __builtin_amdgcn_update_dpp(h, h, CTRL, ROWMASK, 0xF, false);
    const unsigned l2 = __builtin_amdgcn_update_dpp(l, l, CTRL, ROWMASK, 0xF, false);
    key_max(h, l, h2, l2);
}

// maximum key over the wave, returned in scalar registers: within each row of 16
// lanes (lane xor 1, xor 2, then rotations by 4 and 8 leave the row maximum in
// every lane of the row), then row 1 takes row 0's and row 3 row 2's (row_bcast
// 15), then row 3 takes row 1's (row_bcast 31): lane 63 holds the maximum.
__device__ __forceinline__ void wave_key_max(unsigned &h, unsigned &l) {
    dpp_key_step<0xB1, 0xF>(h, l);   // quad_perm [1, 0, 3, 2]
    dpp_key_step<0x4E, 0xF>(h, l);   // quad_perm [2, 3, 0, 1]
    dpp_key_step<0x124, 0xF>(h, l);  // row_ror 4
    dpp_key_step<0x128, 0xF>(h, l);  // row_ror 8
    dpp_key_step<0x142, 0xA>(h, l);  // row_bcast 15 into rows 1 and 3
    dpp_key_step<0x143, 0xC>(h, l);  // row_bcast 31 into rows 2 and 3
    h = __builtin_amdgcn_readlane(h, 63);
    l = __builtin_amdgcn_readlane(l, 63);
}

// Routing in one block of 1024 threads. Rows go in passes of up to 16 (and
// rows * E <= ROUTE_Z logits): every thread sums the router partials of its
// (row, expert) entries into LDS (the first pass also sums each row's shared-expert
// gate logit, so those loads go out in the same round trip), then wave w picks the
// top_k of the pass's row w with no block barrier between picks: lane l holds the
// selection keys of experts l, l + 64, ... and its best one not yet picked; a pick
// is the wave-wide maximum of those, after which the picked key is cleared and the
// lanes rescan their (at most 16) keys. The touched experts are compacted in ascending order with a
// ballot prefix, and each (slot, row) coefficient is written exactly once. A NaN
// logit ranks as -inf, so every pick is an in-range expert.
constexpr int ROUTE_THREADS = 1024;         // one thread per expert at E = 1024
constexpr int ROUTE_WAVES = ROUTE_THREADS / 64;
constexpr int ROUTE_Z = 8192;               // router logits held in LDS per pass

// EPL: experts per lane, a power of two >= E / 64 (at most 16 at E = 1024)
template <int EPL>
__global__ __launch_bounds__(ROUTE_THREADS) void k_moe_route(MoeRouteArgs a) {
    // the arguments into scalar registers in one round trip
    asm volatile("" ::"s"(a.p_router), "s"(a.ks_router), "s"(a.p_sgi), "s"(a.ks_sgi), "s"(a.ssp), "s"(a.ncb),
                 "s"(a.H), "s"(a.eps), "s"(a.M), "s"(a.E), "s"(a.top_k), "s"(a.max_slots), "s"(a.nslots),
                 "s"(a.slot_expert), "s"(a.coef), "s"(a.shared_scale), "s"(a.sel));
    __shared__ float z[ROUTE_Z];            // unscaled router sums, [pass row][E]
    __shared__ float gz[16];                // unscaled shared-expert gate sums
    __shared__ float rscale[16];
    __shared__ unsigned char used[1024];
    __shared__ int esel[16 * DBF_MAX_TOPK_DEV];
    __shared__ float wsel[16 * DBF_MAX_TOPK_DEV];
    __shared__ int sexp[1024];
    __shared__ int wtot[ROUTE_WAVES];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int E = a.E, K = a.top_k, M = a.M;
    const int rg = ROUTE_Z / E < ROUTE_WAVES ? ROUTE_Z / E : ROUTE_WAVES;  // >= 8
    const int ks_max = a.ks_router > a.ks_sgi ? a.ks_router : a.ks_sgi;
    for (int e = tid; e < E; e += ROUTE_THREADS) used[e] = 0;
    // row scale, one wave per row (rows <= 16 = ROUTE_WAVES): the first 128 norm
    // partials load with the router partials; the scale is finished after them
    const float *sr = a.ssp + (size_t)(wv < M ? wv : 0) * a.ncb;
    float f0 = 0.f, f1 = 0.f;  // added only after the router sums: no wait before them
    if (wv < M) {
        f0 = lane < a.ncb ? sr[lane] : 0.f;
        f1 = lane + 64 < a.ncb ? sr[lane + 64] : 0.f;
    }
    for (int m0 = 0; m0 < M; m0 += rg) {
        const int rows = M - m0 < rg ? M - m0 : rg;
        const int nz = rows * E, nall = nz + (m0 == 0 ? M : 0);
        for (int i = tid; i < nall; i += ROUTE_THREADS) {
            const float *b[1];
            int ks;
            size_t stride;
            float *dst;
            if (i < nz) {
                const int r = i / E;
                b[0] = a.p_router + (size_t)(m0 + r) * E + (i - r * E);
                ks = a.ks_router;
                stride = (size_t)16 * E;
                dst = &z[i];
            } else {
                b[0] = a.p_sgi + (i - nz);
                ks = a.ks_sgi;
                stride = 16;
                dst = &gz[i - nz];
            }
            float o[1];
            if (ks_max > PARTIAL_BATCH)
                sum_partials_n<1, 24>(b, ks, stride, o);
            else
                sum_partials_n<1>(b, ks, stride, o);
            *dst = o[0];
        }
        __syncthreads();
        if (m0 == 0 && wv < M) {
            asm volatile("" : "+v"(f0));  // keeps the add (and its wait) from being hoisted
            float s = f0 + f1;
            for (int i = lane + 128; i < a.ncb; i += 64) s += sr[i];
            s = wave_sum(s);
            s = 1.0f / sqrtf(s / (float)a.H + a.eps);
            if (lane == 0) {
                rscale[wv] = s;
                a.shared_scale[wv] = sigmoidf_(s * gz[wv]);
            }
        }
        __syncthreads();
        if (wv < rows) {
            const int m = m0 + wv;
            const float s = rscale[m];
            unsigned kh[EPL], kl[EPL];  // keys of experts lane + 64 j
#pragma unroll
            for (int j = 0; j < EPL; j++) {
                const int e = lane + 64 * j;
                // the read is clamped into the row, not branched around
                float v = s * z[wv * E + (e < E ? e : E - 1)] + 0.f;  // + 0 folds -0 into +0
                v = v != v ? -INFINITY : v;
                kh[j] = e < E ? order_key(v) : 0u;
                kl[j] = e < E ? ~(unsigned)e : 0u;
            }
            unsigned bh = 0u, bl = 0u;  // this lane's best key
#pragma unroll
            for (int j = 0; j < EPL; j++) key_max(bh, bl, kh[j], kl[j]);
            float myv = 0.f;  // lane t keeps pick t
            int myi = 0;
            for (int t = 0; t < K; t++) {
                unsigned h = bh, l = bl;
                wave_key_max(h, l);
                // K <= E real keys existed, so the maximum is a real, untaken expert;
                // the clamp only keeps an index in range whatever the keys hold
                int e = (int)~l;
                e = e < 0 ? 0 : (e >= E ? E - 1 : e);
                if (lane == t) {
                    myv = key_value(h);
                    myi = e;
                }
                if (t + 1 < K) {
                    // the low word names the expert: clear its key and rescan
                    bh = 0u;
                    bl = 0u;
#pragma unroll
                    for (int j = 0; j < EPL; j++) {
                        const bool hit = kl[j] == l;
                        kh[j] = hit ? 0u : kh[j];
                        kl[j] = hit ? 0u : kl[j];
                        key_max(bh, bl, kh[j], kl[j]);
                    }
                }
            }
            // renormalised top-k weights: softmax over the kept logits, summed in pick order
            const float zmax = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(myv), 0));
            const float ex = lane < K ? expf(myv - zmax) : 0.f;
            float den = 0.f;
            for (int t = 0; t < K; t++) den += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), t));
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
    const int epl = (a.E + 63) / 64;  // E <= 1024
    if (epl <= 1)
        launch_k(PROF_ROWS, "k_moe_route", k_moe_route<1>, dim3(1), dim3(ROUTE_THREADS), 0, s, a);
    else if (epl <= 2)
        launch_k(PROF_ROWS, "k_moe_route", k_moe_route<2>, dim3(1), dim3(ROUTE_THREADS), 0, s, a);
    else if (epl <= 4)
        launch_k(PROF_ROWS, "k_moe_route", k_moe_route<4>, dim3(1), dim3(ROUTE_THREADS), 0, s, a);
    else if (epl <= 8)
        launch_k(PROF_ROWS, "k_moe_route", k_moe_route<8>, dim3(1), dim3(ROUTE_THREADS), 0, s, a);
    else
        launch_k(PROF_ROWS, "k_moe_route", k_moe_route<16>, dim3(1), dim3(ROUTE_THREADS), 0, s, a);
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
