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

__device__ __forceinline__ float moe_row_scale(const float *ssp_row, int ncb, int H, float eps) {
    const int lane = threadIdx.x & 63;
    float s = 0.f;
    for (int i = lane; i < ncb; i += 64) s += ssp_row[i];
    s = wave_sum(s);
    return 1.0f / sqrtf(s / (float)H + eps);
}

// (value, index) with ties to the lower index
__device__ __forceinline__ void better_pair(float &v, int &i, float v2, int i2) {
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

// One block: route every row, then build the slot list.
__global__ __launch_bounds__(256) void k_moe_route(MoeRouteArgs a) {
    __shared__ float z[1024];
    __shared__ unsigned char taken[1024];
    __shared__ unsigned char used[1024];
    __shared__ float rv[4];
    __shared__ int ri[4];
    __shared__ int esel[16 * DBF_MAX_TOPK_DEV];
    __shared__ float wsel[16 * DBF_MAX_TOPK_DEV];
    __shared__ int slot_of[1024];
    __shared__ int nsl;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int E = a.E, K = a.top_k;
    for (int e = tid; e < E; e += 256) used[e] = 0;
    __syncthreads();
    for (int m = 0; m < a.M; m++) {
        const float s = moe_row_scale(a.ssp + (size_t)m * a.ncb, a.ncb, a.H, a.eps);
        for (int e = tid; e < E; e += 256) {
            z[e] = s * sum_partials(a.p_router, a.ks_router, 16, E, m, e);
            taken[e] = 0;
        }
        __syncthreads();
        for (int t = 0; t < K; t++) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
            for (int e = tid; e < E; e += 256)
                if (!taken[e]) better_pair(bv, bi, z[e], e);
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const float v2 = __shfl_xor(bv, o, 64);
                const int i2 = __shfl_xor(bi, o, 64);
                better_pair(bv, bi, v2, i2);
            }
            if (lane == 0) {
                rv[wv] = bv;
                ri[wv] = bi;
            }
            __syncthreads();
            if (tid == 0) {
                float v = rv[0];
                int i = ri[0];
                for (int w = 1; w < 4; w++) better_pair(v, i, rv[w], ri[w]);
                esel[m * DBF_MAX_TOPK_DEV + t] = i;
                wsel[m * DBF_MAX_TOPK_DEV + t] = v;  // logit for now
                taken[i] = 1;
                used[i] = 1;
            }
            __syncthreads();
        }
        if (tid == 0) {
            // renormalised top-k weights: softmax over the kept logits
            const float zmax = wsel[m * DBF_MAX_TOPK_DEV];
            float den = 0.f;
            for (int t = 0; t < K; t++) {
                const float e = expf(wsel[m * DBF_MAX_TOPK_DEV + t] - zmax);
                wsel[m * DBF_MAX_TOPK_DEV + t] = e;
                den += e;
            }
            for (int t = 0; t < K; t++) {
                wsel[m * DBF_MAX_TOPK_DEV + t] /= den;
                a.sel[m * K + t] = esel[m * DBF_MAX_TOPK_DEV + t];
            }
        }
        if (wv == 0) {
            const float g = s * sum_partials(a.p_sgi, a.ks_sgi, 16, 1, m, 0);
            if (lane == 0) a.shared_scale[m] = sigmoidf_(g);
        }
        __syncthreads();
    }
    if (tid == 0) {
        int n = 0;
        for (int e = 0; e < E; e++) {
            slot_of[e] = -1;
            if (used[e]) {
                slot_of[e] = n;
                a.slot_expert[n] = e;
                n++;
            }
        }
        nsl = n;
        *a.nslots = n;
    }
    __syncthreads();
    for (int i = tid; i < nsl * 16; i += 256) a.coef[i] = 0.f;
    __syncthreads();
    if (tid < 16 && tid < a.M) {
        const int m = tid;
        for (int t = 0; t < K; t++)
            a.coef[(size_t)slot_of[esel[m * DBF_MAX_TOPK_DEV + t]] * 16 + m] = wsel[m * DBF_MAX_TOPK_DEV + t];
    }
}

void launch_moe_route(const MoeRouteArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_moe_route, dim3(1), dim3(256), 0, s, a);
}

// Expert (and shared-expert) SwiGLU: h = silu(s_m * sum P_gate) * (s_m * sum P_up),
// split for the down projections. Grid (cols/64, 4 row groups, max_slots + 1); the
// last z-slice is the shared expert.
__global__ __launch_bounds__(256) void k_moe_swiglu(MoeSwigluArgs a) {
    const int slot = blockIdx.z;
    const bool shared = slot == a.max_slots;
    if (!shared && slot >= *a.nslots) return;
    const int I = shared ? a.Is : a.Ie;
    const int m = blockIdx.y * 4 + (threadIdx.x >> 6);
    const int k = blockIdx.x * 64 + (threadIdx.x & 63);
    const int Ip = (I + 31) & ~31;
    float h = 0.f;
    if (m < a.M) {
        float g = 0.f, u = 0.f;
        if (k < I) {  // partial loads first; the row scale forms while they arrive
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
        const float s = moe_row_scale(a.ssp + (size_t)m * a.ncb, a.ncb, a.H, a.eps);
        if (k < I) {
            g *= s;
            u *= s;
            h = g / (1.0f + expf(-g)) * u;
        }
    }
    uint16_t *xs = shared ? a.xs_sh : a.xs_e + (size_t)slot * (split_tile_bytes(a.Ie) / 2);
    if (k < Ip) split_store(xs, m, k, h);
}

void launch_moe_swiglu(const MoeSwigluArgs &a, hipStream_t s) {
    const int I = a.Ie > a.Is ? a.Ie : a.Is;
    hipLaunchKernelGGL(k_moe_swiglu, dim3((I + 63) / 64, 4, a.max_slots + 1), dim3(256), 0, s, a);
}

// x = x1 + sum_slots coef[slot][m] * down_slot + shared_scale[m] * down_shared; then the
// same outputs as the column kernel (copies, split of x * w, norm partials).
__global__ __launch_bounds__(256) void k_moe_combine(MoeCombineArgs a) {
    const int m = blockIdx.y * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int k = blockIdx.x * 64 + lane;
    const bool row_ok = m < a.M;
    const bool ok = row_ok && k < a.H;
    float v = 0.f;
    if (ok) {
        v = a.base[(size_t)m * a.H + k];
        const int ns = *a.nslots;
        float y = 0.f;
        for (int sl = 0; sl < ns; sl++) {
            const float c = a.coef[(size_t)sl * 16 + m];
            if (c != 0.f)
                y += c * sum_partials(a.pd + (size_t)sl * a.ks * 16 * a.H, a.ks, 16, a.H, m, k);
        }
        y += a.shared_scale[m] * sum_partials(a.psd, a.ks_sh, 16, a.H, m, k);
        v += y;
        if (a.out) a.out[(size_t)m * a.H + k] = v;
        if (a.copy0) a.copy0[(size_t)m * a.H + k] = v;
        if (a.copy1) a.copy1[(size_t)m * a.H + k] = v;
    }
    if (row_ok && a.ssp_out) {
        const float ss = wave_sum(v * v);
        if (lane == 0) a.ssp_out[(size_t)m * a.ncb + blockIdx.x] = ss;
    }
    if (a.xs && k < ((a.H + 31) & ~31)) split_store(a.xs, m, k, ok ? v * (a.w ? a.w[k] : 1.f) : 0.f);
}

void launch_moe_combine(const MoeCombineArgs &a, hipStream_t s) {
    const int ncb = (a.H + 63) / 64;
    hipLaunchKernelGGL(k_moe_combine, dim3(ncb, a.xs ? 4 : (a.M + 3) / 4), dim3(256), 0, s, a);
}

}  // namespace dbf
