// rows.hip -- the column-parallel row kernels of the drafter block.
//
// RMSNorm (hf2q qwen35/mtp.rs `rms_norm_with_weight`: y = x / sqrt(mean(x^2)+eps) * w)
// is applied in two halves. Its row scale s_m = 1/sqrt(mean_k x_mk^2 + eps) is a
// per-row scalar, and a projection is linear, so
//     Linear(x_m * s_m (.) w, W) = s_m * Linear(x_m (.) w, W).
// The producer of a normalized input therefore only writes x (.) w (split for the
// matrix cores) plus per-64-column partial sums of x^2 ("ssp", [16][ncb]); the
// consumer of the projection's output applies s_m. No kernel needs a whole row,
// so every row kernel runs one wavefront per (row, 64 columns): many blocks, no
// serial row loop. All sums run in a fixed order.
#include "internal.hpp"
#include "kernels.hpp"

namespace dbf {

// Row scale from the per-column-block partial sums of squares; called by a whole
// wavefront (lane-strided sum, then a fixed xor tree).
__device__ __forceinline__ float row_scale(const float *ssp_row, int ncb, int H, float eps) {
    const int lane = threadIdx.x & 63;
    float s = 0.f;
    for (int i = lane; i < ncb; i += 64) s += ssp_row[i];
    s = wave_sum(s);
    return 1.0f / sqrtf(s / (float)H + eps);
}

// sum over ks split-K partials of element (row, col) in a [ks][rows][N] buffer
__device__ __forceinline__ float sum_partials(const float *p, int ks, int rows, int N, int row,
                                              int col) {
    const size_t stride = (size_t)rows * N;
    const float *q = p + (size_t)row * N + col;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    int t = 0;
    for (; t + 3 < ks; t += 4) {
        a0 += q[(t + 0) * stride];
        a1 += q[(t + 1) * stride];
        a2 += q[(t + 2) * stride];
        a3 += q[(t + 3) * stride];
    }
    for (; t < ks; t++) a0 += q[t * stride];
    return (a0 + a1) + (a2 + a3);
}

// ---------------------------------------------------------------------------
// Generic column kernel. Grid (ncb = ceil(H/64), 4), 256 threads: wave w handles
// row m = 4*blockIdx.y + w, lane the column blockIdx.x*64 + lane.
//   v = [gather embed row | base] + scale0 * sum P0 + scale1 * sum P1
//   out/copies <- v;  xs <- split(v (.) w);  ssp_out[m][cb] <- sum over the 64 columns of v^2
// Rows m >= M and padding columns write zeros into the split tile.
__global__ __launch_bounds__(256) void k_colsum(ColArgs a) {
    const int m = blockIdx.y * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int k = blockIdx.x * 64 + lane;
    const bool row_ok = m < a.M;
    const bool ok = row_ok && k < a.H;
    float v = 0.f;
    if (row_ok) {
        float sc0 = 1.f, sc1 = 1.f;
        if (a.p0 && a.ssp0) sc0 = row_scale(a.ssp0 + (size_t)m * a.ncb_in, a.ncb_in, a.H, a.eps0);
        if (a.p1 && a.ssp1) sc1 = row_scale(a.ssp1 + (size_t)m * a.ncb_in, a.ncb_in, a.H, a.eps1);
        if (ok) {
            if (a.tokens) {
                int t = a.tokens[m];
                t = t < 0 ? 0 : (t >= a.V ? a.V - 1 : t);
                v = bf16_to_f32(a.embed[(size_t)t * a.H + k]);
            } else if (a.base) {
                v = a.base[(size_t)m * a.ldb + k];
            }
            if (a.p0) v += sc0 * sum_partials(a.p0, a.ks0, a.rows0, a.H, m, k);
            if (a.p1) v += sc1 * sum_partials(a.p1, a.ks1, a.rows1, a.H, m, k);
            if (a.out) a.out[(size_t)m * a.H + k] = v;
            if (a.copy0) a.copy0[(size_t)m * a.H + k] = v;
            if (a.copy1) a.copy1[(size_t)m * a.H + k] = v;
        }
        if (a.ssp_out) {
            float ss = wave_sum(v * v);
            if (lane == 0) a.ssp_out[(size_t)m * a.ncb_out + blockIdx.x] = ss;
        }
    }
    if (a.xs && k < ((a.H + 31) & ~31)) split_store(a.xs, m, k, ok ? v * (a.w ? a.w[k] : 1.f) : 0.f);
}

void launch_colsum(const ColArgs &a, hipStream_t s) {
    const int ncb = (a.H + 63) / 64;
    const int rg = a.xs ? 4 : (a.M + 3) / 4;  // split tiles need all 16 rows written
    hipLaunchKernelGGL(k_colsum, dim3(ncb, rg), dim3(256), 0, s, a);
}

// ---------------------------------------------------------------------------
// Final norm: h_final = x * s_m (.) w.
__global__ __launch_bounds__(256) void k_final_norm(const float *x, const float *ssp, int ncb, int M,
                                                    int H, const float *w, float eps, float *out) {
    const int m = blockIdx.y * 4 + (threadIdx.x >> 6);
    const int k = blockIdx.x * 64 + (threadIdx.x & 63);
    if (m >= M) return;
    const float s = row_scale(ssp + (size_t)m * ncb, ncb, H, eps);
    if (k < H) out[(size_t)m * H + k] = x[(size_t)m * H + k] * s * w[k];
}

void launch_final_norm(const float *x, const float *ssp, int M, int H, const float *w, float eps,
                       float *out, hipStream_t s) {
    const int ncb = (H + 63) / 64;
    hipLaunchKernelGGL(k_final_norm, dim3(ncb, (M + 3) / 4), dim3(256), 0, s, x, ssp, ncb, M, H, w,
                       eps, out);
}

// ---------------------------------------------------------------------------
// Q/K/V post-processing, one wavefront per head vector (qwen35/mtp.rs
// `forward_full_attention`): sum split-K partials and apply the row's RMSNorm
// scale; per-head RMSNorm (q_norm / k_norm); rotate-half RoPE over the first
// rotary_dim lanes with angle pos * theta^(-2j/rotary_dim) formed in F64 (an F32
// product is off by ~1e-3 rad at 32k positions); store q (block rows) and the raw
// gate, or the key and value rows of the cache (F32, or BF16 with RNE).
// Blocks [0, M*nq) are q heads of block rows; then (R+M)*nkv k/v heads, context
// rows first. DFlash context rows sit at positions P0+r, block rows at P0+R+m.
__global__ __launch_bounds__(64) void k_qkv_post(QkvPostArgs a) {
    __shared__ float vec[256];
    const int lane = threadIdx.x;
    const int hd = a.hd, qt = a.nq * hd, kt = a.nkv * hd;
    const int b = blockIdx.x;
    const bool isq = b < a.M * a.nq;
    int row, head;         // row within its group (block rows or all kv rows), head index
    long long pos;
    float s;               // RMSNorm scale of the source row
    const float *src, *wn; // partial buffer, head-norm weight
    int ks, prow, N;
    if (isq) {
        row = b / a.nq;
        head = b % a.nq;
        pos = a.P0 + a.R + row;
        s = row_scale(a.ssp_x + (size_t)row * a.ncb, a.ncb, a.H, a.eps);
        src = a.pq;
        ks = a.ksq;
        prow = row;
        N = qt;
        wn = a.q_norm;
    } else {
        const int idx = b - a.M * a.nq;
        row = idx / a.nkv;  // 0..R+M-1, context rows first
        head = idx % a.nkv;
        const bool ctx = row < a.R;
        const int m = ctx ? row : row - a.R;
        pos = ctx ? a.P0 + row : a.P0 + a.R + m;
        s = ctx ? row_scale(a.ssp_ctx + (size_t)m * a.ncb, a.ncb, a.H, a.eps)
                : row_scale(a.ssp_x + (size_t)m * a.ncb, a.ncb, a.H, a.eps);
        src = a.pk;
        ks = a.ksk;
        prow = ctx ? m : a.kv_block_row0 + m;
        N = kt;
        wn = a.k_norm;
    }
    const int rows = isq ? 16 : a.rows_kv;
    float raw[4];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int d = lane + 64 * i;
        raw[i] = 0.f;
        if (d < hd) {
            raw[i] = s * sum_partials(src, ks, rows, N, prow, head * hd + d);
            ss += raw[i] * raw[i];
        }
    }
    const float hs = 1.0f / sqrtf(wave_sum(ss) / (float)hd + a.eps);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int d = lane + 64 * i;
        if (d < hd) vec[d] = raw[i] * hs * wn[d];
    }
    __syncthreads();
    const int half = a.rotary_dim / 2;
    const size_t cache_off = ((size_t)head * a.capacity + pos) * hd;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int d = lane + 64 * i;
        if (d >= hd) continue;
        float val = vec[d];
        if (d < 2 * half) {
            const int j = d < half ? d : d - half;
            const float pv = vec[d < half ? d + half : d - half];
            const double ang = (double)pos * pow(a.theta, -2.0 * (double)j / (double)a.rotary_dim);
            double sn, cs;
            sincos(ang, &sn, &cs);
            const float c = (float)cs, sv = (float)sn;
            val = d < half ? val * c - pv * sv : pv * sv + val * c;
        }
        if (isq) {
            a.q_out[(size_t)row * qt + head * hd + d] = val;
        } else {
            if (a.kv_bf16) ((uint16_t *)a.cache_k)[cache_off + d] = f32_to_bf16(val);
            else ((float *)a.cache_k)[cache_off + d] = val;
        }
    }
    // the gate (q blocks) and the value row (k blocks): same source row, no head norm
    if (isq && a.pg) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int d = lane + 64 * i;
            if (d < hd)
                a.g_out[(size_t)row * qt + head * hd + d] =
                    s * sum_partials(a.pg, a.ksg, 16, qt, row, head * hd + d);
        }
    }
    if (!isq) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int d = lane + 64 * i;
            if (d >= hd) continue;
            const float v = s * sum_partials(a.pv, a.ksv, a.rows_kv, kt, prow, head * hd + d);
            if (a.kv_bf16) ((uint16_t *)a.cache_v)[cache_off + d] = f32_to_bf16(v);
            else ((float *)a.cache_v)[cache_off + d] = v;
        }
    }
}

void launch_qkv_post(const QkvPostArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_qkv_post, dim3(a.M * a.nq + (a.R + a.M) * a.nkv), dim3(64), 0, s, a);
}

// ---------------------------------------------------------------------------
// SwiGLU: h = silu(s_m * sum P_gate) * (s_m * sum P_up), split for the down
// projection (s_m: RMSNorm scale of the FFN input row).
__global__ __launch_bounds__(256) void k_swiglu(SwigluArgs a) {
    const int m = blockIdx.y * 4 + (threadIdx.x >> 6);
    const int k = blockIdx.x * 64 + (threadIdx.x & 63);
    const int Ip = (a.I + 31) & ~31;
    float h = 0.f;
    if (m < a.M) {
        const float s = row_scale(a.ssp + (size_t)m * a.ncb, a.ncb, a.H, a.eps);
        if (k < a.I) {
            const float g = s * sum_partials(a.pg, a.ksg, 16, a.I, m, k);
            const float u = s * sum_partials(a.pu, a.ksu, 16, a.I, m, k);
            h = g / (1.0f + expf(-g)) * u;
        }
    }
    if (k < Ip) split_store(a.xs, m, k, h);
}

void launch_swiglu(const SwigluArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_swiglu, dim3((a.I + 63) / 64, 4), dim3(256), 0, s, a);
}

}  // namespace dbf
