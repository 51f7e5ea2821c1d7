// rows.hip -- per-row kernels of the drafter block: input gathers, the fused
// "sum split-K partials + residual + RMSNorm + activation split" epilogues, the
// Q/K/V post-processing (per-head RMSNorm, RoPE, KV store) and SwiGLU.
//
// One 256-thread block per activation row; every reduction runs in a fixed order
// (thread-strided partial sums, then a fixed wave/block tree), so results are
// bit-reproducible run to run.
#include "internal.hpp"
#include "kernels.hpp"

namespace dbf {

// RMSNorm scale of a row held in `v` (n elements, strided over the block):
// 1 / sqrt(mean(v^2) + eps), hf2q qwen35/mtp.rs `rms_norm_with_weight`.
__device__ __forceinline__ float rms_scale(float ss, int n, float eps, float *sh4) {
    float tot = block_sum_256(ss, sh4);
    return 1.0f / sqrtf(tot / (float)n + eps);
}

// Write row r of a split tile from a shared/global row buffer (zeros when !valid).
__device__ __forceinline__ void split_row(uint16_t *tile, int r, const float *row, int K,
                                          bool valid, float scale, const float *w) {
    const int Kp = (K + 31) & ~31;
    for (int k = threadIdx.x; k < Kp; k += blockDim.x) {
        float a = 0.f;
        if (valid && k < K) a = row[k] * scale * (w ? w[k] : 1.0f);
        split_store(tile, r, k, a);
    }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_split_rows(const float *X, int rows, int K, int ldx,
                                                    uint16_t *tile) {
    const int r = blockIdx.x;
    split_row(tile, r, X + (size_t)r * ldx, K, r < rows, 1.0f, nullptr);
}

void launch_split_rows(const float *X, int rows, int K, int ldx, uint16_t *tile, hipStream_t s) {
    hipLaunchKernelGGL(k_split_rows, dim3(16), dim3(256), 0, s, X, rows, K, ldx, tile);
}

// ---------------------------------------------------------------------------
// DFlash block input: x = embed[token] (BF16 -> F32 exact) or x0; xres = x;
// split(RMSNorm(x, in_norm of layer 0)).
__global__ __launch_bounds__(256) void k_input_dflash(const int32_t *tokens, const float *x0,
                                                      const uint16_t *embed, int V, int M, int H,
                                                      const float *w, float eps, float *xres,
                                                      uint16_t *xs) {
    __shared__ float sh4[4];
    extern __shared__ float row[];
    const int m = blockIdx.x;
    const bool valid = m < M;
    float ss = 0.f;
    if (valid) {
        if (tokens) {
            int t = tokens[m];
            t = t < 0 ? 0 : (t >= V ? V - 1 : t);
            const uint16_t *e = embed + (size_t)t * H;
            for (int k = threadIdx.x; k < H; k += 256) row[k] = bf16_to_f32(e[k]);
        } else {
            for (int k = threadIdx.x; k < H; k += 256) row[k] = x0[(size_t)m * H + k];
        }
        for (int k = threadIdx.x; k < H; k += 256) {
            xres[(size_t)m * H + k] = row[k];
            ss += row[k] * row[k];
        }
    }
    float sc = rms_scale(ss, H, eps, sh4);
    split_row(xs, m, row, H, valid, sc, w);
}

void launch_input_dflash(const int32_t *tokens, const float *x0, const uint16_t *embed, int V,
                         int M, int H, const float *norm_w, float eps, float *xres, uint16_t *xs,
                         hipStream_t s) {
    hipLaunchKernelGGL(k_input_dflash, dim3(16), dim3(256), H * sizeof(float), s, tokens, x0,
                       embed, V, M, H, norm_w, eps, xres, xs);
}

// ---------------------------------------------------------------------------
// MTP input halves: split(RMSNorm(e, enorm, 1e-6)) and split(RMSNorm(h, hnorm, 1e-6))
// (qwen35/mtp.rs `project_embedding_and_hidden`, eps fixed at 1e-6 there).
__global__ __launch_bounds__(256) void k_mtp_input(const float *e, const float *hp, int M, int H,
                                                   const float *enorm, const float *hnorm,
                                                   uint16_t *xs_e, uint16_t *xs_h) {
    __shared__ float sh4[4];
    const int m = blockIdx.x % 16;
    const bool second = blockIdx.x >= 16;
    const float *src = second ? hp : e;
    const float *w = second ? hnorm : enorm;
    uint16_t *xs = second ? xs_h : xs_e;
    const bool valid = m < M;
    const float *row = src + (size_t)(valid ? m : 0) * H;
    float ss = 0.f;
    if (valid)
        for (int k = threadIdx.x; k < H; k += 256) ss += row[k] * row[k];
    float sc = rms_scale(ss, H, 1e-6f, sh4);
    split_row(xs, m, row, H, valid, sc, w);
}

void launch_mtp_input(const float *e, const float *hp, int M, int H, const float *enorm,
                      const float *hnorm, uint16_t *xs_e, uint16_t *xs_h, hipStream_t s) {
    hipLaunchKernelGGL(k_mtp_input, dim3(32), dim3(256), 0, s, e, hp, M, H, enorm, hnorm, xs_e,
                       xs_h);
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_sum_norm_split(SumNormArgs a) {
    __shared__ float sh4[4];
    extern __shared__ float row[];
    const int m = blockIdx.x;
    const int H = a.H;
    const bool valid = m < a.M;
    float ss = 0.f;
    if (valid) {
        for (int k = threadIdx.x; k < H; k += 256) {
            float v = a.base ? a.base[(size_t)m * H + k] : 0.f;
            float p = 0.f;
            for (int t = 0; t < a.ks0; t++) p += a.p0[((size_t)t * a.rows0 + m) * H + k];
            if (a.p1) {
                float p1 = 0.f;
                for (int t = 0; t < a.ks1; t++) p1 += a.p1[((size_t)t * a.rows1 + m) * H + k];
                p += p1;
            }
            v += p;
            row[k] = v;
            ss += v * v;
        }
        for (int k = threadIdx.x; k < H; k += 256) {
            float v = row[k];
            a.out[(size_t)m * H + k] = v;
            if (a.copy0) a.copy0[(size_t)m * H + k] = v;
            if (a.copy1) a.copy1[(size_t)m * H + k] = v;
        }
    }
    float sc = rms_scale(ss, H, a.eps, sh4);
    if (valid && a.normed)
        for (int k = threadIdx.x; k < H; k += 256) a.normed[(size_t)m * H + k] = row[k] * sc * a.w[k];
    split_row(a.xs, m, row, H, valid, sc, a.w);
}

void launch_sum_norm_split(const SumNormArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_sum_norm_split, dim3(16), dim3(256), a.H * sizeof(float), s, a);
}

// ---------------------------------------------------------------------------
// DFlash context rows: h_ctx = RMSNorm(sum_ks P_fc, hidden_norm), split once and
// reused as the K/V input of every layer.
__global__ __launch_bounds__(256) void k_hctx(const float *p, int ks, int R, int H, const float *w,
                                              float eps, uint16_t *xs) {
    __shared__ float sh4[4];
    extern __shared__ float row[];
    const int r = blockIdx.x;
    const bool valid = r < R;
    float ss = 0.f;
    if (valid)
        for (int k = threadIdx.x; k < H; k += 256) {
            float v = 0.f;
            for (int t = 0; t < ks; t++) v += p[((size_t)t * 16 + r) * H + k];
            row[k] = v;
            ss += v * v;
        }
    float sc = rms_scale(ss, H, eps, sh4);
    split_row(xs, r, row, H, valid, sc, w);
}

void launch_hctx(const float *p, int ks, int R, int H, const float *w, float eps, uint16_t *xs,
                 hipStream_t s) {
    hipLaunchKernelGGL(k_hctx, dim3(16), dim3(256), H * sizeof(float), s, p, ks, R, H, w, eps, xs);
}

// ---------------------------------------------------------------------------
// Q/K/V post-processing for one row (block row or DFlash context row):
// sum partials; per-head RMSNorm of q (q_norm) and k (k_norm); rotate-half RoPE on
// the first rotary_dim lanes of every head with angle pos * theta^(-2j/rotary_dim)
// formed in F64 (at 32k positions an F32 product errs by ~1e-3 rad); store q (block
// rows), the raw gate, and k/v into the cache row `pos` (F32, or BF16 with RNE).
// (qwen35/mtp.rs `forward_full_attention`: q/k per-head norms, IMROPE with four
// equal text positions = RoPE, SDPA-with-KV-cache append.)
__global__ __launch_bounds__(256) void k_qkv_post(QkvPostArgs a) {
    extern __shared__ float smem[];
    const int hd = a.hd, qt = a.nq * hd, kt = a.nkv * hd;
    const bool is_ctx = (int)blockIdx.x < a.R;
    const int m = is_ctx ? (int)blockIdx.x : (int)blockIdx.x - a.R;  // row in its group
    const long long pos = is_ctx ? a.P0 + m : a.P0 + a.R + m;
    const int kvrow = is_ctx ? m : a.kv_block_row0 + m;
    float *qs = smem;                 // [qt] (block rows only)
    float *ksb = smem + qt;           // [kt]
    float *vs = ksb + kt;             // [kt]
    float *hscale = vs + kt;          // [nq + nkv]
    const int nscale = a.nq + a.nkv;
    double *angle_base = (double *)(hscale + nscale + ((qt + 2 * kt + nscale) & 1));  // [rotary_dim/2]

    const int half = a.rotary_dim / 2;
    for (int j = threadIdx.x; j < half; j += 256)
        angle_base[j] = pow(a.theta, -2.0 * (double)j / (double)a.rotary_dim);

    // 1. sums of split-K partials
    for (int i = threadIdx.x; i < kt; i += 256) {
        float k = 0.f, v = 0.f;
        for (int t = 0; t < a.ksk; t++) k += a.pk[((size_t)t * a.rows_kv + kvrow) * kt + i];
        for (int t = 0; t < a.ksv; t++) v += a.pv[((size_t)t * a.rows_kv + kvrow) * kt + i];
        ksb[i] = k;
        vs[i] = v;
    }
    if (!is_ctx) {
        for (int i = threadIdx.x; i < qt; i += 256) {
            float q = 0.f;
            for (int t = 0; t < a.ksq; t++) q += a.pq[((size_t)t * 16 + m) * qt + i];
            qs[i] = q;
            if (a.pg) {
                float g = 0.f;
                for (int t = 0; t < a.ksg; t++) g += a.pg[((size_t)t * 16 + m) * qt + i];
                a.g_out[(size_t)m * qt + i] = g;
            }
        }
    }
    __syncthreads();
    // 2. per-head mean squares: wave w takes heads w, w+4, ...
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nh_q = is_ctx ? 0 : a.nq;
    for (int h = wv; h < nh_q + a.nkv; h += 4) {
        const float *src = h < nh_q ? qs + h * hd : ksb + (h - nh_q) * hd;
        float ss = 0.f;
        for (int d = lane; d < hd; d += 64) ss += src[d] * src[d];
        ss = wave_sum(ss);
        if (lane == 0) hscale[h] = 1.0f / sqrtf(ss / (float)hd + a.eps);
    }
    __syncthreads();
    // 3. normalize, rotate, store
    const int nel = (nh_q + a.nkv) * hd;
    for (int i = threadIdx.x; i < nel; i += 256) {
        const int h = i / hd, d = i - h * hd;
        const bool isq = h < nh_q;
        const float *src = isq ? qs + h * hd : ksb + (h - nh_q) * hd;
        const float *w = isq ? a.q_norm : a.k_norm;
        const float sc = hscale[h];
        float val = src[d] * sc * w[d];
        if (d < 2 * half) {
            const int j = d < half ? d : d - half;
            const int pd = d < half ? d + half : d - half;
            const float pv = src[pd] * sc * w[pd];
            double ang = (double)pos * angle_base[j];
            double sn, cs;
            sincos(ang, &sn, &cs);
            const float c = (float)cs, s = (float)sn;
            val = d < half ? val * c - pv * s : pv * s + val * c;
        }
        if (isq) {
            a.q_out[(size_t)m * qt + h * hd + d] = val;
        } else {
            const int kh = h - nh_q;
            const size_t off = ((size_t)kh * a.capacity + pos) * hd + d;
            if (a.kv_bf16) ((uint16_t *)a.cache_k)[off] = f32_to_bf16(val);
            else ((float *)a.cache_k)[off] = val;
        }
    }
    for (int i = threadIdx.x; i < kt; i += 256) {
        const int kh = i / hd, d = i - kh * hd;
        const size_t off = ((size_t)kh * a.capacity + pos) * hd + d;
        if (a.kv_bf16) ((uint16_t *)a.cache_v)[off] = f32_to_bf16(vs[i]);
        else ((float *)a.cache_v)[off] = vs[i];
    }
}

void launch_qkv_post(const QkvPostArgs &a, hipStream_t s) {
    const int qt = a.nq * a.hd, kt = a.nkv * a.hd;
    size_t sm = (size_t)(qt + 2 * kt + a.nq + a.nkv + 1) * sizeof(float) +
                (size_t)(a.rotary_dim / 2 + 1) * sizeof(double);
    hipLaunchKernelGGL(k_qkv_post, dim3(a.R + a.M), dim3(256), sm, s, a);
}

// ---------------------------------------------------------------------------
// SwiGLU: h = silu(sum P_gate) * (sum P_up), split for the down projection.
__global__ __launch_bounds__(256) void k_swiglu_split(const float *pg, int ksg, const float *pu,
                                                      int ksu, int M, int I, uint16_t *xs) {
    const int m = blockIdx.x;
    const bool valid = m < M;
    const int Ip = (I + 31) & ~31;
    for (int k = threadIdx.x; k < Ip; k += 256) {
        float h = 0.f;
        if (valid && k < I) {
            float g = 0.f, u = 0.f;
            for (int t = 0; t < ksg; t++) g += pg[((size_t)t * 16 + m) * I + k];
            for (int t = 0; t < ksu; t++) u += pu[((size_t)t * 16 + m) * I + k];
            h = g / (1.0f + expf(-g)) * u;
        }
        split_store(xs, m, k, h);
    }
}

void launch_swiglu_split(const float *pg, int ksg, const float *pu, int ksu, int M, int I,
                         uint16_t *xs, hipStream_t s) {
    hipLaunchKernelGGL(k_swiglu_split, dim3(16), dim3(256), 0, s, pg, ksg, pu, ksu, M, I, xs);
}

}  // namespace dbf
