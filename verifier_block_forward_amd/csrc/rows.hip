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

// ---------------------------------------------------------------------------
// Generic column kernel. Grid (ncb = ceil(H/64), 4), 256 threads: wave w handles
// row m = 4*blockIdx.y + w, lane the column blockIdx.x*64 + lane.
//   v = [gather embed row | base] + scale0 * sum P0 + scale1 * sum P1
//   out/copies <- v;  xs <- split(v (.) w);  ssp_out[m][cb] <- sum over the 64 columns of v^2
// Rows m >= M and padding columns write zeros into the split tile.
__device__ __forceinline__ int colsum_row_groups(const ColArgs &a) {
    return a.xs ? 4 : (a.M + 3) / 4;  // split tiles need all 16 rows written
}

// Input modes: SRC_BASE when the rows come from `base` (or are zero), SRC_ANY for
// the token gather. The base-only form has no branch joins between its independent
// loads, so the compiler issues them together.
constexpr int SRC_ANY = 0, SRC_BASE = 1;

template <int SRC>
__device__ __forceinline__ void colsum_body(const ColArgs &a) {
    // the arguments into scalar registers in one round trip
    if constexpr (SRC == SRC_BASE)
        asm volatile("" ::"s"(a.M), "s"(a.H), "s"(a.base), "s"(a.ldb), "s"(a.p0), "s"(a.ks0), "s"(a.rows0),
                     "s"(a.ssp0), "s"(a.eps0), "s"(a.p1), "s"(a.ks1), "s"(a.rows1), "s"(a.ssp1), "s"(a.eps1),
                     "s"(a.ncb_in), "s"(a.out), "s"(a.copy0), "s"(a.copy1), "s"(a.w), "s"(a.xs),
                     "s"(a.ssp_out), "s"(a.ncb_out));
    else
        asm volatile("" ::"s"(a.M), "s"(a.H), "s"(a.base), "s"(a.ldb), "s"(a.p0), "s"(a.ks0), "s"(a.rows0),
                     "s"(a.ssp0), "s"(a.eps0), "s"(a.p1), "s"(a.ks1), "s"(a.rows1), "s"(a.ssp1), "s"(a.eps1),
                     "s"(a.ncb_in), "s"(a.out), "s"(a.copy0), "s"(a.copy1), "s"(a.w), "s"(a.xs),
                     "s"(a.ssp_out), "s"(a.ncb_out), "s"(a.tokens), "s"(a.embed), "s"(a.V));
    if ((int)blockIdx.x >= (a.H + 63) / 64 || (int)blockIdx.y >= colsum_row_groups(a)) return;
    const int m = blockIdx.y * 4 + wave_id();
    const int lane = threadIdx.x & 63;
    const int k = blockIdx.x * 64 + lane;
    const bool row_ok = m < a.M;
    const bool ok = row_ok && k < a.H;
    // Loads that depend on no other load go out first (this lane's share of the
    // row-scale partials, the base or gathered value, the token id, the norm
    // weight), then the split-K partials in one batch, so a single wait covers them
    // all; the row scales are reduced after it.
    const bool sc0on = row_ok && a.p0 && a.ssp0, sc1on = row_ok && a.p1 && a.ssp1;
    const float *sr0 = a.ssp0 + (size_t)m * a.ncb_in, *sr1 = a.ssp1 + (size_t)m * a.ncb_in;
    float f0 = 0.f, f1 = 0.f, bv = 0.f, wk = 1.f;
    int tok = 0;
    if (sc0on) f0 = row_scale_first(sr0, a.ncb_in);
    if (sc1on) f1 = row_scale_first(sr1, a.ncb_in);
    if (ok) {
        if constexpr (SRC == SRC_BASE) {
            if (a.base) bv = a.base[(size_t)m * a.ldb + k];
        } else if (a.tokens) {
            tok = a.tokens[m];
        } else if (a.base) {
            bv = a.base[(size_t)m * a.ldb + k];
        }
        if (a.xs && a.w) wk = a.w[k];
    }
    float v = 0.f;
    if (row_ok) {
        float s0 = 0.f, s1 = 0.f;
        if (ok && a.p0) s0 = sum_partials(a.p0, a.ks0, a.rows0, a.H, m, k);
        if (ok && a.p1) s1 = sum_partials(a.p1, a.ks1, a.rows1, a.H, m, k);
        float sc0 = 1.f, sc1 = 1.f;
        if (sc0on) sc0 = row_scale_finish(f0, sr0, a.ncb_in, a.H, a.eps0);
        if (sc1on) sc1 = row_scale_finish(f1, sr1, a.ncb_in, a.H, a.eps1);
        if (ok) {
            if (SRC != SRC_BASE && a.tokens) {
                const int t = tok < 0 ? 0 : (tok >= a.V ? a.V - 1 : tok);
                v = bf16_to_f32(a.embed[(size_t)t * a.H + k]);
            } else {
                v = bv;  // base value (0 when there is none)
            }
            if (a.p0) v += sc0 * s0;
            if (a.p1) v += sc1 * s1;
            if (a.out) a.out[(size_t)m * a.H + k] = v;
            if (a.copy0) a.copy0[(size_t)m * a.H + k] = v;
            if (a.copy1) a.copy1[(size_t)m * a.H + k] = v;
        }
        if (a.ssp_out) {
            float ss = wave_sum(v * v);
            if (lane == 0) a.ssp_out[(size_t)m * a.ncb_out + blockIdx.x] = ss;
        }
    }
    if (a.xs && k < ((a.H + 31) & ~31)) split_store(a.xs, m, k, ok ? v * wk : 0.f);
}

template <int SRC>
__global__ __launch_bounds__(256) void k_colsum(ColArgs a) { colsum_body<SRC>(a); }

// two independent column jobs in one launch (blockIdx.z selects the job)
__global__ __launch_bounds__(256) void k_colsum2(ColArgs a0, ColArgs a1) {
    if (blockIdx.z == 0) colsum_body<SRC_ANY>(a0);
    else colsum_body<SRC_ANY>(a1);
}

static dim3 colsum_grid(const ColArgs &a) {
    return dim3((a.H + 63) / 64, a.xs ? 4 : (a.M + 3) / 4);
}

void launch_colsum(const ColArgs &a, hipStream_t s) {
    if (!a.tokens)
        launch_k(PROF_ROWS, "k_colsum", k_colsum<SRC_BASE>, colsum_grid(a), dim3(256), 0, s, a);
    else
        launch_k(PROF_ROWS, "k_colsum", k_colsum<SRC_ANY>, colsum_grid(a), dim3(256), 0, s, a);
}

void launch_colsum2(const ColArgs &a0, const ColArgs &a1, hipStream_t s) {
    const dim3 g0 = colsum_grid(a0), g1 = colsum_grid(a1);
    const dim3 g(g0.x > g1.x ? g0.x : g1.x, g0.y > g1.y ? g0.y : g1.y, 2);
    launch_k(PROF_ROWS, "k_colsum2", k_colsum2, g, dim3(256), 0, s, a0, a1);
}

// ---------------------------------------------------------------------------
// Final norm: h_final = x * s_m (.) w.
__global__ __launch_bounds__(256) void k_final_norm(const float *x, const float *ssp, const float *w,
                                                    float *out, int ncb, int M, int H, float eps) {
    // the arguments into scalar registers in one round trip
    asm volatile("" ::"s"(x), "s"(ssp), "s"(w), "s"(out), "s"(ncb), "s"(M), "s"(H), "s"(eps));
    const int m = blockIdx.y * 4 + wave_id();
    const int k = blockIdx.x * 64 + (threadIdx.x & 63);
    if (m >= M) return;
    const float *sr = ssp + (size_t)m * ncb;
    const float f = row_scale_first(sr, ncb);  // in flight with the row and weight loads
    const float xv = k < H ? x[(size_t)m * H + k] : 0.f, wv = k < H ? w[k] : 0.f;
    const float s = row_scale_finish(f, sr, ncb, H, eps);
    if (k < H) out[(size_t)m * H + k] = xv * s * wv;
}

void launch_final_norm(const float *x, const float *ssp, int ncb, int M, int H, const float *w, float eps,
                       float *out, hipStream_t s) {
    launch_k(PROF_ROWS, "k_final_norm", k_final_norm, dim3((H + 63) / 64, (M + 3) / 4), dim3(256), 0, s, x,
             ssp, w, out, ncb, M, H, eps);
}

// ---------------------------------------------------------------------------
// Q/K/V post-processing, one wavefront per head vector (qwen35/mtp.rs
// `forward_full_attention`): sum split-K partials and apply the row's RMSNorm
// scale; per-head RMSNorm (q_norm / k_norm); rotate-half RoPE over the first
// rotary_dim lanes; store q (block rows) and the raw gate, or the key and value
// rows of the cache (F32, or BF16 with RNE). The RoPE angle pos * inv_freq[j] is
// formed in F64 from the host's F64 table theta^(-2j/rotary_dim) and reduced
// modulo 2 pi in F64 (an F32 product is off by ~1e-3 rad at 32k positions), then
// sin/cos are taken in F32 on the reduced angle. The partial sums of the head and
// of its companion (gate or value) are loaded together. Each lane owns CPL =
// hd/64 columns d = lane + 64 i.
// Blocks [0, M*nq) are q heads of block rows; then (R+M)*nkv k/v heads, context
// rows first. DFlash context rows sit at positions P0+r, block rows at P0+R+m.
template <int CPL>
__global__ __launch_bounds__(64) void k_qkv_post(QkvPostArgs a) {
    // the arguments into scalar registers in one round trip
    asm volatile("" ::"s"(a.pq), "s"(a.pk), "s"(a.pv), "s"(a.pg), "s"(a.ksq), "s"(a.ksk), "s"(a.ksv),
                 "s"(a.ksg), "s"(a.rows_kv), "s"(a.kv_block_row0), "s"(a.ssp_x), "s"(a.ssp_ctx),
                 "s"(a.ncb), "s"(a.ncb_ctx), "s"(a.H), "s"(a.q_norm), "s"(a.k_norm), "s"(a.eps), "s"(a.rotary_dim),
                 "s"(a.M), "s"(a.R), "s"(a.nq), "s"(a.nkv), "s"(a.P0), "s"(a.q_out), "s"(a.g_out),
                 "s"(a.cache_k), "s"(a.cache_v), "s"(a.kv_bf16), "s"(a.capacity));
    __shared__ float vec[64 * CPL];
    const int lane = threadIdx.x;
    const int hd = 64 * CPL, qt = a.nq * hd, kt = a.nkv * hd;
    const int b = blockIdx.x;
    const bool isq = b < a.M * a.nq;
    int row, head;         // row within its group (block rows or all kv rows), head index
    long long pos;
    const float *sspr;     // norm partials of the source row (its RMSNorm scale)
    int ncb;               // partials per row in sspr
    const float *src, *src2, *wn;  // partials of the head and of its gate / value, head-norm weight
    int ks, ks2, prow, N, rows;
    if (isq) {
        row = b / a.nq;
        head = b % a.nq;
        pos = a.P0 + a.R + row;
        sspr = a.ssp_x + (size_t)row * a.ncb;
        ncb = a.ncb;
        src = a.pq;
        ks = a.ksq;
        src2 = a.pg;
        ks2 = a.ksg;
        prow = row;
        N = qt;
        rows = 16;
        wn = a.q_norm;
    } else {
        const int idx = b - a.M * a.nq;
        row = idx / a.nkv;  // 0..R+M-1, context rows first
        head = idx % a.nkv;
        const bool ctx = row < a.R;
        const int m = ctx ? row : row - a.R;
        pos = ctx ? a.P0 + row : a.P0 + a.R + m;
        sspr = ctx ? a.ssp_ctx + (size_t)m * a.ncb_ctx : a.ssp_x + (size_t)m * a.ncb;
        ncb = ctx ? a.ncb_ctx : a.ncb;
        src = a.pk;
        ks = a.ksk;
        src2 = a.pv;
        ks2 = a.ksv;
        prow = ctx ? m : a.kv_block_row0 + m;
        N = kt;
        rows = a.rows_kv;
        wn = a.k_norm;
    }
    const size_t stride = (size_t)rows * N;
    const size_t rowoff = (size_t)prow * N + (size_t)head * hd + lane;
    // the row-scale share, the head-norm weights and the RoPE frequencies go out
    // with the partials (one wait)
    const float f = row_scale_first(sspr, ncb);
    const int half = a.rotary_dim / 2;
    float wnv[CPL];
    double ifr[CPL];
#pragma unroll
    for (int i = 0; i < CPL; i++) {
        const int d = lane + 64 * i;
        wnv[i] = wn[d];
        ifr[i] = d < 2 * half ? a.inv_freq[d < half ? d : d - half] : 0.0;
    }
    float raw[CPL], side[CPL] = {};
    if (src2 && ks2 == ks) {
        const float *bb[2 * CPL];
#pragma unroll
        for (int i = 0; i < CPL; i++) {
            bb[i] = src + rowoff + 64 * i;
            bb[CPL + i] = src2 + rowoff + 64 * i;
        }
        float o[2 * CPL];
        sum_partials_n<2 * CPL>(bb, ks, stride, o);
#pragma unroll
        for (int i = 0; i < CPL; i++) {
            raw[i] = o[i];
            side[i] = o[CPL + i];
        }
    } else {
        const float *bb[CPL];
#pragma unroll
        for (int i = 0; i < CPL; i++) bb[i] = src + rowoff + 64 * i;
        sum_partials_n<CPL>(bb, ks, stride, raw);
        if (src2) {
#pragma unroll
            for (int i = 0; i < CPL; i++) bb[i] = src2 + rowoff + 64 * i;
            sum_partials_n<CPL>(bb, ks2, stride, side);
        }
    }
    const float s = row_scale_finish(f, sspr, ncb, a.H, a.eps);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; i++) {
        raw[i] *= s;
        side[i] *= s;
        ss += raw[i] * raw[i];
    }
    const float hs = 1.0f / sqrtf(wave_sum(ss) / (float)hd + a.eps);
#pragma unroll
    for (int i = 0; i < CPL; i++) {
        const int d = lane + 64 * i;
        vec[d] = raw[i] * hs * wnv[i];
    }
    __syncthreads();
    const size_t cache_off = ((size_t)head * a.capacity + pos) * hd;
    const double two_pi = 6.283185307179586;
#pragma unroll
    for (int i = 0; i < CPL; i++) {
        const int d = lane + 64 * i;
        float val = vec[d];
        if (d < 2 * half) {
            const float pv = vec[d < half ? d + half : d - half];
            const double ang = (double)pos * ifr[i];
            const double red = fma(-rint(ang * (1.0 / two_pi)), two_pi, ang);  // |red| <= pi
            float sv, c;
            sincosf((float)red, &sv, &c);
            val = d < half ? val * c - pv * sv : pv * sv + val * c;
        }
        if (isq) {
            a.q_out[(size_t)row * qt + head * hd + d] = val;
            if (src2) a.g_out[(size_t)row * qt + head * hd + d] = side[i];
        } else {
            if (a.kv_bf16) {
                ((uint16_t *)a.cache_k)[cache_off + d] = f32_to_bf16(val);
                ((uint16_t *)a.cache_v)[cache_off + d] = f32_to_bf16(side[i]);
            } else {
                ((float *)a.cache_k)[cache_off + d] = val;
                ((float *)a.cache_v)[cache_off + d] = side[i];
            }
        }
    }
}

void launch_qkv_post(const QkvPostArgs &a, hipStream_t s) {
    const dim3 grid(a.M * a.nq + (a.R + a.M) * a.nkv);
    if (a.hd == 64) launch_k(PROF_ROWS, "k_qkv_post", k_qkv_post<1>, grid, dim3(64), 0, s, a);
    else if (a.hd == 128) launch_k(PROF_ROWS, "k_qkv_post", k_qkv_post<2>, grid, dim3(64), 0, s, a);
    else launch_k(PROF_ROWS, "k_qkv_post", k_qkv_post<4>, grid, dim3(64), 0, s, a);
}

// ---------------------------------------------------------------------------
// SwiGLU: h = silu(s_m * sum P_gate) * (s_m * sum P_up), split for the down
// projection (s_m: RMSNorm scale of the FFN input row).
__global__ __launch_bounds__(256) void k_swiglu(SwigluArgs a) {
    // the arguments into scalar registers in one round trip
    asm volatile("" ::"s"(a.pg), "s"(a.pu), "s"(a.ksg), "s"(a.ksu), "s"(a.ssp), "s"(a.ncb), "s"(a.H),
                 "s"(a.eps), "s"(a.M), "s"(a.I), "s"(a.xs));
    const int m = blockIdx.y * 4 + wave_id();
    const int k = blockIdx.x * 64 + (threadIdx.x & 63);
    const int Ip = (a.I + 31) & ~31;
    float h = 0.f;
    if (m < a.M) {
        const float *sr = a.ssp + (size_t)m * a.ncb;
        const float f = row_scale_first(sr, a.ncb);  // in flight with the partials
        float g = 0.f, u = 0.f;
        if (k < a.I) {
            if (a.ksg == a.ksu) {
                const size_t off = (size_t)m * a.I + k;
                const float *b[2] = {a.pg + off, a.pu + off};
                float o[2];
                sum_partials_n<2>(b, a.ksg, (size_t)16 * a.I, o);
                g = o[0];
                u = o[1];
            } else {
                g = sum_partials(a.pg, a.ksg, 16, a.I, m, k);
                u = sum_partials(a.pu, a.ksu, 16, a.I, m, k);
            }
        }
        const float s = row_scale_finish(f, sr, a.ncb, a.H, a.eps);
        if (k < a.I) {
            g *= s;
            u *= s;
            h = g / (1.0f + expf(-g)) * u;
        }
    }
    if (k < Ip) split_store(a.xs, m, k, h);
}

void launch_swiglu(const SwigluArgs &a, hipStream_t s) {
    launch_k(PROF_ROWS, "k_swiglu", k_swiglu, dim3((a.I + 63) / 64, 4), dim3(256), 0, s, a);
}

}  // namespace dbf
