// attn.hip -- GQA attention of the block rows over the KV cache, split over key
// chunks, then a combine pass; and the greedy accept-prefix walk.
//
// Block row i (position P0+R+i) attends to cache rows [0, P0+R+i]: the cached
// prefix, this call's context rows and the block rows up to itself (causal within
// the block). q head h reads kv head h*nkv/nq (contiguous GQA groups). Scores are
// scaled by 1/sqrt(hd) and normalised with an online softmax (running max m, sum
// l, accumulator acc); each (chunk, kv head) block writes (acc, m, l) for its
// queries and the combine pass merges chunks. (qwen35/mtp.rs
// `forward_full_attention`: `apply_sdpa_with_kv_cache`, then
// `apply_sigmoid_gate_multiply`.)
#include "internal.hpp"
#include "kernels.hpp"

namespace dbf {

constexpr int ATT_MAX_CHUNKS = 64;

void attn_plan(long long n_keys, int *chunk, int *n_chunks) {
    long long per = (n_keys + ATT_MAX_CHUNKS - 1) / ATT_MAX_CHUNKS;
    long long c = ((per + 63) / 64) * 64;
    if (c < 64) c = 64;
    *chunk = (int)c;
    *n_chunks = (int)((n_keys + c - 1) / c);
}

// HD head_dim, QB queries per block, KT keys per LDS tile; TPQ = 256/QB threads
// share one query: each scores KT/TPQ keys and accumulates HD/TPQ output lanes.
template <int HD, int QB, int KT>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a) {
    constexpr int TPQ = 256 / QB, KPT = KT / TPQ, DPT = HD / TPQ, HDP = HD + 1;
    static_assert(KPT >= 1 && DPT >= 1, "tile shape");
    __shared__ float Qs[QB * HDP];   // pre-scaled queries
    __shared__ float Ks[KT * HDP];
    __shared__ float Vs[KT * HD];
    __shared__ float Ps[QB * (KT + 1)];

    const int c = blockIdx.x, kvh = blockIdx.y, qg = blockIdx.z;
    const int G = a.nq / a.nkv;
    const int NQ = G * a.M;
    const int q0 = qg * QB;
    const int t = threadIdx.x, qi = t / TPQ, sub = t % TPQ;
    const long long n_all = a.n_ctx + a.M;
    const long long k_lo = (long long)c * a.chunk;
    long long k_hi = k_lo + a.chunk;
    if (k_hi > n_all) k_hi = n_all;
    const float scale = 1.0f / sqrtf((float)HD);

    const bool qvalid = q0 + qi < NQ;
    const int gq = qvalid ? q0 + qi : NQ - 1;  // padding slots recompute a valid query
    const int qm = gq / G, qh = kvh * G + gq % G;
    const long long qlim = a.n_ctx + qm;  // last visible key position

    for (int i = t; i < QB * HD; i += 256) {
        const int r = i / HD, d = i - r * HD;
        const int g2 = q0 + r < NQ ? q0 + r : NQ - 1;
        const int m2 = g2 / G, h2 = kvh * G + g2 % G;
        Qs[r * HDP + d] = a.q[(size_t)m2 * a.nq * HD + (size_t)h2 * HD + d] * scale;
    }

    const size_t head_off = (size_t)kvh * a.capacity * HD;
    float m_run = -INFINITY, l_run = 0.f;
    float acc[DPT];
#pragma unroll
    for (int i = 0; i < DPT; i++) acc[i] = 0.f;

    for (long long kb = k_lo; kb < k_hi; kb += KT) {
        __syncthreads();
        const int nk = (int)((k_hi - kb) < KT ? (k_hi - kb) : KT);
        for (int i = t; i < KT * HD; i += 256) {
            const int r = i / HD, d = i - r * HD;
            float kv = 0.f, vv = 0.f;
            if (r < nk) {
                const size_t off = head_off + (size_t)(kb + r) * HD + d;
                if (a.kv_bf16) {
                    kv = bf16_to_f32(((const uint16_t *)a.cache_k)[off]);
                    vv = bf16_to_f32(((const uint16_t *)a.cache_v)[off]);
                } else {
                    kv = ((const float *)a.cache_k)[off];
                    vv = ((const float *)a.cache_v)[off];
                }
            }
            Ks[r * HDP + d] = kv;
            Vs[r * HD + d] = vv;
        }
        __syncthreads();
        float s[KPT];
#pragma unroll
        for (int u = 0; u < KPT; u++) s[u] = 0.f;
        const float *qr = Qs + qi * HDP;
        for (int d = 0; d < HD; d++) {
            const float qv = qr[d];
#pragma unroll
            for (int u = 0; u < KPT; u++) s[u] += qv * Ks[(sub + TPQ * u) * HDP + d];
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int u = 0; u < KPT; u++) {
            const int j = sub + TPQ * u;
            if (!(j < nk && kb + j <= qlim)) s[u] = -INFINITY;
            tmax = fmaxf(tmax, s[u]);
        }
#pragma unroll
        for (int o = 1; o < TPQ; o <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o, 64));
        const float m_new = fmaxf(m_run, tmax);
        float alpha = 1.f, psum = 0.f;
        if (m_new != -INFINITY) {
            alpha = expf(m_run - m_new);
#pragma unroll
            for (int u = 0; u < KPT; u++) {
                s[u] = expf(s[u] - m_new);
                psum += s[u];
            }
        } else {
#pragma unroll
            for (int u = 0; u < KPT; u++) s[u] = 0.f;
        }
#pragma unroll
        for (int o = 1; o < TPQ; o <<= 1) psum += __shfl_xor(psum, o, 64);
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int u = 0; u < KPT; u++) Ps[qi * (KT + 1) + sub + TPQ * u] = s[u];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < DPT; i++) acc[i] *= alpha;
        for (int j = 0; j < KT; j++) {
            const float p = Ps[qi * (KT + 1) + j];
#pragma unroll
            for (int i = 0; i < DPT; i++) acc[i] += p * Vs[j * HD + sub + TPQ * i];
        }
    }
    if (qvalid) {
        const size_t qidx = (size_t)qm * a.nq + qh;
        float *o = a.part + ((size_t)c * a.M * a.nq + qidx) * (HD + 2);
#pragma unroll
        for (int i = 0; i < DPT; i++) o[sub + TPQ * i] = acc[i];
        if (sub == 0) {
            o[HD] = m_run;
            o[HD + 1] = l_run;
        }
    }
}

bool attn_supported(int hd) { return hd == 64 || hd == 128 || hd == 256; }

void launch_attn(const AttnArgs &a, hipStream_t s) {
    const int G = a.nq / a.nkv;
    const int NQ = G * a.M;
    const int QB = a.hd == 256 ? 16 : 32;
    dim3 grid(a.n_chunks, a.nkv, (NQ + QB - 1) / QB);
    if (a.hd == 64) hipLaunchKernelGGL((k_attn<64, 32, 32>), grid, dim3(256), 0, s, a);
    else if (a.hd == 128) hipLaunchKernelGGL((k_attn<128, 32, 32>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_attn<256, 16, 16>), grid, dim3(256), 0, s, a);
}

// Merge chunk partials of query (m, h), apply the optional sigmoid gate and write
// the attention output row into the split tile of the O projection. Rows m >= M
// and the padding columns are written as zeros.
__global__ __launch_bounds__(256) void k_attn_combine(CombineArgs a) {
    const int m = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
    const int hd = a.hd, K = a.nq * hd;
    if (d < hd) {
        float o = 0.f;
        if (m < a.M) {
            const size_t q = (size_t)m * a.nq + h;
            const size_t stride = (size_t)a.M * a.nq * (hd + 2);
            float mx = -INFINITY;
            for (int c = 0; c < a.n_chunks; c++) {
                const float *p = a.part + c * stride + q * (hd + 2);
                if (p[hd + 1] > 0.f) mx = fmaxf(mx, p[hd]);
            }
            float l = 0.f, acc = 0.f;
            for (int c = 0; c < a.n_chunks; c++) {
                const float *p = a.part + c * stride + q * (hd + 2);
                if (p[hd + 1] > 0.f) {
                    const float e = expf(p[hd] - mx);
                    l += p[hd + 1] * e;
                    acc += p[d] * e;
                }
            }
            o = acc / l;
            if (a.g) o *= sigmoidf_(a.g[(size_t)m * K + h * hd + d]);
        }
        split_store(a.xs, m, h * hd + d, o);
    }
    if (h == a.nq - 1) {
        const int Kp = (K + 31) & ~31;
        for (int k = K + d; k < Kp; k += blockDim.x) split_store(a.xs, m, k, 0.f);
    }
}

void launch_attn_combine(const CombineArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_attn_combine, dim3(16, a.nq), dim3(256), 0, s, a);
}

// ---------------------------------------------------------------------------
// Greedy accept-prefix walk (hf2q dflash/qwen35_orchestrator.rs, module doc:
// greedy accept-walk invariant; per-round steps 7-8). One wavefront.
__global__ __launch_bounds__(64) void k_accept(const int32_t *d, const int32_t *t, int K,
                                               const int32_t *eos, int n_eos, int32_t *res,
                                               int32_t *committed) {
    const int lane = threadIdx.x;
    int a = K;
    for (int base = 0; base < K; base += 64) {
        const int i = base + lane;
        const bool mis = i < K && d[i] != t[i];
        const unsigned long long b = __ballot(mis);
        if (b) {
            a = base + __ffsll((long long)b) - 1;
            break;
        }
    }
    int first_eos = a + 1;
    if (n_eos > 0) {
        for (int base = 0; base <= a; base += 64) {
            const int i = base + lane;
            bool ise = false;
            if (i <= a) {
                const int tok = t[i];
                for (int e = 0; e < n_eos; e++) ise |= tok == eos[e];
            }
            const unsigned long long b = __ballot(ise);
            if (b) {
                first_eos = base + __ffsll((long long)b) - 1;
                break;
            }
        }
    }
    const bool hit = first_eos <= a;
    const int n = hit ? first_eos + 1 : a + 1;
    if (committed)
        for (int i = lane; i < n; i += 64) committed[i] = t[i];
    if (lane == 0) {
        res[0] = a;
        res[1] = t[a];
        res[2] = K - a;
        res[3] = hit ? 1 : 0;
        res[4] = n;
    }
}

void launch_accept(const int32_t *drafts, const int32_t *target, int K, const int32_t *eos,
                   int n_eos, int32_t *result, int32_t *committed, hipStream_t s) {
    hipLaunchKernelGGL(k_accept, dim3(1), dim3(64), 0, s, drafts, target, K, eos, n_eos, result,
                       committed);
}

}  // namespace dbf
