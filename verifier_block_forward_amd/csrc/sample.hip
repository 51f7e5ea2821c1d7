// sample.hip -- draws from softmax(logits / T) by inverse CDF, and the sampled
// acceptance of one drafted token (MTP K = 1).
//
// ([ORCH] module doc, "Non-greedy (Metropolis-Hastings)": stochastic acceptance
// is named for the MTP K = 1 path, without its rule. The rule taken is standard
// speculative sampling: accept the draft d with probability min(1, p0(d)/q(d));
// otherwise draw from max(0, p0 - q) normalised; on acceptance draw the bonus
// token from p1. The random numbers are inputs.)
//
// A logits row of V values is split into nb <= SMP_BLOCKS_MAX segments of at
// least SMP_SEG_MIN values. Values are scaled to base 2, y = z * log2(e) / T, so
// every weight is exp2(y - m). Kernels:
//   k_smp_stats      per (segment, row): (max y, sum exp2(y - max)).
//   k_smp_residual   per segment: sum of max(0, p0 - q) (acceptance path only).
//   k_smp_draw       one workgroup per row: draw with u[row].
//   k_smp_accept     one workgroup: the acceptance test and the free token.
// A draw scans the segment weights in segment order to find the segment where
// the running sum passes u * total, then scans that segment's values in index
// order; the element weights there are computed by the same function that formed
// the segment sums. Sums over threads use fixed trees, so results do not depend on
// timing. Where rounding leaves u * total at or past the last running sum, the
// draw is the last index of nonzero weight.
#include "internal.hpp"
#include "kernels.hpp"

namespace dbf {

constexpr int SMP_THREADS = 256;
constexpr int SMP_WAVES = SMP_THREADS / 64;
constexpr int SMP_SEG_MIN = 1024;
constexpr int SMP_BLOCKS_MAX = 256;  // <= SMP_THREADS: one segment record per thread

int smp_blocks(int V) {
    const int nb = (V + SMP_SEG_MIN - 1) / SMP_SEG_MIN;
    return nb < 1 ? 1 : (nb > SMP_BLOCKS_MAX ? SMP_BLOCKS_MAX : nb);
}

static __device__ __forceinline__ int smp_seg(int V, int nb) { return (V + nb - 1) / nb; }

// ---------------------------------------------------------------------------
// workgroup reductions and scans (fixed trees; every thread gets the result)
struct SmpShared {
    float f[SMP_WAVES];
    int i[SMP_WAVES];
};

__device__ __forceinline__ float wave_maxf(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ int wave_mini(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ int wave_maxi(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float block_maxf(float v, SmpShared &sh) {
    v = wave_maxf(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh.f[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = sh.f[0];
#pragma unroll
    for (int w = 1; w < SMP_WAVES; w++) r = fmaxf(r, sh.f[w]);
    return r;
}

__device__ __forceinline__ float block_sumf(float v, SmpShared &sh) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh.f[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = sh.f[0];
#pragma unroll
    for (int w = 1; w < SMP_WAVES; w++) r += sh.f[w];
    return r;
}

__device__ __forceinline__ int block_mini(int v, SmpShared &sh) {
    v = wave_mini(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh.i[threadIdx.x >> 6] = v;
    __syncthreads();
    int r = sh.i[0];
#pragma unroll
    for (int w = 1; w < SMP_WAVES; w++) r = min(r, sh.i[w]);
    return r;
}

__device__ __forceinline__ int block_maxi(int v, SmpShared &sh) {
    v = wave_maxi(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh.i[threadIdx.x >> 6] = v;
    __syncthreads();
    int r = sh.i[0];
#pragma unroll
    for (int w = 1; w < SMP_WAVES; w++) r = max(r, sh.i[w]);
    return r;
}

// inclusive prefix sum over the workgroup's threads in thread order
__device__ __forceinline__ float block_scanf(float v, SmpShared &sh) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    __syncthreads();
    if (lane == 63) sh.f[wv] = v;
    __syncthreads();
    float off = 0.f;
#pragma unroll
    for (int w = 0; w < SMP_WAVES; w++) off += w < wv ? sh.f[w] : 0.f;
    return v + off;
}

// ---------------------------------------------------------------------------
// per-segment statistics of one row: (max y, sum exp2(y - max)), y = z * c
__global__ __launch_bounds__(SMP_THREADS) void k_smp_stats(SmpStatArgs a) {
    // the arguments into scalar registers in one round trip
    asm volatile("" ::"s"(a.z[0]), "s"(a.z[1]), "s"(a.z[2]), "s"(a.nptr), "s"(a.ld), "s"(a.V), "s"(a.nb),
                 "s"(a.c), "s"(a.stats));
    __shared__ SmpShared sh;
    const int b = blockIdx.x, row = blockIdx.y;
    // row pointer chosen among the loaded arguments (no indexed argument load)
    const float *zr = row == 0 ? a.z[0] : (row == 1 ? a.z[1] : a.z[2]);
    const float *z = a.nptr > 1 ? zr : a.z[0] + (size_t)row * a.ld;
    const int seg = smp_seg(a.V, a.nb);
    const int lo = b * seg, hi = min(a.V, lo + seg);
    float m = -INFINITY;
    for (int i = lo + (int)threadIdx.x; i < hi; i += SMP_THREADS) m = fmaxf(m, z[i] * a.c);
    m = block_maxf(m, sh);
    float s = 0.f;
    if (m > -INFINITY)
        for (int i = lo + (int)threadIdx.x; i < hi; i += SMP_THREADS) s += exp2f(z[i] * a.c - m);
    s = block_sumf(s, sh);
    if (threadIdx.x == 0) a.stats[(size_t)row * a.nb + b] = make_float2(m, s);
}

void launch_smp_stats(const SmpStatArgs &a, int rows, hipStream_t s) {
    launch_k(PROF_SAMPLE, "k_smp_stats", k_smp_stats, dim3(a.nb, rows), dim3(SMP_THREADS), 0, s, a);
}

// Row totals from the segment records: M = max m_b, S = sum_b s_b 2^(m_b - M).
// Thread t < nb also gets its segment's weight w_t = s_t 2^(m_t - M) (0 beyond).
struct RowTotal {
    float m, inv_s, s, w;
};

__device__ __forceinline__ RowTotal row_total(const float2 *st, int nb, SmpShared &sh) {
    const int t = threadIdx.x;
    const float2 r = t < nb ? st[t] : make_float2(-INFINITY, 0.f);
    RowTotal o;
    o.m = block_maxf(r.x, sh);
    o.w = (r.y > 0.f) ? r.y * exp2f(r.x - o.m) : 0.f;
    o.s = block_sumf(o.w, sh);
    o.inv_s = 1.0f / o.s;
    return o;
}

// weight of one value in the residual max(0, p0 - q), identical wherever formed
__device__ __forceinline__ float resid_w(float zq, float zp, float c, const RowTotal &q,
                                         const RowTotal &p) {
    const float d = exp2f(zp * c - p.m) * p.inv_s - exp2f(zq * c - q.m) * q.inv_s;
    return d > 0.f ? d : 0.f;
}

// per-segment sums of the residual (segment b)
__global__ __launch_bounds__(SMP_THREADS) void k_smp_residual(SmpResidualArgs a) {
    // the arguments into scalar registers in one round trip
    asm volatile("" ::"s"(a.zq), "s"(a.zp), "s"(a.stats), "s"(a.V), "s"(a.nb), "s"(a.c), "s"(a.rsum));
    __shared__ SmpShared sh;
    const int b = blockIdx.x;
    const RowTotal q = row_total(a.stats, a.nb, sh);
    const RowTotal p = row_total(a.stats + a.nb, a.nb, sh);
    const int seg = smp_seg(a.V, a.nb);
    const int lo = b * seg, hi = min(a.V, lo + seg);
    float s = 0.f;
    for (int i = lo + (int)threadIdx.x; i < hi; i += SMP_THREADS) s += resid_w(a.zq[i], a.zp[i], a.c, q, p);
    s = block_sumf(s, sh);
    if (threadIdx.x == 0) a.rsum[b] = s;
}

void launch_smp_residual(const SmpResidualArgs &a, hipStream_t s) {
    launch_k(PROF_SAMPLE, "k_smp_residual", k_smp_residual, dim3(a.nb), dim3(SMP_THREADS), 0, s, a);
}

// ---------------------------------------------------------------------------
// Inverse-CDF draw, one workgroup. Thread t < nb holds segment t's weight w; the
// element weight of index i is wfn(i). Returns the drawn index (every thread).
template <class WFn>
__device__ int smp_search(float w, int V, int nb, float u, WFn wfn, SmpShared &sh) {
    const int t = threadIdx.x;
    // segment: first t with running sum past u * total
    const float incl = block_scanf(w, sh);
    __shared__ float total_sh;
    if (t == SMP_THREADS - 1) total_sh = incl;
    __syncthreads();
    const float target = u * total_sh;
    const int hit = (t < nb && w > 0.f && incl > target) ? t : 0x7fffffff;
    int bsel = block_mini(hit, sh);
    float rem;
    if (bsel == 0x7fffffff) {  // past the end: last segment of nonzero weight
        bsel = block_maxi((t < nb && w > 0.f) ? t : -1, sh);
        if (bsel < 0) bsel = 0;
        rem = INFINITY;
    } else {
        __shared__ float excl_sh;
        if (t == bsel) excl_sh = incl - w;
        __syncthreads();
        rem = target - excl_sh;
    }
    // inside the segment: thread t takes a contiguous run of ept values
    const int seg = (V + nb - 1) / nb;
    const int lo = bsel * seg, hi = min(V, lo + seg);
    const int ept = (seg + SMP_THREADS - 1) / SMP_THREADS;
    const int a0 = min(hi, lo + t * ept), a1 = min(hi, a0 + ept);
    float s = 0.f;
    for (int i = a0; i < a1; i++) s += wfn(i);
    const float tin = block_scanf(s, sh);
    const int th = (s > 0.f && tin > rem) ? t : 0x7fffffff;
    int tsel = block_mini(th, sh);
    bool past = false;
    if (tsel == 0x7fffffff) {
        tsel = block_maxi(s > 0.f ? t : -1, sh);
        past = true;
    }
    __shared__ int idx_sh;
    if (t == 0) idx_sh = -1;
    __syncthreads();
    if (t == tsel) {
        float c = tin - s;
        int last = -1, found = -1;
        for (int i = a0; i < a1; i++) {
            const float e = wfn(i);
            if (e > 0.f) {
                last = i;
                c += e;
                if (!past && c > rem) {
                    found = i;
                    break;
                }
            }
        }
        idx_sh = found >= 0 ? found : last;
    }
    __syncthreads();
    int idx = idx_sh;
    if (idx < 0) idx = lo < V ? lo : V - 1;  // no weight anywhere (all rows -inf): first index
    return idx;
}

// one draw per row
__global__ __launch_bounds__(SMP_THREADS) void k_smp_draw(SmpDrawArgs a) {
    // the arguments into scalar registers in one round trip
    asm volatile("" ::"s"(a.z), "s"(a.stats), "s"(a.u), "s"(a.V), "s"(a.nb), "s"(a.c), "s"(a.token),
                 "s"(a.prob));
    __shared__ SmpShared sh;
    const int row = blockIdx.x;
    const float *z = a.z + (size_t)row * a.V;
    const RowTotal rt = row_total(a.stats + (size_t)row * a.nb, a.nb, sh);
    const float c = a.c;
    const int idx = smp_search(rt.w, a.V, a.nb, a.u[row],
                               [&](int i) { return exp2f(z[i] * c - rt.m); }, sh);
    if (threadIdx.x == 0) {
        a.token[row] = idx;
        if (a.prob) a.prob[row] = exp2f(z[idx] * c - rt.m) * rt.inv_s;
    }
}

void launch_smp_draw(const SmpDrawArgs &a, int M, hipStream_t s) {
    launch_k(PROF_SAMPLE, "k_smp_draw", k_smp_draw, dim3(M), dim3(SMP_THREADS), 0, s, a);
}

// acceptance test and free token, one workgroup
__global__ __launch_bounds__(SMP_THREADS) void k_smp_accept(SmpAcceptArgs a) {
    // the arguments into scalar registers in one round trip
    asm volatile("" ::"s"(a.zq), "s"(a.zp0), "s"(a.zp1), "s"(a.stats), "s"(a.rsum), "s"(a.draft), "s"(a.u),
                 "s"(a.eos), "s"(a.n_eos), "s"(a.V), "s"(a.nb), "s"(a.c), "s"(a.result), "s"(a.committed));
    __shared__ SmpShared sh;
    const int t = threadIdx.x;
    const int d = *a.draft;
    if (d < 0 || d >= a.V) {  // not a token of this vocabulary: nothing is read at d
        if (t < 5) a.result[t] = t < 3 ? -1 : 0;
        return;
    }
    const float c = a.c;
    const RowTotal q = row_total(a.stats, a.nb, sh);
    const RowTotal p0 = row_total(a.stats + a.nb, a.nb, sh);
    const RowTotal p1 = row_total(a.stats + 2 * a.nb, a.nb, sh);
    const float qd = exp2f(a.zq[d] * c - q.m) * q.inv_s;
    const float pd = exp2f(a.zp0[d] * c - p0.m) * p0.inv_s;
    const float u0 = a.u[0], u1 = a.u[1];
    const bool acc = u0 * qd < pd;
    const float *zq = a.zq, *zp0 = a.zp0, *zp1 = a.zp1;
    int tok;
    if (acc) {
        tok = smp_search(p1.w, a.V, a.nb, u1, [&](int i) { return exp2f(zp1[i] * c - p1.m); }, sh);
    } else {
        const float rw = t < a.nb ? a.rsum[t] : 0.f;
        const float rtot = block_sumf(rw, sh);
        if (rtot > 0.f)
            tok = smp_search(rw, a.V, a.nb, u1, [&](int i) { return resid_w(zq[i], zp0[i], c, q, p0); }, sh);
        else  // p0 == q to rounding: the residual is empty, draw from p0
            tok = smp_search(p0.w, a.V, a.nb, u1, [&](int i) { return exp2f(zp0[i] * c - p0.m); }, sh);
    }
    if (t == 0) {
        const int seq[2] = {d, tok};
        const int first = acc ? 0 : 1;
        int n = 0, hit = 0;
        for (int i = first; i < 2; i++) {
            if (a.committed) a.committed[n] = seq[i];
            n++;
            for (int e = 0; e < a.n_eos; e++)
                if (seq[i] == a.eos[e]) hit = 1;
            if (hit) break;
        }
        a.result[0] = acc ? 1 : 0;
        a.result[1] = tok;
        a.result[2] = acc ? 0 : 1;
        a.result[3] = hit;
        a.result[4] = n;
    }
}

void launch_smp_accept(const SmpAcceptArgs &a, hipStream_t s) {
    launch_k(PROF_SAMPLE, "k_smp_accept", k_smp_accept, dim3(1), dim3(SMP_THREADS), 0, s, a);
}

}  // namespace dbf
