// attn.hip -- GQA attention of the block rows over the KV cache, split over key
// chunks, then a combine pass; and the greedy accept-prefix walk.
//
// Block row i (position P0+R+i) attends to cache rows [0, P0+R+i]: the cached
// prefix, this call's context rows and the block rows up to itself (causal within
// the block). q head h reads kv head h*nkv/nq (contiguous GQA groups). Scores are
// scaled by 1/sqrt(hd) and normalised with an online softmax (running max m, sum
// l, accumulator acc) kept in base 2: the scores carry an extra factor log2(e), so
// exp(s - m) is formed as 2^(s' - m') and m is stored in log2 units. Each (chunk,
// kv head) block writes (acc, m, l) for its queries and the combine pass merges
// chunks. (qwen35/mtp.rs
// `forward_full_attention`: `apply_sdpa_with_kv_cache`, then
// `apply_sigmoid_gate_multiply`.)
#include <atomic>

#include "internal.hpp"
#include "kernels.hpp"

namespace dbf {

constexpr int ATT_KT = 16;     // keys per sub-tile
constexpr int ATT_WAVES = 4;   // waves per workgroup, each on a quarter of the chunk

// Chunking of the keys. Keys per wave are sized so that the launch has about one
// 4-wave workgroup per CU: on MI355X fewer, longer chunks were measured faster than
// more parallelism, since every workgroup pays for staging the queries and merging
// its waves, and every chunk adds a partial record to the combine. At least one
// 16-key sub-tile per wave, and at most ATT_CHUNKS_MAX chunks.
void attn_plan_keys(long long n_keys, int keys_per_wave, int *chunk, int *n_chunks) {
    long long pw = (keys_per_wave + ATT_KT - 1) / ATT_KT * ATT_KT;
    if (pw < ATT_KT) pw = ATT_KT;
    const long long per = (n_keys + ATT_CHUNKS_MAX - 1) / ATT_CHUNKS_MAX;  // keys per chunk
    const long long pw_min = (per + ATT_WAVES * ATT_KT - 1) / (ATT_WAVES * ATT_KT) * ATT_KT;
    if (pw < pw_min) pw = pw_min;
    *chunk = (int)(ATT_WAVES * pw);
    *n_chunks = (int)((n_keys + *chunk - 1) / *chunk);
}

// compute units of the current device, queried once per device
static int device_cus() {
    constexpr int MAXDEV = 64;
    static std::atomic<int> cached[MAXDEV];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < MAXDEV) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    if (dev < MAXDEV) cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

void attn_plan(long long n_keys, int groups, int *chunk, int *n_chunks) {
    const int cus = device_cus();
    const long long chunks = cus / groups > 1 ? cus / groups : 1;
    const long long per = (n_keys + chunks - 1) / chunks;
    attn_plan_keys(n_keys, (int)((per + ATT_WAVES - 1) / ATT_WAVES), chunk, n_chunks);
}

// Query tiles (16 queries each) one workgroup may take: the accumulators
// (QT * hd / 16 float4 per lane) and one sub-tile of raw K/V must fit a wave's
// registers without spilling. F32 caches hold twice the raw bytes of BF16 ones.
constexpr int attn_qt_cap(int hd, bool kv_bf16) {
    return kv_bf16 ? (hd == 256 ? 2 : 4) : (hd == 256 ? 1 : (hd == 128 ? 2 : 4));
}

int attn_qtiles(int hd, int nq_group, bool kv_bf16) {
    const int need = (nq_group + 15) / 16;
    const int cap = attn_qt_cap(hd, kv_bf16);
    return need < cap ? (need <= 1 ? 1 : (need <= 2 ? 2 : 4)) : cap;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_att __attribute__((ext_vector_type(2)));

// four values (the 4-key operands of the P*V product) split into hi/lo
__device__ __forceinline__ void split4(float x0, float x1, float x2, float x3, s16x4 &hi, s16x4 &lo) {
    unsigned h0, l0, h1, l1;
    split2(x0, x1, h0, l0);
    split2(x2, x3, h1, l1);
    hi = __builtin_bit_cast(s16x4, u32x2_att{h0, h1});
    lo = __builtin_bit_cast(s16x4, u32x2_att{l0, l1});
}

template <int HD, int QT, bool KVB>
struct AttnLds {
    static constexpr int S = HD / 32, DT = HD / 16, VTW = HD + 8;  // V row pitch (elements)
    static constexpr int Q_BYTES = QT * S * 2 * 64 * 16;
    static constexpr int VPLANE = ATT_KT * VTW * 2;  // bytes of one wave's V rows (BF16 caches)
    static constexpr int V_BYTES = KVB ? ATT_WAVES * VPLANE : 0;
    static constexpr int LOOP = Q_BYTES + V_BYTES;
    static constexpr int ACC_BYTES = (ATT_WAVES - 1) * QT * DT * 64 * 16;
    static constexpr int ML_BYTES = ATT_WAVES * QT * 64 * 8;
    static constexpr int MERGE = ACC_BYTES + ML_BYTES;
    static constexpr int BYTES = LOOP > MERGE ? LOOP : MERGE;
};

// Raw K/V of one 16-key sub-tile as a lane (r16, g) loads it. K: key row r16, dims
// 32*st + 8g .. +7 of every 32-dim step st (the A operand of the score product).
// F32 V: already in the A-operand order of the P*V product, v[4*dt + j] = V[key
// 4g + j][dim 16*dt + r16] (each load instruction reads 4 key rows x 64 contiguous
// bytes). BF16 V: whole rows per load (attn_v_slot), transposed through LDS later.
template <int HD, bool KVB>
struct KvRaw;
template <int HD>
struct KvRaw<HD, false> {
    float4 k[HD / 16];
    float v[HD / 4];
};
template <int HD>
struct KvRaw<HD, true> {
    uint4 k[HD / 32], v[HD / 32];
};

constexpr int ATT_WPE = 2;
// Waves per SIMD the register allocation is sized for. The planner launches about
// one workgroup per CU, so the F32-cache variants that would spill inside the key
// loop at two waves per SIMD take the whole register file (one wave) instead. The
// 128-dim two-tile F32 variant keeps two: at that budget it parks two addresses
// in scratch outside the loop only, and measured faster than at one wave.
template <int HD, int QT, bool KVB>
constexpr int attn_wpe() {
    return (!KVB && (HD == 256 || (HD == 64 && QT == 4))) ? 1 : ATT_WPE;
}

// Sub-tiles held in registers ahead of use: every wave issues its first PF
// sub-tiles' loads before anything else, then refills a slot as soon as it has
// been converted. Two slots only where they fit the register budget of two
// workgroups per CU (BF16 caches up to 128 dims).
template <int HD, bool KVB>
constexpr int attn_prefetch() {
    return (KVB && HD <= 128) ? 2 : 1;
}

// BF16 V sub-tile element (row, col) that load st of lane (r16, g) fetches: whole
// rows per load instruction (64 lanes x 8 elements), so every cache line is read by
// one instruction; the rows are stored to LDS as they are and read back transposed.
template <int HD>
__device__ __forceinline__ void attn_v_slot(int st, int g, int r16, int &row, int &col) {
    const int e = (64 * st + 16 * g + r16) * 8;
    row = e / HD;
    col = e % HD;
}

typedef unsigned int u32x4_att __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_v16(const uint16_t *p) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load((const u32x4_att *)p));
}

template <int HD, bool KVB>
__device__ __forceinline__ void attn_load_k(KvRaw<HD, KVB> &r, const AttnArgs &a, size_t head_off,
                                            long long kb, long long n_all, int g, int r16) {
    long long krow = kb + r16;  // rows past the last key re-read a valid row (masked later)
    if (krow > n_all - 1) krow = n_all - 1;
#pragma unroll
    for (int st = 0; st < HD / 32; st++) {
        const size_t off = head_off + (size_t)krow * HD + 32 * st + 8 * g;
        if constexpr (KVB) {
            r.k[st] = *(const uint4 *)((const uint16_t *)a.cache_k + off);
            int row, col;
            attn_v_slot<HD>(st, g, r16, row, col);
            long long vrow = kb + row;
            if (vrow > n_all - 1) vrow = n_all - 1;
            r.v[st] = ld_v16((const uint16_t *)a.cache_v + head_off + (size_t)vrow * HD + col);
        } else {
            const float4 *kp = (const float4 *)((const float *)a.cache_k + off);
            r.k[2 * st] = kp[0];
            r.k[2 * st + 1] = kp[1];
        }
    }
}

// F32 V in the A-operand order of the P*V product (BF16 V comes with attn_load_k)
template <int HD, bool KVB>
__device__ __forceinline__ void attn_load_v(KvRaw<HD, KVB> &r, const AttnArgs &a, size_t head_off,
                                            long long kb, long long n_all, int g, int r16) {
    if constexpr (!KVB) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            long long vrow = kb + 4 * g + j;
            if (vrow > n_all - 1) vrow = n_all - 1;
            const float *vp = (const float *)a.cache_v + head_off + (size_t)vrow * HD + r16;
#pragma unroll
            for (int dt = 0; dt < HD / 16; dt++) r.v[4 * dt + j] = vp[16 * dt];
        }
    }
}

// BF16 V sub-tile -> this wave's LDS rows: row j holds key j, pitch VTW elements
// (HD + 8: the 16 rows of a transposed read then fall on different banks).
template <int HD, int VTW>
__device__ __forceinline__ void attn_v_store(const KvRaw<HD, true> &r, uint16_t *vrows, int g, int r16) {
#pragma unroll
    for (int st = 0; st < HD / 32; st++) {
        int row, col;
        attn_v_slot<HD>(st, g, r16, row, col);
        *(uint4 *)(vrows + row * VTW + col) = r.v[st];
    }
}

// The A operand of the P*V product for dims 16*dt..+15, read transposed out of the
// V rows with ds_read_b64_tr_b16 (gfx950). Within each 16-lane group that read
// hands lane i, element j, element i%4 of the 8-byte chunk addressed by lane
// 4j + i/4; so lane (i, g) addresses key 4g + i/4, dims 16*dt + 4*(i%4) .. +3, and
// receives V[4g + j][16*dt + i] for j = 0..3: keys 4g..4g+3 of dim i (layout checked
// with a probe on MI355X).
typedef short s16x4_lds __attribute__((ext_vector_type(4)));
template <int VTW>
__device__ __forceinline__ s16x4_lds attn_v_operand(const uint16_t *vrows, int dt, int g, int r16) {
    const uint16_t *p = vrows + (4 * g + (r16 >> 2)) * VTW + 16 * dt + 4 * (r16 & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_lds *)p);
}

// A operand(s) of the score product for 32-dim step st: BF16 K as is, F32 K split hi/lo
template <int HD, bool KVB>
__device__ __forceinline__ void attn_k_step(const KvRaw<HD, KVB> &r, int st, bf16x8 &kh, bf16x8 &kl) {
    if constexpr (KVB) {
        kh = __builtin_bit_cast(bf16x8, r.k[st]);
    } else {
        const float4 k0 = r.k[2 * st], k1 = r.k[2 * st + 1];
        const float kf[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
        split8(kf, kh, kl);
    }
}

// Reductions over the four 16-lane groups of a wave (lanes l, l^16, l^32, l^48)
// with the gfx950 lane-swap instructions. Given two copies of a value, a swap
// leaves this lane's value in one register and its partner's (lane ^ 16, resp.
// lane ^ 32) in the other (layout checked with a probe on MI355X), so combining
// the two reduces the pair without a trip through LDS; both lanes of a pair get
// the same result. The swaps are written as inline assembly because this
// compiler folds max(first output, second output) of the swap builtin into the
// first output when both inputs are one value. The s_nop gives the two wait
// states a swap needs after a VALU write of its operands.
__device__ __forceinline__ void lane_swap16(float &x, float &y) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void lane_swap32(float &x, float &y) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ float group4_max(float x) {
    float y = x;
    lane_swap16(x, y);
    x = fmaxf(x, y);
    y = x;
    lane_swap32(x, y);
    return fmaxf(x, y);
}
__device__ __forceinline__ float group4_sum(float x) {
    float y = x;
    lane_swap16(x, y);
    x = x + y;
    y = x;
    lane_swap32(x, y);
    return x + y;
}

// The running max of a query moves only when a score passes it by more than
// ATT_RESCALE (log2 units); until then probabilities are formed against the old
// max and may reach 2^ATT_RESCALE. The result is the same softmax (acc and l share
// the reference point), and the accumulator rescale runs on few sub-tiles.
constexpr float ATT_RESCALE = 8.0f;

// Order this wave's LDS writes before its following reads (and reads before later
// writes). A wavefront's LDS instructions execute in issue order, so only the
// compiler has to be kept from moving them across this point.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One workgroup (4 waves) per (key chunk, kv head, group of up to 16*QT queries);
// wave w takes the w-th quarter of the chunk and the four online-softmax states are
// merged through LDS at the end, so the chunk writes a single (acc, m, l) partial.
// Scores are formed transposed, S^T[key][q] = K Q^T (v_mfma_f32_16x16x32_bf16,
// A = 16 keys x 32 dims straight from the cache rows, B = pre-scaled queries split
// hi/lo, staged in LDS and, for BF16 caches where they fit, held in registers).
// That accumulator layout (lane: keys 4g..4g+3 of query l%16) is the B operand of
// v_mfma_f32_16x16x16_bf16 for O^T[d][q] += V^T[d][key] P^T[key][q], so the
// probabilities never leave their lanes. The V^T operand (4 keys x 1 dim per lane)
// is loaded straight in that order for F32 caches and split in registers; BF16
// caches load whole V rows, store them in LDS (a region private to the wave) and
// read the operand back transposed with ds_read_b64_tr_b16. The key loop has no
// workgroup barrier. F32 caches are split hi/lo (three products: hh, hl, lh); BF16
// caches are exact (two products: h*K, l*K). The K/V loads of the first sub-tiles
// are issued before the queries are staged, so their latency overlaps the staging.
template <int HD, int QT, bool KVB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(attn_wpe<HD, QT, KVB>()))) void k_attn(AttnArgs a) {
    // the arguments into scalar registers in one round trip
    asm volatile("" ::"s"(a.q), "s"(a.cache_k), "s"(a.cache_v), "s"(a.kv_bf16), "s"(a.capacity),
                 "s"(a.n_ctx), "s"(a.M), "s"(a.nq), "s"(a.nkv), "s"(a.chunk), "s"(a.bidir), "s"(a.part));
    using L = AttnLds<HD, QT, KVB>;
    constexpr int S = L::S, DT = L::DT, VTW = L::VTW;
    constexpr int PF = attn_prefetch<HD, KVB>();
    // F32 caches run the key loop peeled (below); the two-slot BF16 variants
    // measured slower that way: their unconditional refills push the registers to
    // the limit and the transposed V reads then go out one at a time.
    constexpr bool PEEL = !KVB;
    __shared__ __align__(16) unsigned char smem[L::BYTES];
    uint4 *qsm = (uint4 *)smem;

    // scalar wave index: the key range, the sub-tile count and every branch on them
    // are then scalar (no exec-mask branches around the reloads)
    const int w = wave_id();
    const int lane = threadIdx.x & 63;
    uint16_t *vth = (uint16_t *)(smem + L::Q_BYTES + (KVB ? w * L::VPLANE : 0));  // BF16 caches
    const int r16 = lane & 15, g = lane >> 4;
    const int c = blockIdx.x, kvh = blockIdx.y;
    const int G = a.nq / a.nkv;
    const int NQ = G * a.M;
    const int q0 = blockIdx.z * 16 * QT;
    const long long n_all = a.n_ctx + a.M;
    const int pw = a.chunk / ATT_WAVES;
    const long long c_hi = (long long)(c + 1) * a.chunk < n_all ? (long long)(c + 1) * a.chunk : n_all;
    const long long k_lo = (long long)c * a.chunk + (long long)w * pw;
    const long long k_hi = k_lo + pw < c_hi ? k_lo + pw : c_hi;  // may be <= k_lo: wave idle
    const int n_sub = k_hi > k_lo ? (int)((k_hi - k_lo + ATT_KT - 1) / ATT_KT) : 0;
    // scores in log2 units: the queries carry log2(e)/sqrt(hd), so p = 2^(s - max)
    const float scale = 1.4426950408889634f / sqrtf((float)HD);
    const size_t head_off = (size_t)kvh * a.capacity * HD;

    // the queries' loads go out ahead of the first K/V sub-tiles (loads return in
    // issue order), and are split and staged after those are issued
    constexpr int QIT = (QT * S + ATT_WAVES - 1) / ATT_WAVES;
    float qraw[QIT][8];
#pragma unroll
    for (int i = 0; i < QIT; i++) {
        const int idx = w + ATT_WAVES * i;
        if (idx < QT * S) {
            const int t = idx / S, st = idx % S;
            const int gq = q0 + 16 * t + r16;
            const int gqc = gq < NQ ? gq : NQ - 1;
            const int h = kvh * G + gqc % G;
            const float *src = a.q + (size_t)(gqc / G) * a.nq * HD + (size_t)h * HD + 32 * st + 8 * g;
#pragma unroll
            for (int j = 0; j < 8; j++) qraw[i][j] = src[j];
        }
    }
    // (issued even past the wave's range: those rows are clamped to the last key,
    // and every slot then has its loads in flight when the key loop starts)
    KvRaw<HD, KVB> rb[PF];
#pragma unroll
    for (int u = 0; u < PF; u++) {
        attn_load_k<HD, KVB>(rb[u], a, head_off, k_lo + (long long)u * ATT_KT, n_all, g, r16);
        attn_load_v<HD, KVB>(rb[u], a, head_off, k_lo + (long long)u * ATT_KT, n_all, g, r16);
    }

    int qm[QT];
    bool qv[QT];
#pragma unroll
    for (int t = 0; t < QT; t++) {
        const int gq = q0 + 16 * t + r16;
        qv[t] = gq < NQ;
        qm[t] = (qv[t] ? gq : NQ - 1) / G;
    }
    // B operand of the score MFMA, written cooperatively: lane holds dims 32s+8g..+7
#pragma unroll
    for (int i = 0; i < QIT; i++) {
        const int idx = w + ATT_WAVES * i;
        if (idx < QT * S) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; j++) v[j] = qraw[i][j] * scale;
            bf16x8 hi, lo;
            split8(v, hi, lo);
            qsm[(idx * 2 + 0) * 64 + lane] = __builtin_bit_cast(uint4, hi);
            qsm[(idx * 2 + 1) * 64 + lane] = __builtin_bit_cast(uint4, lo);
        }
    }

    // BF16 caches keep the query operands in registers where they fit (the F32
    // path needs those registers for its raw sub-tiles and re-reads them from LDS)
    constexpr bool QREG = KVB && QT * HD <= 256;
    bf16x8 qreg[QREG ? QT * S * 2 : 1];

    float m_run[QT], l_run[QT];  // l_run: this lane's share; summed over the groups at the end
    f32x4 acc[QT][DT];
#pragma unroll
    for (int t = 0; t < QT; t++) {
        m_run[t] = -INFINITY;
        l_run[t] = 0.f;
#pragma unroll
        for (int d = 0; d < DT; d++) acc[t][d] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();  // queries staged
    if constexpr (QREG) {
#pragma unroll
        for (int i = 0; i < QT * S * 2; i++) qreg[i] = __builtin_bit_cast(bf16x8, qsm[i * 64 + lane]);
    }
    // every query sees the keys up to lim_all; sub-tiles below it skip the mask
    const long long lim_all = a.n_ctx + (a.bidir ? a.M - 1 : 0);

    // Sub-tile it from slot rbu; with more, the slot's loads of sub-tile it + PF go
    // out as soon as its registers are free.
    auto sub_tile = [&](KvRaw<HD, KVB> &rbu, const int it, const bool more) __attribute__((always_inline)) {
        const long long kb = k_lo + (long long)it * ATT_KT;
        const long long kb_next = kb + (long long)PF * ATT_KT;
        if constexpr (KVB) attn_v_store<HD, VTW>(rbu, vth, g, r16);
        f32x4 sc[QT];
#pragma unroll
        for (int t = 0; t < QT; t++) sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < S; st++) {
            bf16x8 kh, kl;
            attn_k_step<HD, KVB>(rbu, st, kh, kl);
#pragma unroll
            for (int t = 0; t < QT; t++) {
                bf16x8 qh, ql;
                if constexpr (QREG) {
                    qh = qreg[(t * S + st) * 2 + 0];
                    ql = qreg[(t * S + st) * 2 + 1];
                } else {
                    qh = __builtin_bit_cast(bf16x8, qsm[((t * S + st) * 2 + 0) * 64 + lane]);
                    ql = __builtin_bit_cast(bf16x8, qsm[((t * S + st) * 2 + 1) * 64 + lane]);
                }
                sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, qh, sc[t], 0, 0, 0);
                sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kh, ql, sc[t], 0, 0, 0);
                if constexpr (!KVB) sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, qh, sc[t], 0, 0, 0);
            }
        }
        if (more) attn_load_k<HD, KVB>(rbu, a, head_off, kb_next, n_all, g, r16);
        // masked scores and their per-query max over the sub-tile
        const bool full = kb + ATT_KT <= k_hi && kb + ATT_KT - 1 <= lim_all;  // wave-uniform
        float sv[QT][4], mx[QT];
        bool grow = false;
#pragma unroll
        for (int t = 0; t < QT; t++) {
            if (full) {
#pragma unroll
                for (int i = 0; i < 4; i++) sv[t][i] = sc[t][i];
            } else {
                const long long lim = a.n_ctx + (a.bidir ? a.M - 1 : qm[t]);  // last visible key
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const long long kp = kb + 4 * g + i;
                    sv[t][i] = (kp < k_hi && kp <= lim) ? sc[t][i] : -INFINITY;
                }
            }
            mx[t] = group4_max(fmaxf(fmaxf(sv[t][0], sv[t][1]), fmaxf(sv[t][2], sv[t][3])));
            grow |= mx[t] > m_run[t] + ATT_RESCALE;  // first finite score: m_run is -inf
        }
        if (__ballot(grow)) {  // move the reference point of every query, rescale acc and l
#pragma unroll
            for (int t = 0; t < QT; t++) {
                const float m_new = fmaxf(m_run[t], mx[t]);
                const float al = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[t] - m_new);
                l_run[t] *= al;
#pragma unroll
                for (int d = 0; d < DT; d++) acc[t][d] *= al;
                m_run[t] = m_new;
            }
        }
        s16x4 ph[QT], pl[QT];
#pragma unroll
        for (int t = 0; t < QT; t++) {
            const float m_use = m_run[t] == -INFINITY ? 0.f : m_run[t];  // all scores -inf: p = 0
            float p[4], ps = 0.f;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                p[i] = __builtin_amdgcn_exp2f(sv[t][i] - m_use);
                ps += p[i];
            }
            split4(p[0], p[1], p[2], p[3], ph[t], pl[t]);
            l_run[t] += ps;
        }
        if constexpr (KVB) wave_lds_sync();  // V rows of this sub-tile written by every lane
#pragma unroll
        for (int d = 0; d < DT; d++) {
            s16x4 va, vb;
            if constexpr (KVB) {
                va = attn_v_operand<VTW>(vth, d, g, r16);
            } else {
                split4(rbu.v[4 * d], rbu.v[4 * d + 1], rbu.v[4 * d + 2], rbu.v[4 * d + 3], va, vb);
            }
#pragma unroll
            for (int t = 0; t < QT; t++) {
                f32x4 o = acc[t][d];
                o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, ph[t], o, 0, 0, 0);
                o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pl[t], o, 0, 0, 0);
                if constexpr (!KVB) o = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vb, ph[t], o, 0, 0, 0);
                acc[t][d] = o;
            }
        }
        if constexpr (KVB) wave_lds_sync();  // V reads done before the next sub-tile overwrites them
        if (more) attn_load_v<HD, KVB>(rbu, a, head_off, kb_next, n_all, g, r16);
    };
    // The main loop refills every slot, so each slot's loads are in flight in a fixed
    // order and the wait for one slot leaves the others' loads outstanding; the last
    // sub-tiles, whose refills depend on the count, run after it (a conditional
    // refill inside the loop makes every wait cover all slots).
    const int n_main = (PEEL && n_sub > PF) ? (n_sub - PF) / PF * PF : 0;
    int it0 = 0;
    for (; it0 < n_main; it0 += PF) {
#pragma unroll
        for (int u = 0; u < PF; u++) sub_tile(rb[u], it0 + u, true);
    }
    for (; it0 < n_sub; it0 += PF) {
#pragma unroll
        for (int u = 0; u < PF; u++) {
            const int it = it0 + u;
            if (it >= n_sub) break;
            sub_tile(rb[u], it, it + PF < n_sub);
        }
    }

    // merge the four waves' (m, l, acc) through LDS (the loop buffers are dead now):
    // wave w finishes the dims tiles [w DPW, (w+1) DPW) of every query tile, so
    // each wave writes the other waves' tiles of its accumulator and reads the
    // three other copies of its own
    constexpr int DPW = DT / ATT_WAVES;
    static_assert(DT % ATT_WAVES == 0, "every wave owns whole dims tiles");
#pragma unroll
    for (int t = 0; t < QT; t++) l_run[t] = group4_sum(l_run[t]);
    __syncthreads();
    // [3][QT][DT][64]: writer v's copy of dims tile d, in slot v (v < owner) or
    // v - 1 (v > owner) of the owner's three
    float4 *accb = (float4 *)smem;
    float2 *mlb = (float2 *)(smem + L::ACC_BYTES);  // [4][QT][64]
#pragma unroll
    for (int t = 0; t < QT; t++) {
        mlb[(w * QT + t) * 64 + lane] = make_float2(m_run[t], l_run[t]);
#pragma unroll
        for (int d = 0; d < DT; d++) {
            const int own = d / DPW;
            if (own == w) continue;
            const int slot = w < own ? w : w - 1;
            accb[((slot * QT + t) * DT + d) * 64 + lane] =
                make_float4(acc[t][d][0], acc[t][d][1], acc[t][d][2], acc[t][d][3]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < QT; t++) {
        float mw[ATT_WAVES], lw[ATT_WAVES];
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < ATT_WAVES; v++) {
            const float2 ml = mlb[(v * QT + t) * 64 + lane];
            mw[v] = ml.x;
            lw[v] = ml.y;
            if (ml.y > 0.f) mx = fmaxf(mx, ml.x);
        }
        float e[ATT_WAVES], lsum = 0.f;
#pragma unroll
        for (int v = 0; v < ATT_WAVES; v++) {
            e[v] = lw[v] > 0.f ? exp2f(mw[v] - mx) : 0.f;
            lsum += lw[v] * e[v];
        }
        if (!qv[t]) continue;
        const int gq = q0 + 16 * t + r16;
        const int h = kvh * G + gq % G;
        const size_t qidx = (size_t)qm[t] * a.nq + h;
        float *o = a.part + ((size_t)c * a.M * a.nq + qidx) * (HD + ATT_PART_EXTRA);
#pragma unroll
        for (int d = 0; d < DT; d++) {
            if (d / DPW != w) continue;
            // waves in order 0..3, this wave's own copy from its registers
            f32x4 s4;
#pragma unroll
            for (int v = 0; v < ATT_WAVES; v++) {
                f32x4 x;
                if (v == w) {
                    x = acc[t][d];
                } else {
                    const float4 q4 = accb[(((v < w ? v : v - 1) * QT + t) * DT + d) * 64 + lane];
                    x = f32x4{q4.x, q4.y, q4.z, q4.w};
                }
                if (v == 0)
                    s4 = x * e[0];
                else
                    s4 += x * e[v];
            }
            *(float4 *)(o + 16 * d + 4 * g) = make_float4(s4[0], s4[1], s4[2], s4[3]);
        }
        if (w == 0 && g == 0) {
            o[HD] = lsum > 0.f ? mx : -INFINITY;
            o[HD + 1] = lsum;
        }
    }
}

bool attn_supported(int hd) { return hd == 64 || hd == 128 || hd == 256; }

// qt comes from attn_qtiles with the same cap, so every value reaching here has a variant
template <int HD, bool KVB>
static void go_attn(const AttnArgs &a, int qt, dim3 grid, hipStream_t s) {
    constexpr int CAP = attn_qt_cap(HD, KVB);
    if (qt == 1) {
        launch_k(PROF_ATTN, "k_attn", (k_attn<HD, 1, KVB>), grid, dim3(256), 0, s, a);
    } else if constexpr (CAP >= 2) {
        if (qt == 2) launch_k(PROF_ATTN, "k_attn", (k_attn<HD, 2, KVB>), grid, dim3(256), 0, s, a);
        else if constexpr (CAP >= 4) launch_k(PROF_ATTN, "k_attn", (k_attn<HD, 4, KVB>), grid, dim3(256), 0, s, a);
    }
}

void launch_attn(const AttnArgs &a, hipStream_t s) {
    const int G = a.nq / a.nkv;
    const int NQ = G * a.M;
    const int qt = attn_qtiles(a.hd, NQ, a.kv_bf16 != 0);
    dim3 grid(a.n_chunks, a.nkv, (NQ + 16 * qt - 1) / (16 * qt));
    if (a.kv_bf16) {
        if (a.hd == 64) go_attn<64, true>(a, qt, grid, s);
        else if (a.hd == 128) go_attn<128, true>(a, qt, grid, s);
        else go_attn<256, true>(a, qt, grid, s);
    } else {
        if (a.hd == 64) go_attn<64, false>(a, qt, grid, s);
        else if (a.hd == 128) go_attn<128, false>(a, qt, grid, s);
        else go_attn<256, false>(a, qt, grid, s);
    }
}

// Merge the chunk partials of query (m, h), apply the optional sigmoid gate and
// write the attention output row into the split tile of the O projection. With NT
// threads, thread t takes dims 4 (t % (hd/4)) .. +3 (one float4) of the chunks
// congruent to t / (hd/4) modulo 4 NT / hd; it reads them in batches of B records,
// every load of a batch in flight at once (a batch past the last chunk re-reads its
// first record and drops it), and folds each batch into a running (max, sum, acc)
// state; the chunk groups are then merged through LDS in a fixed order. The host
// picks NT and B from the chunk count so that a thread issues about as many loads
// as it has chunks. The grid is M x nq; block (m, h) also writes zeros into the
// padding rows m + M, m + 2M, ... < SPLIT_ROWS of its columns. (hd is 64, 128 or 256, so the
// split tile of nq * hd columns has no padding columns.)
template <int HD, int NT, int B>
__global__ __launch_bounds__(NT) void k_attn_combine(CombineArgs a) {
    // the arguments into scalar registers in one round trip
    asm volatile("" ::"s"(a.part), "s"(a.n_chunks), "s"(a.M), "s"(a.nq), "s"(a.hd), "s"(a.g), "s"(a.xs));
    __shared__ float4 sm_o[NT];
    __shared__ float sm_m[NT], sm_l[NT];
    const int m = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    constexpr int hd = HD, tpg = HD / 4, ngrp = NT / tpg;  // threads per chunk group, chunk groups
    const int K = a.nq * hd, rec = hd + ATT_PART_EXTRA;
    const int d4 = tid % tpg, grp = tid / tpg;
    // the gate values go out with the partial loads instead of after the merge
    float4 gv = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.g && grp == 0) gv = *(const float4 *)(a.g + (size_t)m * K + h * hd + 4 * d4);
    float mr = -INFINITY, lr = 0.f;
    f32x4 orun = {0.f, 0.f, 0.f, 0.f};
    {
        const size_t stride = (size_t)a.M * a.nq * rec;
        const float *p = a.part + ((size_t)m * a.nq + h) * rec;
        for (int c0 = grp; c0 < a.n_chunks; c0 += B * ngrp) {
            float mv[B], lv[B];
            f32x4 ov[B];
#pragma unroll
            for (int j = 0; j < B; j++) {
                const int cc = c0 + j * ngrp;
                const float *pc = p + (size_t)(cc < a.n_chunks ? cc : c0) * stride;
                mv[j] = pc[hd];
                lv[j] = cc < a.n_chunks ? pc[hd + 1] : 0.f;
                const float4 o4 = *(const float4 *)(pc + 4 * d4);
                ov[j] = f32x4{o4.x, o4.y, o4.z, o4.w};
            }
            float bm = -INFINITY;
#pragma unroll
            for (int j = 0; j < B; j++)
                if (lv[j] > 0.f) bm = fmaxf(bm, mv[j]);
            const float mn = fmaxf(mr, bm);
            if (mn != -INFINITY) {
                const float sc = lr > 0.f ? exp2f(mr - mn) : 0.f;
                orun *= sc;
                lr *= sc;
#pragma unroll
                for (int j = 0; j < B; j++) {
                    const float e = lv[j] > 0.f ? exp2f(mv[j] - mn) : 0.f;
                    orun += ov[j] * e;
                    lr += lv[j] * e;
                }
                mr = mn;
            }
        }
    }
    sm_m[tid] = mr;
    sm_l[tid] = lr;
    sm_o[tid] = make_float4(orun[0], orun[1], orun[2], orun[3]);
    __syncthreads();
    if (grp != 0) return;
    float o[4];
    {
        // unrolled 8 at a time: a full unroll over the 32 or 64 groups of the
        // 1024-thread blocks held every group's record in registers at once and
        // spilled (the additions keep their order either way)
        float mx = -INFINITY;
#pragma unroll 8
        for (int q = 0; q < ngrp; q++)
            if (sm_l[q * tpg + d4] > 0.f) mx = fmaxf(mx, sm_m[q * tpg + d4]);
        f32x4 osum = {0.f, 0.f, 0.f, 0.f};
        float lsum = 0.f;
#pragma unroll 8
        for (int q = 0; q < ngrp; q++) {
            const float lq = sm_l[q * tpg + d4];
            const float e = lq > 0.f ? exp2f(sm_m[q * tpg + d4] - mx) : 0.f;
            const float4 oq = sm_o[q * tpg + d4];
            osum += f32x4{oq.x, oq.y, oq.z, oq.w} * e;
            lsum += lq * e;
        }
        const float gvv[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            o[i] = osum[i] / lsum;
            if (a.g) o[i] *= sigmoidf_(gvv[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; i++) split_store(a.xs, m, h * hd + 4 * d4 + i, o[i]);
    for (int r = m + a.M; r < SPLIT_ROWS; r += a.M)
#pragma unroll
        for (int i = 0; i < 4; i++) split_store(a.xs, r, h * hd + 4 * d4 + i, 0.f);
}

template <int HD>
static void launch_combine_hd(const CombineArgs &a, hipStream_t s) {
    // chunks per thread with 256 threads; past 8 the block takes 1024 threads
    constexpr int g256 = 1024 / HD, g1024 = 4096 / HD;
    const int per256 = (a.n_chunks + g256 - 1) / g256;
    const int per1024 = (a.n_chunks + g1024 - 1) / g1024;
    const dim3 grid(a.M, a.nq);
    if (per256 <= 4) {
        launch_k(PROF_ATTN, "k_attn_combine", k_attn_combine<HD, 256, 4>, grid, dim3(256), 0, s, a);
    } else if (per256 <= 8) {
        launch_k(PROF_ATTN, "k_attn_combine", k_attn_combine<HD, 256, 8>, grid, dim3(256), 0, s, a);
    } else if (per1024 <= 8) {
        launch_k(PROF_ATTN, "k_attn_combine", k_attn_combine<HD, 1024, 8>, grid, dim3(1024), 0, s, a);
    } else if constexpr ((ATT_CHUNKS_MAX + g1024 - 1) / g1024 > 8) {
        // only 256-dim heads reach 16 chunks per thread within ATT_CHUNKS_MAX chunks
        launch_k(PROF_ATTN, "k_attn_combine", k_attn_combine<HD, 1024, 16>, grid, dim3(1024), 0, s, a);
    }
}

void launch_attn_combine(const CombineArgs &a, hipStream_t s) {
    if (a.hd == 64)
        launch_combine_hd<64>(a, s);
    else if (a.hd == 128)
        launch_combine_hd<128>(a, s);
    else
        launch_combine_hd<256>(a, s);
}

// ---------------------------------------------------------------------------
// Greedy accept-prefix walk (hf2q dflash/qwen35_orchestrator.rs, module doc:
// greedy accept-walk invariant; per-round steps 7-8). One wavefront.
__global__ __launch_bounds__(64) void k_accept(const int32_t *d, const int32_t *t, int K,
                                               const int32_t *eos, int n_eos, int32_t *res,
                                               int32_t *committed) {
    // the arguments into scalar registers in one round trip
    asm volatile("" ::"s"(d), "s"(t), "s"(K), "s"(eos), "s"(n_eos), "s"(res), "s"(committed));
    accept_walk(d, t, K, eos, n_eos, res, committed);
}

void launch_accept(const int32_t *drafts, const int32_t *target, int K, const int32_t *eos,
                   int n_eos, int32_t *result, int32_t *committed, hipStream_t s) {
    launch_k(PROF_ACCEPT, "k_accept", k_accept, dim3(1), dim3(64), 0, s, drafts, target, K, eos, n_eos, result,
                       committed);
}

}  // namespace dbf
