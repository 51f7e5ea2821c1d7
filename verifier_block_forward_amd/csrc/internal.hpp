// internal.hpp -- device helpers and launch declarations shared by the libdbf kernels.
//
// Activation "split" layout. Every projection in the block multiplies BF16 weights
// by F32 activations. The kernels run these products on the gfx950 matrix cores
// (v_mfma_f32_16x16x32_bf16) by splitting each F32 activation a into two BF16
// terms, hi = rne(a) and lo = rne(a - hi), so that a = hi + lo + r with
// |r| <= 2^-16 |a|; each BF16*BF16 product is exact in the F32 accumulator. This
// is the multi-word BF16 splitting of Henry, Tang and Heinecke ("Leveraging the
// bfloat16 artificial intelligence datatype for higher-precision computations",
// ARITH 2019).
//
// A split buffer holds up to 16 activation rows ("one tile") of length K, padded
// to a multiple of 32 columns, in the order the MFMA B operand is read: for k-step
// s (columns 32s..32s+31), half h (0 = hi, 1 = lo) and lane l of a wavefront,
// 8 consecutive BF16 at element offset ((s*2 + h)*64 + l)*8. Lane l carries
// activation row (l % 16) and columns 32s + 8*(l/16) .. +7. A wave therefore reads
// each half of a k-step as one contiguous, fully coalesced 1 KiB line.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dbf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
#define DBF_MAX_TOPK_DEV 16

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// F32 -> BF16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

constexpr int SPLIT_ROWS = 16;  // rows of a split tile

// bytes of one split tile for K columns
__host__ __device__ inline size_t split_tile_bytes(int K) {
    return (size_t)((K + 31) / 32) * 2 * 64 * 8 * sizeof(uint16_t);
}

// element offset (in uint16 units) of activation (row r < 16, column k), half h
__device__ __forceinline__ size_t split_index(int r, int k, int h) {
    int s = k >> 5, g = (k & 31) >> 3, j = k & 7;
    return ((size_t)(s * 2 + h) * 64 + (g * 16 + r)) * 8 + j;
}

typedef float f32x2_split __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_split __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_split __attribute__((ext_vector_type(4)));

// Two F32 values split into BF16 hi (round to nearest even) and lo = BF16(x - hi),
// each pair packed in one dword (first value in the low half): the same values as
// split_store, with one v_cvt_pk_bf16_f32 per pair instead of one per value plus
// a repack.
__device__ __forceinline__ void split2(float a, float b, unsigned &hi, unsigned &lo) {
    const f32x2_split f = {a, b};
    const bf16x2_split h = __builtin_convertvector(f, bf16x2_split);
    const f32x2_split hf = __builtin_convertvector(h, f32x2_split);
    const bf16x2_split l = __builtin_convertvector(f - hf, bf16x2_split);
    hi = __builtin_bit_cast(unsigned, h);
    lo = __builtin_bit_cast(unsigned, l);
}

// eight consecutive values (one lane's run of a k-step) into hi and lo operands
__device__ __forceinline__ void split8(const float *v, bf16x8 &hi, bf16x8 &lo) {
    u32x4_split h, l;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        unsigned a, b;
        split2(v[2 * j], v[2 * j + 1], a, b);
        h[j] = a;
        l[j] = b;
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

__device__ __forceinline__ void split_store(uint16_t *tile, int r, int k, float a) {
    uint16_t hi = f32_to_bf16(a);
    float rem = a - bf16_to_f32(hi);
    tile[split_index(r, k, 0)] = hi;
    tile[split_index(r, k, 1)] = f32_to_bf16(rem);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
    return v;
}

// Sum over a 256-thread block in a fixed order (wave sums, then waves 0..3).
__device__ __forceinline__ float block_sum_256(float v, float *sh4) {
    v = wave_sum(v);
    int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh4[w] = v;
    __syncthreads();
    return (sh4[0] + sh4[1]) + (sh4[2] + sh4[3]);
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }

// RMSNorm row scale s_m = 1/sqrt(mean x^2 + eps) from the per-64-column partial sums
// of squares of the row, formed by a whole wavefront (lane-strided sum, then a
// fixed xor tree). Split in two so that a kernel can issue the first load (this
// lane's element of the first 64) together with its other independent loads, and
// finish the sum after one wait for all of them.
__device__ __forceinline__ float row_scale_first(const float *ssp_row, int ncb) {
    const int lane = threadIdx.x & 63;
    return lane < ncb ? ssp_row[lane] : 0.f;
}

__device__ __forceinline__ float row_scale_finish(float first, const float *ssp_row, int ncb, int H,
                                                  float eps) {
    const int lane = threadIdx.x & 63;
    float s = first;
    for (int i = lane + 64; i < ncb; i += 64) s += ssp_row[i];
    s = wave_sum(s);
    return 1.0f / sqrtf(s / (float)H + eps);
}

// This thread's wavefront within the workgroup, as a value the compiler knows to
// be uniform across the wave (readfirstlane): indexes and branches derived from it
// stay in scalar registers instead of vector registers and exec-mask branches.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Kernel arguments are read with scalar loads, and the compiler fetches each one
// where a branch first needs it, so a kernel that tests several pointers pays a
// chain of dependent scalar round trips before its first global load. The row
// kernels therefore start with an empty asm statement that takes every argument
// they read as an "s" (scalar register) operand: all the loads go out together and
// one wait covers them. One statement per kernel, not one per value: separate
// statements were scheduled one wait apart in some kernels.

// Split-K partial sums. A projection writes its ks partial products as
// [ks][rows][N] F32; consumers add them in increasing ks order. The loads go out
// in batches of PARTIAL_BATCH (indexes past ks re-read the last partial and are
// not added), so a sum over ks partials costs ceil(ks / PARTIAL_BATCH) memory
// round trips instead of one per few partials.
constexpr int PARTIAL_BATCH = 16;

// NV sums sharing ks and the partial stride: out[v] = sum_t base[v][t * stride],
// loaded B partials at a time. The additions run in increasing t whatever B is.
template <int NV, int B = PARTIAL_BATCH>
__device__ __forceinline__ void sum_partials_n(const float *const base[NV], int ks, size_t stride,
                                               float out[NV]) {
#pragma unroll
    for (int v = 0; v < NV; v++) out[v] = 0.f;
    for (int t0 = 0; t0 < ks; t0 += B) {
        float x[NV][B];
#pragma unroll
        for (int u = 0; u < B; u++) {
            const int t = t0 + u < ks ? t0 + u : ks - 1;
#pragma unroll
            for (int v = 0; v < NV; v++) x[v][u] = base[v][(size_t)t * stride];
        }
#pragma unroll
        for (int u = 0; u < B; u++)
#pragma unroll
            for (int v = 0; v < NV; v++) out[v] += t0 + u < ks ? x[v][u] : 0.f;
    }
}

// element (row, col) summed over the ks partials of a [ks][rows][N] buffer. Up to
// 24 partials (the long-K projections split 22 ways) take one round trip.
__device__ __forceinline__ float sum_partials(const float *p, int ks, int rows, int N, int row,
                                              int col) {
    const float *b[1] = {p + (size_t)row * N + col};
    float o[1];
    if (ks > PARTIAL_BATCH)
        sum_partials_n<1, 24>(b, ks, (size_t)rows * N, o);
    else
        sum_partials_n<1>(b, ks, (size_t)rows * N, o);
    return o[0];
}

// Greedy accept-prefix walk (hf2q dflash/qwen35_orchestrator.rs, module doc:
// greedy accept-walk invariant; per-round steps 7-8), run by one whole wavefront:
// a = length of the longest prefix with d[i] == t[i]; res = {a, t[a], K - a,
// hit_eos, n_committed}; committed = t[0..a], cut after the first EOS (inclusive).
// d may point to LDS (generic address).
__device__ __forceinline__ void accept_walk(const int32_t *d, const int32_t *t, int K, const int32_t *eos,
                                            int n_eos, int32_t *res, int32_t *committed) {
    const int lane = threadIdx.x & 63;
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

}  // namespace dbf
