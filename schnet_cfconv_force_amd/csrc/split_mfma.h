// Split-fp16 matrix products on v_mfma_f32_16x16x32_f16 at close to fp32
// accuracy (the atom-wise layers and the filter network share them).
//
// An fp32 operand x is first scaled by a power of two (exact) so that
// |x| < 2^14, then held as hi = fp16(x) and lo = fp16(x - hi).  x - hi is
// exact in fp32, and for |x| >= 2^-3 its fp16 rounding keeps 11 bits, so
// hi + lo carries about 22 significant bits; smaller values lose low bits of
// lo, an absolute error below 2^-25 (below 2^-39 of the operand's scale).
// A product a.b is accumulated in one fp32 accumulator as hi.hi + hi.lo +
// lo.hi; the dropped lo.lo term is below 2^-22 |a||b|.  The weights (the A
// operands, staged once per block in LDS) are scaled per matrix from the
// block-wide maximum, the per-atom or per-pair data (the B operands, in
// registers) by exponents from their own maxima or bounds, and the result is
// unscaled by one ldexp.
//
// Layout of one 16x16x32 product (64 lanes): A fragment of lane l = row
// l%16, k = 8(l/16) + j; B fragment = column l%16, k = 8(l/16) + j; the
// accumulator of lane l = column l%16, rows 4(l/16) + r.
#pragma once

#include "sn_internal.h"

namespace sn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

// |x| < 2^kSplitTop after scaling
constexpr int kSplitTop = 14;

__device__ inline void split8(const float (&v)[8], half8 &hi, half8 &lo) {
    // The values are opaque to the compiler: otherwise it may fuse the
    // product that made one into its conversion to hi at one use but not at
    // another, and hi would then differ between them by a rounding.
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        x[j] = v[j];
        asm("" : "+v"(x[j]));
    }
    half8 h;
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = (_Float16)x[j];
    // hi is converted once (packed pairs); lo = x - hi (exact) is one
    // mixed-precision fma per value that reads hi from its packed half, for
    // which -1 is kept opaque too (folded, x - hi would become a conversion
    // back to fp32 and a subtraction)
    asm("" : "+v"(h));
    float m1 = -1.0f;
    asm("" : "+s"(m1));
    half8 l;
#pragma unroll
    for (int j = 0; j < 8; ++j) l[j] = (_Float16)fmaf((float)h[j], m1, x[j]);
    hi = h;
    lo = l;
}

// The same for four values (half of one B operand).
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
__device__ inline void split4(const float (&v)[4], half4 &hi, half4 &lo) {
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[j] = v[j];
        asm("" : "+v"(x[j]));
    }
    half4 h;
#pragma unroll
    for (int j = 0; j < 4; ++j) h[j] = (_Float16)x[j];
    asm("" : "+v"(h));
    float m1 = -1.0f;
    asm("" : "+s"(m1));
    half4 l;
#pragma unroll
    for (int j = 0; j < 4; ++j) l[j] = (_Float16)fmaf((float)h[j], m1, x[j]);
    hi = h;
    lo = l;
}

// One fp16 operand (no low half), for products taken in plain fp16.
__device__ inline half8 to_half8(const float (&v)[8]) {
    half8 h;
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = (_Float16)v[j];
    return h;
}

// Power-of-two exponent s with amax 2^s in [2^(kSplitTop-1), 2^kSplitTop)
// (0 for a zero or non-finite maximum).
__device__ inline int split_scale(float amax) {
    return (amax > 0.0f && amax < INFINITY) ? (kSplitTop - 1) - ilogbf(amax) : 0;
}

// Stage nf (<= NF) fragments of one weight matrix into LDS: fragment idx
// holds the eight weights that val(idx, v) writes to v, scaled by 2^sc and
// split (hi and lo in separate arrays, so that a wavefront's 16-byte reads
// are contiguous and free of bank conflicts).  sc comes from the matrix's largest
// magnitude, a block-wide maximum through *s_max, which must hold 0 on
// entry.  All of a thread's global loads are issued before the first is
// used.  Every thread of the block must call it (it holds a barrier);
// returns sc.
template <int NF, int NTHR, typename Val>
__device__ inline int stage_split(half8 *hi, half8 *lo, int nf, unsigned *s_max, Val val) {
    constexpr int IT = (NF + NTHR - 1) / NTHR;
    float v[IT][8];
    float mx = 0.0f;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int idx = (int)threadIdx.x + it * NTHR;
        if (idx < nf) {
            val(idx, v[it]);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[it][j] = 0.0f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(v[it][j]));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if ((threadIdx.x & 63) == 0) atomicMax(s_max, __float_as_uint(mx));
    __syncthreads();
    const int sc = split_scale(__uint_as_float(*s_max));
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int idx = (int)threadIdx.x + it * NTHR;
        if (idx < nf) {
            float w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] = ldexpf(v[it][j], sc);
            split8(w, hi[idx], lo[idx]);
        }
    }
    return sc;
}

// Copy nf (<= NF) pre-split fragments (a weight-pack slot) into LDS; all of
// a thread's loads are issued before the first store.
template <int NF, int NTHR>
__device__ inline void copy_frags(half8 *hi, half8 *lo, const half8 *src_hi, const half8 *src_lo, int nf) {
    constexpr int IT = (NF + NTHR - 1) / NTHR;
    half8 vh[IT], vl[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int idx = (int)threadIdx.x + it * NTHR;
        if (idx < nf) {
            vh[it] = src_hi[idx];
            vl[it] = src_lo[idx];
        }
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int idx = (int)threadIdx.x + it * NTHR;
        if (idx < nf) {
            hi[idx] = vh[it];
            lo[idx] = vl[it];
        }
    }
}

// acc[m][n] += A_m B_n in split form for MG weight tiles (fragments at
// whi[m * stride], wlo[m * stride]) and NT B operands; dependent matrix
// instructions on one accumulator are MG*NT instructions apart.
template <int MG, int NT>
__device__ inline void mma_split(const half8 *whi, const half8 *wlo, int stride, const half8 *bh, const half8 *bl,
                                 floatx4 (*acc)[NT]) {
    half8 ah[MG], al[MG];
#pragma unroll
    for (int m = 0; m < MG; ++m) {
        ah[m] = whi[m * stride];
        al[m] = wlo[m * stride];
    }
#pragma unroll
    for (int m = 0; m < MG; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[m], bh[n], acc[m][n], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < MG; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[m], bl[n], acc[m][n], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < MG; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[m], bh[n], acc[m][n], 0, 0, 0);
}

// acc[m][n] += A_m B_n with one fp16 product per pair of operands (the hi
// halves only): fp32 accumulation of fp16-rounded operands.
template <int MG, int NT>
__device__ inline void mma_one(const half8 *whi, int stride, const half8 *bh, floatx4 (*acc)[NT]) {
    half8 ah[MG];
#pragma unroll
    for (int m = 0; m < MG; ++m) ah[m] = whi[m * stride];
#pragma unroll
    for (int m = 0; m < MG; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[m], bh[n], acc[m][n], 0, 0, 0);
}

}  // namespace sn
