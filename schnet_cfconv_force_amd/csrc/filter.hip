// Filter network on the matrix cores ("How", flash radial basis and the
// filter network with channel-wise 16-bit weights -- FlashSchNet summary
// page; OpenAlex abstract techniques (1) and (4)).
//
// Per pair p with distance d_p (one row shared by both directed edges):
//   a   = rbf(d) A1 + b1            rbf_k = exp(-gamma (d - mu_k)^2), K <= 64
//   phi = ssp(a) A2 + b2            (the envelope fc(d) is applied by the CFConv)
// and, in the backward pass, with G_p = g_y_i (.) x_j + g_y_j (.) x_i (the
// gradient of E with respect to the shared filter row):
//   g_fc = <G, phi>,  g_phi = fc G,  g_a = (g_phi A2^T) (.) sigmoid(a),
//   g_rbf = g_a A1^T,  S_p += sum_k g_rbf_k rbf_k'(d) + g_fc fc'(d).
//
// Precision.  The products run on v_mfma_f32_16x16x32_f16 in split form:
// every fp32 operand x is held as hi = fp16(x) and lo = fp16((x - hi) 2^11),
// and a.b is accumulated as hi.hi into one fp32 accumulator and
// hi.lo + lo.hi into a second one that is scaled by 2^-11 at the end.  The
// dropped lo.lo term is below 2^-22 |a||b|, so the result carries close to
// fp32 accuracy at 3/16 of the cost of fp32 matrix instructions.  Backward
// operands are first scaled per pair by a power of two (exact) so that no
// value falls into the fp16 subnormal range.
//
// Matrix-core mapping.  Everything is computed transposed: features are the
// M dimension and 16 pairs are the N dimension.  Lane l always owns pair
// l%16; the accumulator layout of one GEMM (lane l: rows 4(l/16)+r of each
// 16-row tile) becomes the B operand of the next one (lane l: k-slot l/16,
// 8 values) once the k index of value j of a 32-wide step t is taken to be
// 32t + 16(j/4) + 4(l/16) + j%4 -- two accumulator tiles make one step.  So
// the chained GEMMs never leave registers.  The weights are pre-split and
// pre-arranged in LDS in the order the lanes consume them: one pair of
// 16-byte reads per lane feeds three matrix instructions.  The radial basis
// is generated in registers from d (no E x K tensor exists anywhere).
//
// Work distribution: persistent blocks (one per CU, weights staged once into
// LDS, int16 codes dequantised while staging); each wavefront loops over
// 16-pair tiles of an XCD-contiguous range.
#include "sn_internal.h"

namespace sn {

namespace {

constexpr int kFwdThreads = 1024;   // 4 wavefronts per SIMD
constexpr int kFwdNT = 1;           // 16-pair tiles per forward wavefront (2 measured slower)
constexpr int kFwdMG = 4;           // forward output tiles per product group
constexpr int kBwdThreads = 1024;   // 4 wavefronts per SIMD
constexpr int kBwdMG = 1;           // backward output tiles per group (register budget of 4 wavefronts)
constexpr float kPi = 3.14159265358979323846f;
constexpr float kLoScale = 2048.0f;        // 2^11
constexpr float kLoUnscale = 1.0f / 2048.0f;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

struct FilterArgs {
    int K;
    float lo, dmu, gamma, cutoff;
    const float *A1, *A2;        // fp32 weights (format 0)
    const int16_t *qA1, *qA2;    // int16 codes (format 1)
    const float *sA1, *sA2;      // per-output-column scales (format 1)
    const float *b1, *b2;
    const float *dsrc;           // distance of pair p at dsrc[p * dstride + doff]
    int dstride, doff;
    int64_t P;
    float *phi;                  // forward output [P][F]
    // backward
    const int2 *pair_ij;
    const float *x, *gy;         // [N][F]
    const float *phi_in;         // [P][F]
    float *S;                    // [P]
    const float *xmax, *gmax;    // [N]: max_f |x_i[f]|, max_f |g_y_i[f]|
    int accumulate;
};

template <int F>
__device__ inline float w1(const FilterArgs &a, int k, int f) {   // A1[k][f], 0 beyond K
    if (k >= a.K) return 0.0f;
    if (a.qA1) return (float)a.qA1[k * F + f] * a.sA1[f];
    return a.A1[k * F + f];
}
template <int F>
__device__ inline float w2(const FilterArgs &a, int g, int f) {   // A2[g][f]
    if (a.qA2) return (float)a.qA2[g * F + f] * a.sA2[f];
    return a.A2[g * F + f];
}

__device__ inline void split8(const float (&v)[8], half8 &hi, half8 &lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const _Float16 h = (_Float16)v[j];
        hi[j] = h;
        lo[j] = (_Float16)fmaf((float)h, -kLoScale, v[j] * kLoScale);   // (x - hi) 2^11, exact
    }
}



// Stage nf (<= NF) weight fragments into LDS: fragment idx holds the eight
// weights val(idx, j), split.  A thread's global loads for all of its
// fragments are issued before the first one is used, so the staging costs
// one memory latency rather than one per fragment.
template <int NF, int NT, typename Val>
__device__ inline void stage_frags(half8 *hi, half8 *lo, int nf, Val val) {
    constexpr int IT = (NF + NT - 1) / NT;
    float v[IT][8];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int idx = (int)threadIdx.x + it * NT;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[it][j] = idx < nf ? val(idx, j) : 0.0f;
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int idx = (int)threadIdx.x + it * NT;
        if (idx < nf) split8(v[it], hi[idx], lo[idx]);
    }
}

// The three split products for MT output tiles that share one B operand,
// ordered so that dependent matrix instructions on the same accumulator are
// MT instructions apart: hi.hi and hi.lo for every tile, then lo.hi.
// Fragment halves of tile m at whi[m * stride], wlo[m * stride] (hi and lo
// live in separate arrays so that a wavefront's 16-byte reads are contiguous
// and free of LDS bank conflicts).
template <int MT>
__device__ inline void mma3_tiles(const half8 *whi, const half8 *wlo, int stride, const half8 &bh, const half8 &bl,
                                  floatx4 *main, floatx4 *corr) {
    half8 lo[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const half8 hi = whi[m * stride];
        main[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, bh, main[m], 0, 0, 0);
        corr[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, bl, corr[m], 0, 0, 0);
        lo[m] = wlo[m * stride];
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) corr[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo[m], bh, corr[m], 0, 0, 0);
}

// The split products for MG weight tiles and NT B operands (16-pair tiles)
// sharing one pair of fragment reads: main[m][n] += hi.hi, corr[m][n] +=
// hi.lo + lo.hi; dependent instructions on one accumulator are MG*NT apart.
template <int MG, int NT>
__device__ inline void mma3_tiles_nt(const half8 *whi, const half8 *wlo, int stride, const half8 (&bh)[NT],
                                     const half8 (&bl)[NT], floatx4 (&main)[MG][NT], floatx4 (&corr)[MG][NT]) {
    half8 lo[MG];
#pragma unroll
    for (int m = 0; m < MG; ++m) {
        const half8 hi = whi[m * stride];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            main[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, bh[n], main[m][n], 0, 0, 0);
            corr[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, bl[n], corr[m][n], 0, 0, 0);
        }
        lo[m] = wlo[m * stride];
    }
#pragma unroll
    for (int m = 0; m < MG; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) corr[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo[m], bh[n], corr[m][n], 0, 0, 0);
}

// Two B operands sharing their A fragments: (main0, corr0) += A B0 and
// (main1, corr1) += A B1 in split form -- one pair of fragment reads for six
// matrix instructions.
template <int MT>
__device__ inline void mma3_tiles2(const half8 *whi, const half8 *wlo, int stride, const half8 &bh0,
                                   const half8 &bl0, floatx4 *main0, floatx4 *corr0, const half8 &bh1,
                                   const half8 &bl1, floatx4 *main1, floatx4 *corr1) {
    half8 lo[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const half8 hi = whi[m * stride];
        main0[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, bh0, main0[m], 0, 0, 0);
        corr0[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, bl0, corr0[m], 0, 0, 0);
        main1[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, bh1, main1[m], 0, 0, 0);
        corr1[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(hi, bl1, corr1[m], 0, 0, 0);
        lo[m] = wlo[m * stride];
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        corr0[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo[m], bh0, corr0[m], 0, 0, 0);
        corr1[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(lo[m], bh1, corr1[m], 0, 0, 0);
    }
}

// k index of value j of the B operand of a chained 32-wide step t (two
// accumulator tiles 2t and 2t+1), for the lane in k-slot s
__device__ inline int chain_k(int t, int s, int j) { return 32 * t + 16 * (j >> 2) + 4 * s + (j & 3); }


// Tiles of 16 pairs handled by this wavefront.  The grid is a multiple of
// the XCD count; the blocks of one XCD share one contiguous range of tiles
// (pairs are in CSR order, so the gathered atom rows of a range stay in
// that XCD's L2), and the wavefronts of those blocks stride through it.
__device__ inline void tile_range(int64_t P, int64_t &tile, int64_t &end, int64_t &stride, int tile_pairs = 16) {
    const int64_t ntiles = (P + tile_pairs - 1) / tile_pairs;
    const int xcd = blockIdx.x % kXcds, nxb = gridDim.x / kXcds;
    const int64_t per = (ntiles + kXcds - 1) / kXcds;
    const int waves = blockDim.x / 64;
    tile = per * xcd + (int64_t)(blockIdx.x / kXcds) * waves + threadIdx.x / 64;
    end = min(ntiles, per * (xcd + 1));
    stride = (int64_t)nxb * waves;
}

__device__ inline float rbf_val(const FilterArgs &a, float d, int k) {
    if (k >= a.K) return 0.0f;
    const float t = d - (a.lo + (float)k * a.dmu);
    return fast_exp(-a.gamma * t * t);
}

// Stage A1 for the first GEMM: s_a1[(m*KS + ks)*64 + l] holds, for output
// feature f = 16m + l%16, the weights A1[k][f], k = 32 ks + 8(l/16) + j.
template <int F, int NT>
__device__ inline void stage_a1(const FilterArgs &a, half8 *s_hi, half8 *s_lo, int KS) {
    constexpr int MT = F / 16;
    stage_frags<MT * 2 * 64, NT>(s_hi, s_lo, MT * KS * 64, [&](int idx, int j) {
        const int m = idx / (KS * 64), ks = (idx / 64) % KS, l = idx % 64;
        return w1<F>(a, 32 * ks + 8 * (l / 16) + j, 16 * m + l % 16);
    });
}

// 2^e such that |x| * 2^-e <= 1 for the largest |x| of the lane's pair
// (the pair's values are spread over the four k-slot lanes l%16 + 16 s).
__device__ inline int pair_exponent(float amax) {
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    return amax > 0.0f ? ilogbf(amax) + 1 : 0;
}

template <int F>
__global__ __launch_bounds__(kFwdThreads) void filter_fwd_kernel(FilterArgs a) {
    constexpr int MT = F / 16;
    constexpr int T2 = MT / 2;                 // 32-wide k steps of the F x F GEMM
    constexpr int NT = kFwdNT;                 // 16-pair tiles per wavefront
    constexpr int MG = MT < kFwdMG ? MT : kFwdMG;   // output tiles per group
    __shared__ half8 s_a1h[MT * 2 * 64], s_a1l[MT * 2 * 64];
    __shared__ half8 s_a2h[MT * T2 * 64], s_a2l[MT * T2 * 64];   // [m][t][l]: A2[chain_k(t, l/16, j)][16 m + l%16]
    __shared__ float s_b1[F], s_b2[F];
    const int KS = (a.K + 31) / 32;
    stage_a1<F, kFwdThreads>(a, s_a1h, s_a1l, KS);
    stage_frags<MT * T2 * 64, kFwdThreads>(s_a2h, s_a2l, MT * T2 * 64, [&](int idx, int j) {
        const int m = idx / (T2 * 64), t = (idx / 64) % T2, l = idx % 64;
        return w2<F>(a, chain_k(t, l / 16, j), 16 * m + l % 16);
    });
    for (int f = threadIdx.x; f < F; f += blockDim.x) { s_b1[f] = a.b1[f]; s_b2[f] = a.b2[f]; }
    __syncthreads();

    int64_t tile, tile_end, stride;
    tile_range(a.P, tile, tile_end, stride, 16 * NT);
    for (; tile < tile_end; tile += stride) {
        // keep the weight-fragment LDS reads inside the loop: hoisted out of
        // it they would need hundreds of registers
        asm volatile("" ::: "memory");
        int lane = threadIdx.x % 64;
        asm volatile("" : "+v"(lane));
        const int slot = lane / 16;
        int64_t p[NT];
        half8 rh[2][NT], rl[2][NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            p[n] = tile * (16 * NT) + 16 * n + lane % 16;
            const float d = (p[n] < a.P) ? a.dsrc[p[n] * a.dstride + a.doff] : 0.0f;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                float v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = ks < KS ? rbf_val(a, d, 32 * ks + 8 * slot + j) : 0.0f;
                split8(v, rh[ks][n], rl[ks][n]);
            }
        }
        // z = ssp(rbf A1 + b1) on features 16 m + 4 slot + r, in groups of MG tiles
        float z[NT][MT][4];
#pragma unroll
        for (int m0 = 0; m0 < MT; m0 += MG) {
            floatx4 am[MG][NT], ac[MG][NT];
#pragma unroll
            for (int g = 0; g < MG; ++g)
#pragma unroll
                for (int n = 0; n < NT; ++n) am[g][n] = ac[g][n] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                if (ks < KS)
                    mma3_tiles_nt<MG, NT>(s_a1h + (m0 * KS + ks) * 64 + lane, s_a1l + (m0 * KS + ks) * 64 + lane,
                                          KS * 64, rh[ks], rl[ks], am, ac);
#pragma unroll
            for (int g = 0; g < MG; ++g) {
                const float4 b = *reinterpret_cast<const float4 *>(s_b1 + 16 * (m0 + g) + 4 * slot);
                const float bb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                for (int n = 0; n < NT; ++n)
#pragma unroll
                    for (int r = 0; r < 4; ++r) z[n][m0 + g][r] = ssp(am[g][n][r] + ac[g][n][r] * kLoUnscale + bb[r]);
            }
        }
        // chained B operands of the second GEMM
        half8 zh[T2][NT], zl[T2][NT];
#pragma unroll
        for (int t = 0; t < T2; ++t)
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                float v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = z[n][2 * t + (j >> 2)][j & 3];
                split8(v, zh[t][n], zl[t][n]);
            }
#pragma unroll
        for (int m0 = 0; m0 < MT; m0 += MG) {
            floatx4 main[MG][NT], corr[MG][NT];
#pragma unroll
            for (int g = 0; g < MG; ++g)
#pragma unroll
                for (int n = 0; n < NT; ++n) main[g][n] = corr[g][n] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < T2; ++t)
                mma3_tiles_nt<MG, NT>(s_a2h + (m0 * T2 + t) * 64 + lane, s_a2l + (m0 * T2 + t) * 64 + lane,
                                      T2 * 64, zh[t], zl[t], main, corr);
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                if (p[n] < a.P) {
#pragma unroll
                    for (int g = 0; g < MG; ++g) {
                        const int f0 = 16 * (m0 + g) + 4 * slot;
                        const float4 b = *reinterpret_cast<const float4 *>(s_b2 + f0);
                        const float4 v = make_float4(main[g][n][0] + corr[g][n][0] * kLoUnscale + b.x,
                                                     main[g][n][1] + corr[g][n][1] * kLoUnscale + b.y,
                                                     main[g][n][2] + corr[g][n][2] * kLoUnscale + b.z,
                                                     main[g][n][3] + corr[g][n][3] * kLoUnscale + b.w);
                        *reinterpret_cast<float4 *>(a.phi + p[n] * F + f0) = v;
                    }
                }
            }
        }
    }
}

template <int F>
__global__ __launch_bounds__(kBwdThreads) void filter_bwd_kernel(FilterArgs a) {
    constexpr int MT = F / 16;
    constexpr int T2 = MT / 2;
    constexpr int MG = MT < kBwdMG ? MT : kBwdMG;
    __shared__ half8 s_a1h[MT * 2 * 64], s_a1l[MT * 2 * 64];      // [m][ks][l] as in the forward pass
    __shared__ half8 s_a2bh[MT * T2 * 64], s_a2bl[MT * T2 * 64];  // [m][t][l]: A2[16 m + l%16][32 t + 8(l/16) + j]
    __shared__ float s_b1[F];
    const int KS = (a.K + 31) / 32;
    stage_a1<F, kBwdThreads>(a, s_a1h, s_a1l, KS);
    stage_frags<MT * T2 * 64, kBwdThreads>(s_a2bh, s_a2bl, MT * T2 * 64, [&](int idx, int j) {
        const int m = idx / (T2 * 64), t = (idx / 64) % T2, l = idx % 64;
        return w2<F>(a, 16 * m + l % 16, 32 * t + 8 * (l / 16) + j);
    });
    for (int f = threadIdx.x; f < F; f += blockDim.x) s_b1[f] = a.b1[f];
    __syncthreads();

    int64_t tile, tile_end, stride;
    tile_range(a.P, tile, tile_end, stride);
    for (; tile < tile_end; tile += stride) {
        asm volatile("" ::: "memory");
        // lane-derived values are recomputed per tile (opaque to the
        // compiler) instead of being hoisted and kept live across the loop
        int lane = threadIdx.x % 64;
        asm volatile("" : "+v"(lane));
        const int slot = lane / 16;
        const int64_t p = tile * 16 + lane % 16;
        const bool live = p < a.P;
        const float d = live ? a.dsrc[p * a.dstride + a.doff] : 0.0f;
        const int2 ij = live ? a.pair_ij[p] : make_int2(0, 0);
        float fc = 0.0f, dfc = 0.0f;
        if (live && d < a.cutoff) {
            float th = 0.5f * kPi * d / a.cutoff;
            float c = cosf(th), sn = sinf(th);
            fc = c * c;
            dfc = -(kPi / a.cutoff) * sn * c;
        }
        // G = g_y_i x_j + g_y_j x_i on the features 32 t + 8 slot + j, times
        // fc 2^-e1 (g_phi scaled; e1 from a bound on |g_phi| through the
        // per-atom row maxima), split into the B operands of all k-steps.
        int e1 = 0;
        {
            const float2 mi = live ? make_float2(a.xmax[ij.x], a.gmax[ij.x]) : make_float2(0.f, 0.f);
            const float2 mj = live ? make_float2(a.xmax[ij.y], a.gmax[ij.y]) : make_float2(0.f, 0.f);
            const float bound = fc * (mi.y * mj.x + mj.y * mi.x);
            e1 = bound > 0.0f ? ilogbf(bound) + 1 : 0;
        }
        const float fs = ldexpf(fc, -e1);
        float gfc = 0.0f;
        half8 gh[T2], gl[T2];
        {
            const int64_t bi = (int64_t)ij.x * F + 8 * slot, bj = (int64_t)ij.y * F + 8 * slot;
            const int64_t bp = (live ? p : 0) * F + 8 * slot;
#pragma unroll
            for (int t = 0; t < T2; ++t) {
                asm volatile("" ::: "memory");   // at most one step's gathers in flight
                float v[8];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int o = 32 * t + 4 * q;
                    const float4 gyi = *reinterpret_cast<const float4 *>(a.gy + bi + o);
                    const float4 gyj = *reinterpret_cast<const float4 *>(a.gy + bj + o);
                    const float4 xi = *reinterpret_cast<const float4 *>(a.x + bi + o);
                    const float4 xj = *reinterpret_cast<const float4 *>(a.x + bj + o);
                    const float4 ph = *reinterpret_cast<const float4 *>(a.phi_in + bp + o);
                    const float g0 = gyi.x * xj.x + gyj.x * xi.x, g1 = gyi.y * xj.y + gyj.y * xi.y;
                    const float g2 = gyi.z * xj.z + gyj.z * xi.z, g3 = gyi.w * xj.w + gyj.w * xi.w;
                    gfc += g0 * ph.x + g1 * ph.y + g2 * ph.z + g3 * ph.w;
                    v[4 * q + 0] = fs * g0; v[4 * q + 1] = fs * g1;
                    v[4 * q + 2] = fs * g2; v[4 * q + 3] = fs * g3;
                }
                split8(v, gh[t], gl[t]);
                // the step is consumed before the next step's gathers issue
                asm volatile("" : "+v"(gh[t]), "+v"(gl[t]), "+v"(gfc));
            }
        }
        // the lane's basis values rbf_k(d) and derivatives rbf_k'(d) =
        // -2 gamma (d - mu_k) rbf_k, k = 32 ks + 8 slot + j, split into the B
        // operands of the recomputed first layer and of its distance tangent
        // (the derivatives scaled by 2^-ep, ep from the pair's largest |rbf'|)
        half8 rh[2], rl[2], qh[2], ql[2];
        int ep;
        {
            // d goes through an opaque copy so that this is not hoisted into
            // the gather phase (register pressure)
            float dr = d;
            asm volatile("" : "+v"(dr)::"memory");
            float rb[2][8], rd[2][8];
            float dmax = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int k = 32 * ks + 8 * slot + j;
                    const float tt = dr - (a.lo + (float)k * a.dmu);
                    const float e = k < a.K ? fast_exp(-a.gamma * tt * tt) : 0.0f;
                    rb[ks][j] = e;
                    rd[ks][j] = -2.0f * a.gamma * tt * e;
                    dmax = fmaxf(dmax, fabsf(rd[ks][j]));
                }
            ep = pair_exponent(dmax);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
                for (int j = 0; j < 8; ++j) rd[ks][j] = ldexpf(rd[ks][j], -ep);
                split8(rb[ks], rh[ks], rl[ks]);
                split8(rd[ks], qh[ks], ql[ks]);
            }
        }
        // per group of MG output tiles (features 16 m ..): g_z = A2 g_phi
        // (2^-e1), the recomputed a = rbf A1 + b1 and its tangent
        // a' = rbf' A1 (2^-ep), then sum_g g_z sigmoid(a) a' -- which is
        // sum_k g_rbf_k rbf_k', the RBF part of dE/dd, without forming g_rbf
        float sk = 0.0f;
#pragma unroll
        for (int m0 = 0; m0 < MT; m0 += MG) {
            floatx4 zm[MG], zc[MG];
#pragma unroll
            for (int m = 0; m < MG; ++m) zm[m] = zc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < T2; ++t)
                mma3_tiles<MG>(s_a2bh + (m0 * T2 + t) * 64 + lane, s_a2bl + (m0 * T2 + t) * 64 + lane, T2 * 64,
                               gh[t], gl[t], zm, zc);
            floatx4 gz[MG];
#pragma unroll
            for (int m = 0; m < MG; ++m) {
#pragma unroll
                for (int r = 0; r < 4; ++r) gz[m][r] = fmaf(zc[m][r], kLoUnscale, zm[m][r]);
                // g_z is complete before the recompute's operands are read
                asm volatile("" : "+v"(gz[m])::"memory");
            }
            floatx4 am[MG], ac[MG], tm[MG], tc[MG];
#pragma unroll
            for (int m = 0; m < MG; ++m) {
                am[m] = *reinterpret_cast<const floatx4 *>(s_b1 + 16 * (m0 + m) + 4 * slot);
                ac[m] = tm[m] = tc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                if (ks < KS)
                    mma3_tiles2<MG>(s_a1h + (m0 * KS + ks) * 64 + lane, s_a1l + (m0 * KS + ks) * 64 + lane, KS * 64,
                                    rh[ks], rl[ks], am, ac, qh[ks], ql[ks], tm, tc);
#pragma unroll
            for (int m = 0; m < MG; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float sg = sigm(fmaf(ac[m][r], kLoUnscale, am[m][r]));
                    sk = fmaf(gz[m][r] * sg, fmaf(tc[m][r], kLoUnscale, tm[m][r]), sk);
                }
            // the group is finished before the next group's fragments are read
            asm volatile("" : "+v"(sk)::"memory");
        }
        // S_p = sum_k g_rbf_k rbf_k' + g_fc fc'(d), summed over the four k-slot lanes
        float sp = fmaf(ldexpf(sk, e1 + ep), 1.0f, gfc * dfc);
        sp += __shfl_xor(sp, 16, 64);
        sp += __shfl_xor(sp, 32, 64);
        if (live && slot == 0) a.S[p] = a.accumulate ? a.S[p] + sp : sp;
    }
}

int num_cus() {
    static int n = 0;
    if (n == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            n = v;
        else
            n = 256;
    }
    return n;
}

FilterArgs make_args(const sn_model &m, int t) {
    const int F = m.n_features, K = m.n_rbf, I = m.n_interactions, T = m.n_types;
    int64_t off[9 * 16 + 6];
    sn_param_offsets(T, I, F, K, off, (int32_t)(sizeof(off) / sizeof(off[0])));
    const int64_t *blk = off + 1 + 9 * t;   // W_in, A1, b1, A2, b2, Wo1, bo1, Wo2, bo2
    FilterArgs a = {};
    a.K = K;
    a.lo = m.rbf_lo;
    a.dmu = (m.rbf_hi - m.rbf_lo) / (float)(K - 1);
    a.gamma = m.rbf_gamma;
    a.cutoff = m.cutoff;
    a.A1 = m.params + blk[1];
    a.b1 = m.params + blk[2];
    a.A2 = m.params + blk[3];
    a.b2 = m.params + blk[4];
    if (m.filter_format == 1) {
        const int64_t qper = (int64_t)K * F + (int64_t)F * F;
        a.qA1 = m.qweights + qper * t;
        a.qA2 = a.qA1 + (int64_t)K * F;
        a.sA1 = m.qscales + (int64_t)2 * F * t;
        a.sA2 = a.sA1 + F;
    }
    return a;
}

template <int F>
sn_status launch_fwd(const FilterArgs &a, hipStream_t s) {
    const int64_t tiles = (a.P + 16 * kFwdNT - 1) / (16 * kFwdNT);
    const int waves = kFwdThreads / 64;
    const int grid = xcd_grid((int)std::min<int64_t>(num_cus(), (tiles + waves - 1) / waves));
    filter_fwd_kernel<F><<<grid, kFwdThreads, 0, s>>>(a);
    return launch_status();
}

template <int F>
sn_status launch_bwd(const FilterArgs &a, hipStream_t s) {
    const int64_t tiles = (a.P + 15) / 16;
    const int waves = kBwdThreads / 64;
    const int grid = xcd_grid((int)std::min<int64_t>(num_cus(), (tiles + waves - 1) / waves));
    filter_bwd_kernel<F><<<grid, kBwdThreads, 0, s>>>(a);
    return launch_status();
}

sn_status fwd_dispatch(const FilterArgs &a, int F, hipStream_t s) {
    if (a.P <= 0) return SN_OK;
    ProfScope ps(K_FILTER_FWD, s);
    switch (F) {
        case 32: return launch_fwd<32>(a, s);
        case 64: return launch_fwd<64>(a, s);
        case 128: return launch_fwd<128>(a, s);
        default: return SN_ERR_INVALID;
    }
}

}  // namespace

sn_status filter_forward(const sn_model &m, int t, const float4 *pgeo, int64_t P, float *phi, hipStream_t s) {
    FilterArgs a = make_args(m, t);
    a.dsrc = reinterpret_cast<const float *>(pgeo);
    a.dstride = 4;
    a.doff = 3;
    a.P = P;
    a.phi = phi;
    return fwd_dispatch(a, m.n_features, s);
}

sn_status filter_forward_plain(const sn_model &m, int t, const float *d, int64_t P, float *phi, hipStream_t s) {
    FilterArgs a = make_args(m, t);
    a.dsrc = d;
    a.dstride = 1;
    a.doff = 0;
    a.P = P;
    a.phi = phi;
    return fwd_dispatch(a, m.n_features, s);
}

sn_status filter_backward(const sn_model &m, int t, const float4 *pgeo, const int2 *pair_ij, int64_t P, int N,
                          const float *phi, const float *x, const float *gy, const float *xmax, const float *gmax,
                          float *S, int accumulate, hipStream_t s) {
    if (P <= 0) return SN_OK;
    (void)N;
    FilterArgs a = make_args(m, t);
    a.dsrc = reinterpret_cast<const float *>(pgeo);
    a.dstride = 4;
    a.doff = 3;
    a.P = P;
    a.pair_ij = pair_ij;
    a.x = x;
    a.gy = gy;
    a.phi_in = phi;
    a.S = S;
    a.xmax = xmax;
    a.gmax = gmax;
    a.accumulate = accumulate;
    ProfScope ps(K_FILTER_BWD, s);
    switch (m.n_features) {
        case 32: return launch_bwd<32>(a, s);
        case 64: return launch_bwd<64>(a, s);
        case 128: return launch_bwd<128>(a, s);
        default: return SN_ERR_INVALID;
    }
}

}  // namespace sn
