// Filter network on the matrix cores ("How", flash radial basis and the
// filter network with channel-wise 16-bit weights -- FlashSchNet summary
// page; OpenAlex abstract techniques (1) and (4)).
//
// Per pair p with distance d_p (one row shared by both directed edges):
//   a   = rbf(d) A1 + b1            rbf_k = exp(-gamma (d - mu_k)^2), K <= 64
//   phi = ssp(a) A2 + b2            (stored times the envelope: W = fc(d) phi, the CFConv's weight)
// and, in the backward pass, with G_p = g_y_i (.) x_j + g_y_j (.) x_i (the
// gradient of E with respect to the shared filter row):
//   g_fc = <G, phi>,  g_phi = fc G,  g_a = (g_phi A2^T) (.) sigmoid(a),
//   g_rbf = g_a A1^T,  S_p += sum_k g_rbf_k rbf_k'(d) + g_fc fc'(d).
// The backward does not read the stored rows back: with z = softplus(a),
// phi = z A2 + b2', b2' = b2 - ln 2 (column sums of A2), so
// g_fc = <A2 G, z> + <G, b2'> comes from the recomputed first layer and the
// product g_z = A2 G that the pass forms anyway.
//
// Precision.  The products use the split form of split_mfma.h: an operand
// scaled by a power of two to below 2^14 is held as fp16 hi and lo halves,
// and a.b accumulates hi.hi + hi.lo + lo.hi in one fp32 accumulator, close
// to fp32 accuracy at 3/16 of the cost of fp32 matrix instructions.  The
// weights take one scale per matrix (from their largest magnitude, found
// while staging).  The per-pair operands take scales from bounds that hold
// for every pair, so no per-pair maximum is searched: the radial basis lies
// in [0, 1] with its largest value near 1; its distance derivative is
// bounded through the basis width; the first layer's activation through the
// column sums of |A1| and |b1|; the gathered filter gradient through the
// per-atom row maxima of x and g_y.  Biases seed the accumulators (scaled
// like them), and the scales are taken out by one multiply per output.
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
// Work distribution: persistent blocks (one per CU, weights copied once into
// LDS from the weight pack, where int16 codes were dequantised); each
// wavefront loops over 16-pair tiles of an XCD-contiguous range.
#include "split_mfma.h"

namespace sn {

namespace {

constexpr int kFwdThreads = 1024;   // 4 wavefronts per SIMD
// Systems with fewer 16-pair tiles than 16 per compute unit run the filter
// kernels in blocks of one wavefront per SIMD instead, so that their tiles
// spread over up to four times as many compute units (one block per CU
// either way: the staged weights take most of the LDS).
constexpr int kSmallThreads = 256;
constexpr int kFwdMG = 4;           // forward output tiles per product group
constexpr int kBwdThreads = 1024;   // 4 wavefronts per SIMD
constexpr int kBwdMG = 1;           // backward output tiles per group (register budget of 4 wavefronts)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kE = 2.7182818284590452f;

struct FilterArgs {
    int K;
    float lo, dmu, gamma, cutoff;
    const float *A1, *A2;        // fp32 weights (format 0)
    const int16_t *qA1, *qA2;    // int16 codes (format 1)
    const float *sA1, *sA2;      // per-output-column scales (format 1)
    const float *b1, *b2;
    const float *dsrc;           // distance of pair p at dsrc[p * dstride + doff]
    int dstride, doff;
    int64_t P;                   // pair count, or the capacity when P_dev is set
    const int *P_dev;            // (may be null) the pair count on the device
    const int *guard;            // (may be null) no pairs while *guard is non-zero
    float *phi;                  // forward output [P][F] (fp32), or
    uint32_t *phi24;             // forward output [P][3F/4] (the 24-bit row format)
    // backward
    const int2 *pair_ij;
    const float *fc, *lfc;       // [P]: envelope fc(d_p) and fc'(d_p) / fc(d_p); the forward
                                 // multiplies the stored rows by fc
    const float *x, *gy;         // [N][F]
    const float *b2f;            // [F]: b2' = b2 - ln 2 (column sums of A2), from the weight pack
    float *S;                    // [P]
    const float *xmax, *gmax;    // [N]: max_f |x_i[f]|, max_f |g_y_i[f]|
    int accumulate;
    // weight pack: the first layer, the pass's second layer, and their
    // scales (first layer: {sa1, sz}; second layer: {sa2, -})
    const half8 *pa1h, *pa1l, *pa2h, *pa2l;
    const int *psc1, *psc2;
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

// k index of value j of the B operand of a chained 32-wide step t (two
// accumulator tiles 2t and 2t+1), for the lane in k-slot s
__device__ inline int chain_k(int t, int s, int j) { return 32 * t + 16 * (j >> 2) + 4 * s + (j & 3); }

// Tiles of 16 pairs handled by this wavefront.  The grid is a multiple of
// the XCD count; the blocks of one XCD share one contiguous range of tiles
// (pairs are in CSR order, so the gathered atom rows of a range stay in
// that XCD's L2), and the wavefronts of those blocks stride through it.
__device__ inline void tile_range(int64_t P, int64_t &tile, int64_t &end, int64_t &stride) {
    const int64_t ntiles = (P + 15) / 16;
    const int xcd = blockIdx.x % kXcds, nxb = gridDim.x / kXcds;
    const int64_t per = (ntiles + kXcds - 1) / kXcds;
    const int waves = blockDim.x / 64;
    tile = per * xcd + (int64_t)(blockIdx.x / kXcds) * waves + threadIdx.x / 64;
    end = min(ntiles, per * (xcd + 1));
    stride = (int64_t)nxb * waves;
}

// Gaussian basis rbf_k(d) = exp(-gamma (d - mu_k)^2), mu_k = lo + k dmu,
// written in u = kappa (d - mu_k) as rbf_k = 2^(c2 u^2), c2 = -gamma log2(e) /
// kappa^2.  kappa is a power of two chosen so that |u rbf_k| < 2^13 for every
// d (max_t |t| exp(-gamma t^2) = 1 / sqrt(2 e gamma)): u rbf_k is the
// derivative rbf_k'(d) times kappa / (-2 gamma), already scaled for the split
// products.  Along one lane's eight consecutive k the u values step by
// kappa dmu.
struct Basis {
    float lo, dmu, kappa, kd, c2;
};
__device__ inline Basis make_basis(const FilterArgs &a) {
    Basis b;
    const float bound = rsqrtf(2.0f * kE * a.gamma);
    b.kappa = (bound > 0.0f && bound < INFINITY) ? ldexpf(1.0f, (kSplitTop - 2) - ilogbf(bound)) : 1.0f;
    b.lo = a.lo;
    b.dmu = a.dmu;
    b.kd = b.kappa * a.dmu;
    b.c2 = -a.gamma * kLog2e / (b.kappa * b.kappa);
    return b;
}
// u of the first of the eight values at k = k0
__device__ inline float basis_u0(const Basis &b, float d, int k0) {
    return b.kappa * (d - fmaf((float)k0, b.dmu, b.lo));
}
// rb[j] = rbf_{k0+j}(d)
__device__ inline void basis8(const Basis &b, float u0, float (&rb)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float u = fmaf(-(float)j, b.kd, u0);
        rb[j] = __builtin_amdgcn_exp2f(b.c2 * u * u);
    }
}
// rb[j] = rbf_{k0+j}(d) and du[j] = u rbf_{k0+j}(d)
__device__ inline void basis8_d(const Basis &b, float u0, float (&rb)[8], float (&du)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float u = fmaf(-(float)j, b.kd, u0);
        const float e = __builtin_amdgcn_exp2f(b.c2 * u * u);
        rb[j] = e;
        du[j] = u * e;
    }
}

// Stage A1 for the first GEMM: s_a1[(m*kKS + ks)*64 + l] holds, for output
// feature f = 16m + l%16, the weights A1[k][f], k = 32 ks + 8(l/16) + j
// (zero for k >= K, so basis values beyond K never contribute; with K <= 32
// the kernels skip the second k-step).  The fixed stride of kKS steps makes
// every fragment offset a compile-time constant.  Returns the scale
// exponent; *s_max must hold 0 on entry.
constexpr int kKS = 2;   // 32-wide k-steps of the first layer (K <= 64)
template <int F, int NTHR>
__device__ inline int stage_a1(const FilterArgs &a, half8 *s_hi, half8 *s_lo, unsigned *s_max) {
    constexpr int MT = F / 16;
    return stage_split<MT * kKS * 64, NTHR>(s_hi, s_lo, MT * kKS * 64, s_max, [&](int idx, float (&v)[8]) {
        const int m = idx / (kKS * 64), ks = (idx / 64) % kKS, l = idx % 64;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = w1<F>(a, 32 * ks + 8 * (l / 16) + j, 16 * m + l % 16);
    });
}

// The largest |a_f| bound over the features, into *s_max (0 on entry; read
// after a barrier): |a_f| <= sum_k |A1[k][f]| + |b1[f]| since 0 <= rbf <= 1.
// z = ssp(a) / ln 2 then satisfies |z| <= bound log2(e) + 1.
template <int F>
__device__ inline void first_layer_bound(const FilterArgs &a, unsigned *s_max) {
    for (int f = threadIdx.x; f < F; f += blockDim.x) {
        float s = fabsf(a.b1[f]);
        for (int k = 0; k < a.K; ++k) s += fabsf(w1<F>(a, k, f));
        atomicMax(s_max, __float_as_uint(s));
    }
}
// Second-layer fragments ([m][t][l]).  Forward: value j = ln 2 A2[chain_k(t,
// l/16, j)][16 m + l%16] (the activation is computed in base 2 and the layer
// absorbs the ln 2).  Backward: A2[16 m + l%16][32 t + 8(l/16) + j].
template <int F>
__device__ inline void a2_fwd_frag(const FilterArgs &a, int idx, float (&v)[8]) {
    constexpr int T2 = F / 32;
    const int m = idx / (T2 * 64), t = (idx / 64) % T2, l = idx % 64;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = kLn2 * w2<F>(a, chain_k(t, l / 16, j), 16 * m + l % 16);
}
template <int F>
__device__ inline void a2_bwd_frag(const FilterArgs &a, int idx, float (&v)[8]) {
    constexpr int T2 = F / 32;
    const int m = idx / (T2 * 64), t = (idx / 64) % T2, l = idx % 64;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = w2<F>(a, 16 * m + l % 16, 32 * t + 8 * (l / 16) + j);
}

// acc0 += A B0 and acc1 += A B1 in split form for MG weight tiles: one pair
// of fragment reads per tile for six matrix instructions; dependent
// instructions on one accumulator are 2 MG apart.
template <int MG>
__device__ inline void mma_split2(const half8 *whi, const half8 *wlo, int stride, const half8 &bh0, const half8 &bl0,
                                  floatx4 *acc0, const half8 &bh1, const half8 &bl1, floatx4 *acc1) {
    half8 ah[MG], al[MG];
#pragma unroll
    for (int m = 0; m < MG; ++m) {
        ah[m] = whi[m * stride];
        al[m] = wlo[m * stride];
    }
#pragma unroll
    for (int m = 0; m < MG; ++m) {
        acc0[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[m], bh0, acc0[m], 0, 0, 0);
        acc1[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[m], bh1, acc1[m], 0, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < MG; ++m) {
        acc0[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[m], bl0, acc0[m], 0, 0, 0);
        acc1[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[m], bl1, acc1[m], 0, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < MG; ++m) {
        acc0[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[m], bh0, acc0[m], 0, 0, 0);
        acc1[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[m], bh1, acc1[m], 0, 0, 0);
    }
}

// The same with one fp16 product per pair of operands.
template <int MG>
__device__ inline void mma_one2(const half8 *whi, int stride, const half8 &bh0, floatx4 *acc0, const half8 &bh1,
                                floatx4 *acc1) {
    half8 ah[MG];
#pragma unroll
    for (int m = 0; m < MG; ++m) ah[m] = whi[m * stride];
#pragma unroll
    for (int m = 0; m < MG; ++m) {
        acc0[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[m], bh0, acc0[m], 0, 0, 0);
        acc1[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[m], bh1, acc1[m], 0, 0, 0);
    }
}

// ONE selects the arithmetic of the products: 0 = three fp16 products per
// fp32 product (split operands), 1 = one fp16 product of the rounded
// operands (the scales and everything else are the same).
template <int F, int NTHR, int ONE>
__device__ inline void filter_fwd_body(const FilterArgs &a) {
    const int64_t P = (a.guard && *a.guard) ? 0 : a.P_dev ? (int64_t)*a.P_dev : a.P;
    constexpr int MT = F / 16;
    constexpr int T2 = MT / 2;                      // 32-wide k steps of the F x F GEMM
    constexpr int MG = MT < kFwdMG ? MT : kFwdMG;   // output tiles per group
    __shared__ half8 s_a1h[MT * kKS * 64], s_a1l[MT * kKS * 64];
    __shared__ half8 s_a2h[MT * T2 * 64], s_a2l[MT * T2 * 64];   // [m][t][l]: ln2 A2[chain_k(t, l/16, j)][16 m + l%16]
    __shared__ float s_b1[F], s_b2[F];
    const int KS = (a.K + 31) / 32;
    // the weights come from the pack
    copy_frags<MT * kKS * 64, NTHR>(s_a1h, s_a1l, a.pa1h, a.pa1l, MT * kKS * 64);
    copy_frags<MT * T2 * 64, NTHR>(s_a2h, s_a2l, a.pa2h, a.pa2l, MT * T2 * 64);
    const int sa1 = a.psc1[0], sz = a.psc1[1], sa2 = a.psc2[0];
    for (int f = threadIdx.x; f < F; f += blockDim.x) {
        s_b1[f] = ldexpf(a.b1[f], sa1);
        s_b2[f] = ldexpf(a.b2[f], sz + sa2);
    }
    __syncthreads();
    const Basis bs = make_basis(a);
    const float cy = ldexpf(kLog2e, -sa1);        // first accumulator -> a log2(e)
    const float zs = ldexpf(1.0f, sz);
    const float os = ldexpf(1.0f, -(sz + sa2));   // second accumulator -> phi

    int64_t tile, tile_end, stride;
    tile_range(P, tile, tile_end, stride);
    // the distance of the wavefront's next tile is loaded one tile ahead, so
    // that its latency (and the wait for the earlier tile's stores, which the
    // same counter tracks) is not paid at the start of every tile
    // (with the envelope factor of the stored rows, when there is one)
    auto load_d = [&](int64_t t) {
        const int64_t q = t * 16 + (threadIdx.x % 16);
        return (t < tile_end && q < P) ? a.dsrc[q * a.dstride + a.doff] : 0.0f;
    };
    auto load_fc = [&](int64_t t) {
        const int64_t q = t * 16 + (threadIdx.x % 16);
        return (a.fc && t < tile_end && q < P) ? a.fc[q] : 1.0f;
    };
    float d_next = load_d(tile), fc_next = load_fc(tile);
    asm volatile("" : "+v"(d_next), "+v"(fc_next));
    for (; tile < tile_end; tile += stride) {
        // keep the weight-fragment LDS reads inside the loop: hoisted out of
        // it they would need hundreds of registers
        asm volatile("" ::: "memory");
        int lane = threadIdx.x % 64;
        asm volatile("" : "+v"(lane));
        const int slot = lane / 16;
        const int64_t p = tile * 16 + lane % 16;
        const float d = d_next, fcp = fc_next;
        d_next = load_d(tile + stride);
        fc_next = load_fc(tile + stride);
        half8 rh[2], rl[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            float v[8];
            basis8(bs, basis_u0(bs, d, 32 * ks + 8 * slot), v);
            if (ONE)
                rh[ks] = to_half8(v);
            else
                split8(v, rh[ks], rl[ks]);
        }
        // z 2^sz = (ssp(rbf A1 + b1) / ln 2) 2^sz on features 16 m + 4 slot + r,
        // in groups of MG tiles; ssp(a) / ln 2 = max(y, 0) + log2(1 + 2^-|y|) - 1
        // with y = a log2(e)
        float z[MT][4];
#pragma unroll
        for (int m0 = 0; m0 < MT; m0 += MG) {
            floatx4 acc[MG][1];
#pragma unroll
            for (int g = 0; g < MG; ++g) acc[g][0] = *reinterpret_cast<const floatx4 *>(s_b1 + 16 * (m0 + g) + 4 * slot);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                if (ks < KS) {
                    if (ONE)
                        mma_one<MG, 1>(s_a1h + (m0 * kKS + ks) * 64 + lane, kKS * 64, &rh[ks], acc);
                    else
                        mma_split<MG, 1>(s_a1h + (m0 * kKS + ks) * 64 + lane, s_a1l + (m0 * kKS + ks) * 64 + lane,
                                         kKS * 64, &rh[ks], &rl[ks], acc);
                }
#pragma unroll
            for (int g = 0; g < MG; ++g)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float y = acc[g][0][r] * cy;
                    const float s = fmaxf(y, 0.0f) + __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(-fabsf(y)));
                    z[m0 + g][r] = fmaf(s, zs, -zs);
                }
        }
        // chained B operands of the second GEMM
        half8 zh[T2], zl[T2];
#pragma unroll
        for (int t = 0; t < T2; ++t) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = z[2 * t + (j >> 2)][j & 3];
            if (ONE)
                zh[t] = to_half8(v);
            else
                split8(v, zh[t], zl[t]);
        }
#pragma unroll
        for (int m0 = 0; m0 < MT; m0 += MG) {
            floatx4 acc[MG][1];
#pragma unroll
            for (int g = 0; g < MG; ++g) acc[g][0] = *reinterpret_cast<const floatx4 *>(s_b2 + 16 * (m0 + g) + 4 * slot);
#pragma unroll
            for (int t = 0; t < T2; ++t) {
                if (ONE)
                    mma_one<MG, 1>(s_a2h + (m0 * T2 + t) * 64 + lane, T2 * 64, &zh[t], acc);
                else
                    mma_split<MG, 1>(s_a2h + (m0 * T2 + t) * 64 + lane, s_a2l + (m0 * T2 + t) * 64 + lane, T2 * 64,
                                     &zh[t], &zl[t], acc);
            }
            // the next distance has arrived long before; taking it here keeps
            // the loop's first wait from also waiting for these stores
            asm volatile("" : "+v"(d_next), "+v"(fc_next));
            if (p < P) {
                const float ws = os * fcp;
#pragma unroll
                for (int g = 0; g < MG; ++g) {
                    const floatx4 v = acc[g][0] * ws;
                    if (a.phi24) {
                        const Packed4 w = pack_fp24(v[0], v[1], v[2], v[3]);
                        *reinterpret_cast<uint3 *>(a.phi24 + p * fp24_words(F) + 3 * (4 * (m0 + g) + slot)) =
                            make_uint3(w.w0, w.w1, w.w2);
                    } else {
                        *reinterpret_cast<floatx4 *>(a.phi + p * F + 16 * (m0 + g) + 4 * slot) = v;
                    }
                }
            }
        }
    }
}

template <int F, int NTHR, int ONE>
__global__ __launch_bounds__(NTHR) void filter_fwd_kernel(FilterArgs a) {
    filter_fwd_body<F, NTHR, ONE>(a);
}

// Systems with few pairs: every interaction's forward filter in one launch
// (blockIdx.y = interaction), which saves I - 1 launch ramps per evaluation.
constexpr int kFusedMaxI = 8;
struct FilterArgsSet {
    FilterArgs a[kFusedMaxI];
};
template <int F, int NTHR, int ONE>
__global__ __launch_bounds__(NTHR) void filter_fwd_all_kernel(FilterArgsSet set) {
    filter_fwd_body<F, NTHR, ONE>(set.a[blockIdx.y]);
}

template <int F, int NTHR, int ONE>
__device__ inline void filter_bwd_body(const FilterArgs &a) {
    const int64_t P = (a.guard && *a.guard) ? 0 : a.P_dev ? (int64_t)*a.P_dev : a.P;
    constexpr int MT = F / 16;
    constexpr int T2 = MT / 2;
    constexpr int MG = MT < kBwdMG ? MT : kBwdMG;
    __shared__ half8 s_a1h[MT * kKS * 64], s_a1l[MT * kKS * 64];      // [m][ks][l] as in the forward pass
    __shared__ half8 s_a2bh[MT * T2 * 64], s_a2bl[MT * T2 * 64];  // [m][t][l]: A2[16 m + l%16][32 t + 8(l/16) + j]
    __shared__ float s_b1[F];
    __shared__ float4 s_b2f[F / 4];
    const int KS = (a.K + 31) / 32;
    // the weights come from the pack (which also holds the folded bias)
    copy_frags<MT * kKS * 64, NTHR>(s_a1h, s_a1l, a.pa1h, a.pa1l, MT * kKS * 64);
    copy_frags<MT * T2 * 64, NTHR>(s_a2bh, s_a2bl, a.pa2h, a.pa2l, MT * T2 * 64);
    const int sa1 = a.psc1[0], sa2 = a.psc2[0];
    for (int f = threadIdx.x; f < F; f += blockDim.x) {
        s_b1[f] = ldexpf(a.b1[f], sa1);
        reinterpret_cast<float *>(s_b2f)[f] = a.b2f[f];
    }
    __syncthreads();
    const Basis bs = make_basis(a);
    const float cs = ldexpf(-kLog2e, -sa1);              // recomputed accumulator -> -a log2(e)
    const float srb = -2.0f * a.gamma / bs.kappa;        // rbf_k'(d) = srb u rbf_k
    const int es = -(kSplitTop - 1) - sa2 - sa1;         // with e1: the scales of g_z and a'

    int64_t tile, tile_end, stride;
    tile_range(P, tile, tile_end, stride);
    for (; tile < tile_end; tile += stride) {
        asm volatile("" ::: "memory");
        // lane-derived values are recomputed per tile (opaque to the
        // compiler) instead of being hoisted and kept live across the loop
        int lane = threadIdx.x % 64;
        asm volatile("" : "+v"(lane));
        const int slot = lane / 16;
        const int64_t p = tile * 16 + lane % 16;
        const bool live = p < P;
        const float d = live ? a.dsrc[p * a.dstride + a.doff] : 0.0f;
        const int2 ij = live ? a.pair_ij[p] : make_int2(0, 0);
        const float fc = live ? a.fc[p] : 0.0f;
        const float lfc = live ? a.lfc[p] : 0.0f;
        // G = g_y_i x_j + g_y_j x_i on the features 32 t + 8 slot + j, times
        // 2^(13 - e1) with |G| < 2^e1 from the per-atom row maxima, split into
        // the B operands of all k-steps
        int e1 = 0;
        {
            const float2 mi = live ? make_float2(a.xmax[ij.x], a.gmax[ij.x]) : make_float2(0.f, 0.f);
            const float2 mj = live ? make_float2(a.xmax[ij.y], a.gmax[ij.y]) : make_float2(0.f, 0.f);
            const float bound = mi.y * mj.x + mj.y * mi.x;
            e1 = (bound > 0.0f && bound < INFINITY) ? ilogbf(bound) + 1 : 0;
        }
        const float fs = ldexpf(1.0f, (kSplitTop - 1) - e1);
        float gfc = 0.0f;   // <G, b2'> here; <A2 G, z> below
        half8 gh[T2], gl[T2];
        {
            const int64_t bi = (int64_t)ij.x * F + 8 * slot, bj = (int64_t)ij.y * F + 8 * slot;
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
                    const float4 bf = s_b2f[(o + 8 * slot) / 4];
                    const float g0 = gyi.x * xj.x + gyj.x * xi.x, g1 = gyi.y * xj.y + gyj.y * xi.y;
                    const float g2 = gyi.z * xj.z + gyj.z * xi.z, g3 = gyi.w * xj.w + gyj.w * xi.w;
                    gfc += g0 * bf.x + g1 * bf.y + g2 * bf.z + g3 * bf.w;
                    v[4 * q + 0] = fs * g0; v[4 * q + 1] = fs * g1;
                    v[4 * q + 2] = fs * g2; v[4 * q + 3] = fs * g3;
                }
                if (ONE)
                    gh[t] = to_half8(v);
                else
                    split8(v, gh[t], gl[t]);
                // the step is consumed before the next step's gathers issue
                asm volatile("" : "+v"(gh[t]), "+v"(gl[t]), "+v"(gfc));
            }
        }
        // the lane's basis values rbf_k(d) and u rbf_k (the derivative up to
        // srb), k = 32 ks + 8 slot + j, split into the B operands of the
        // recomputed first layer and of its distance tangent
        half8 rh[2], rl[2], qh[2], ql[2];
        {
            // d goes through an opaque copy so that this is not hoisted into
            // the gather phase (register pressure)
            float dr = d;
            asm volatile("" : "+v"(dr)::"memory");
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                float rb[8], du[8];
                basis8_d(bs, basis_u0(bs, dr, 32 * ks + 8 * slot), rb, du);
                if (ONE) {
                    rh[ks] = to_half8(rb);
                    qh[ks] = to_half8(du);
                } else {
                    split8(rb, rh[ks], rl[ks]);
                    split8(du, qh[ks], ql[ks]);
                }
            }
        }
        // per group of MG output tiles (features 16 m ..): g_z = A2 G, the
        // recomputed a = rbf A1 + b1 and its tangent a' = (u rbf) A1 (all
        // scaled), then sum_g g_z sigmoid(a) a' -- which is sum_k g_rbf_k
        // rbf_k' up to the envelope and the scales, the RBF part of dE/dd,
        // without forming g_rbf
        float sk = 0.0f, zg = 0.0f;
#pragma unroll
        for (int m0 = 0; m0 < MT; m0 += MG) {
            floatx4 gz[MG][1];
#pragma unroll
            for (int m = 0; m < MG; ++m) gz[m][0] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < T2; ++t) {
                if (ONE)
                    mma_one<MG, 1>(s_a2bh + (m0 * T2 + t) * 64 + lane, T2 * 64, &gh[t], gz);
                else
                    mma_split<MG, 1>(s_a2bh + (m0 * T2 + t) * 64 + lane, s_a2bl + (m0 * T2 + t) * 64 + lane,
                                     T2 * 64, &gh[t], &gl[t], gz);
            }
            // g_z is complete before the recompute's operands are read
#pragma unroll
            for (int m = 0; m < MG; ++m) asm volatile("" : "+v"(gz[m][0])::"memory");
            floatx4 am[MG], tm[MG];
#pragma unroll
            for (int m = 0; m < MG; ++m) {
                am[m] = *reinterpret_cast<const floatx4 *>(s_b1 + 16 * (m0 + m) + 4 * slot);
                tm[m] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                if (ks < KS) {
                    if (ONE)
                        mma_one2<MG>(s_a1h + (m0 * kKS + ks) * 64 + lane, kKS * 64, rh[ks], am, qh[ks], tm);
                    else
                        mma_split2<MG>(s_a1h + (m0 * kKS + ks) * 64 + lane, s_a1l + (m0 * kKS + ks) * 64 + lane,
                                       kKS * 64, rh[ks], rl[ks], am, qh[ks], ql[ks], tm);
                }
#pragma unroll
            for (int m = 0; m < MG; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    // with y = -a log2(e): sigmoid(a) = 1 / u and softplus(a) log2(e)
                    // = log2(u) - y, u = 1 + 2^y.  y is capped at 64: beyond it both
                    // are below 2^-64 (the cap leaves 2^-64 and 0)
                    const float y = fminf(am[m][r] * cs, 64.0f);
                    const float u = 1.0f + __builtin_amdgcn_exp2f(y);
                    const float sg = __builtin_amdgcn_rcpf(u);
                    sk = fmaf(gz[m][0][r] * sg, tm[m][r], sk);
                    zg = fmaf(__builtin_amdgcn_logf(u) - y, gz[m][0][r], zg);
                }
            // the group is finished before the next group's fragments are read
            asm volatile("" : "+v"(sk), "+v"(zg)::"memory");
        }
        // S_p = fc sum_k g_rbf_k rbf_k' + g_fc fc'(d), summed over the four k-slot lanes;
        // g_fc = <G, phi> = <G, b2'> + ln 2 <A2 G, softplus(a) log2(e)>, and fc' = fc lfc
        gfc = fmaf(kLn2, ldexpf(zg, e1 + es + sa1), gfc);
        float sp = fc * fmaf(srb, ldexpf(sk, e1 + es), gfc * lfc);
        sp += __shfl_xor(sp, 16, 64);
        sp += __shfl_xor(sp, 32, 64);
        if (live && slot == 0) a.S[p] = a.accumulate ? a.S[p] + sp : sp;
    }
}


template <int F, int NTHR, int ONE>
__global__ __launch_bounds__(NTHR) void filter_bwd_kernel(FilterArgs a) {
    filter_bwd_body<F, NTHR, ONE>(a);
}

// Systems with few pairs: every interaction's backward filter in one launch
// (blockIdx.y = interaction), each writing its own S slice.
template <int F, int NTHR, int ONE>
__global__ __launch_bounds__(NTHR) void filter_bwd_all_kernel(FilterArgsSet set) {
    filter_bwd_body<F, NTHR, ONE>(set.a[blockIdx.y]);
}


// The filter's slots of the weight pack: one block per (interaction,
// matrix), each staging one matrix exactly as the kernels above would, but
// into the pack.
struct FilterWeights {
    const float *A1, *A2, *b1, *b2;
    const int16_t *qA1, *qA2;
    const float *sA1, *sA2;
};
struct FilterPackArgs {
    FilterWeights w[16];
    char *pack;
    int I, K;
};

template <int F>
__global__ __launch_bounds__(kFwdThreads) void filter_pack_kernel(FilterPackArgs pa) {
    constexpr int MT = F / 16, T2 = MT / 2;
    __shared__ unsigned s_max[2];
    if (threadIdx.x < 2) s_max[threadIdx.x] = 0u;
    __syncthreads();
    const int t = blockIdx.x / 3, kind = blockIdx.x % 3;
    FilterArgs a = {};
    a.K = pa.K;
    a.A1 = pa.w[t].A1;
    a.A2 = pa.w[t].A2;
    a.b1 = pa.w[t].b1;
    a.qA1 = pa.w[t].qA1;
    a.qA2 = pa.w[t].qA2;
    a.sA1 = pa.w[t].sA1;
    a.sA2 = pa.w[t].sA2;
    const PackRef r = pack_ref(pa.pack, pa.I, pack_slot(t, kind));
    half8 *hi = const_cast<half8 *>(static_cast<const half8 *>(r.hi));
    half8 *lo = const_cast<half8 *>(static_cast<const half8 *>(r.lo));
    int sc0 = 0, sc1 = 0;
    if (kind == PK_FA1) {
        first_layer_bound<F>(a, &s_max[1]);
        sc0 = stage_a1<F, kFwdThreads>(a, hi, lo, &s_max[0]);   // its barrier completes s_max[1]
        sc1 = split_scale(__uint_as_float(s_max[1]) * kLog2e + 1.0f);
    } else if (kind == PK_FA2) {
        sc0 = stage_split<MT * T2 * 64, kFwdThreads>(hi, lo, MT * T2 * 64, &s_max[0],
                                                     [&](int idx, float (&v)[8]) { a2_fwd_frag<F>(a, idx, v); });
    } else {
        sc0 = stage_split<MT * T2 * 64, kFwdThreads>(hi, lo, MT * T2 * 64, &s_max[0],
                                                     [&](int idx, float (&v)[8]) { a2_bwd_frag<F>(a, idx, v); });
        // the backward's folded bias b2' = b2 - ln 2 sum_g A2[g][.]: each of
        // NP thread groups sums F / NP rows, then the parts are added in order
        constexpr int NP = kFwdThreads / F;
        __shared__ float s_part[kFwdThreads];
        const int f = threadIdx.x % F, part = threadIdx.x / F;
        float c = 0.0f;
        for (int g = part * (F / NP); g < (part + 1) * (F / NP); ++g) c += w2<F>(a, g, f);
        s_part[threadIdx.x] = c;
        __syncthreads();
        if (threadIdx.x < F) {
            float sum = 0.0f;
            for (int q = 0; q < NP; ++q) sum += s_part[q * F + f];
            const_cast<float *>(pack_vec(pa.pack, pa.I, t))[f] = fmaf(-kLn2, sum, pa.w[t].b2[f]);
        }
    }
    if (threadIdx.x == 0) {
        int *sc = const_cast<int *>(r.sc);
        sc[0] = sc0;
        sc[1] = sc1;
    }
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

template <int F, int ONE>
sn_status launch_fwd(const FilterArgs &a, hipStream_t s) {
    const int64_t tiles = (a.P + 15) / 16;
    if (tiles < (int64_t)num_cus() * (kFwdThreads / 64)) {
        const int waves = kSmallThreads / 64;
        const int grid = xcd_grid((int)std::min<int64_t>(num_cus(), (tiles + waves - 1) / waves));
        filter_fwd_kernel<F, kSmallThreads, ONE><<<grid, kSmallThreads, 0, s>>>(a);
        return launch_status();
    }
    const int waves = kFwdThreads / 64;
    const int grid = xcd_grid((int)std::min<int64_t>(num_cus(), (tiles + waves - 1) / waves));
    filter_fwd_kernel<F, kFwdThreads, ONE><<<grid, kFwdThreads, 0, s>>>(a);
    return launch_status();
}

template <int F, int ONE>
sn_status launch_bwd(const FilterArgs &a, hipStream_t s) {
    const int64_t tiles = (a.P + 15) / 16;
    if (tiles < (int64_t)num_cus() * (kBwdThreads / 64)) {
        const int waves = kSmallThreads / 64;
        const int grid = xcd_grid((int)std::min<int64_t>(num_cus(), (tiles + waves - 1) / waves));
        filter_bwd_kernel<F, kSmallThreads, ONE><<<grid, kSmallThreads, 0, s>>>(a);
        return launch_status();
    }
    const int waves = kBwdThreads / 64;
    const int grid = xcd_grid((int)std::min<int64_t>(num_cus(), (tiles + waves - 1) / waves));
    filter_bwd_kernel<F, kBwdThreads, ONE><<<grid, kBwdThreads, 0, s>>>(a);
    return launch_status();
}

// All interactions at once (systems with few pair tiles): one pass over the
// compute units, each interaction taking a multiple of the XCD count of
// blocks (one block per CU: the staged weights take most of the LDS).  When
// the tiles outnumber one wavefront per SIMD of those blocks, the blocks get
// two wavefronts per SIMD, so that no wavefront runs two tiles in sequence.
inline int fused_blocks_per_interaction(int I) { return std::max(kXcds, num_cus() / I / kXcds * kXcds); }

template <int F, int ONE>
sn_status launch_fwd_all(const FilterArgsSet &set, int I, int64_t P, hipStream_t s) {
    const int64_t tiles = (P + 15) / 16;
    const int per = fused_blocks_per_interaction(I);
    if (tiles > (int64_t)per * (kSmallThreads / 64)) {
        constexpr int T = 2 * kSmallThreads;
        const int gx = xcd_grid((int)std::min<int64_t>(per, (tiles + T / 64 - 1) / (T / 64)));
        filter_fwd_all_kernel<F, T, ONE><<<dim3(gx, I), T, 0, s>>>(set);
        return launch_status();
    }
    const int waves = kSmallThreads / 64;
    const int gx = xcd_grid((int)std::min<int64_t>(per, (tiles + waves - 1) / waves));
    filter_fwd_all_kernel<F, kSmallThreads, ONE><<<dim3(gx, I), kSmallThreads, 0, s>>>(set);
    return launch_status();
}

template <int F, int ONE>
sn_status launch_bwd_all(const FilterArgsSet &set, int I, int64_t P, hipStream_t s) {
    const int64_t tiles = (P + 15) / 16;
    const int per = fused_blocks_per_interaction(I);
    if (tiles > (int64_t)per * (kSmallThreads / 64)) {
        constexpr int T = 2 * kSmallThreads;
        const int gx = xcd_grid((int)std::min<int64_t>(per, (tiles + T / 64 - 1) / (T / 64)));
        filter_bwd_all_kernel<F, T, ONE><<<dim3(gx, I), T, 0, s>>>(set);
        return launch_status();
    }
    const int waves = kSmallThreads / 64;
    const int gx = xcd_grid((int)std::min<int64_t>(per, (tiles + waves - 1) / waves));
    filter_bwd_all_kernel<F, kSmallThreads, ONE><<<dim3(gx, I), kSmallThreads, 0, s>>>(set);
    return launch_status();
}

sn_status fwd_dispatch(const FilterArgs &a, int F, int one, hipStream_t s) {
    if (a.P <= 0) return SN_OK;
    ProfScope ps(K_FILTER_FWD, s);
    switch (F) {
        case 32: return one ? launch_fwd<32, 1>(a, s) : launch_fwd<32, 0>(a, s);
        case 64: return one ? launch_fwd<64, 1>(a, s) : launch_fwd<64, 0>(a, s);
        case 128: return one ? launch_fwd<128, 1>(a, s) : launch_fwd<128, 0>(a, s);
        default: return SN_ERR_INVALID;
    }
}

void attach_pack(FilterArgs &a, const sn_model &m, int t, const char *pack, int second) {
    if (!pack) return;
    const PackRef r1 = pack_ref(pack, m.n_interactions, pack_slot(t, PK_FA1));
    const PackRef r2 = pack_ref(pack, m.n_interactions, pack_slot(t, second));
    a.pa1h = static_cast<const half8 *>(r1.hi);
    a.pa1l = static_cast<const half8 *>(r1.lo);
    a.psc1 = r1.sc;
    a.pa2h = static_cast<const half8 *>(r2.hi);
    a.pa2l = static_cast<const half8 *>(r2.lo);
    a.psc2 = r2.sc;
}

}  // namespace

// Compute units of the current device (read once per process; the
// initialisation of a function-local static is thread-safe).
int num_cus() {
    static const int n = [] {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            return v;
        return 256;
    }();
    return n;
}


sn_status filter_pack(const sn_model &m, char *pack, hipStream_t s) {
    const int I = m.n_interactions;
    if (I < 1 || I > 16) return SN_ERR_INVALID;
    FilterPackArgs pa = {};
    pa.pack = pack;
    pa.I = I;
    pa.K = m.n_rbf;
    for (int t = 0; t < I; ++t) {
        const FilterArgs a = make_args(m, t);
        pa.w[t] = FilterWeights{a.A1, a.A2, a.b1, a.b2, a.qA1, a.qA2, a.sA1, a.sA2};
    }
    ProfScope ps(K_PACK, s);
    switch (m.n_features) {
        case 32: filter_pack_kernel<32><<<3 * I, kFwdThreads, 0, s>>>(pa); break;
        case 64: filter_pack_kernel<64><<<3 * I, kFwdThreads, 0, s>>>(pa); break;
        case 128: filter_pack_kernel<128><<<3 * I, kFwdThreads, 0, s>>>(pa); break;
        default: return SN_ERR_INVALID;
    }
    return launch_status();
}

sn_status filter_forward(const sn_model &m, int t, const float4 *pgeo, const float *pfc, int64_t P, uint32_t *phi24,
                         const char *pack, const int *p_dev, const int *guard, hipStream_t s) {
    if (!pack) return SN_ERR_INVALID;
    FilterArgs a = make_args(m, t);
    attach_pack(a, m, t, pack, PK_FA2);
    a.dsrc = reinterpret_cast<const float *>(pgeo);
    a.dstride = 4;
    a.doff = 3;
    a.P = P;
    a.P_dev = p_dev;
    a.guard = guard;
    a.phi24 = phi24;
    a.fc = pfc;
    return fwd_dispatch(a, m.n_features, m.filter_math, s);
}

bool filter_forward_fused(const sn_model &m, int64_t P) {
    return P > 0 && m.n_interactions <= kFusedMaxI && (P + 15) / 16 < (int64_t)num_cus() * (kFwdThreads / 64);
}

sn_status filter_forward_all(const sn_model &m, const float4 *pgeo, const float *pfc, int64_t P,
                             uint32_t *const *phi24, const char *pack, const int *p_dev, const int *guard,
                             hipStream_t s) {
    if (!pack || !filter_forward_fused(m, P)) return SN_ERR_INVALID;
    FilterArgsSet set = {};
    const int I = m.n_interactions;
    for (int t = 0; t < I; ++t) {
        FilterArgs &a = set.a[t];
        a = make_args(m, t);
        attach_pack(a, m, t, pack, PK_FA2);
        a.dsrc = reinterpret_cast<const float *>(pgeo);
        a.dstride = 4;
        a.doff = 3;
        a.P = P;
        a.P_dev = p_dev;
        a.guard = guard;
        a.phi24 = phi24[t];
        a.fc = pfc;
    }
    ProfScope ps(K_FILTER_FWD, s);
    switch (m.n_features) {
        case 32: return m.filter_math ? launch_fwd_all<32, 1>(set, I, P, s) : launch_fwd_all<32, 0>(set, I, P, s);
        case 64: return m.filter_math ? launch_fwd_all<64, 1>(set, I, P, s) : launch_fwd_all<64, 0>(set, I, P, s);
        case 128: return m.filter_math ? launch_fwd_all<128, 1>(set, I, P, s) : launch_fwd_all<128, 0>(set, I, P, s);
        default: return SN_ERR_INVALID;
    }
}

sn_status filter_forward_plain(const sn_model &m, int t, const float *d, int64_t P, float *phi, const char *pack,
                               hipStream_t s) {
    if (!pack) return SN_ERR_INVALID;
    FilterArgs a = make_args(m, t);
    attach_pack(a, m, t, pack, PK_FA2);
    a.dsrc = d;
    a.dstride = 1;
    a.doff = 0;
    a.P = P;
    a.phi = phi;
    return fwd_dispatch(a, m.n_features, m.filter_math, s);
}

sn_status filter_backward(const sn_model &m, int t, const float4 *pgeo, const float *pfc, const float *plfc,
                          const int2 *pair_ij, int64_t P, int N, const float *x, const float *gy, const float *xmax,
                          const float *gmax, float *S, int accumulate, const char *pack, const int *p_dev,
                          const int *guard, hipStream_t s) {
    if (P <= 0) return SN_OK;
    if (!pack) return SN_ERR_INVALID;
    (void)N;
    FilterArgs a = make_args(m, t);
    attach_pack(a, m, t, pack, PK_FA2B);
    a.b2f = pack_vec(pack, m.n_interactions, t);
    a.dsrc = reinterpret_cast<const float *>(pgeo);
    a.dstride = 4;
    a.doff = 3;
    a.P = P;
    a.pair_ij = pair_ij;
    a.P_dev = p_dev;
    a.guard = guard;
    a.fc = pfc;
    a.lfc = plfc;
    a.x = x;
    a.gy = gy;
    a.S = S;
    a.xmax = xmax;
    a.gmax = gmax;
    a.accumulate = accumulate;
    ProfScope ps(K_FILTER_BWD, s);
    switch (m.n_features) {
        case 32: return m.filter_math ? launch_bwd<32, 1>(a, s) : launch_bwd<32, 0>(a, s);
        case 64: return m.filter_math ? launch_bwd<64, 1>(a, s) : launch_bwd<64, 0>(a, s);
        case 128: return m.filter_math ? launch_bwd<128, 1>(a, s) : launch_bwd<128, 0>(a, s);
        default: return SN_ERR_INVALID;
    }
}


sn_status filter_backward_all(const sn_model &m, const float4 *pgeo, const float *pfc, const float *plfc,
                              const int2 *pair_ij, int64_t P, const float *const *x, const float *const *gy,
                              const float *const *xmax, const float *const *gmax, float *S, const char *pack,
                              const int *p_dev, const int *guard, hipStream_t s) {
    if (P <= 0) return SN_OK;
    if (!pack || !filter_forward_fused(m, P)) return SN_ERR_INVALID;
    FilterArgsSet set = {};
    const int I = m.n_interactions;
    for (int t = 0; t < I; ++t) {
        FilterArgs &a = set.a[t];
        a = make_args(m, t);
        attach_pack(a, m, t, pack, PK_FA2B);
        a.b2f = pack_vec(pack, m.n_interactions, t);
        a.dsrc = reinterpret_cast<const float *>(pgeo);
        a.dstride = 4;
        a.doff = 3;
        a.P = P;
        a.pair_ij = pair_ij;
        a.P_dev = p_dev;
        a.guard = guard;
        a.fc = pfc;
        a.lfc = plfc;
        a.x = x[t];
        a.gy = gy[t];
        a.S = S + P * t;
        a.xmax = xmax[t];
        a.gmax = gmax[t];
        a.accumulate = 0;
    }
    ProfScope ps(K_FILTER_BWD, s);
    switch (m.n_features) {
        case 32: return m.filter_math ? launch_bwd_all<32, 1>(set, I, P, s) : launch_bwd_all<32, 0>(set, I, P, s);
        case 64: return m.filter_math ? launch_bwd_all<64, 1>(set, I, P, s) : launch_bwd_all<64, 0>(set, I, P, s);
        case 128: return m.filter_math ? launch_bwd_all<128, 1>(set, I, P, s) : launch_bwd_all<128, 0>(set, I, P, s);
        default: return SN_ERR_INVALID;
    }
}

}  // namespace sn
