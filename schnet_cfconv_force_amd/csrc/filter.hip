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
// Matrix-core mapping.  Everything is computed transposed: features are the
// M dimension and 16 pairs are the N dimension of v_mfma_f32_16x16x4f32.
// Lane l then always owns pair l%16, and the accumulator layout of one GEMM
// (lane l: rows 4(l/16)+r of a 16-row tile, r = 0..3) is directly a valid
// B operand of the next GEMM (lane l: k-slot l/16) once the k index of step
// (tile m, register r) is taken to be 16m + 4(l/16) + r.  So the three
// chained GEMMs never leave registers; only the weights are read from LDS,
// pre-arranged so that each lane's operands for four consecutive steps are
// one conflict-free 16-byte read.  The radial basis values are generated in
// registers from d (no E x K tensor exists anywhere).
//
// Work distribution: persistent blocks (one per CU, weights staged once into
// LDS, int16 codes dequantised while staging); each wavefront loops over
// 16-pair tiles.
#include "sn_internal.h"

namespace sn {

namespace {

constexpr int kFwdThreads = 1024;   // 4 wavefronts per SIMD (<= 128 VGPRs)
constexpr int kBwdThreads = 512;    // 2 wavefronts per SIMD (<= 256 VGPRs)
constexpr float kPi = 3.14159265358979323846f;

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
    int accumulate;
};

template <int F>
__device__ inline float w1(const FilterArgs &a, int k, int f) {   // A1[k][f]
    if (k >= a.K) return 0.0f;
    if (a.qA1) return (float)a.qA1[k * F + f] * a.sA1[f];
    return a.A1[k * F + f];
}
template <int F>
__device__ inline float w2(const FilterArgs &a, int g, int f) {   // A2[g][f]
    if (a.qA2) return (float)a.qA2[g * F + f] * a.sA2[f];
    return a.A2[g * F + f];
}

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

__device__ inline float rbf(const FilterArgs &a, float d, int k) {
    if (k >= a.K) return 0.0f;
    const float t = d - (a.lo + (float)k * a.dmu);
    return fast_exp(-a.gamma * t * t);
}

// GEMM 1 shared by both passes: acc[m] = (rbf(d) A1)^T for the lane's pair.
// s_f1 layout: [m][kq][lane] float4, component r = step 4kq + r, holding
// A1[4 step + lane/16][16 m + lane%16].  KS = ceil(K/4) steps are issued;
// the zero padding of the last group of four is skipped.
template <int F>
__device__ inline void gemm_rbf(const FilterArgs &a, const float4 *s_f1, int KQ, int KS, float d, int lane,
                                floatx4 (&acc)[F / 16]) {
    constexpr int MT = F / 16;
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int kq = 0; kq < KQ; ++kq) {
        const int nstep = min(4, KS - 4 * kq);
        float bv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) bv[r] = rbf(a, d, 4 * (4 * kq + r) + lane / 16);
        if (nstep == 4) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float4 w = s_f1[(m * KQ + kq) * 64 + lane];
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(w.x, bv[0], acc[m], 0, 0, 0);
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(w.y, bv[1], acc[m], 0, 0, 0);
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(w.z, bv[2], acc[m], 0, 0, 0);
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(w.w, bv[3], acc[m], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float4 w = s_f1[(m * KQ + kq) * 64 + lane];
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(w.x, bv[0], acc[m], 0, 0, 0);
                if (nstep > 1) acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(w.y, bv[1], acc[m], 0, 0, 0);
                if (nstep > 2) acc[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(w.z, bv[2], acc[m], 0, 0, 0);
            }
        }
    }
}

template <int F>
__device__ inline void stage_f1(const FilterArgs &a, float4 *s_f1, int KQ) {
    constexpr int MT = F / 16;
    for (int idx = threadIdx.x; idx < MT * KQ * 64; idx += blockDim.x) {
        const int m = idx / (KQ * 64), kq = (idx / 64) % KQ, l = idx % 64;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = w1<F>(a, 4 * (4 * kq + r) + l / 16, 16 * m + l % 16);
        s_f1[idx] = make_float4(v[0], v[1], v[2], v[3]);
    }
}

template <int F>
__global__ __launch_bounds__(kFwdThreads) void filter_fwd_kernel(FilterArgs a) {
    constexpr int MT = F / 16;
    __shared__ float4 s_f1[MT * 4 * 64];          // K <= 64: at most 4 groups of 4 steps
    __shared__ float4 s_f2[MT * MT * 64];         // [m][m2][lane]: A2[16 m2 + 4(l/16) + r][16 m + l%16]
    __shared__ float s_b1[F], s_b2[F];
    const int KS = (a.K + 3) / 4;
    const int KQ = (KS + 3) / 4;
    stage_f1<F>(a, s_f1, KQ);
    for (int idx = threadIdx.x; idx < MT * MT * 64; idx += blockDim.x) {
        const int m = idx / (MT * 64), m2 = (idx / 64) % MT, l = idx % 64;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = w2<F>(a, 16 * m2 + 4 * (l / 16) + r, 16 * m + l % 16);
        s_f2[idx] = make_float4(v[0], v[1], v[2], v[3]);
    }
    for (int f = threadIdx.x; f < F; f += blockDim.x) { s_b1[f] = a.b1[f]; s_b2[f] = a.b2[f]; }
    __syncthreads();

    const int lane = threadIdx.x % 64;
    int64_t tile, tile_end, stride;
    tile_range(a.P, tile, tile_end, stride);
    for (; tile < tile_end; tile += stride) {
        // keep the weight-fragment LDS reads inside the loop: hoisted out of
        // it they would need hundreds of registers
        asm volatile("" ::: "memory");
        const int64_t p = tile * 16 + lane % 16;
        const float d = (p < a.P) ? a.dsrc[p * a.dstride + a.doff] : 0.0f;
        floatx4 acc1[MT];
        gemm_rbf<F>(a, s_f1, KQ, KS, d, lane, acc1);
        float z[MT][4];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) z[m][r] = ssp(acc1[m][r] + s_b1[16 * m + 4 * (lane / 16) + r]);
        floatx4 acc2[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) acc2[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m2 = 0; m2 < MT; ++m2) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float4 w = s_f2[(m * MT + m2) * 64 + lane];
                acc2[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(w.x, z[m2][0], acc2[m], 0, 0, 0);
                acc2[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(w.y, z[m2][1], acc2[m], 0, 0, 0);
                acc2[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(w.z, z[m2][2], acc2[m], 0, 0, 0);
                acc2[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(w.w, z[m2][3], acc2[m], 0, 0, 0);
            }
        }
        if (p < a.P) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int f0 = 16 * m + 4 * (lane / 16);
                float4 v = make_float4(acc2[m][0] + s_b2[f0], acc2[m][1] + s_b2[f0 + 1], acc2[m][2] + s_b2[f0 + 2],
                                       acc2[m][3] + s_b2[f0 + 3]);
                *reinterpret_cast<float4 *>(a.phi + p * F + f0) = v;
            }
        }
    }
}

template <int F>
__global__ __launch_bounds__(kBwdThreads) void filter_bwd_kernel(FilterArgs a) {
    constexpr int MT = F / 16;
    constexpr int FS = F / 4;        // features per k-slot in the g_phi GEMM
    constexpr int SQ = FS / 4;
    __shared__ float4 s_f1[MT * 4 * 64];
    __shared__ float4 s_f2b[MT * SQ * 64];   // [m][sq][lane]: A2[16 m + l%16][FS (l/16) + 4 sq + r]
    __shared__ float4 s_f1b[4 * MT * 64];    // [kt][m2][lane]: A1[16 kt + l%16][16 m2 + 4(l/16) + r]
    __shared__ float s_b1[F];
    const int KS = (a.K + 3) / 4;
    const int KQ = (KS + 3) / 4;
    const int KT = (a.K + 15) / 16;
    stage_f1<F>(a, s_f1, KQ);
    for (int idx = threadIdx.x; idx < MT * SQ * 64; idx += blockDim.x) {
        const int m = idx / (SQ * 64), sq = (idx / 64) % SQ, l = idx % 64;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = w2<F>(a, 16 * m + l % 16, FS * (l / 16) + 4 * sq + r);
        s_f2b[idx] = make_float4(v[0], v[1], v[2], v[3]);
    }
    for (int idx = threadIdx.x; idx < KT * MT * 64; idx += blockDim.x) {
        const int kt = idx / (MT * 64), m2 = (idx / 64) % MT, l = idx % 64;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = w1<F>(a, 16 * kt + l % 16, 16 * m2 + 4 * (l / 16) + r);
        s_f1b[idx] = make_float4(v[0], v[1], v[2], v[3]);
    }
    for (int f = threadIdx.x; f < F; f += blockDim.x) s_b1[f] = a.b1[f];
    __syncthreads();

    const int lane = threadIdx.x % 64;
    const int slot = lane / 16;
    int64_t tile, tile_end, stride;
    tile_range(a.P, tile, tile_end, stride);
    for (; tile < tile_end; tile += stride) {
        asm volatile("" ::: "memory");
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
        // G = g_y_i x_j + g_y_j x_i over this lane's quarter of the features,
        // gathered in two halves to bound the loads in flight
        float gphi[FS];
        float gfc = 0.0f;
        {
            const int64_t bi = (int64_t)ij.x * F + FS * slot, bj = (int64_t)ij.y * F + FS * slot;
            const int64_t bp = (live ? p : 0) * F + FS * slot;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                asm volatile("" ::: "memory");
#pragma unroll
                for (int qq = 0; qq < SQ / 2; ++qq) {
                    const int q = half * (SQ / 2) + qq;
                    const float4 gyi = *reinterpret_cast<const float4 *>(a.gy + bi + 4 * q);
                    const float4 gyj = *reinterpret_cast<const float4 *>(a.gy + bj + 4 * q);
                    const float4 xi = *reinterpret_cast<const float4 *>(a.x + bi + 4 * q);
                    const float4 xj = *reinterpret_cast<const float4 *>(a.x + bj + 4 * q);
                    const float4 ph = *reinterpret_cast<const float4 *>(a.phi_in + bp + 4 * q);
                    const float g0 = gyi.x * xj.x + gyj.x * xi.x, g1 = gyi.y * xj.y + gyj.y * xi.y;
                    const float g2 = gyi.z * xj.z + gyj.z * xi.z, g3 = gyi.w * xj.w + gyj.w * xi.w;
                    gfc += g0 * ph.x + g1 * ph.y + g2 * ph.z + g3 * ph.w;
                    gphi[4 * q + 0] = fc * g0; gphi[4 * q + 1] = fc * g1;
                    gphi[4 * q + 2] = fc * g2; gphi[4 * q + 3] = fc * g3;
                }
            }
        }
        // g_z^T = A2 g_phi^T  (k = feature f = FS slot + step)
        floatx4 gz[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) gz[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sq = 0; sq < SQ; ++sq) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float4 w = s_f2b[(m * SQ + sq) * 64 + lane];
                gz[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(w.x, gphi[4 * sq + 0], gz[m], 0, 0, 0);
                gz[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(w.y, gphi[4 * sq + 1], gz[m], 0, 0, 0);
                gz[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(w.z, gphi[4 * sq + 2], gz[m], 0, 0, 0);
                gz[m] = __builtin_amdgcn_mfma_f32_16x16x4f32(w.w, gphi[4 * sq + 3], gz[m], 0, 0, 0);
            }
        }
        // recompute a = rbf A1 + b1;  g_a = g_z (.) sigmoid(a)
        floatx4 acc1[MT];
        gemm_rbf<F>(a, s_f1, KQ, KS, d, lane, acc1);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) gz[m][r] *= sigm(acc1[m][r] + s_b1[16 * m + 4 * slot + r]);
        // g_rbf^T = A1 g_a^T
        floatx4 ge[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) ge[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m2 = 0; m2 < MT; ++m2) {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                if (kt < KT) {
                    const float4 w = s_f1b[(kt * MT + m2) * 64 + lane];
                    ge[kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(w.x, gz[m2][0], ge[kt], 0, 0, 0);
                    ge[kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(w.y, gz[m2][1], ge[kt], 0, 0, 0);
                    ge[kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(w.z, gz[m2][2], ge[kt], 0, 0, 0);
                    ge[kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(w.w, gz[m2][3], ge[kt], 0, 0, 0);
                }
            }
        }
        // S_p = sum_k g_rbf_k rbf_k'(d) + g_fc fc'(d), summed over the four k-slots
        float sp = gfc * dfc;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            if (kt < KT) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int k = 16 * kt + 4 * slot + r;
                    if (k < a.K) {
                        const float t = d - (a.lo + (float)k * a.dmu);
                        sp += ge[kt][r] * (-2.0f * a.gamma * t * fast_exp(-a.gamma * t * t));
                    }
                }
            }
        }
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
    int64_t off[3 + 9 * 16 + 2 + 1];
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
    const int64_t tiles = (a.P + 15) / 16;
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

sn_status filter_backward(const sn_model &m, int t, const float4 *pgeo, const int2 *pair_ij, int64_t P,
                          const float *phi, const float *x, const float *gy, float *S, int accumulate,
                          hipStream_t s) {
    if (P <= 0) return SN_OK;
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
