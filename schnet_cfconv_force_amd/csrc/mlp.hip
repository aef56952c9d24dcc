// Atom-wise layers of the interaction blocks and the readout, fused per
// block of 16 atoms and run on the matrix cores.
//
// Same mapping as the filter network: computed transposed (output features
// are the M dimension, 16 atoms the N dimension of
// v_mfma_f32_16x16x32_f16), operands held in split form (hi = fp16(x),
// lo = fp16((x - hi) 2^11), accumulated as hi.hi + 2^-11 (hi.lo + lo.hi)),
// and the accumulator layout of the first GEMM fed directly as the B operand
// of the second.  Each atom's operands are scaled by a power of two first
// (exact), so no value is lost to the fp16 range.
//
// Kernels (one launch each):
//   OUT      o = y Wo1 + bo1 (stored);  h += ssp(o) Wo2 + bo2
//   X        x = h W_in
//   READOUT  q = h R1 + c1;  eps = ssp(q) . R2 + c2;  g_h = (sigmoid(q) (.) R2) R1^T
//   BWD_OUT  g_o = (g_h Wo2^T) (.) sigmoid(o);  g_y = g_o Wo1^T (stored)
//   BWD_X    g_h += g_x W_in^T
#include "sn_internal.h"

namespace sn {

namespace {

constexpr float kLoScale = 2048.0f;
constexpr float kLoUnscale = 1.0f / 2048.0f;
// 8 wavefronts (128 atoms) per block: one block per CU holds the staged
// weights, and the grid of the largest systems fits in one pass of the CUs
constexpr int kMlpThreads = 512;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

__device__ inline void split8(const float (&v)[8], half8 &hi, half8 &lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const _Float16 h = (_Float16)v[j];
        hi[j] = h;
        lo[j] = (_Float16)fmaf((float)h, -kLoScale, v[j] * kLoScale);   // (x - hi) 2^11, exact
    }
}

// The three split products for MT output tiles sharing one B operand, with
// dependent instructions on one accumulator MT instructions apart.
// Weight hi and lo halves live in separate arrays, so a wavefront's 16-byte
// reads are contiguous and free of LDS bank conflicts.
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

__device__ inline int chain_k(int t, int s, int j) { return 32 * t + 16 * (j >> 2) + 4 * s + (j & 3); }

// exponent e with |x| 2^-e <= 1 over the atom's values (four k-slot lanes)
__device__ inline int atom_exponent(float amax) {
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    return amax > 0.0f ? ilogbf(amax) + 1 : 0;
}

enum { MLP_X = 0, MLP_OUT = 1, MLP_READOUT = 2, MLP_BWD_OUT = 3, MLP_BWD_X = 4 };

template <int F, int MODE>
struct Shape {
    static constexpr int FI1 = F;
    static constexpr int FO1 = MODE == MLP_READOUT ? F / 2 : F;
    static constexpr bool TWO = MODE == MLP_OUT || MODE == MLP_READOUT || MODE == MLP_BWD_OUT;
    static constexpr int FI2 = FO1;
    static constexpr int FO2 = F;
    static constexpr int M1 = FO1 / 16, T1 = (FI1 + 31) / 32;
    static constexpr int M2 = FO2 / 16, T2 = (FI2 + 31) / 32;
};

struct MlpArgs {
    int N;
    const float *in;            // [N][F] input of the first layer
    const float *W1, *b1;       // first layer weights (layout depends on the mode) and bias
    const float *W2, *b2;       // second layer
    const float *aux;           // BWD_OUT: the stored pre-activation o
    const float *R2, *c2;       // READOUT
    float *mid;                 // OUT: o is stored here
    float *out;                 // X: x;  OUT: h (+=);  READOUT: g_h;  BWD_OUT: g_y;  BWD_X: g_h (+=)
    float *eps;                 // READOUT: per-atom energy
};

// Weight of output row `mrow`, input column `k` for a layer y = x W
// (W[in][out], trans = 0) or y = x W^T (W[out][in], trans = 1).
__device__ inline float wval(const float *W, int trans, int kdim, int mdim, int k, int mrow) {
    if (k >= kdim) return 0.0f;
    return trans ? W[mrow * kdim + k] : W[k * mdim + mrow];
}

// Stage a layer's A fragments: [m][t][l], value j = weight(row 16m + l%16,
// column kfn(t, l/16, j)); chained = 1 uses the accumulator-chain k order.
__device__ inline void stage(half8 *dhi, half8 *dlo, const float *W, int trans, int kdim, int mdim, int MT, int T, int chained) {
    for (int idx = threadIdx.x; idx < MT * T * 64; idx += blockDim.x) {
        const int m = idx / (T * 64), t = (idx / 64) % T, l = idx % 64;
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int k = chained ? chain_k(t, l / 16, j) : 32 * t + 8 * (l / 16) + j;
            v[j] = wval(W, trans, kdim, mdim, k, 16 * m + l % 16);
        }
        split8(v, dhi[idx], dlo[idx]);
    }
}

template <int F, int MODE>
__global__ __launch_bounds__(kMlpThreads) void mlp_kernel(MlpArgs a) {
    using S = Shape<F, MODE>;
    constexpr int M1 = S::M1, T1 = S::T1, M2 = S::M2, T2 = S::T2;
    constexpr int TRANS1 = (MODE == MLP_BWD_OUT || MODE == MLP_BWD_X) ? 1 : 0;
    constexpr int TRANS2 = (MODE == MLP_READOUT || MODE == MLP_BWD_OUT) ? 1 : 0;
    __shared__ half8 s_w1h[M1 * T1 * 64], s_w1l[M1 * T1 * 64];
    __shared__ half8 s_w2h[S::TWO ? M2 * T2 * 64 : 1], s_w2l[S::TWO ? M2 * T2 * 64 : 1];
    stage(s_w1h, s_w1l, a.W1, TRANS1, S::FI1, S::FO1, M1, T1, 0);
    if (S::TWO) stage(s_w2h, s_w2l, a.W2, TRANS2, S::FI2, S::FO2, M2, T2, 1);
    __syncthreads();

    const int lane = threadIdx.x % 64, slot = lane / 16;
    const int atom0 = (blockIdx.x * (kMlpThreads / 64) + threadIdx.x / 64) * 16;
    if (atom0 >= a.N) return;
    const int atom = atom0 + lane % 16;
    const bool live = atom < a.N;

    // first layer input: features 32 t + 8 slot + j of the lane's atom
    float xin[T1][8];
    float xmax = 0.0f;
#pragma unroll
    for (int t = 0; t < T1; ++t)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int f0 = 32 * t + 8 * slot + 4 * q;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (live && f0 < S::FI1) v = *reinterpret_cast<const float4 *>(a.in + (int64_t)atom * F + f0);
            xin[t][4 * q + 0] = v.x; xin[t][4 * q + 1] = v.y; xin[t][4 * q + 2] = v.z; xin[t][4 * q + 3] = v.w;
            xmax = fmaxf(xmax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
    const int e1 = atom_exponent(xmax);
    floatx4 am[M1], ac[M1];
#pragma unroll
    for (int m = 0; m < M1; ++m) am[m] = ac[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < T1; ++t) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = ldexpf(xin[t][j], -e1);
        half8 bh, bl;
        split8(v, bh, bl);
        mma3_tiles<M1>(s_w1h + t * 64 + lane, s_w1l + t * 64 + lane, T1 * 64, bh, bl, am, ac);
    }
    // first-layer result for output features 16 m + 4 slot + r
    float r1[M1][4];
#pragma unroll
    for (int m = 0; m < M1; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) r1[m][r] = ldexpf(am[m][r] + ac[m][r] * kLoUnscale, e1);

    if (MODE == MLP_X || MODE == MLP_BWD_X) {
        if (!live) return;
#pragma unroll
        for (int m = 0; m < M1; ++m) {
            float4 *dst = reinterpret_cast<float4 *>(a.out + (int64_t)atom * F + 16 * m + 4 * slot);
            float4 v = make_float4(r1[m][0], r1[m][1], r1[m][2], r1[m][3]);
            if (MODE == MLP_BWD_X) {
                const float4 o = *dst;
                v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
            }
            *dst = v;
        }
        return;
    }

    // activation between the layers -> B operand of the second GEMM
    float z[M1][4];
    float zmax = 0.0f;
    float eps_part = 0.0f;
#pragma unroll
    for (int m = 0; m < M1; ++m) {
        const int n0 = 16 * m + 4 * slot;
        if (MODE == MLP_OUT) {
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                o[r] = r1[m][r] + a.b1[n0 + r];
                z[m][r] = ssp(o[r]);
            }
            if (live)
                *reinterpret_cast<float4 *>(a.mid + (int64_t)atom * F + n0) = make_float4(o[0], o[1], o[2], o[3]);
        } else if (MODE == MLP_READOUT) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float q = r1[m][r] + a.b1[n0 + r];
                eps_part += ssp(q) * a.R2[n0 + r];
                z[m][r] = sigm(q) * a.R2[n0 + r];
            }
        } else {   // MLP_BWD_OUT
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
            if (live) o = *reinterpret_cast<const float4 *>(a.aux + (int64_t)atom * F + n0);
            z[m][0] = r1[m][0] * sigm(o.x);
            z[m][1] = r1[m][1] * sigm(o.y);
            z[m][2] = r1[m][2] * sigm(o.z);
            z[m][3] = r1[m][3] * sigm(o.w);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) zmax = fmaxf(zmax, fabsf(z[m][r]));
    }
    if (MODE == MLP_READOUT) {
        eps_part += __shfl_xor(eps_part, 16, 64);
        eps_part += __shfl_xor(eps_part, 32, 64);
        if (live && slot == 0) a.eps[atom] = eps_part + a.c2[0];
    }
    const int e2 = atom_exponent(zmax);
    floatx4 bm[M2], bc[M2];
#pragma unroll
    for (int m = 0; m < M2; ++m) bm[m] = bc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < T2; ++t) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int m = 2 * t + (j >> 2);
            v[j] = m < M1 ? ldexpf(z[m < M1 ? m : 0][j & 3], -e2) : 0.0f;
        }
        half8 bh, bl;
        split8(v, bh, bl);
        mma3_tiles<M2>(s_w2h + t * 64 + lane, s_w2l + t * 64 + lane, T2 * 64, bh, bl, bm, bc);
    }
    if (!live) return;
#pragma unroll
    for (int m = 0; m < M2; ++m) {
        const int n0 = 16 * m + 4 * slot;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = ldexpf(bm[m][r] + bc[m][r] * kLoUnscale, e2);
        float4 *dst = reinterpret_cast<float4 *>(a.out + (int64_t)atom * F + n0);
        if (MODE == MLP_OUT) {
            const float4 h = *dst;
            *dst = make_float4(h.x + v[0] + a.b2[n0], h.y + v[1] + a.b2[n0 + 1], h.z + v[2] + a.b2[n0 + 2],
                               h.w + v[3] + a.b2[n0 + 3]);
        } else {
            *dst = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
}

template <int MODE>
sn_status launch_mlp(int F, const MlpArgs &a, hipStream_t s) {
    if (a.N <= 0) return SN_OK;
    ProfScope ps(K_MLP, s);
    const int atoms_per_block = 16 * (kMlpThreads / 64);
    const int grid = (a.N + atoms_per_block - 1) / atoms_per_block;
    switch (F) {
        case 32: mlp_kernel<32, MODE><<<grid, kMlpThreads, 0, s>>>(a); break;
        case 64: mlp_kernel<64, MODE><<<grid, kMlpThreads, 0, s>>>(a); break;
        case 128: mlp_kernel<128, MODE><<<grid, kMlpThreads, 0, s>>>(a); break;
        default: return SN_ERR_INVALID;
    }
    return launch_status();
}

}  // namespace

sn_status mlp_x(int N, int F, const float *h, const float *W_in, float *x, hipStream_t s) {
    MlpArgs a = {};
    a.N = N; a.in = h; a.W1 = W_in; a.out = x;
    return launch_mlp<MLP_X>(F, a, s);
}

sn_status mlp_out(int N, int F, const float *y, const float *Wo1, const float *bo1, const float *Wo2,
                  const float *bo2, float *o, float *h, hipStream_t s) {
    MlpArgs a = {};
    a.N = N; a.in = y; a.W1 = Wo1; a.b1 = bo1; a.W2 = Wo2; a.b2 = bo2; a.mid = o; a.out = h;
    return launch_mlp<MLP_OUT>(F, a, s);
}

sn_status mlp_readout(int N, int F, const float *h, const float *R1, const float *c1, const float *R2,
                      const float *c2, float *eps, float *gh, hipStream_t s) {
    MlpArgs a = {};
    a.N = N; a.in = h; a.W1 = R1; a.b1 = c1; a.W2 = R1; a.R2 = R2; a.c2 = c2; a.eps = eps; a.out = gh;
    return launch_mlp<MLP_READOUT>(F, a, s);
}

sn_status mlp_bwd_out(int N, int F, const float *gh, const float *Wo2, const float *o, const float *Wo1, float *gy,
                      hipStream_t s) {
    MlpArgs a = {};
    a.N = N; a.in = gh; a.W1 = Wo2; a.aux = o; a.W2 = Wo1; a.out = gy;
    return launch_mlp<MLP_BWD_OUT>(F, a, s);
}

sn_status mlp_bwd_x(int N, int F, const float *gx, const float *W_in, float *gh, hipStream_t s) {
    MlpArgs a = {};
    a.N = N; a.in = gx; a.W1 = W_in; a.out = gh;
    return launch_mlp<MLP_BWD_X>(F, a, s);
}

}  // namespace sn
