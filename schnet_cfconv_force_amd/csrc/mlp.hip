// Atom-wise layers of the interaction blocks and the readout, fused per
// wavefront of 16 atoms and run on the matrix cores.
//
// Same mapping as the filter network: computed transposed (output features
// are the M dimension, atoms the N dimension of v_mfma_f32_16x16x32_f16),
// operands in the split-fp16 form of split_mfma.h, and the accumulator
// layout of the first GEMM fed directly as the B operand of the second.
// At these sizes a launch is bound by its chain of latencies (input and
// weight loads, the dependent matrix instructions of one tile, the stores),
// so wavefronts stay small (one 16-atom tile; kNT > 1 would share each
// weight fragment read between tiles) and many (two per SIMD).  Each atom's
// operands are scaled by a power of two from the atom's own maximum.
//
// Kernels (one launch each):
//   OUT      o = y Wo1 + bo1 (stored);  h += ssp(o) Wo2 + bo2
//   X        x = h W_in
//   READOUT  q = h R1 + c1;  eps = ssp(q) . R2 + c2;  g_h = (sigmoid(q) (.) R2) R1^T
//   BWD_OUT  g_o = (g_h Wo2^T) (.) sigmoid(o);  g_y = g_o Wo1^T (stored)
//   BWD_X    g_h += g_x W_in^T
#include "split_mfma.h"

namespace sn {

namespace {

// 8 wavefronts of 16 atoms per block: one block per CU holds the staged
// weights of both layers, and 17k-atom systems fit in one pass of the CUs
constexpr int kMlpWaves = 8;
constexpr int kMlpThreads = 64 * kMlpWaves;
constexpr int kNT = 1;   // 16-atom tiles per wavefront

__device__ inline int chain_k(int t, int s, int j) { return 32 * t + 16 * (j >> 2) + 4 * s + (j & 3); }

// the atom's largest magnitude over its four k-slot lanes
__device__ inline float atom_max(float amax) {
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    return fmaxf(amax, __shfl_xor(amax, 32, 64));
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
    // weights stored [out][in] (read transposed)
    static constexpr int TR1 = (MODE == MLP_BWD_OUT || MODE == MLP_BWD_X) ? 1 : 0;
    static constexpr int TR2 = (MODE == MLP_READOUT || MODE == MLP_BWD_OUT) ? 1 : 0;
};

struct MlpArgs {
    int N;
    const float *in;            // [N][F] input of the first layer
    const half8 *w1h, *w1l;     // first layer, pre-split (weight-pack slot)
    const half8 *w2h, *w2l;     // second layer
    const int *sc1, *sc2;       // their split scales
    const float *b1, *b2;       // biases
    const float *aux;           // BWD_OUT: the stored pre-activation o
    const float *R2, *c2;       // READOUT
    float *mid;                 // OUT: o is stored here
    float *out;                 // X: x;  OUT: h (+=);  READOUT: g_h;  BWD_OUT: g_y;  BWD_X: g_h (+=)
    float *eps;                 // READOUT: per-atom energy
    float *rmax;                // X: max_f |x|;  BWD_OUT: max_f |g_y| (per atom; optional)
};

// Weights of A fragment idx of a layer ([m][t][l]): value j = weight(row
// 16m + l%16, column k(t, l/16, j)), k in the plain order (32t + 8s + j) or
// the accumulator-chain order.  In both orders values 0-3 and 4-7 are runs
// of four consecutive k, read as one 16-byte load each when W is stored
// [out][in] (TRANS); 0 beyond kdim.
template <int T, int TRANS, int CHAINED>
__device__ inline void layer_frag(const float *W, int kdim, int mdim, int idx, float (&v)[8]) {
    const int m = idx / (T * 64), t = (idx / 64) % T, l = idx % 64, s = l / 16;
    const int mrow = 16 * m + l % 16;
    const int k0 = CHAINED ? 32 * t + 4 * s : 32 * t + 8 * s;
    const int k1 = CHAINED ? k0 + 16 : k0 + 4;
    if (TRANS) {
        float4 p = make_float4(0.f, 0.f, 0.f, 0.f), q = p;
        if (k0 < kdim) p = *reinterpret_cast<const float4 *>(W + (int64_t)mrow * kdim + k0);
        if (k1 < kdim) q = *reinterpret_cast<const float4 *>(W + (int64_t)mrow * kdim + k1);
        v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w;
        v[4] = q.x; v[5] = q.y; v[6] = q.z; v[7] = q.w;
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int k = (j < 4 ? k0 : k1) + (j & 3);
            v[j] = k < kdim ? W[(int64_t)k * mdim + mrow] : 0.0f;
        }
    }
}

template <int F, int MODE>
__global__ __launch_bounds__(kMlpThreads) void mlp_kernel(MlpArgs a) {
    using S = Shape<F, MODE>;
    constexpr int M1 = S::M1, T1 = S::T1, M2 = S::M2, T2 = S::T2;
    constexpr int MG1 = M1 < 4 ? M1 : 4, MG2 = M2 < 4 ? M2 : 4;
    __shared__ half8 s_w1h[M1 * T1 * 64], s_w1l[M1 * T1 * 64];
    __shared__ half8 s_w2h[S::TWO ? M2 * T2 * 64 : 1], s_w2l[S::TWO ? M2 * T2 * 64 : 1];

    const int lane = threadIdx.x % 64, slot = lane / 16;
    const int base = (blockIdx.x * kMlpWaves + threadIdx.x / 64) * (16 * kNT);
    int atom[kNT];
    bool live[kNT];
    // first layer input: features 32 t + 8 slot + j of the lane's atoms
    // (loaded before the weights are staged, so that the two latencies overlap)
    float xin[kNT][T1][8];
    float xmax[kNT];
#pragma unroll
    for (int n = 0; n < kNT; ++n) {
        atom[n] = base + 16 * n + lane % 16;
        live[n] = atom[n] < a.N;
        xmax[n] = 0.0f;
#pragma unroll
        for (int t = 0; t < T1; ++t)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int f0 = 32 * t + 8 * slot + 4 * q;
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (live[n] && f0 < S::FI1) v = *reinterpret_cast<const float4 *>(a.in + (int64_t)atom[n] * F + f0);
                xin[n][t][4 * q + 0] = v.x; xin[n][t][4 * q + 1] = v.y;
                xin[n][t][4 * q + 2] = v.z; xin[n][t][4 * q + 3] = v.w;
                xmax[n] = fmaxf(xmax[n], fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
            }
    }
    copy_frags<M1 * T1 * 64, kMlpThreads>(s_w1h, s_w1l, a.w1h, a.w1l, M1 * T1 * 64);
    if (S::TWO) copy_frags<M2 * T2 * 64, kMlpThreads>(s_w2h, s_w2l, a.w2h, a.w2l, M2 * T2 * 64);
    const int sw1 = a.sc1[0];
    const int sw2 = S::TWO ? a.sc2[0] : 0;
    __syncthreads();
    if (base >= a.N) return;

    // first layer: r1 = in W1 for output features 16 m + 4 slot + r
    float r1[kNT][M1][4];
    {
        int sx[kNT];
        half8 bh[T1][kNT], bl[T1][kNT];
#pragma unroll
        for (int n = 0; n < kNT; ++n) {
            sx[n] = split_scale(atom_max(xmax[n]));
#pragma unroll
            for (int t = 0; t < T1; ++t) {
                float v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = ldexpf(xin[n][t][j], sx[n]);
                split8(v, bh[t][n], bl[t][n]);
            }
        }
#pragma unroll
        for (int m0 = 0; m0 < M1; m0 += MG1) {
            floatx4 acc[MG1][kNT];
#pragma unroll
            for (int m = 0; m < MG1; ++m)
#pragma unroll
                for (int n = 0; n < kNT; ++n) acc[m][n] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < T1; ++t)
                mma_split<MG1, kNT>(s_w1h + (m0 * T1 + t) * 64 + lane, s_w1l + (m0 * T1 + t) * 64 + lane, T1 * 64,
                                    bh[t], bl[t], acc);
#pragma unroll
            for (int m = 0; m < MG1; ++m)
#pragma unroll
                for (int n = 0; n < kNT; ++n)
#pragma unroll
                    for (int r = 0; r < 4; ++r) r1[n][m0 + m][r] = ldexpf(acc[m][n][r], -(sw1 + sx[n]));
        }
    }

    if (MODE == MLP_X || MODE == MLP_BWD_X) {
        if (MODE == MLP_X && a.rmax) {   // the per-atom row maximum of x, for the filter backward's scales
#pragma unroll
            for (int n = 0; n < kNT; ++n) {
                float mx = 0.0f;
#pragma unroll
                for (int m = 0; m < M1; ++m)
#pragma unroll
                    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(r1[n][m][r]));
                mx = atom_max(mx);
                if (live[n] && slot == 0) a.rmax[atom[n]] = mx;
            }
        }
#pragma unroll
        for (int n = 0; n < kNT; ++n) {
            if (!live[n]) continue;
#pragma unroll
            for (int m = 0; m < M1; ++m) {
                float4 *dst = reinterpret_cast<float4 *>(a.out + (int64_t)atom[n] * F + 16 * m + 4 * slot);
                float4 v = make_float4(r1[n][m][0], r1[n][m][1], r1[n][m][2], r1[n][m][3]);
                if (MODE == MLP_BWD_X) {
                    const float4 o = *dst;
                    v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
                }
                *dst = v;
            }
        }
        return;
    }

    // activation between the layers -> B operands of the second GEMM
    half8 bh[T2][kNT], bl[T2][kNT];
    int sz[kNT];
#pragma unroll
    for (int n = 0; n < kNT; ++n) {
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
                    o[r] = r1[n][m][r] + a.b1[n0 + r];
                    z[m][r] = ssp(o[r]);
                }
                if (live[n])
                    *reinterpret_cast<float4 *>(a.mid + (int64_t)atom[n] * F + n0) = make_float4(o[0], o[1], o[2], o[3]);
            } else if (MODE == MLP_READOUT) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float q = r1[n][m][r] + a.b1[n0 + r];
                    eps_part += ssp(q) * a.R2[n0 + r];
                    z[m][r] = sigm(q) * a.R2[n0 + r];
                }
            } else {   // MLP_BWD_OUT
                float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
                if (live[n]) o = *reinterpret_cast<const float4 *>(a.aux + (int64_t)atom[n] * F + n0);
                z[m][0] = r1[n][m][0] * sigm(o.x);
                z[m][1] = r1[n][m][1] * sigm(o.y);
                z[m][2] = r1[n][m][2] * sigm(o.z);
                z[m][3] = r1[n][m][3] * sigm(o.w);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) zmax = fmaxf(zmax, fabsf(z[m][r]));
        }
        if (MODE == MLP_READOUT) {
            eps_part += __shfl_xor(eps_part, 16, 64);
            eps_part += __shfl_xor(eps_part, 32, 64);
            if (live[n] && slot == 0) a.eps[atom[n]] = eps_part + a.c2[0];
        }
        sz[n] = split_scale(atom_max(zmax));
#pragma unroll
        for (int t = 0; t < T2; ++t) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int m = 2 * t + (j >> 2);
                v[j] = m < M1 ? ldexpf(z[m < M1 ? m : 0][j & 3], sz[n]) : 0.0f;
            }
            split8(v, bh[t][n], bl[t][n]);
        }
    }
    float omax[kNT];
#pragma unroll
    for (int n = 0; n < kNT; ++n) omax[n] = 0.0f;
#pragma unroll
    for (int m0 = 0; m0 < M2; m0 += MG2) {
        floatx4 acc[MG2][kNT];
#pragma unroll
        for (int m = 0; m < MG2; ++m)
#pragma unroll
            for (int n = 0; n < kNT; ++n) acc[m][n] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < T2; ++t)
            mma_split<MG2, kNT>(s_w2h + (m0 * T2 + t) * 64 + lane, s_w2l + (m0 * T2 + t) * 64 + lane, T2 * 64,
                                bh[t], bl[t], acc);
#pragma unroll
        for (int n = 0; n < kNT; ++n) {
            if (!live[n]) continue;
#pragma unroll
            for (int m = 0; m < MG2; ++m) {
                const int n0 = 16 * (m0 + m) + 4 * slot;
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = ldexpf(acc[m][n][r], -(sw2 + sz[n]));
                float4 *dst = reinterpret_cast<float4 *>(a.out + (int64_t)atom[n] * F + n0);
                if (MODE == MLP_OUT) {
                    const float4 h = *dst;
                    *dst = make_float4(h.x + v[0] + a.b2[n0], h.y + v[1] + a.b2[n0 + 1], h.z + v[2] + a.b2[n0 + 2],
                                       h.w + v[3] + a.b2[n0 + 3]);
                } else {
                    *dst = make_float4(v[0], v[1], v[2], v[3]);
                }
                if (MODE == MLP_BWD_OUT)
                    omax[n] = fmaxf(omax[n], fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
            }
        }
    }
    if (MODE == MLP_BWD_OUT && a.rmax) {   // the per-atom row maximum of g_y
#pragma unroll
        for (int n = 0; n < kNT; ++n) {
            const float mx = atom_max(omax[n]);
            if (live[n] && slot == 0) a.rmax[atom[n]] = mx;
        }
    }
}

// Pre-split one layer of a mode into a weight-pack slot (as the kernel's
// staging would into LDS); returns the split scale.
template <int F, int MODE, int LAYER>
__device__ inline int pack_layer(const float *W, half8 *hi, half8 *lo, unsigned *s_max) {
    using S = Shape<F, MODE>;
    if (LAYER == 1)
        return stage_split<S::M1 * S::T1 * 64, kMlpThreads>(hi, lo, S::M1 * S::T1 * 64, s_max,
            [&](int idx, float (&v)[8]) { layer_frag<S::T1, S::TR1, 0>(W, S::FI1, S::FO1, idx, v); });
    return stage_split<S::M2 * S::T2 * 64, kMlpThreads>(hi, lo, S::M2 * S::T2 * 64, s_max,
        [&](int idx, float (&v)[8]) { layer_frag<S::T2, S::TR2, 1>(W, S::FI2, S::FO2, idx, v); });
}

struct MlpPackArgs {
    const float *W_in[16], *Wo1[16], *Wo2[16];
    const float *R1;
    char *pack;
    int I;
};

// The atom-wise slots of the weight pack: one block per matrix (six per
// interaction, then the two readout layers).
template <int F>
__global__ __launch_bounds__(kMlpThreads) void mlp_pack_kernel(MlpPackArgs pa) {
    __shared__ unsigned s_max;
    if (threadIdx.x == 0) s_max = 0u;
    __syncthreads();
    const int b = blockIdx.x;
    const int t = b / 6, k = b % 6;
    const int slot = b < 6 * pa.I ? pack_slot(t, PK_XW + k) : pack_readout_slot(pa.I, b - 6 * pa.I);
    const PackRef r = pack_ref(pa.pack, pa.I, slot);
    half8 *hi = const_cast<half8 *>(static_cast<const half8 *>(r.hi));
    half8 *lo = const_cast<half8 *>(static_cast<const half8 *>(r.lo));
    int sc = 0;
    if (b >= 6 * pa.I) {
        sc = b == 6 * pa.I ? pack_layer<F, MLP_READOUT, 1>(pa.R1, hi, lo, &s_max)
                           : pack_layer<F, MLP_READOUT, 2>(pa.R1, hi, lo, &s_max);
    } else {
        switch (PK_XW + k) {
            case PK_XW: sc = pack_layer<F, MLP_X, 1>(pa.W_in[t], hi, lo, &s_max); break;
            case PK_OW1: sc = pack_layer<F, MLP_OUT, 1>(pa.Wo1[t], hi, lo, &s_max); break;
            case PK_OW2: sc = pack_layer<F, MLP_OUT, 2>(pa.Wo2[t], hi, lo, &s_max); break;
            case PK_BOW1: sc = pack_layer<F, MLP_BWD_OUT, 1>(pa.Wo2[t], hi, lo, &s_max); break;
            case PK_BOW2: sc = pack_layer<F, MLP_BWD_OUT, 2>(pa.Wo1[t], hi, lo, &s_max); break;
            default: sc = pack_layer<F, MLP_BWD_X, 1>(pa.W_in[t], hi, lo, &s_max); break;
        }
    }
    if (threadIdx.x == 0) const_cast<int *>(r.sc)[0] = sc;
}

template <int MODE>
sn_status launch_mlp(int F, const MlpArgs &a, hipStream_t s) {
    if (a.N <= 0) return SN_OK;
    ProfScope ps(K_MLP, s);
    const int atoms_per_block = 16 * kNT * kMlpWaves;
    const int grid = (a.N + atoms_per_block - 1) / atoms_per_block;
    switch (F) {
        case 32: mlp_kernel<32, MODE><<<grid, kMlpThreads, 0, s>>>(a); break;
        case 64: mlp_kernel<64, MODE><<<grid, kMlpThreads, 0, s>>>(a); break;
        case 128: mlp_kernel<128, MODE><<<grid, kMlpThreads, 0, s>>>(a); break;
        default: return SN_ERR_INVALID;
    }
    return launch_status();
}

void set_layers(MlpArgs &a, PackRef w1, const PackRef *w2) {
    a.w1h = static_cast<const half8 *>(w1.hi);
    a.w1l = static_cast<const half8 *>(w1.lo);
    a.sc1 = w1.sc;
    if (w2) {
        a.w2h = static_cast<const half8 *>(w2->hi);
        a.w2l = static_cast<const half8 *>(w2->lo);
        a.sc2 = w2->sc;
    }
}

}  // namespace

sn_status mlp_pack(const sn_model &m, char *pack, hipStream_t s) {
    const int T = m.n_types, I = m.n_interactions, F = m.n_features, K = m.n_rbf;
    if (I < 1 || I > 16) return SN_ERR_INVALID;
    int64_t off[9 * 16 + 6];
    sn_param_offsets(T, I, F, K, off, (int32_t)(sizeof(off) / sizeof(off[0])));
    MlpPackArgs pa = {};
    pa.pack = pack;
    pa.I = I;
    for (int t = 0; t < I; ++t) {
        const int64_t *blk = off + 1 + 9 * t;   // W_in, A1, b1, A2, b2, Wo1, bo1, Wo2, bo2
        pa.W_in[t] = m.params + blk[0];
        pa.Wo1[t] = m.params + blk[5];
        pa.Wo2[t] = m.params + blk[7];
    }
    pa.R1 = m.params + off[1 + 9 * I];
    ProfScope ps(K_PACK, s);
    const int grid = 6 * I + 2;
    switch (F) {
        case 32: mlp_pack_kernel<32><<<grid, kMlpThreads, 0, s>>>(pa); break;
        case 64: mlp_pack_kernel<64><<<grid, kMlpThreads, 0, s>>>(pa); break;
        case 128: mlp_pack_kernel<128><<<grid, kMlpThreads, 0, s>>>(pa); break;
        default: return SN_ERR_INVALID;
    }
    return launch_status();
}

sn_status mlp_x(int N, int F, const float *h, PackRef W_in, float *x, float *xmax, hipStream_t s) {
    MlpArgs a = {};
    a.N = N; a.in = h; a.out = x; a.rmax = xmax;
    set_layers(a, W_in, nullptr);
    return launch_mlp<MLP_X>(F, a, s);
}

sn_status mlp_out(int N, int F, const float *y, PackRef Wo1, const float *bo1, PackRef Wo2, const float *bo2,
                  float *o, float *h, hipStream_t s) {
    MlpArgs a = {};
    a.N = N; a.in = y; a.b1 = bo1; a.b2 = bo2; a.mid = o; a.out = h;
    set_layers(a, Wo1, &Wo2);
    return launch_mlp<MLP_OUT>(F, a, s);
}

sn_status mlp_readout(int N, int F, const float *h, PackRef R1, const float *c1, PackRef R1t, const float *R2,
                      const float *c2, float *eps, float *gh, hipStream_t s) {
    MlpArgs a = {};
    a.N = N; a.in = h; a.b1 = c1; a.R2 = R2; a.c2 = c2; a.eps = eps; a.out = gh;
    set_layers(a, R1, &R1t);
    return launch_mlp<MLP_READOUT>(F, a, s);
}

sn_status mlp_bwd_out(int N, int F, const float *gh, PackRef Wo2t, const float *o, PackRef Wo1t, float *gy,
                      float *gymax, hipStream_t s) {
    MlpArgs a = {};
    a.N = N; a.in = gh; a.aux = o; a.out = gy; a.rmax = gymax;
    set_layers(a, Wo2t, &Wo1t);
    return launch_mlp<MLP_BWD_OUT>(F, a, s);
}

sn_status mlp_bwd_x(int N, int F, const float *gx, PackRef W_int, float *gh, hipStream_t s) {
    MlpArgs a = {};
    a.N = N; a.in = gx; a.out = gh;
    set_layers(a, W_int, nullptr);
    return launch_mlp<MLP_BWD_X>(F, a, s);
}

}  // namespace sn
