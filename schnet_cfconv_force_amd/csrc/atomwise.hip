// Atom-wise layers: embedding lookup, the dense F x F layers of the
// interaction blocks and the readout (forward and backward), and the
// per-replica energy sum.
//
// Dense layer Y = epi(pro(X) @ B) on the matrix cores: a wavefront owns 16
// atoms and all output columns; v_mfma_f32_16x16x4f32 with
//   A (16 atoms x 4 k)    : lane l holds X[atom l%16][k-slot l/16]
//   B (4 k x 16 columns)  : lane l holds B[k-slot l/16][column l%16]
//   D (16 atoms x 16 col) : lane l holds rows 4(l/16)+r, column l%16
// The k index of slot s at step t is (FI/4) s + t, so every lane reads one
// contiguous quarter of its atom's row.  B is staged once per block in LDS
// in exactly the order the lanes consume it (one 16-byte read per lane per
// four steps, conflict free).
#include "sn_internal.h"

namespace sn {

namespace {

template <int FI, int FO, int TRANS, int PRO, int EPI>
__global__ __launch_bounds__(256) void dense_kernel(int N, const float *__restrict__ X, const float *__restrict__ W,
                                                    const float *__restrict__ bias, const float *__restrict__ aux,
                                                    float *Y) {
    constexpr int QK = FI / 4;         // k values per slot
    constexpr int MO = FO / 16;        // output column tiles
    constexpr int SQ = QK / 4;         // float4 groups per slot
    __shared__ float4 s_w[MO * SQ * 64];
    const int tid = threadIdx.x;
    for (int idx = tid; idx < MO * SQ * 64; idx += 256) {
        const int mo = idx / (SQ * 64), sq = (idx / 64) % SQ, l = idx % 64;
        const int n = 16 * mo + (l % 16);
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int k = QK * (l / 16) + 4 * sq + r;
            v[r] = TRANS ? W[n * FI + k] : W[k * FO + n];
        }
        s_w[idx] = make_float4(v[0], v[1], v[2], v[3]);
    }
    __syncthreads();
    const int lane = tid % 64;
    const int row0 = (blockIdx.x * 4 + tid / 64) * 16;
    if (row0 >= N) return;
    const int arow = row0 + (lane % 16);
    float a[QK];
#pragma unroll
    for (int q = 0; q < SQ; ++q) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (arow < N) v = *reinterpret_cast<const float4 *>(X + (int64_t)arow * FI + QK * (lane / 16) + 4 * q);
        a[4 * q + 0] = v.x; a[4 * q + 1] = v.y; a[4 * q + 2] = v.z; a[4 * q + 3] = v.w;
    }
    if (PRO == PRO_SSP) {
#pragma unroll
        for (int k = 0; k < QK; ++k) a[k] = ssp(a[k]);
    }
    floatx4 acc[MO];
#pragma unroll
    for (int mo = 0; mo < MO; ++mo) acc[mo] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sq = 0; sq < SQ; ++sq) {
#pragma unroll
        for (int mo = 0; mo < MO; ++mo) {
            const float4 b = s_w[(mo * SQ + sq) * 64 + lane];
            acc[mo] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * sq + 0], b.x, acc[mo], 0, 0, 0);
            acc[mo] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * sq + 1], b.y, acc[mo], 0, 0, 0);
            acc[mo] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * sq + 2], b.z, acc[mo], 0, 0, 0);
            acc[mo] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[4 * sq + 3], b.w, acc[mo], 0, 0, 0);
        }
    }
#pragma unroll
    for (int mo = 0; mo < MO; ++mo) {
        const int n = 16 * mo + (lane % 16);
        const float bn = bias ? bias[n] : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = row0 + 4 * (lane / 16) + r;
            if (row >= N) continue;
            float v = acc[mo][r] + bn;
            const int64_t o = (int64_t)row * FO + n;
            if (EPI == EPI_SIGMUL) v *= sigm(aux[o]);
            if (EPI == EPI_ACCUM) v += Y[o];
            Y[o] = v;
        }
    }
}

__global__ void embed_kernel(int N, int F, int T, const int32_t *types, const float *emb, float *h, int *status) {
    int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)N * F) return;
    int i = (int)(idx / F), f = (int)(idx % F);
    int z = types[i];
    if (z < 0 || z >= T) {
        if (f == 0) flag_status(status, SN_ERR_INVALID);
        z = 0;
    }
    h[idx] = emb[(int64_t)z * F + f];
}

// eps_i = sum_m ssp(q_im) R2_m + c2 ;  gq_im = sigmoid(q_im) R2_m
__global__ void readout_kernel(int N, int H, const float *q, const float *R2, const float *c2, float *eps,
                               float *gq) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N) return;
    float e = c2[0];
    for (int m = 0; m < H; ++m) {
        float v = q[(int64_t)i * H + m];
        e += ssp(v) * R2[m];
        gq[(int64_t)i * H + m] = sigm(v) * R2[m];
    }
    eps[i] = e;
}

// one block per replica, fixed-order tree reduction (deterministic)
__global__ __launch_bounds__(256) void replica_sum_kernel(const int32_t *rptr, const float *eps, float *energy) {
    __shared__ double red[256];
    const int b = blockIdx.x;
    double s = 0.0;
    for (int i = rptr[b] + threadIdx.x; i < rptr[b + 1]; i += 256) s += (double)eps[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) energy[b] = (float)red[0];
}

template <int FI, int FO>
sn_status dense_dispatch(int N, const float *X, const float *W, int transW, const float *bias, int pro, int epi,
                         const float *aux, float *Y, hipStream_t s) {
    const int grid = (N + 63) / 64;
#define SN_DENSE_CASE(T, P, E)                                                                  \
    if (transW == T && pro == P && epi == E) {                                                  \
        dense_kernel<FI, FO, T, P, E><<<grid, 256, 0, s>>>(N, X, W, bias, aux, Y);              \
        return launch_status();                                                                 \
    }
    SN_DENSE_CASE(0, PRO_NONE, EPI_STORE)
    SN_DENSE_CASE(0, PRO_SSP, EPI_ACCUM)
    SN_DENSE_CASE(1, PRO_NONE, EPI_SIGMUL)
    SN_DENSE_CASE(1, PRO_NONE, EPI_STORE)
    SN_DENSE_CASE(1, PRO_NONE, EPI_ACCUM)
#undef SN_DENSE_CASE
    return SN_ERR_INVALID;
}

}  // namespace

sn_status dense(int N, int Fi, int Fo, const float *X, const float *W, int transW, const float *bias, int pro,
                int epi, const float *aux, float *Y, hipStream_t s) {
    if (N <= 0) return SN_OK;
    ProfScope ps(K_DENSE, s);
#define SN_SHAPE(A, B) \
    if (Fi == A && Fo == B) return dense_dispatch<A, B>(N, X, W, transW, bias, pro, epi, aux, Y, s);
    SN_SHAPE(32, 32) SN_SHAPE(32, 16) SN_SHAPE(16, 32)
    SN_SHAPE(64, 64) SN_SHAPE(64, 32) SN_SHAPE(32, 64)
    SN_SHAPE(128, 128) SN_SHAPE(128, 64) SN_SHAPE(64, 128)
#undef SN_SHAPE
    return SN_ERR_INVALID;
}

sn_status embed(int N, int F, int T, const int32_t *types, const float *emb, float *h, int *status,
                hipStream_t s) {
    if (N <= 0) return SN_OK;
    ProfScope ps(K_EMBED, s);
    int64_t n = (int64_t)N * F;
    embed_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(N, F, T, types, emb, h, status);
    return launch_status();
}

sn_status readout(int N, int H, const float *q, const float *R2, const float *c2, float *eps, float *gq,
                  hipStream_t s) {
    if (N <= 0) return SN_OK;
    ProfScope ps(K_READOUT, s);
    readout_kernel<<<(N + 255) / 256, 256, 0, s>>>(N, H, q, R2, c2, eps, gq);
    return launch_status();
}

sn_status replica_sum(int B, const int32_t *replica_ptr, const float *eps, float *energy, hipStream_t s) {
    ProfScope ps(K_ENERGY, s);
    replica_sum_kernel<<<B, 256, 0, s>>>(replica_ptr, eps, energy);
    return launch_status();
}

}  // namespace sn
