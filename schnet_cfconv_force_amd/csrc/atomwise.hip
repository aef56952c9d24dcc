// Atom-wise helpers: embedding lookup and the per-replica energy sum.
#include "sn_internal.h"

namespace sn {

namespace {

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

}  // namespace

sn_status embed(int N, int F, int T, const int32_t *types, const float *emb, float *h, int *status,
                hipStream_t s) {
    if (N <= 0) return SN_OK;
    ProfScope ps(K_EMBED, s);
    int64_t n = (int64_t)N * F;
    embed_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(N, F, T, types, emb, h, status);
    return launch_status();
}

sn_status replica_sum(int B, const int32_t *replica_ptr, const float *eps, float *energy, hipStream_t s) {
    ProfScope ps(K_ENERGY, s);
    replica_sum_kernel<<<B, 256, 0, s>>>(replica_ptr, eps, energy);
    return launch_status();
}

}  // namespace sn
