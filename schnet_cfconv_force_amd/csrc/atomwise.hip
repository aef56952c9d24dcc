// The per-replica energy sum.
#include "sn_internal.h"

namespace sn {

namespace {

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

sn_status replica_sum(int B, const int32_t *replica_ptr, const float *eps, float *energy, hipStream_t s) {
    ProfScope ps(K_ENERGY, s);
    replica_sum_kernel<<<B, 256, 0, s>>>(replica_ptr, eps, energy);
    return launch_status();
}

}  // namespace sn
