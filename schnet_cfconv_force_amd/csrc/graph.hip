// Edge-side kernels: pair setup, the CFConv CSR segment reduce, and force
// assembly.
//
// Pair indexing.  The filter W(d) depends only on the distance, so the two
// directed edges (i, j) and (j, i) share one filter row.  Each unordered
// pair {i < j} gets an index p, numbered in CSR order of the "upper" edges
// (j > i); edge_pair[e] maps every directed edge to its pair, so the filter
// network runs once per pair (half the directed edges) and the CFConv reads
// the shared row from both ends.
//
// CFConv ("How", flash message passing and flash aggregation -- FlashSchNet
// summary page): y_i = sum_{e in row i} fc(d_e) phi_{p(e)} (.) x_{col(e)}.
// One group of F/4 lanes owns a row and accumulates it in registers, so no
// atomics are needed and the summation order is fixed.  Because W is the
// same for (i, j) and (j, i), the same kernel applied to g_y gives the
// input gradient of the backward pass.
//
// Forces: F_i = sum_{e in row i} S_{p(e)} u_e, with u_e = (r_j - r_i)/d and
// S_p = dE/dd_p -- again one lane group per row, no atomics.
#include "sn_internal.h"

namespace sn {

namespace {

// thread per row: first upper edge and number of upper edges
__global__ void pair_count_kernel(int N, const int32_t *row_ptr, const int32_t *col, int32_t *up_first,
                                  int32_t *up_cnt, const int *guard, const int *run_flag) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N || (run_flag && *run_flag == 0)) return;
    if (guard && *guard) {               // the pair count is then 0: nothing reads these
        up_cnt[i] = 0;
        return;
    }
    int lo = row_ptr[i], hi = row_ptr[i + 1];
    const int end = hi;
    while (lo < hi) {                     // first e with col[e] > i
        int mid = (lo + hi) >> 1;
        if (col[mid] > i) hi = mid; else lo = mid + 1;
    }
    up_first[i] = lo;
    up_cnt[i] = end - lo;
}

struct PairArgs {
    int N;
    const int32_t *row_ptr, *col, *rev, *up_first, *up_ptr;
    const float *pos;
    int32_t *edge_pair;
    int2 *pair_ij;
    float4 *pgeo;
    float *pfc, *plfc;
    int periodic;
    float L[3], invL[3];
    float cutoff;
    int64_t E;
    int *status;
    const int *guard;
    const int *run_flag;
};

// one wavefront per row: pair index of every edge; geometry of upper edges
__global__ __launch_bounds__(256) void pair_fill_kernel(PairArgs a) {
    const int lane = threadIdx.x % 64;
    const int i = blockIdx.x * 4 + threadIdx.x / 64;
    if (i >= a.N || (a.guard && *a.guard) || (a.run_flag && *a.run_flag == 0)) return;
    const int64_t P = a.status[kPairTotal];   // written by the pair count check
    const int e0 = a.row_ptr[i], e1 = a.row_ptr[i + 1];
    const int uf = a.up_first[i], up = a.up_ptr[i];
    for (int e = e0 + lane; e < e1; e += 64) {
        const int j = a.col[e];
        if (j < 0 || j >= a.N || j == i) {
            flag_status(a.status, SN_ERR_INVALID);
            a.edge_pair[e] = 0;
            continue;
        }
        if (j > i) {
            const int p = up + (e - uf);
            if (p >= P) {                         // more upper edges than E/2: not symmetric
                flag_status(a.status, SN_ERR_INVALID);
                a.edge_pair[e] = 0;
                continue;
            }
            a.edge_pair[e] = p;
            a.pair_ij[p] = make_int2(i, j);
            float4 g;
            float fc, lfc;
            pair_geometry(a.pos + 3 * i, a.pos + 3 * j, a.periodic, a.L, a.invL, a.cutoff, g, fc, lfc);
            a.pgeo[p] = g;
            a.pfc[p] = fc;
            a.plfc[p] = lfc;
        } else {
            // the reverse edge (j, i) is an upper edge of row j
            const int r = a.rev[e];
            const int p = (r >= a.up_first[j] && r < a.row_ptr[j + 1] && a.col[r] == i)
                              ? a.up_ptr[j] + (r - a.up_first[j]) : -1;
            if (p < 0 || p >= P) {
                flag_status(a.status, SN_ERR_INVALID);
                a.edge_pair[e] = 0;
                continue;
            }
            a.edge_pair[e] = p;
        }
    }
}

struct RefreshArgs {
    const float *pos;
    float *ref_pos;
    int N;
    const int2 *pair_ij;
    float4 *pgeo;
    float *pfc, *plfc;
    int periodic;
    float L[3], invL[3];
    float cutoff;
    const int *status;
};

// Neighbour skin: on a step that rebuilt the list, record the positions it
// was built from; on the others, the pairs of the kept list get their
// geometry from the current positions (pairs now beyond the cutoff get a
// zero envelope and contribute nothing).
__global__ __launch_bounds__(256) void pair_refresh_kernel(RefreshArgs a) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (a.status[kStatusWord] != 0) return;   // the list may be unfilled after an error
    if (a.status[kBuildFlag] != 0) {
        if (idx < 3 * (int64_t)a.N) a.ref_pos[idx] = a.pos[idx];
        return;
    }
    if (idx >= a.status[kPairTotal]) return;
    const int2 ij = a.pair_ij[idx];
    float4 g;
    float fc, lfc;
    pair_geometry(a.pos + 3 * ij.x, a.pos + 3 * ij.y, a.periodic, a.L, a.invL, a.cutoff, g, fc, lfc);
    a.pgeo[idx] = g;
    a.pfc[idx] = fc;
    a.plfc[idx] = lfc;
}

// y_i = sum_{e in row i} W[p] (.) in[col(e)], W = fc phi in the 24-bit row
// format (three words per four features).  One block of kCfWaves wavefronts
// per row: wavefront w takes the row's edge chunks w, w + kCfWaves, ... of
// kCfChunk edges; in a wavefront F/FPL lanes cover the features (FPL
// consecutive ones each: FPL/4 loads of three filter words and of a float4)
// and the 64/(F/FPL) lane groups take interleaved edges of the chunk.  The
// lane groups, then the wavefronts, are combined in a fixed order
// (deterministic).  Per XCD this keeps about one replica's rows in flight,
// so the second read of a pair's filter row (from the other row) mostly hits
// L2; 8 features per lane were 7 % faster than 4 and 4 % faster than 16,
// and a block per row 6 % faster than four rows per block.
constexpr int kCfFPL = 8;
constexpr int kCfWaves = 4;
constexpr int kCfChunk = 16;
// Systems of fewer rows than this are latency-bound: their CFConv issues
// every round of a chunk's loads at once, and their force assembly gives a
// wavefront to each row.
constexpr int kSmallRows = 4096;

template <int F, int FPL, int UNROLL>
__global__ __launch_bounds__(64 * kCfWaves) void cfconv_kernel(int N, const int32_t *row_ptr, const int32_t *col,
                                                               const int32_t *edge_pair, const uint32_t *phi24,
                                                               const float *in, float *out, const int *guard) {
    constexpr int LPR = F / FPL;          // lanes per feature row
    constexpr int G = 64 / LPR;           // edges in flight per wavefront
    constexpr int Q = FPL / 4;            // float4 pieces per lane
    __shared__ float4 s_part[kCfWaves][LPR * Q];
    const int lane = threadIdx.x % 64, wv = threadIdx.x / 64;
    const int sub = lane % LPR, grp = lane / LPR;
    const int row = xcd_block(N);
    if (row < 0 || (guard && *guard)) return;   // the whole block leaves together
    const int e0 = row_ptr[row], e1 = row_ptr[row + 1];
    float4 acc[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) acc[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int eb = e0 + kCfChunk * wv; eb < e1; eb += kCfWaves * kCfChunk) {
        // the chunk's indices loaded once, coalesced, then broadcast
        const int k = eb + lane;
        int cj = 0, cp = 0;
        if (lane < kCfChunk && k < e1) {
            cj = col[k];
            cp = edge_pair[k];
        }
        const int n = min(kCfChunk, e1 - eb);
        const int rounds = (n + G - 1) / G;     // uniform over the wavefront
#pragma unroll UNROLL
        for (int r = 0; r < rounds; ++r) {
            const int t = r * G + grp;
            const int src = t < n ? t : n - 1;  // shuffle sources are always live lanes
            const int j = __shfl(cj, src, 64);
            const int p = __shfl(cp, src, 64);
            if (t < n) {
                const uint32_t *pw = phi24 + (int64_t)p * fp24_words(F) + 3 * Q * sub;
                const float *px = in + (int64_t)j * F + FPL * sub;
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const uint3 fw = *reinterpret_cast<const uint3 *>(pw + 3 * q);
                    const float4 f = unpack_fp24(fw.x, fw.y, fw.z);
                    const float4 x = *reinterpret_cast<const float4 *>(px + 4 * q);
                    acc[q].x = fmaf(f.x, x.x, acc[q].x);
                    acc[q].y = fmaf(f.y, x.y, acc[q].y);
                    acc[q].z = fmaf(f.z, x.z, acc[q].z);
                    acc[q].w = fmaf(f.w, x.w, acc[q].w);
                }
            }
        }
    }
#pragma unroll
    for (int o = 32; o >= LPR; o >>= 1)
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            acc[q].x += __shfl_xor(acc[q].x, o, 64);
            acc[q].y += __shfl_xor(acc[q].y, o, 64);
            acc[q].z += __shfl_xor(acc[q].z, o, 64);
            acc[q].w += __shfl_xor(acc[q].w, o, 64);
        }
    if (grp == 0)
#pragma unroll
        for (int q = 0; q < Q; ++q) s_part[wv][sub * Q + q] = acc[q];
    __syncthreads();
    if (wv == 0 && grp == 0)
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            float4 r = s_part[0][sub * Q + q];
#pragma unroll
            for (int w = 1; w < kCfWaves; ++w) {
                const float4 v = s_part[w][sub * Q + q];
                r.x += v.x; r.y += v.y; r.z += v.z; r.w += v.w;
            }
            *reinterpret_cast<float4 *>(out + (int64_t)row * F + FPL * sub + 4 * q) = r;
        }
}

// lanes per row of the force assembly: 16 (32 was faster for forces alone,
// slower with the MD kicks); 64 for systems of fewer than kSmallRows rows,
// whose rows are then summed in one round of loads instead of four
constexpr int kFrLanes = 16;
constexpr int kFrLanesSmall = 64;

struct ForcesArgs {
    int N, row_blocks;
    const int32_t *row_ptr, *col, *edge_pair;
    const float4 *pgeo;
    const float *S;
    int s_parts;          // S_p = S[(s_parts - 1) s_stride + p] + ... + S[p]
    int64_t s_stride;
    float *forces;
    const int32_t *rptr;
    const float *eps;
    float *energy;        // (may be null) energy[b]
    double *elog;         // (may be null) MD log: elog[b], or elog[step B + b] with elog_by_step
    int elog_by_step;     // step = status[kMdStep] - 1 (device-driven steps)
    VerletFuse vf;   // vf.vel null: no integrator part
    int *status;
    const int *guard;
};

__device__ inline int load_status(const int *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Blocks [0, row_blocks): F_i = sum_{e in row i} S[p(e)] u_e, LANES lanes
// per row, then the Verlet part for atom i.  Blocks past them: the energy of one
// replica each (fixed-order tree, deterministic).
template <int LANES>
__global__ __launch_bounds__(256) void forces_kernel(ForcesArgs a) {
    __shared__ double red[256];
    __shared__ int s_go, s_open;
    // device-driven steps: this step's index (the words are written only by
    // the step's first launch, so every block reads the same value)
    const int step = a.vf.n_total >= 0 || a.elog_by_step ? a.status[kMdStep] - 1 : 0;
    if ((int)blockIdx.x >= a.row_blocks) {
        const int b = blockIdx.x - a.row_blocks;
        double s = 0.0;
        for (int i = a.rptr[b] + threadIdx.x; i < a.rptr[b + 1]; i += 256) s += (double)a.eps[i];
        red[threadIdx.x] = s;
        __syncthreads();
        for (int w = 128; w > 0; w >>= 1) {
            if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
            __syncthreads();
        }
        if (threadIdx.x == 0) {
            if (a.energy) a.energy[b] = (float)red[0];
            if (a.elog) a.elog[(a.elog_by_step ? (int64_t)step * (gridDim.x - a.row_blocks) : 0) + b] = red[0];
        }
    } else {
        if (threadIdx.x == 0) {
            s_go = a.vf.vel && load_status(a.status) == 0;
            s_open = a.vf.open && (a.vf.n_total < 0 || step + 1 < a.vf.n_total);
        }
        __syncthreads();
        const int sub = threadIdx.x % LANES;
        const int i = (blockIdx.x * 256 + threadIdx.x) / LANES;
        if (i < a.N && !(a.guard && *a.guard)) {
            const int e0 = a.row_ptr[i], e1 = a.row_ptr[i + 1];
            float fx = 0.f, fy = 0.f, fz = 0.f;
            for (int e = e0 + sub; e < e1; e += LANES) {
                const int p = a.edge_pair[e];
                const float4 g = a.pgeo[p];
                float sv = a.S[(a.s_parts - 1) * a.s_stride + p];
                for (int t = a.s_parts - 2; t >= 0; --t) sv += a.S[t * a.s_stride + p];
                const float s = (a.col[e] > i) ? sv : -sv;
                fx += s * g.x;
                fy += s * g.y;
                fz += s * g.z;
            }
            for (int o = LANES / 2; o > 0; o >>= 1) {
                fx += __shfl_xor(fx, o, LANES);
                fy += __shfl_xor(fy, o, LANES);
                fz += __shfl_xor(fz, o, LANES);
            }
            if (sub == 0) {
                a.forces[3 * i] = fx;
                a.forces[3 * i + 1] = fy;
                a.forces[3 * i + 2] = fz;
                const bool finite = isfinite(fx) && isfinite(fy) && isfinite(fz);
                if (!finite) flag_status(a.status, SN_ERR_NONFINITE);
                if (s_go && finite) {
                    const float im = a.vf.inv_mass[i];
                    const float f3[3] = {fx, fy, fz};
                    float r2 = 0.0f;
#pragma unroll
                    for (int c = 0; c < 3; ++c) {
                        // the kicks and the drift as explicit fused multiply-adds,
                        // as in open_step_kernel: the same bits whichever launch
                        // applies them
                        const float hf = a.vf.half * f3[c];
                        float v = a.vf.vel[3 * i + c];
                        if (a.vf.close) v = fmaf(hf, im, v);
                        if (s_open) {
                            v = fmaf(hf, im, v);
                            const float r = fmaf(a.vf.dt, v, a.vf.pos[3 * i + c]);
                            a.vf.pos[3 * i + c] = r;
                            if (a.vf.ref_pos) {
                                const float dr = r - a.vf.ref_pos[3 * i + c];
                                r2 = fmaf(dr, dr, r2);
                            }
                        }
                        a.vf.vel[3 * i + c] = v;
                    }
                    // beyond half the skin from where the list was built: the
                    // next step rebuilds (every writer stores the same value)
                    if (a.vf.ref_pos && !(r2 <= a.vf.half_skin2))
                        __hip_atomic_store(a.status + kDisplaced, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0 && a.vf.close) {
        if (a.vf.edge_slot) *a.vf.edge_slot = a.status[kEdgeTotal];
        if (a.vf.edge_log) a.vf.edge_log[step] = a.status[kEdgeTotal];
    }
}

}  // namespace

sn_status pairs_setup(const sn_system &sys, const float *pos, const int32_t *row_ptr, const int32_t *col,
                      const int32_t *rev, int64_t E, float cutoff, char *ws, const EfLayout &L, int *status,
                      const int *guard, hipStream_t s, const int *run_flag) {
    const int N = sys.n_atoms;
    ProfScope ps(K_PAIRS, s);
    int32_t *up_first = reinterpret_cast<int32_t *>(ws + L.up_first);
    int32_t *up_cnt = reinterpret_cast<int32_t *>(ws + L.up_cnt);
    int32_t *up_ptr = reinterpret_cast<int32_t *>(ws + L.up_ptr);
    pair_count_kernel<<<(N + 255) / 256, 256, 0, s>>>(N, row_ptr, col, up_first, up_cnt, guard, run_flag);
    SN_TRY(launch_status());
    SN_TRY(scan_exclusive(up_cnt, up_ptr, N, nullptr, nullptr, s, PairCountCheck{status, row_ptr, N, E, guard != nullptr},
                          run_flag));
    PairArgs a;
    a.N = N;
    a.row_ptr = row_ptr; a.col = col; a.rev = rev; a.up_first = up_first; a.up_ptr = up_ptr;
    a.pos = pos;
    a.edge_pair = reinterpret_cast<int32_t *>(ws + L.edge_pair);
    a.pair_ij = reinterpret_cast<int2 *>(ws + L.pair_ij);
    a.pgeo = reinterpret_cast<float4 *>(ws + L.pgeo);
    a.pfc = reinterpret_cast<float *>(ws + L.pfc);
    a.plfc = reinterpret_cast<float *>(ws + L.plfc);
    a.periodic = sys.periodic ? 1 : 0;
    for (int c = 0; c < 3; ++c) {
        a.L[c] = sys.periodic ? sys.box[c] : 1.0f;
        a.invL[c] = (float)(1.0 / (double)a.L[c]);
    }
    a.cutoff = cutoff;
    a.E = E;
    a.status = status;
    a.guard = guard;
    a.run_flag = run_flag;
    pair_fill_kernel<<<(N + 3) / 4, 256, 0, s>>>(a);
    return launch_status();
}

sn_status pairs_refresh(const sn_system &sys, const float *pos, float cutoff, char *ws, const EfLayout &L,
                        int *status, int64_t P_cap, hipStream_t s) {
    ProfScope ps(K_PAIRS, s);
    RefreshArgs a;
    a.pos = pos;
    a.ref_pos = reinterpret_cast<float *>(ws + L.ref_pos);
    a.N = sys.n_atoms;
    a.pair_ij = reinterpret_cast<const int2 *>(ws + L.pair_ij);
    a.pgeo = reinterpret_cast<float4 *>(ws + L.pgeo);
    a.pfc = reinterpret_cast<float *>(ws + L.pfc);
    a.plfc = reinterpret_cast<float *>(ws + L.plfc);
    a.periodic = sys.periodic ? 1 : 0;
    for (int c = 0; c < 3; ++c) {
        a.L[c] = sys.periodic ? sys.box[c] : 1.0f;
        a.invL[c] = (float)(1.0 / (double)a.L[c]);
    }
    a.cutoff = cutoff;
    a.status = status;
    const int64_t n = std::max<int64_t>(P_cap, 3 * (int64_t)sys.n_atoms);
    if (n <= 0) return SN_OK;
    pair_refresh_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a);
    return launch_status();
}

sn_status cfconv(int F, int N, const int32_t *row_ptr, const int32_t *col, const int32_t *edge_pair,
                 const uint32_t *phi24, const float *in, float *out, const int *guard, hipStream_t s) {
    ProfScope ps(K_CFCONV, s);
    const int grid = xcd_grid(N);        // one block per row
    constexpr int T = 64 * kCfWaves;
    const bool small = N < kSmallRows;
#define SN_CF(FF)                                                                                          \
    (small ? cfconv_kernel<FF, kCfFPL, 4><<<grid, T, 0, s>>>(N, row_ptr, col, edge_pair, phi24, in, out, guard) \
           : cfconv_kernel<FF, kCfFPL, 2><<<grid, T, 0, s>>>(N, row_ptr, col, edge_pair, phi24, in, out, guard))
    switch (F) {
        case 32: SN_CF(32); break;
        case 64: SN_CF(64); break;
        case 128: SN_CF(128); break;
        default: return SN_ERR_INVALID;
    }
#undef SN_CF
    return launch_status();
}

sn_status forces_rows(int N, int B, const int32_t *replica_ptr, const float *eps, float *energy,
                      const int32_t *row_ptr, const int32_t *col, const int32_t *edge_pair, const float4 *pgeo,
                      const float *S, int s_parts, int64_t s_stride, float *forces, int *status, const int *guard,
                      const VerletFuse *vf, hipStream_t s, double *elog, int elog_by_step) {
    ProfScope ps(K_FORCES, s);
    ForcesArgs a;
    a.N = N;
    const int lanes = N < kSmallRows ? kFrLanesSmall : kFrLanes;
    a.row_blocks = (N + 256 / lanes - 1) / (256 / lanes);
    a.row_ptr = row_ptr; a.col = col; a.edge_pair = edge_pair; a.pgeo = pgeo; a.S = S; a.forces = forces;
    a.s_parts = s_parts;
    a.s_stride = s_stride;
    a.rptr = replica_ptr; a.eps = eps; a.energy = energy;
    a.elog = elog;
    a.elog_by_step = elog_by_step;
    a.vf = vf ? *vf : VerletFuse{};
    if (!vf) a.vf.n_total = -1;
    a.status = status;
    a.guard = guard;
    if (lanes == kFrLanesSmall)
        forces_kernel<kFrLanesSmall><<<a.row_blocks + B, 256, 0, s>>>(a);
    else
        forces_kernel<kFrLanes><<<a.row_blocks + B, 256, 0, s>>>(a);
    return launch_status();
}

}  // namespace sn
