// Atom-wise layers of the interaction blocks and the readout, fused per
// wavefront of 16 atoms and run on the matrix cores.
//
// Computed transposed (output features are the M dimension, atoms the N
// dimension of v_mfma_f32_16x16x32_f16), with operands in the split-fp16
// form of split_mfma.h.  Every layer's weights sit in the weight pack in
// the accumulator-chained order, so a layer's input is always held the way
// an accumulator leaves it (lane = atom l%16, features 16 m + 4 (l/16) + r):
// rows load with one float4 per tile, and a layer's output feeds the next
// layer as its B operand without leaving the registers.  Each atom's
// operands are scaled by a power of two from the atom's own maximum.
//
// One launch runs a chain of layers between two CFConvs:
//   EMBED_X   h = Emb[type];  x_0 = h W_in
//   OUT_X     o = y Wo1 + bo1 (stored);  h += ssp(o) Wo2 + bo2;  x_{t+1} = h W_in
//   TAIL      the last interaction's OUT, then the readout
//             q = h R1 + c1, eps = ssp(q) . R2 + c2, g_h = (sigmoid(q) (.) R2) R1^T,
//             then the first backward block g_o = (g_h Wo2^T) (.) sigmoid(o),
//             g_y = g_o Wo1^T
//   BX_BO     g_h += g_x W_in^T (interaction t), then for t - 1:
//             g_o = (g_h Wo2^T) (.) sigmoid(o), g_y = g_o Wo1^T
// x and g_y also get their per-atom row maxima (the filter backward's
// scales).  A block stages its chain's weights in two LDS buffers: while one
// layer runs, the next layer's fragments are already loaded into registers
// and go to the freed buffer after a block barrier.
#include "split_mfma.h"

namespace sn {

namespace {

// 5 wavefronts of 16 atoms per block (one block per CU: two buffers of
// F x F weights take 128 KB of LDS): a 17k-atom system spreads over 216
// CUs in one pass; 8 wavefronts (135 CUs) were 8 % slower per launch
constexpr int kMlpWaves = 5;
constexpr int kMlpThreads = 64 * kMlpWaves;

template <int F>
struct Dims {
    static constexpr int M = F / 16;                 // 16-feature tiles of a row
    static constexpr int MR = F / 32;                // tiles of the readout's hidden layer (F / 2)
    static constexpr int T = (F + 31) / 32;          // 32-wide k steps over F inputs
    static constexpr int TR = (F / 2 + 31) / 32;     // ... over F / 2 inputs
    static constexpr int LAYER = M * T * 64;         // fragments of an F x F layer
    static constexpr int R1F = MR * T * 64;          // readout first layer (F -> F / 2)
    static constexpr int R2F = M * TR * 64;          // readout second layer (F / 2 -> F)
    static constexpr int BUF = LAYER > R1F + R2F ? LAYER : R1F + R2F;
    static constexpr int IT = (BUF + kMlpThreads - 1) / kMlpThreads;   // fragments per thread
};

// the atom's largest magnitude over its four k-slot lanes
__device__ inline float atom_max(float amax) {
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    return fmaxf(amax, __shfl_xor(amax, 32, 64));
}

// Weights of fragment idx of a layer ([m][t][l], T k steps) in the
// accumulator-chained order: value j = weight(row 16 m + l%16, column
// 32 t + 16 (j / 4) + 4 (l / 16) + j % 4); 0 beyond kdim.  W is [kdim][mdim]
// (row-vector convention) or, with TRANS, [mdim][kdim]; runs of four
// consecutive k are then one 16-byte load.
template <int T, int TRANS>
__device__ inline void layer_frag(const float *W, int kdim, int mdim, int idx, float (&v)[8]) {
    const int m = idx / (T * 64), t = (idx / 64) % T, l = idx % 64, s = l / 16;
    const int mrow = 16 * m + l % 16;
    const int k0 = 32 * t + 4 * s, k1 = k0 + 16;
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

// One wavefront's 16 atoms.
struct Wave {
    int lane, slot, atom;
    bool live;
};

template <int M>
__device__ inline void load_rows(const float *src, int F, const Wave &w, float (&v)[M][4]) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
        float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
        if (w.live) q = *reinterpret_cast<const float4 *>(src + (int64_t)w.atom * F + 16 * m + 4 * w.slot);
        v[m][0] = q.x; v[m][1] = q.y; v[m][2] = q.z; v[m][3] = q.w;
    }
}

template <int M>
__device__ inline void store_rows(float *dst, int F, const Wave &w, const float (&v)[M][4]) {
    if (!w.live) return;
#pragma unroll
    for (int m = 0; m < M; ++m)
        *reinterpret_cast<float4 *>(dst + (int64_t)w.atom * F + 16 * m + 4 * w.slot) =
            make_float4(v[m][0], v[m][1], v[m][2], v[m][3]);
}

// per-atom max_f |v| (every lane of the atom gets it)
template <int M>
__device__ inline float row_absmax(const float (&v)[M][4]) {
    float mx = 0.0f;
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(v[m][r]));
    return atom_max(mx);
}

// out = in W for 16 atoms: MI input tiles, MO output tiles; W as fragments
// [m][t][l] in LDS (hi at wh, lo at wl) with split scale sw.
template <int MI, int MO>
__device__ inline void layer(const float (&in)[MI][4], const half8 *wh, const half8 *wl, int sw, int lane,
                             float (&out)[MO][4]) {
    constexpr int T = (16 * MI + 31) / 32;
    constexpr int MG = MO < 4 ? MO : 4;
    const int sx = split_scale(row_absmax(in));
    half8 bh[T], bl[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int m = 2 * t + (j >> 2);
            v[j] = m < MI ? ldexpf(in[m < MI ? m : 0][j & 3], sx) : 0.0f;
        }
        split8(v, bh[t], bl[t]);
    }
#pragma unroll
    for (int m0 = 0; m0 < MO; m0 += MG) {
        floatx4 acc[MG][1];
#pragma unroll
        for (int m = 0; m < MG; ++m) acc[m][0] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < T; ++t)
            mma_split<MG, 1>(wh + (m0 * T + t) * 64 + lane, wl + (m0 * T + t) * 64 + lane, T * 64, &bh[t], &bl[t],
                             acc);
#pragma unroll
        for (int m = 0; m < MG; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) out[m0 + m][r] = ldexpf(acc[m][0][r], -(sw + sx));
    }
}

// A weight slot's fragments on their way from the pack to an LDS buffer:
// loaded into registers before a layer runs, stored after the barrier that
// frees the buffer.
template <int F>
struct Prefetch {
    half8 h[Dims<F>::IT], l[Dims<F>::IT];
};

// (fragments 0..nf-1 of slot r go to buffer positions at..at+nf-1)
template <int F>
__device__ inline void prefetch_load(Prefetch<F> &p, const PackRef &r, int nf, int at = 0) {
#pragma unroll
    for (int it = 0; it < Dims<F>::IT; ++it) {
        const int idx = (int)threadIdx.x + it * kMlpThreads - at;
        if (idx >= 0 && idx < nf) {
            p.h[it] = static_cast<const half8 *>(r.hi)[idx];
            p.l[it] = static_cast<const half8 *>(r.lo)[idx];
        }
    }
}

template <int F>
__device__ inline void prefetch_store(const Prefetch<F> &p, half8 *dh, half8 *dl, int nf) {
#pragma unroll
    for (int it = 0; it < Dims<F>::IT; ++it) {
        const int idx = (int)threadIdx.x + it * kMlpThreads;
        if (idx < nf) {
            dh[idx] = p.h[it];
            dl[idx] = p.l[it];
        }
    }
}

enum Prog { P_EMBED_X = 0, P_OUT_X, P_TAIL, P_BX_BO };

struct ChainArgs {
    int N;
    const float *in;             // OUT_X, TAIL: y;  BX_BO: g_x
    const int32_t *types;        // EMBED_X
    const float *emb;
    int n_types;
    int *status;
    PackRef w[6];                // the chain's weight slots, in layer order
    const float *bo1, *bo2;      // OUT biases
    const float *c1, *R2, *c2;   // readout
    float *o;                    // OUT_X: o (stored)
    const float *o_prev;         // BX_BO: o of interaction t - 1
    const float *h_in;           // OUT_X, TAIL: h before this interaction's update
    float *h;                    // EMBED_X, OUT_X: h written
    float *x, *xmax;             // x_{t+1} and its row maxima
    float *eps;                  // TAIL
    float *gh;                   // TAIL: written; BX_BO: updated
    float *gy, *gmax;            // TAIL, BX_BO: g_y and its row maxima
};

template <int F, int PROG>
__global__ __launch_bounds__(kMlpThreads) void chain_kernel(ChainArgs a) {
    using D = Dims<F>;
    constexpr int M = D::M, MR = D::MR;
    __shared__ half8 s_ah[D::BUF], s_al[D::BUF], s_bh[D::BUF], s_bl[D::BUF];
    Wave w;
    w.lane = threadIdx.x % 64;
    w.slot = w.lane / 16;
    const int base = (blockIdx.x * kMlpWaves + threadIdx.x / 64) * 16;
    w.atom = base + w.lane % 16;
    w.live = w.atom < a.N;
    const bool active = base < a.N;   // the wavefront has atoms (all waves join the barriers)
    const int lane = w.lane;
    Prefetch<F> pf;

    if (PROG == P_EMBED_X) {
        copy_frags<D::BUF, kMlpThreads>(s_ah, s_al, static_cast<const half8 *>(a.w[0].hi),
                                        static_cast<const half8 *>(a.w[0].lo), D::LAYER);
        const int sw0 = a.w[0].sc[0];
        float h[M][4];
        if (active) {
            int z = w.live ? a.types[w.atom] : 0;
            if (z < 0 || z >= a.n_types) {
                if (w.slot == 0) flag_status(a.status, SN_ERR_INVALID);
                z = 0;
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const float4 q = *reinterpret_cast<const float4 *>(a.emb + (int64_t)z * F + 16 * m + 4 * w.slot);
                h[m][0] = q.x; h[m][1] = q.y; h[m][2] = q.z; h[m][3] = q.w;
            }
            store_rows<M>(a.h, F, w, h);
        }
        __syncthreads();
        if (!active) return;
        float x[M][4];
        layer<M, M>(h, s_ah, s_al, sw0, lane, x);
        store_rows<M>(a.x, F, w, x);
        const float mx = row_absmax(x);
        if (w.live && w.slot == 0) a.xmax[w.atom] = mx;
        return;
    }

    // the first two layers' weights; the first layer's input
    copy_frags<D::BUF, kMlpThreads>(s_ah, s_al, static_cast<const half8 *>(a.w[0].hi),
                                    static_cast<const half8 *>(a.w[0].lo), D::LAYER);
    copy_frags<D::BUF, kMlpThreads>(s_bh, s_bl, static_cast<const half8 *>(a.w[1].hi),
                                    static_cast<const half8 *>(a.w[1].lo), D::LAYER);
    const int sw0 = a.w[0].sc[0], sw1 = a.w[1].sc[0];
    float in[M][4];
    if (active) load_rows<M>(a.in, F, w, in);
    __syncthreads();

    if (PROG == P_OUT_X) {
        prefetch_load<F>(pf, a.w[2], D::LAYER);
        const int sw2 = a.w[2].sc[0];
        float o[M][4], z[M][4];
        if (active) {
            layer<M, M>(in, s_ah, s_al, sw0, lane, o);
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    o[m][r] += a.bo1[16 * m + 4 * w.slot + r];
                    z[m][r] = ssp(o[m][r]);
                }
            store_rows<M>(a.o, F, w, o);
        }
        __syncthreads();                                  // buffer A is free
        prefetch_store<F>(pf, s_ah, s_al, D::LAYER);
        float h[M][4];
        if (active) {
            float d[M][4];
            layer<M, M>(z, s_bh, s_bl, sw1, lane, d);
            load_rows<M>(a.h_in, F, w, h);
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) h[m][r] = h[m][r] + d[m][r] + a.bo2[16 * m + 4 * w.slot + r];
            store_rows<M>(a.h, F, w, h);
        }
        __syncthreads();                                  // W_in is in buffer A
        if (!active) return;
        float x[M][4];
        layer<M, M>(h, s_ah, s_al, sw2, lane, x);
        store_rows<M>(a.x, F, w, x);
        const float mx = row_absmax(x);
        if (w.live && w.slot == 0) a.xmax[w.atom] = mx;
        return;
    }

    if (PROG == P_TAIL) {
        // layers: Wo1 (A), Wo2 (B), R1 and R1^T (A), Wo2^T (B), Wo1^T (A)
        prefetch_load<F>(pf, a.w[2], D::R1F);
        prefetch_load<F>(pf, a.w[3], D::R2F, D::R1F);
        const int sw2 = a.w[2].sc[0], sw3 = a.w[3].sc[0], sw4 = a.w[4].sc[0], sw5 = a.w[5].sc[0];
        float o[M][4], z[M][4];
        if (active) {
            layer<M, M>(in, s_ah, s_al, sw0, lane, o);
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    o[m][r] += a.bo1[16 * m + 4 * w.slot + r];
                    z[m][r] = ssp(o[m][r]);
                }
        }
        __syncthreads();                                  // buffer A is free
        prefetch_store<F>(pf, s_ah, s_al, D::R1F + D::R2F);
        float h[M][4];
        if (active) {
            float d[M][4];
            layer<M, M>(z, s_bh, s_bl, sw1, lane, d);
            load_rows<M>(a.h_in, F, w, h);
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) h[m][r] = h[m][r] + d[m][r] + a.bo2[16 * m + 4 * w.slot + r];
        }
        prefetch_load<F>(pf, a.w[4], D::LAYER);
        __syncthreads();                                  // R1, R1^T in A; buffer B is free
        prefetch_store<F>(pf, s_bh, s_bl, D::LAYER);
        float gh[M][4];
        if (active) {
            float q[MR][4], zq[MR][4];
            layer<M, MR>(h, s_ah, s_al, sw2, lane, q);
            float eps_part = 0.0f;
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n0 = 16 * m + 4 * w.slot + r;
                    const float qq = q[m][r] + a.c1[n0];
                    eps_part += ssp(qq) * a.R2[n0];
                    zq[m][r] = sigm(qq) * a.R2[n0];
                }
            eps_part += __shfl_xor(eps_part, 16, 64);
            eps_part += __shfl_xor(eps_part, 32, 64);
            if (w.live && w.slot == 0) a.eps[w.atom] = eps_part + a.c2[0];
            layer<MR, M>(zq, s_ah + D::R1F, s_al + D::R1F, sw3, lane, gh);
            store_rows<M>(a.gh, F, w, gh);
        }
        prefetch_load<F>(pf, a.w[5], D::LAYER);
        __syncthreads();                                  // Wo2^T in B; buffer A is free
        prefetch_store<F>(pf, s_ah, s_al, D::LAYER);
        float go[M][4];
        if (active) {
            layer<M, M>(gh, s_bh, s_bl, sw4, lane, go);
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) go[m][r] *= sigm(o[m][r]);
        }
        __syncthreads();                                  // Wo1^T in A
        if (!active) return;
        float gy[M][4];
        layer<M, M>(go, s_ah, s_al, sw5, lane, gy);
        store_rows<M>(a.gy, F, w, gy);
        const float mx = row_absmax(gy);
        if (w.live && w.slot == 0) a.gmax[w.atom] = mx;
        return;
    }

    // P_BX_BO: layers W_in^T (A), Wo2^T (B), Wo1^T (A)
    prefetch_load<F>(pf, a.w[2], D::LAYER);
    const int sw2 = a.w[2].sc[0];
    float gh[M][4];
    if (active) {
        float d[M][4];
        layer<M, M>(in, s_ah, s_al, sw0, lane, d);
        load_rows<M>(a.gh, F, w, gh);
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) gh[m][r] += d[m][r];
        store_rows<M>(a.gh, F, w, gh);
    }
    __syncthreads();                                      // buffer A is free
    prefetch_store<F>(pf, s_ah, s_al, D::LAYER);
    float go[M][4];
    if (active) {
        float op[M][4];
        layer<M, M>(gh, s_bh, s_bl, sw1, lane, go);
        load_rows<M>(a.o_prev, F, w, op);
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) go[m][r] *= sigm(op[m][r]);
    }
    __syncthreads();                                      // Wo1^T in A
    if (!active) return;
    float gy[M][4];
    layer<M, M>(go, s_ah, s_al, sw2, lane, gy);
    store_rows<M>(a.gy, F, w, gy);
    const float mx = row_absmax(gy);
    if (w.live && w.slot == 0) a.gmax[w.atom] = mx;
}

// Pre-split one matrix into a weight-pack slot (as a block's staging would
// into LDS); returns the split scale.  TRANS: W is read transposed.
template <int F, int KDIM, int MDIM, int TRANS>
__device__ inline int pack_layer(const float *W, half8 *hi, half8 *lo, unsigned *s_max) {
    constexpr int T = (KDIM + 31) / 32, NF = (MDIM / 16) * T * 64;
    return stage_split<NF, kMlpThreads>(hi, lo, NF, s_max,
                                        [&](int idx, float (&v)[8]) { layer_frag<T, TRANS>(W, KDIM, MDIM, idx, v); });
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
        sc = b == 6 * pa.I ? pack_layer<F, F, F / 2, 0>(pa.R1, hi, lo, &s_max)     // q = h R1
                           : pack_layer<F, F / 2, F, 1>(pa.R1, hi, lo, &s_max);    // g_h = g_q R1^T
    } else {
        switch (PK_XW + k) {
            case PK_XW: sc = pack_layer<F, F, F, 0>(pa.W_in[t], hi, lo, &s_max); break;
            case PK_OW1: sc = pack_layer<F, F, F, 0>(pa.Wo1[t], hi, lo, &s_max); break;
            case PK_OW2: sc = pack_layer<F, F, F, 0>(pa.Wo2[t], hi, lo, &s_max); break;
            case PK_BOW1: sc = pack_layer<F, F, F, 1>(pa.Wo2[t], hi, lo, &s_max); break;
            case PK_BOW2: sc = pack_layer<F, F, F, 1>(pa.Wo1[t], hi, lo, &s_max); break;
            default: sc = pack_layer<F, F, F, 1>(pa.W_in[t], hi, lo, &s_max); break;
        }
    }
    if (threadIdx.x == 0) const_cast<int *>(r.sc)[0] = sc;
}

template <int PROG>
sn_status launch_chain(int F, const ChainArgs &a, hipStream_t s) {
    if (a.N <= 0) return SN_OK;
    ProfScope ps(K_MLP, s);
    const int atoms_per_block = 16 * kMlpWaves;
    const int grid = (a.N + atoms_per_block - 1) / atoms_per_block;
    switch (F) {
        case 32: chain_kernel<32, PROG><<<grid, kMlpThreads, 0, s>>>(a); break;
        case 64: chain_kernel<64, PROG><<<grid, kMlpThreads, 0, s>>>(a); break;
        case 128: chain_kernel<128, PROG><<<grid, kMlpThreads, 0, s>>>(a); break;
        default: return SN_ERR_INVALID;
    }
    return launch_status();
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

sn_status mlp_embed_x(int N, int F, int T, const int32_t *types, const float *emb, PackRef W_in, float *h, float *x,
                      float *xmax, int *status, hipStream_t s) {
    ChainArgs a = {};
    a.N = N; a.types = types; a.emb = emb; a.n_types = T; a.status = status;
    a.w[0] = W_in;
    a.h = h; a.x = x; a.xmax = xmax;
    return launch_chain<P_EMBED_X>(F, a, s);
}

sn_status mlp_out_x(int N, int F, const float *y, PackRef Wo1, const float *bo1, PackRef Wo2, const float *bo2,
                    PackRef W_in, float *o, const float *h_in, float *h, float *x, float *xmax, hipStream_t s) {
    ChainArgs a = {};
    a.N = N; a.in = y; a.bo1 = bo1; a.bo2 = bo2;
    a.w[0] = Wo1; a.w[1] = Wo2; a.w[2] = W_in;
    a.o = o; a.h_in = h_in; a.h = h; a.x = x; a.xmax = xmax;
    return launch_chain<P_OUT_X>(F, a, s);
}

sn_status mlp_tail(int N, int F, const float *y, PackRef Wo1, const float *bo1, PackRef Wo2, const float *bo2,
                   const float *h, PackRef R1, const float *c1, PackRef R1t, const float *R2, const float *c2,
                   PackRef Wo2t, PackRef Wo1t, float *eps, float *gh, float *gy, float *gymax, hipStream_t s) {
    ChainArgs a = {};
    a.N = N; a.in = y; a.bo1 = bo1; a.bo2 = bo2; a.c1 = c1; a.R2 = R2; a.c2 = c2;
    a.w[0] = Wo1; a.w[1] = Wo2; a.w[2] = R1; a.w[3] = R1t; a.w[4] = Wo2t; a.w[5] = Wo1t;
    a.h_in = h; a.eps = eps; a.gh = gh; a.gy = gy; a.gmax = gymax;
    return launch_chain<P_TAIL>(F, a, s);
}

sn_status mlp_bx_bo(int N, int F, const float *gx, PackRef W_int, PackRef Wo2t, const float *o_prev, PackRef Wo1t,
                    float *gh, float *gy, float *gymax, hipStream_t s) {
    ChainArgs a = {};
    a.N = N; a.in = gx; a.o_prev = o_prev;
    a.w[0] = W_int; a.w[1] = Wo2t; a.w[2] = Wo1t;
    a.gh = gh; a.gy = gy; a.gmax = gymax;
    return launch_chain<P_BX_BO>(F, a, s);
}

}  // namespace sn
