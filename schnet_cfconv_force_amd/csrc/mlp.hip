// Atom-wise layers of the interaction blocks and the readout, fused per
// chain of layers and run on the matrix cores.
//
// Computed transposed (output features are the M dimension, atoms the N
// dimension of v_mfma_f32_16x16x32_f16), with operands in the split-fp16
// form of split_mfma.h.  Every layer's weights sit in the weight pack in
// the accumulator-chained order, so a layer's output, as an accumulator
// leaves it (lane = atom l%16, features 16 m + 4 (l/16) + r), is already
// laid out as the next layer's B operand; rows load with one float4 per
// tile.  Each atom's operands are scaled by a power of two from the atom's
// own maximum.
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
// scales).  How a block divides a layer among its wavefronts and passes
// operands between layers is described at kMlpWaves below.
#include "split_mfma.h"

namespace sn {

namespace {

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

// Blocks of eight wavefronts (two per SIMD) take NA tiles of 16 atoms
// (NA = 1..5, from the system size, so that small systems still spread over
// many compute units).  In every layer the output tiles of 16 features are
// split over the wavefronts (over four groups, the other factor of two over
// the atom tiles; over all eight when the block has one atom tile): a
// wavefront loads only its own weight fragments, from the pack straight
// into registers, and applies each to all of its atom tiles.  A layer's
// output becomes the next layer's B operands through LDS: each wavefront
// publishes per-atom partial maxima, takes every atom's scale from all of
// them, and writes its part of the split operands; the next layer reads each
// atom tile's operands.  Barriers synchronise LDS only, so weight loads for
// the next layer and row stores stay in flight across them.
constexpr int kMlpWaves = 8;
constexpr int kMlpThreads = 64 * kMlpWaves;
constexpr int kMlpMaxTiles = 5;

template <int F>
struct Dims {
    static constexpr int M = F / 16;                 // 16-feature tiles of a row
    static constexpr int MR = F / 32;                // tiles of the readout's hidden layer (F / 2)
    static constexpr int T = (F + 31) / 32;          // 32-wide k steps over F inputs
    static constexpr int TR = (F / 2 + 31) / 32;     // ... over F / 2 inputs
};

// A layer with MO output tiles: WM wavefront groups along the features, WA
// along the atom tiles.  Wavefront w owns the output tiles NI (w % WM) + i,
// i < NI, of the atom tiles w / WM + WA k, k < NK.
template <int MO, int NA>
struct Units {
    static constexpr int WMAX = NA == 1 ? kMlpWaves : kMlpWaves / 2;
    static constexpr int WM = MO < WMAX ? MO : WMAX;
    static constexpr int WA = kMlpWaves / WM;
    static constexpr int NI = MO / WM;
    static constexpr int NK = (NA + WA - 1) / WA;
    static_assert(MO % WM == 0 && kMlpWaves % WM == 0, "output tiles: a power of two");
};

// The wavefront's view of its block.
struct Blk {
    int lane, slot, w;   // lane, its k-slot (lane / 16), wavefront
    int tile0, nt;       // the block's first atom tile, and its number of tiles
    int N;
    __device__ int atom(int a) const { return (tile0 + a) * 16 + lane % 16; }
};

template <int MO, int NA>
__device__ inline int unit_m(const Blk &b, int i) { return Units<MO, NA>::NI * (b.w % Units<MO, NA>::WM) + i; }
template <int MO, int NA>
__device__ inline int unit_a(const Blk &b, int k) { return b.w / Units<MO, NA>::WM + Units<MO, NA>::WA * k; }

// value v[i][k][r]: output tile unit_m(i), atom lane % 16 of tile unit_a(k),
// feature 16 unit_m(i) + 4 slot + r
template <int MO, int NA>
using Vals = float[Units<MO, NA>::NI][Units<MO, NA>::NK][4];
template <int MO, int NA>
using Accs = floatx4[Units<MO, NA>::NI][Units<MO, NA>::NK];

template <int F, int NA>
struct ChainSmem {
    half8 bh[2][NA * Dims<F>::T * 64];   // split B operands [buffer][(tile T + t) 64 + lane]
    half8 bl[2][NA * Dims<F>::T * 64];
    float pmax[NA * 16][kMlpWaves];      // per-atom partial maxima of the wavefront groups
    float psum[NA * 16][kMlpWaves];      // per-atom partial readout sums
    int sx[NA * 16];                     // per-atom split exponents of the published operands
    float bias[2][F];                    // OUT biases bo1, bo2
    float rc1[F / 2], rr2[F / 2];        // readout c1, R2
    float rc2;                           // readout c2
    int sc[6];                           // split scales of the chain's layers
};

// A bias's four features 16 m + 4 slot .. + 3 of the lane.
template <int F, int NA>
__device__ inline float4 bias4(const ChainSmem<F, NA> &sm, int which, int m, int slot) {
    return *reinterpret_cast<const float4 *>(&sm.bias[which][16 * m + 4 * slot]);
}

// LDS-only block barrier: pending LDS operations complete first; global
// loads and stores stay in flight.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// the atom's largest magnitude over its four k-slot lanes
__device__ inline float atom_max(float amax) {
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    return fmaxf(amax, __shfl_xor(amax, 32, 64));
}

template <int F, int MO, int NA>
__device__ inline void load_vals(const float *src, const Blk &b, Vals<MO, NA> &v) {
    using U = Units<MO, NA>;
#pragma unroll
    for (int k = 0; k < U::NK; ++k) {
        const int at = unit_a<MO, NA>(b, k);
        const bool live = at < b.nt && b.atom(at) < b.N;
#pragma unroll
        for (int i = 0; i < U::NI; ++i) {
            float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
            if (live)
                q = *reinterpret_cast<const float4 *>(src + (int64_t)b.atom(at) * F + 16 * unit_m<MO, NA>(b, i) +
                                                      4 * b.slot);
            v[i][k][0] = q.x; v[i][k][1] = q.y; v[i][k][2] = q.z; v[i][k][3] = q.w;
        }
    }
}

template <int F, int MO, int NA>
__device__ inline void store_vals(float *dst, const Blk &b, const Vals<MO, NA> &v) {
    using U = Units<MO, NA>;
#pragma unroll
    for (int k = 0; k < U::NK; ++k) {
        const int at = unit_a<MO, NA>(b, k);
        if (at < b.nt && b.atom(at) < b.N)
#pragma unroll
            for (int i = 0; i < U::NI; ++i)
                *reinterpret_cast<float4 *>(dst + (int64_t)b.atom(at) * F + 16 * unit_m<MO, NA>(b, i) + 4 * b.slot) =
                    make_float4(v[i][k][0], v[i][k][1], v[i][k][2], v[i][k][3]);
    }
}

// Per-atom partial maxima of |v| into pmax (lanes of k-slot 0 write).
template <int F, int MO, int NA>
__device__ inline void partial_max(ChainSmem<F, NA> &sm, const Blk &b, const Vals<MO, NA> &v) {
    using U = Units<MO, NA>;
#pragma unroll
    for (int k = 0; k < U::NK; ++k) {
        const int at = unit_a<MO, NA>(b, k);
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < U::NI; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(v[i][k][r]));
        mx = atom_max(mx);
        if (at < b.nt && b.slot == 0) sm.pmax[at * 16 + b.lane][b.w % U::WM] = mx;
    }
}

// Publish v (a layer's output, MO tiles) as the next layer's B operands in
// buffer buf, each atom scaled by 2^sx from its largest magnitude over all
// MO tiles (sx goes to sm.sx for the next layer's unscaling).  A k-step with
// only one 16-feature tile gets zeros in its other half.  Holds two block
// barriers; sm.sx is written between them, after every wavefront has
// unscaled with the previous exponents.
template <int F, int MO, int NA>
__device__ inline void publish(ChainSmem<F, NA> &sm, int buf, const Blk &b, const Vals<MO, NA> &v) {
    using U = Units<MO, NA>;
    constexpr int T = Dims<F>::T;
    partial_max<F, MO, NA>(sm, b, v);
    lds_barrier();
#pragma unroll
    for (int k = 0; k < U::NK; ++k) {
        const int at = unit_a<MO, NA>(b, k);
        if (at >= b.nt) continue;
        float mx = 0.0f;
#pragma unroll
        for (int g = 0; g < U::WM; ++g) mx = fmaxf(mx, sm.pmax[at * 16 + b.lane % 16][g]);
        const int s = split_scale(mx);
        if (b.w % U::WM == 0 && b.slot == 0) sm.sx[at * 16 + b.lane] = s;
        if (U::NI % 2 == 0) {
#pragma unroll
            for (int i = 0; i < U::NI; i += 2) {
                float x[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = ldexpf(v[i + j / 4][k][j % 4], s);
                half8 hi, lo;
                split8(x, hi, lo);
                const int idx = (at * T + unit_m<MO, NA>(b, i) / 2) * 64 + b.lane;
                sm.bh[buf][idx] = hi;
                sm.bl[buf][idx] = lo;
            }
        } else {
            const int m = unit_m<MO, NA>(b, 0);
            float x[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = ldexpf(v[0][k][j], s);
            half4 hi, lo;
            split4(x, hi, lo);
            const int idx = (at * T + m / 2) * 64 + b.lane;
            reinterpret_cast<half4 *>(&sm.bh[buf][idx])[m % 2] = hi;
            reinterpret_cast<half4 *>(&sm.bl[buf][idx])[m % 2] = lo;
            if (MO % 2 == 1 && m == MO - 1) {
                const half4 z = {0, 0, 0, 0};
                reinterpret_cast<half4 *>(&sm.bh[buf][idx])[1] = z;
                reinterpret_cast<half4 *>(&sm.bl[buf][idx])[1] = z;
            }
        }
    }
    lds_barrier();
}

// The wavefront's weight fragments of a layer (MO output tiles, TIN k
// steps; [m][t][l] in the pack).
template <int MO, int TIN, int NA>
struct AFrag {
    half8 h[Units<MO, NA>::NI][TIN], l[Units<MO, NA>::NI][TIN];
};

template <int MO, int TIN, int NA>
__device__ inline void load_a(const PackRef &W, const Blk &b, AFrag<MO, TIN, NA> &A) {
    const half8 *wh = static_cast<const half8 *>(W.hi), *wl = static_cast<const half8 *>(W.lo);
#pragma unroll
    for (int i = 0; i < Units<MO, NA>::NI; ++i)
#pragma unroll
        for (int t = 0; t < TIN; ++t) {
            const int idx = (unit_m<MO, NA>(b, i) * TIN + t) * 64 + b.lane;
            A.h[i][t] = wh[idx];
            A.l[i][t] = wl[idx];
        }
}

// acc = B W for the wavefront's units, B from buffer buf; per accumulator
// the products run hi.hi, hi.lo, lo.hi per k step, in k order.  Tiles past
// the block's last are computed too (their columns are never used).
template <int F, int MO, int TIN, int NA>
__device__ inline void layer_mma(const ChainSmem<F, NA> &sm, int buf, const Blk &b, const AFrag<MO, TIN, NA> &A,
                                 Accs<MO, NA> &acc) {
    using U = Units<MO, NA>;
    constexpr int T = Dims<F>::T;
#pragma unroll
    for (int i = 0; i < U::NI; ++i)
#pragma unroll
        for (int k = 0; k < U::NK; ++k) acc[i][k] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < TIN; ++t) {
        half8 bh[U::NK], bl[U::NK];
#pragma unroll
        for (int k = 0; k < U::NK; ++k) {
            const int at = min(unit_a<MO, NA>(b, k), NA - 1);
            bh[k] = sm.bh[buf][(at * T + t) * 64 + b.lane];
            bl[k] = sm.bl[buf][(at * T + t) * 64 + b.lane];
        }
#pragma unroll
        for (int i = 0; i < U::NI; ++i)
#pragma unroll
            for (int k = 0; k < U::NK; ++k)
                acc[i][k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A.h[i][t], bh[k], acc[i][k], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < U::NI; ++i)
#pragma unroll
            for (int k = 0; k < U::NK; ++k)
                acc[i][k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A.h[i][t], bl[k], acc[i][k], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < U::NI; ++i)
#pragma unroll
            for (int k = 0; k < U::NK; ++k)
                acc[i][k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A.l[i][t], bh[k], acc[i][k], 0, 0, 0);
    }
}

// out = acc 2^-(sw + sx) (the layer's unscaled output; sx of the layer's
// input, from sm.sx)
template <int F, int MO, int NA>
__device__ inline void unscale(const ChainSmem<F, NA> &sm, const Accs<MO, NA> &acc, int sw, const Blk &b,
                               Vals<MO, NA> &out) {
    using U = Units<MO, NA>;
#pragma unroll
    for (int k = 0; k < U::NK; ++k) {
        const int at = min(unit_a<MO, NA>(b, k), NA - 1);
        const int e = -(sw + sm.sx[at * 16 + b.lane % 16]);
#pragma unroll
        for (int i = 0; i < U::NI; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) out[i][k][r] = ldexpf(acc[i][k][r], e);
    }
}

// dst[atom] = max_f |v[atom][f]| (after a block barrier)
template <int F, int MO, int NA>
__device__ inline void store_row_max(ChainSmem<F, NA> &sm, const Blk &b, const Vals<MO, NA> &v, float *dst) {
    partial_max<F, MO, NA>(sm, b, v);
    lds_barrier();
    if (b.w == 0 && b.lane < 16)
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            float mx = 0.0f;
#pragma unroll
            for (int g = 0; g < Units<MO, NA>::WM; ++g) mx = fmaxf(mx, sm.pmax[a * 16 + b.lane][g]);
            if (a < b.nt && b.atom(a) < b.N) dst[b.atom(a)] = mx;
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

// The chain's small constants (biases, readout vectors, layer scales) go
// to LDS at the start, so that no layer waits on a global load of them: each
// thread loads its share into registers before the chain's row loads issue,
// and writes it to LDS after they have (the first publish's barriers make
// it visible).  Loads issued together overlap; a load and its LDS write in
// sequence would cost one round trip each.
struct ChainConsts {
    float b0, b1, c1, r2, c2;
    int sc;
};
template <int F>
__device__ inline ChainConsts load_consts(const ChainArgs &a) {
    ChainConsts c = {0.f, 0.f, 0.f, 0.f, 0.f, 0};
    const int f = threadIdx.x;   // F <= 128: threads 0..F-1 take a feature each
    if (f < F) {
        if (a.bo1) c.b0 = a.bo1[f];
        if (a.bo2) c.b1 = a.bo2[f];
        if (a.c1 && f < F / 2) {
            c.c1 = a.c1[f];
            c.r2 = a.R2[f];
        }
    }
    if (a.c2 && f == 255) c.c2 = a.c2[0];
    const int k = f - 256;      // threads 256..261: the six layer scales
    if (k >= 0 && k < 6) {
        const int *p = k == 0 ? a.w[0].sc : k == 1 ? a.w[1].sc : k == 2 ? a.w[2].sc
                     : k == 3 ? a.w[3].sc : k == 4 ? a.w[4].sc : a.w[5].sc;
        if (p) c.sc = *p;
    }
    return c;
}
template <int F, int NA>
__device__ inline void store_consts(ChainSmem<F, NA> &sm, const ChainArgs &a, const ChainConsts &c) {
    const int f = threadIdx.x;
    if (f < F) {
        sm.bias[0][f] = c.b0;
        sm.bias[1][f] = c.b1;
        if (f < F / 2) {
            sm.rc1[f] = c.c1;
            sm.rr2[f] = c.r2;
        }
    }
    if (f == 255) sm.rc2 = c.c2;
    if (f >= 256 && f < 262) sm.sc[f - 256] = c.sc;
}

template <int F, int PROG, int NA>
__global__ __launch_bounds__(kMlpThreads) void chain_kernel(ChainArgs a) {
    using D = Dims<F>;
    constexpr int M = D::M, MR = D::MR, T = D::T, TR = D::TR;
    using U = Units<M, NA>;
    __shared__ ChainSmem<F, NA> sm;
    Blk b;
    b.lane = threadIdx.x % 64;
    b.slot = b.lane / 16;
    b.w = threadIdx.x / 64;
    b.tile0 = blockIdx.x * NA;
    b.nt = min(NA, (a.N + 15) / 16 - b.tile0);
    b.N = a.N;
    Accs<M, NA> acc;
    const ChainConsts cst = load_consts<F>(a);

    if (PROG == P_EMBED_X) {
        AFrag<M, T, NA> A0;
        load_a<M, T, NA>(a.w[0], b, A0);
        Vals<M, NA> h;
#pragma unroll
        for (int k = 0; k < U::NK; ++k) {
            const int at = unit_a<M, NA>(b, k);
            const bool live = at < b.nt && b.atom(at) < b.N;
            int z = live ? a.types[b.atom(at)] : 0;
            if (z < 0 || z >= a.n_types) {
                flag_status(a.status, SN_ERR_INVALID);
                z = 0;
            }
#pragma unroll
            for (int i = 0; i < U::NI; ++i) {
                const float4 q = *reinterpret_cast<const float4 *>(a.emb + (int64_t)z * F + 16 * unit_m<M, NA>(b, i) +
                                                                   4 * b.slot);
                h[i][k][0] = q.x; h[i][k][1] = q.y; h[i][k][2] = q.z; h[i][k][3] = q.w;
            }
        }
        store_vals<F, M, NA>(a.h, b, h);
        store_consts<F, NA>(sm, a, cst);
        publish<F, M, NA>(sm, 0, b, h);
        layer_mma<F, M, T, NA>(sm, 0, b, A0, acc);
        Vals<M, NA> x;
        unscale<F, M, NA>(sm, acc, sm.sc[0], b, x);
        store_vals<F, M, NA>(a.x, b, x);
        store_row_max<F, M, NA>(sm, b, x, a.xmax);
        return;
    }

    if (PROG == P_OUT_X) {
        // layers: Wo1, Wo2, W_in of the next interaction
        AFrag<M, T, NA> A;
        load_a<M, T, NA>(a.w[0], b, A);
        Vals<M, NA> v, hin;   // every row load is issued up front
        load_vals<F, M, NA>(a.in, b, v);
        load_vals<F, M, NA>(a.h_in, b, hin);
        store_consts<F, NA>(sm, a, cst);
        publish<F, M, NA>(sm, 0, b, v);
        layer_mma<F, M, T, NA>(sm, 0, b, A, acc);
        load_a<M, T, NA>(a.w[1], b, A);
        {
            Vals<M, NA> o;
            unscale<F, M, NA>(sm, acc, sm.sc[0], b, o);
#pragma unroll
            for (int i = 0; i < U::NI; ++i) {
                const float4 c = bias4(sm, 0, unit_m<M, NA>(b, i), b.slot);
#pragma unroll
                for (int k = 0; k < U::NK; ++k) {
                    o[i][k][0] += c.x; o[i][k][1] += c.y; o[i][k][2] += c.z; o[i][k][3] += c.w;
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[i][k][r] = ssp(o[i][k][r]);
                }
            }
            store_vals<F, M, NA>(a.o, b, o);
        }
        publish<F, M, NA>(sm, 1, b, v);
        layer_mma<F, M, T, NA>(sm, 1, b, A, acc);
        load_a<M, T, NA>(a.w[2], b, A);
        {
            Vals<M, NA> d;
            unscale<F, M, NA>(sm, acc, sm.sc[1], b, d);
#pragma unroll
            for (int i = 0; i < U::NI; ++i) {
                const float4 c = bias4(sm, 1, unit_m<M, NA>(b, i), b.slot);
                const float cb[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
                for (int k = 0; k < U::NK; ++k)
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[i][k][r] = hin[i][k][r] + d[i][k][r] + cb[r];
            }
            store_vals<F, M, NA>(a.h, b, v);
        }
        publish<F, M, NA>(sm, 0, b, v);
        layer_mma<F, M, T, NA>(sm, 0, b, A, acc);
        unscale<F, M, NA>(sm, acc, sm.sc[2], b, v);
        store_vals<F, M, NA>(a.x, b, v);
        store_row_max<F, M, NA>(sm, b, v, a.xmax);
        return;
    }

    if (PROG == P_TAIL) {
        // layers: Wo1, Wo2, R1, R1^T, Wo2^T, Wo1^T
        using UR = Units<MR, NA>;
        AFrag<M, T, NA> A;
        load_a<M, T, NA>(a.w[0], b, A);
        Vals<M, NA> v, o, hin;   // every row load is issued up front
        load_vals<F, M, NA>(a.in, b, v);
        load_vals<F, M, NA>(a.h_in, b, hin);
        store_consts<F, NA>(sm, a, cst);
        publish<F, M, NA>(sm, 0, b, v);
        layer_mma<F, M, T, NA>(sm, 0, b, A, acc);
        load_a<M, T, NA>(a.w[1], b, A);
        unscale<F, M, NA>(sm, acc, sm.sc[0], b, o);
#pragma unroll
        for (int i = 0; i < U::NI; ++i) {
            const float4 c = bias4(sm, 0, unit_m<M, NA>(b, i), b.slot);
#pragma unroll
            for (int k = 0; k < U::NK; ++k) {
                o[i][k][0] += c.x; o[i][k][1] += c.y; o[i][k][2] += c.z; o[i][k][3] += c.w;
#pragma unroll
                for (int r = 0; r < 4; ++r) v[i][k][r] = ssp(o[i][k][r]);
            }
        }
        publish<F, M, NA>(sm, 1, b, v);
        layer_mma<F, M, T, NA>(sm, 1, b, A, acc);
        AFrag<MR, T, NA> AR;
        load_a<MR, T, NA>(a.w[2], b, AR);
        {
            Vals<M, NA> d;
            unscale<F, M, NA>(sm, acc, sm.sc[1], b, d);
#pragma unroll
            for (int i = 0; i < U::NI; ++i) {
                const float4 c = bias4(sm, 1, unit_m<M, NA>(b, i), b.slot);
                const float cb[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
                for (int k = 0; k < U::NK; ++k)
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[i][k][r] = hin[i][k][r] + d[i][k][r] + cb[r];
            }
        }
        publish<F, M, NA>(sm, 0, b, v);
        {
            // readout: q = h R1 + c1; eps = ssp(q) . R2 + c2; its gradient
            // sigmoid(q) (.) R2 goes on through R1^T
            Accs<MR, NA> accr;
            layer_mma<F, MR, T, NA>(sm, 0, b, AR, accr);
            AFrag<M, TR, NA> AT;
            load_a<M, TR, NA>(a.w[3], b, AT);
            Vals<MR, NA> q;
            unscale<F, MR, NA>(sm, accr, sm.sc[2], b, q);
#pragma unroll
            for (int k = 0; k < UR::NK; ++k) {
                const int at = unit_a<MR, NA>(b, k);
                float e = 0.0f;
#pragma unroll
                for (int i = 0; i < UR::NI; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int n0 = 16 * unit_m<MR, NA>(b, i) + 4 * b.slot + r;
                        const float qq = q[i][k][r] + sm.rc1[n0];
                        e += ssp(qq) * sm.rr2[n0];
                        q[i][k][r] = sigm(qq) * sm.rr2[n0];
                    }
                e += __shfl_xor(e, 16, 64);
                e += __shfl_xor(e, 32, 64);
                if (at < b.nt && b.slot == 0) sm.psum[at * 16 + b.lane][b.w % UR::WM] = e;
            }
            publish<F, MR, NA>(sm, 1, b, q);   // its barriers also order the partial sums
            if (b.w == 0 && b.lane < 16)
#pragma unroll
                for (int at = 0; at < NA; ++at) {
                    float e = sm.psum[at * 16 + b.lane][0];
#pragma unroll
                    for (int g = 1; g < UR::WM; ++g) e += sm.psum[at * 16 + b.lane][g];
                    if (at < b.nt && b.atom(at) < b.N) a.eps[b.atom(at)] = e + sm.rc2;
                }
            layer_mma<F, M, TR, NA>(sm, 1, b, AT, acc);
        }
        load_a<M, T, NA>(a.w[4], b, A);
        unscale<F, M, NA>(sm, acc, sm.sc[3], b, v);
        store_vals<F, M, NA>(a.gh, b, v);
        publish<F, M, NA>(sm, 0, b, v);
        layer_mma<F, M, T, NA>(sm, 0, b, A, acc);
        load_a<M, T, NA>(a.w[5], b, A);
        unscale<F, M, NA>(sm, acc, sm.sc[4], b, v);
#pragma unroll
        for (int i = 0; i < U::NI; ++i)
#pragma unroll
            for (int k = 0; k < U::NK; ++k)
#pragma unroll
                for (int r = 0; r < 4; ++r) v[i][k][r] *= sigm(o[i][k][r]);
        publish<F, M, NA>(sm, 1, b, v);
        layer_mma<F, M, T, NA>(sm, 1, b, A, acc);
        unscale<F, M, NA>(sm, acc, sm.sc[5], b, v);
        store_vals<F, M, NA>(a.gy, b, v);
        store_row_max<F, M, NA>(sm, b, v, a.gmax);
        return;
    }

    // P_BX_BO: layers W_in^T, Wo2^T, Wo1^T
    AFrag<M, T, NA> A;
    load_a<M, T, NA>(a.w[0], b, A);
    Vals<M, NA> v, gh, op;   // every row load is issued up front
    load_vals<F, M, NA>(a.in, b, v);
    load_vals<F, M, NA>(a.gh, b, gh);
    load_vals<F, M, NA>(a.o_prev, b, op);
    store_consts<F, NA>(sm, a, cst);
    publish<F, M, NA>(sm, 0, b, v);
    layer_mma<F, M, T, NA>(sm, 0, b, A, acc);
    load_a<M, T, NA>(a.w[1], b, A);
    {
        Vals<M, NA> d;
        unscale<F, M, NA>(sm, acc, sm.sc[0], b, d);
#pragma unroll
        for (int i = 0; i < U::NI; ++i)
#pragma unroll
            for (int k = 0; k < U::NK; ++k)
#pragma unroll
                for (int r = 0; r < 4; ++r) v[i][k][r] = gh[i][k][r] + d[i][k][r];
        store_vals<F, M, NA>(a.gh, b, v);
    }
    publish<F, M, NA>(sm, 1, b, v);
    layer_mma<F, M, T, NA>(sm, 1, b, A, acc);
    load_a<M, T, NA>(a.w[2], b, A);
    {
        unscale<F, M, NA>(sm, acc, sm.sc[1], b, v);
#pragma unroll
        for (int i = 0; i < U::NI; ++i)
#pragma unroll
            for (int k = 0; k < U::NK; ++k)
#pragma unroll
                for (int r = 0; r < 4; ++r) v[i][k][r] *= sigm(op[i][k][r]);
    }
    publish<F, M, NA>(sm, 0, b, v);
    layer_mma<F, M, T, NA>(sm, 0, b, A, acc);
    unscale<F, M, NA>(sm, acc, sm.sc[2], b, v);
    store_vals<F, M, NA>(a.gy, b, v);
    store_row_max<F, M, NA>(sm, b, v, a.gmax);
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

template <int PROG, int NA>
void launch_na(int F, int grid, const ChainArgs &a, hipStream_t s) {
    switch (F) {
        case 32: chain_kernel<32, PROG, NA><<<grid, kMlpThreads, 0, s>>>(a); break;
        case 64: chain_kernel<64, PROG, NA><<<grid, kMlpThreads, 0, s>>>(a); break;
        default: chain_kernel<128, PROG, NA><<<grid, kMlpThreads, 0, s>>>(a); break;
    }
}

// Atom tiles per block: as few as fill the compute units once.
template <int PROG>
sn_status launch_chain(int F, const ChainArgs &a, hipStream_t s) {
    if (a.N <= 0) return SN_OK;
    if (F != 32 && F != 64 && F != 128) return SN_ERR_INVALID;
    ProfScope ps(K_MLP, s);
    const int tiles = (a.N + 15) / 16, cus = num_cus();
    const int na = std::min(kMlpMaxTiles, std::max(1, (tiles + cus - 1) / cus));
    const int grid = (tiles + na - 1) / na;
    switch (na) {
        case 1: launch_na<PROG, 1>(F, grid, a, s); break;
        case 2: launch_na<PROG, 2>(F, grid, a, s); break;
        case 3: launch_na<PROG, 3>(F, grid, a, s); break;
        case 4: launch_na<PROG, 4>(F, grid, a, s); break;
        default: launch_na<PROG, 5>(F, grid, a, s); break;
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
