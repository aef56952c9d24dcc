// Internal declarations shared by the translation units of libsn.so.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/sn.h"

namespace sn {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// --------------------------------------------------------------- status

// Device status words at the head of the workspace (int32, the first 256
// bytes): the first error code (0 = none), the longest row and the edge
// total of the last neighbour build, the pair count of the last pair setup,
// the MD steps completed, and the state of device-driven MD steps.
enum StatusSlot {
    kStatusWord = 0, kMaxRow = 1, kEdgeTotal = 2, kPairTotal = 3,
    kStepsDone = 4,    // MD: index of the last step that began with no error flagged
    // device-driven MD steps (a rebuild interval or a replayed graph): the
    // launches of every step are identical and these words carry what varies
    kMdStep = 5,       // steps begun in this call (the current step's index + 1)
    kBuildFlag = 6,    // 1: the current step rebuilds the neighbour list
    kDisplaced = 7,    // set when an atom drifted beyond half the skin since the last build
    kLastBuild = 8,    // index of the step that last rebuilt the list
    kStatusSlots = 64
};

#define SN_TRY(expr)                               \
    do {                                           \
        sn_status _st = (expr);                    \
        if (_st != SN_OK) return _st;              \
    } while (0)

#define SN_HIP(expr)                               \
    do {                                           \
        if ((expr) != hipSuccess) return SN_ERR_HIP; \
    } while (0)

inline sn_status launch_status() {
    return hipGetLastError() == hipSuccess ? SN_OK : SN_ERR_HIP;
}

// Record the first error code in the device status word.
__device__ inline void flag_status(int *status, int code) { atomicCAS(status, 0, code); }

// --------------------------------------------------------------- math

// exp and log on the hardware exp2/log2 units (about 1 ulp on their own;
// the scaling by log2(e) or ln 2 adds one rounding).
__device__ inline float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ inline float fast_log(float x) { return __builtin_amdgcn_logf(x) * 0.69314718055994531f; }

// Shifted softplus ln(e^x/2 + 1/2) = max(x,0) + ln(1 + exp(-|x|)) - ln 2.
__device__ inline float ssp(float x) {
    return fmaxf(x, 0.0f) + fast_log(1.0f + fast_exp(-fabsf(x))) - 0.69314718055994531f;
}
// Its derivative, the logistic sigmoid.
__device__ inline float sigm(float x) { return __builtin_amdgcn_rcpf(1.0f + fast_exp(-x)); }

// --------------------------------------------------------------- filter-row storage

// The filter rows that the pipeline keeps in HBM between its kernels are
// stored in a 24-bit float: an fp32 value rounded to its upper three bytes
// (sign, exponent, 15 mantissa bits; the magnitude rounded half up), so the
// relative error of a stored value is at most 2^-16.  Four consecutive
// features pack into three 32-bit words.
struct Packed4 {
    uint32_t w0, w1, w2;
};
__device__ inline Packed4 pack_fp24(float a, float b, float c, float d) {
    // adding half of the dropped byte's weight to the bit pattern rounds the
    // magnitude (a carry runs into the exponent as it should)
    const uint32_t r0 = __float_as_uint(a) + 0x80u, r1 = __float_as_uint(b) + 0x80u;
    const uint32_t r2 = __float_as_uint(c) + 0x80u, r3 = __float_as_uint(d) + 0x80u;
    // v_perm_b32 selector: byte k of the result = byte sel_k of {src0 : src1}
    // (src1 bytes 0-3, src0 bytes 4-7)
    Packed4 p;
    p.w0 = __builtin_amdgcn_perm(r1, r0, 0x05030201u);   // r0.b1 r0.b2 r0.b3 r1.b1
    p.w1 = __builtin_amdgcn_perm(r2, r1, 0x06050302u);   // r1.b2 r1.b3 r2.b1 r2.b2
    p.w2 = __builtin_amdgcn_perm(r3, r2, 0x07060503u);   // r2.b3 r3.b1 r3.b2 r3.b3
    return p;
}
__device__ inline float4 unpack_fp24(uint32_t w0, uint32_t w1, uint32_t w2) {
    // selector byte 0x0c gives a zero byte
    return make_float4(__uint_as_float(__builtin_amdgcn_perm(w1, w0, 0x0201000cu)),
                       __uint_as_float(__builtin_amdgcn_perm(w1, w0, 0x0504030cu)),
                       __uint_as_float(__builtin_amdgcn_perm(w2, w1, 0x0403020cu)),
                       __uint_as_float(__builtin_amdgcn_perm(w2, w2, 0x0302010cu)));
}
// 32-bit words per stored filter row of F features
__host__ __device__ constexpr int fp24_words(int F) { return 3 * F / 4; }

// --------------------------------------------------------------- XCD mapping

// MI355X places consecutive workgroup ids on its 8 XCDs in turn, and each
// XCD has its own L2.  xcd_block() renumbers the launched blocks so that
// each XCD gets one contiguous slab of the logical block range (rows of the
// same replicas share an L2).  The grid must be launched with
// xcd_grid(n) blocks; ids that map beyond n - 1 return -1.
constexpr int kXcds = 8;
inline int xcd_grid(int n) { return (n + kXcds - 1) / kXcds * kXcds; }
__device__ inline int xcd_block(int n) {
    const int per = (n + kXcds - 1) / kXcds;
    const int b = (int)blockIdx.x;
    const int logical = (b % kXcds) * per + b / kXcds;
    return logical < n ? logical : -1;
}

// --------------------------------------------------------------- timing

enum KernelClass {
    K_NB_GRID = 0, K_NB_BIN, K_NB_SCAN, K_NB_COUNT, K_NB_FILL, K_NB_REV,
    K_PAIRS, K_MLP, K_FILTER_FWD, K_CFCONV, K_FILTER_BWD, K_FORCES, K_VERLET, K_KINETIC, K_PACK,
    K_NUM_CLASSES
};

void prof_begin(int cls, hipStream_t s);
void prof_end(int cls, hipStream_t s);

struct ProfScope {
    int cls; hipStream_t s;
    ProfScope(int c, hipStream_t st) : cls(c), s(st) { prof_begin(c, st); }
    ~ProfScope() { prof_end(cls, s); }
};

// --------------------------------------------------------------- workspace

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace: [0, 256) status words, then the scratch of the neighbour
// builder or of the energy/force pipeline (they are never live at the same
// time).
constexpr size_t kWsBase = 256;

struct NbLayout {            // neighbour-builder scratch (offsets from ws base)
    size_t grid, gpart, rep_of, cell_of, cell_cnt, cell_start, cell_fill, spos, row_cnt, keep, rep, mask, total;
    int64_t n_cells;         // capacity of the cell table
};

struct EfLayout {            // energy/force scratch (offsets from ws base)
    size_t up_first, up_cnt, up_ptr, edge_pair, pair_ij, pgeo, pfc, plfc, phi, x, o, gy, h, y, gh, eps, S, xmax, gmax, pack,
        rep, mask, h0, ref_pos, total;
};

// Weight pack: every weight matrix of the model pre-split into fp16 hi / lo
// halves and pre-arranged in the fragment order in which a kernel stages it
// into LDS, written once per evaluation so that each block's staging is a
// straight copy.  One slot per matrix: hi [kPackSlotFrags] then lo
// [kPackSlotFrags] 16-byte fragments; after all slots, two ints per slot
// (the power-of-two scale of the split, and one more scale where a kernel
// needs it); then, per interaction, kPackVecFloats floats of per-feature
// constants (the filter backward's folded second-layer bias).
enum PackKind {
    PK_FA1 = 0,   // filter first layer (both passes)
    PK_FA2,       // filter second layer, forward (chained order, times ln 2)
    PK_FA2B,      // filter second layer, backward (transposed)
    PK_XW,        // atom-wise W_in
    PK_OW1,       // Wo1
    PK_OW2,       // Wo2 (chained)
    PK_BOW1,      // Wo2 transposed
    PK_BOW2,      // Wo1 transposed (chained)
    PK_BXW,       // W_in transposed
    PK_PER_T
};
constexpr int kPackSlotFrags = 2048;
constexpr size_t kPackSlotBytes = 2 * size_t(kPackSlotFrags) * 16;
constexpr int kPackVecFloats = 128;   // the largest feature count
__host__ __device__ inline int pack_slot(int t, int kind) { return t * PK_PER_T + kind; }
__host__ __device__ inline int pack_readout_slot(int I, int k) { return I * PK_PER_T + k; }   // k = 0: R1, 1: R1 transposed (chained)
__host__ __device__ inline int pack_slots(int I) { return I * PK_PER_T + 2; }
__host__ __device__ inline size_t pack_vec_offset(int I) {
    return pack_slots(I) * kPackSlotBytes + align256(8 * size_t(pack_slots(I)));
}
inline size_t pack_bytes(int I) { return pack_vec_offset(I) + align256(4 * size_t(kPackVecFloats) * I); }
__host__ __device__ inline const float *pack_vec(const char *pack, int I, int t) {
    return reinterpret_cast<const float *>(pack + pack_vec_offset(I)) + kPackVecFloats * t;
}
struct PackRef {             // device pointers of one slot
    const void *hi, *lo;
    const int *sc;
};
__host__ __device__ inline PackRef pack_ref(const char *pack, int I, int slot) {
    PackRef r;
    r.hi = pack + slot * kPackSlotBytes;
    r.lo = pack + slot * kPackSlotBytes + kPackSlotBytes / 2;
    r.sc = reinterpret_cast<const int *>(pack + pack_slots(I) * kPackSlotBytes) + 2 * slot;
    return r;
}

NbLayout nb_layout(const sn_system &sys, size_t base);
EfLayout ef_layout(const sn_model &m, const sn_system &sys, int64_t n_edges, size_t base);

// Per-replica cell grid (device struct).
struct CellGrid {
    float lo[3];
    float inv[3];      // 1 / cell edge per dimension
    int n[3];
    int offset;        // first cell of this replica in the global cell table
};

// sin and cos of th in [0, pi/2]: Taylor polynomials about 0 (through x^9
// for sin, x^10 for cos; the first omitted terms are below 3e-9 relative on
// [0, pi/4]) on u = th, or on u = pi/2 - th above pi/4 (sin and cos then
// swap).  pi/2 is split in two floats, so u = pi/2 - th is exact to the
// rounding of the last addition.
__host__ __device__ inline void sincos_quadrant(float th, float &sn, float &cs) {
    const float kPio2Hi = 1.57079637050628662109375f;   // float(pi/2)
    const float kPio2Lo = -4.37113900018624283e-8f;     // pi/2 - kPio2Hi
    const bool flip = th > 0.785398163397448309616f;    // pi/4
    const float u = flip ? (kPio2Hi - th) + kPio2Lo : th;
    const float u2 = u * u;
    const float ps = fmaf(fmaf(fmaf(u2, 1.0f / 362880.0f, -1.0f / 5040.0f), u2, 1.0f / 120.0f), u2, -1.0f / 6.0f);
    const float s_u = fmaf(u * u2, ps, u);
    const float pc = fmaf(fmaf(fmaf(fmaf(u2, -1.0f / 3628800.0f, 1.0f / 40320.0f), u2, -1.0f / 720.0f), u2,
                               1.0f / 24.0f), u2, -0.5f);
    const float c_u = fmaf(u2, pc, 1.0f);
    sn = flip ? c_u : s_u;
    cs = flip ? s_u : c_u;
}

// Geometry of the pair (i, j) at positions ri, rj (three floats each): unit
// vector from i to j and distance in pgeo, the cosine envelope
// fc = (cos(pi d / rc) + 1) / 2 and lfc = fc'(d) / fc(d), the derivative of
// ln fc (both 0 at and beyond rc; the filter rows are stored multiplied by
// fc, so the backward pass needs fc' only in this ratio).  Every fused
// multiply-add is written out, so the bits do not depend on a file's
// contraction setting.
__device__ inline void pair_geometry(const float *ri, const float *rj, int periodic, const float (&L)[3],
                                     const float (&invL)[3], float cutoff, float4 &pgeo, float &fc, float &lfc) {
    float dx = rj[0] - ri[0], dy = rj[1] - ri[1], dz = rj[2] - ri[2];
    if (periodic) {
        dx = fmaf(-L[0], rintf(dx * invL[0]), dx);
        dy = fmaf(-L[1], rintf(dy * invL[1]), dy);
        dz = fmaf(-L[2], rintf(dz * invL[2]), dz);
    }
    const float d = sqrtf(fmaf(dz, dz, fmaf(dy, dy, dx * dx)));
    const float inv = 1.0f / d;
    pgeo = make_float4(dx * inv, dy * inv, dz * inv, d);
    fc = 0.0f;
    lfc = 0.0f;
    if (d < cutoff) {
        // written as cos^2(pi d / (2 rc)): no cancellation near rc; its
        // derivative -(pi / (2 rc)) sin(pi d / rc) = -(pi / rc) sin cos of the
        // half angle, so fc' / fc = -(pi / rc) sin / cos (cos > 0 for d < rc)
        constexpr float kPi = 3.14159265358979323846f;
        const float th = (0.5f * kPi) * d / cutoff;
        float sn, c;
        sincos_quadrant(th, sn, c);
        fc = c * c;
        lfc = -(kPi / cutoff) * sn / c;
    }
}

// --------------------------------------------------------------- launchers

// neighbors.hip
// Pair outputs of the neighbour build (the arrays the pair setup writes),
// plus scratch that must not overlap them: mask [N][kRepMaxAtoms / 64]
// words and rep [2 kTileMaxSplit B] ints.
struct NbPairOut {
    int32_t *edge_pair;
    int2 *pair_ij;
    float4 *pgeo;
    float *pfc, *plfc;
    float cutoff;
    uint64_t *mask;
    int32_t *rep;
};
// Largest replica (atoms), read from the device (synchronises `s`); -1 on error.
int max_replica_atoms(const sn_system &sys, hipStream_t s);
// Replicas of at most this many atoms are built by one block each from
// all-pairs bit masks in LDS (two launches for the whole build; one for a
// system of a single replica of at most kTileOneMax atoms).
constexpr int kRepMaxAtoms = 512;
constexpr int kRepMaxReplicas = 4096;   // each block of that build reads every replica's count
constexpr int kTileMaxSplit = 16;       // blocks per replica in that build
constexpr int kTileOneMax = 128;        // one replica of at most this many atoms: one launch
// sync: read the edge count back (into *n_edges) and check it on the host
// before the rows are filled.  Otherwise nothing is read back: the fill
// checks the capacity and row lengths on the device and flags errors; every
// kernel that reads the CSR afterwards returns at once when the status word
// is set (the rows may then be unfilled).  max_rep: the largest replica's atom count
// (-1: unknown); when it is at most kRepMaxAtoms the tile build
// runs, and with `pairs` set it also writes the pair arrays and the pair
// count (status slot kPairTotal; 0 after an error) and sets *pairs_done.
// step_mark >= 0: the first kernel writes it to status slot kStepsDone if no
// error is flagged by then (MD steps).  run_flag (may be null): every kernel
// of the build returns at once unless *run_flag is non-zero (device-driven MD
// steps that rebuild only some of the time).
sn_status nb_build(const sn_system &sys, const float *pos, float r_list, int32_t *row_ptr, int32_t *col,
                   int32_t *rev, int64_t capacity, int64_t *n_edges, char *ws, hipStream_t s, bool sync = true,
                   int max_rep = -1, const NbPairOut *pairs = nullptr, bool *pairs_done = nullptr,
                   int step_mark = -1, const int *run_flag = nullptr);
// Check run by the scan's last block once the total is known: the pair
// count is E / 2 (E >= 0), or row_ptr[N] / 2 (E < 0), and must equal the
// total (the number of upper edges).  status[kPairTotal] receives it, or 0
// when the check fails (flagged SN_ERR_INVALID) or when `guard` is set and
// an error is already flagged.
struct PairCountCheck {
    int *status;                 // null: no check
    const int32_t *row_ptr;
    int N;
    int64_t E;
    bool guard;
};
// Exclusive prefix sum (one launch); out[n] = total; optional device slots
// receive the total and the maximum input.  in and out must not overlap.
// run_flag (may be null): nothing happens unless *run_flag is non-zero.
sn_status scan_exclusive(const int32_t *in, int32_t *out, int n, int32_t *total_slot, int32_t *max_slot,
                         hipStream_t s, PairCountCheck chk = PairCountCheck{}, const int *run_flag = nullptr);

// filter.hip
// Writes the filter slots of the weight pack (all interactions).
sn_status filter_pack(const sn_model &m, char *pack, hipStream_t s);
// pack: the weight pack written by filter_pack (required).
// phi24: the filter rows [P][3F/4] in the 24-bit row format (see pack_fp24).
// P: the pair capacity (launch size); p_dev (may be null): the device pair
// count; guard (may be null): no pairs are processed while *guard is set.
// The rows are stored multiplied by the envelope pfc[p] (the CFConv's weight W_p).
sn_status filter_forward(const sn_model &m, int t, const float4 *pgeo, const float *pfc, int64_t P, uint32_t *phi24,
                         const char *pack, const int *p_dev, const int *guard, hipStream_t s);
// Whether a system of P pairs (capacity) runs every interaction's forward
// filter in one launch (few pair tiles, at most 8 interactions), and that
// launch: phi24[t] receives interaction t's rows.
bool filter_forward_fused(const sn_model &m, int64_t P);
sn_status filter_forward_all(const sn_model &m, const float4 *pgeo, const float *pfc, int64_t P,
                             uint32_t *const *phi24, const char *pack, const int *p_dev, const int *guard,
                             hipStream_t s);
// phi [P][F] in fp32 without the envelope, for n = P distances d (the same kernel).
sn_status filter_forward_plain(const sn_model &m, int t, const float *d, int64_t P, float *phi, const char *pack,
                               hipStream_t s);
// xmax / gmax: per-atom max_f |x[i][f]| and max_f |g_y[i][f]| of interaction t
// pfc / plfc: per-pair envelope fc(d) and fc'(d) / fc(d).  The stored rows are
// not read (the pass recomputes what it needs of them).  pack: the weight pack
// (required).
sn_status filter_backward(const sn_model &m, int t, const float4 *pgeo, const float *pfc, const float *plfc,
                          const int2 *pair_ij, int64_t P, int N, const float *x, const float *gy, const float *xmax,
                          const float *gmax, float *S, int accumulate, const char *pack, const int *p_dev,
                          const int *guard, hipStream_t s);

// The backward filter of every interaction in one launch (the systems of
// filter_forward_fused), interaction t writing S[t P ...]; x, gy, xmax and
// gmax are per-interaction arrays of pointers.
sn_status filter_backward_all(const sn_model &m, const float4 *pgeo, const float *pfc, const float *plfc,
                              const int2 *pair_ij, int64_t P, const float *const *x, const float *const *gy,
                              const float *const *xmax, const float *const *gmax, float *S, const char *pack,
                              const int *p_dev, const int *guard, hipStream_t s);

// graph.hip
// E: the edge count, or -1 to take it from row_ptr[N] on the device.  Writes
// the pair count to the status slot kPairTotal (0 after a failed check).
// guard (here and below; may be null): the kernels return at once while
// *guard is non-zero, for a CSR that a flagged neighbour build may have left
// unfilled (the pair count is then 0).
// run_flag (may be null): the kernels return at once unless *run_flag is
// non-zero (the list was rebuilt in this device-driven MD step).
sn_status pairs_setup(const sn_system &sys, const float *pos, const int32_t *row_ptr, const int32_t *col,
                      const int32_t *rev, int64_t E, float cutoff, char *ws, const EfLayout &L, int *status,
                      const int *guard, hipStream_t s, const int *run_flag = nullptr);
// Neighbour skin, on the steps of a device-driven MD call: when the step
// rebuilt the list (status slot kBuildFlag set) the positions are recorded
// in ref_pos [N][3]; otherwise the geometry of every pair of the kept list
// (pair_ij, status slot kPairTotal pairs) is recomputed from the positions.
// P_cap: the pair capacity (launch size).
sn_status pairs_refresh(const sn_system &sys, const float *pos, float cutoff, char *ws, const EfLayout &L,
                        int *status, int64_t P_cap, hipStream_t s);
// phi24: the filter rows W = fc phi in the 24-bit row format
sn_status cfconv(int F, int N, const int32_t *row_ptr, const int32_t *col, const int32_t *edge_pair,
                 const uint32_t *phi24, const float *in, float *out, const int *guard, hipStream_t s);
// The integrator's part of an MD step that the force assembly applies as it
// writes each atom's force: close = the step's closing half kick
// v += half F / m (and its edge count to edge_slot if set); open = the next
// step's opening half kick with the same force and the drift r += dt v.
// Atoms do not move once an error is flagged.
// Device-driven steps (n_total >= 0): the step index is status slot kMdStep
// minus one; the opening part runs only when step + 1 < n_total, the edge
// count goes to edge_log[step] (if set); with ref_pos set, an atom that the
// drift leaves more than sqrt(half_skin2) from ref_pos sets status slot
// kDisplaced.
struct VerletFuse {
    float *pos, *vel;
    const float *inv_mass;
    float half, dt;
    int close, open;
    int *edge_slot;
    int n_total;
    int *edge_log;
    const float *ref_pos;
    float half_skin2;
};
// F_i = sum_{e in row i} S_p(e) u_e with S_p = S[(s_parts - 1) stride + p] +
// ... + S[p] (parts added from the last, as the filter backward accumulates
// them when it runs interaction by interaction), one launch that also sums the atom
// energies eps per replica (in fp64) into energy[b] (fp32, if energy is set)
// and elog[b] (fp64, if elog is set; elog[step B + b] when elog_by_step is
// set: device-driven steps, step = status[kMdStep] - 1) and, with vf,
// applies its Verlet part.
sn_status forces_rows(int N, int B, const int32_t *replica_ptr, const float *eps, float *energy,
                      const int32_t *row_ptr, const int32_t *col, const int32_t *edge_pair, const float4 *pgeo,
                      const float *S, int s_parts, int64_t s_stride, float *forces, int *status, const int *guard,
                      const VerletFuse *vf, hipStream_t s, double *elog = nullptr, int elog_by_step = 0);


// Compute units of the current device (filter.hip; read once per process).
int num_cus();

// mlp.hip (fused atom-wise layers; see the kernel comments there).  The
// weights come from the weight pack (slots written by mlp_pack).
sn_status mlp_pack(const sn_model &m, char *pack, hipStream_t s);
// The chains of layers between CFConvs.  xmax / gymax: per-atom row maxima.
// h = Emb[type]; x = h W_in (first interaction)
sn_status mlp_embed_x(int N, int F, int T, const int32_t *types, const float *emb, PackRef W_in, float *h, float *x,
                      float *xmax, int *status, hipStream_t s);
// o = y Wo1 + bo1; h = h_in + ssp(o) Wo2 + bo2; x = h W_in (of the next interaction)
sn_status mlp_out_x(int N, int F, const float *y, PackRef Wo1, const float *bo1, PackRef Wo2, const float *bo2,
                    PackRef W_in, float *o, const float *h_in, float *h, float *x, float *xmax, hipStream_t s);
// the last interaction's OUT, the readout (eps, g_h) and the first backward block (g_y)
sn_status mlp_tail(int N, int F, const float *y, PackRef Wo1, const float *bo1, PackRef Wo2, const float *bo2,
                   const float *h, PackRef R1, const float *c1, PackRef R1t, const float *R2, const float *c2,
                   PackRef Wo2t, PackRef Wo1t, float *eps, float *gh, float *gy, float *gymax, hipStream_t s);
// g_h += g_x W_in^T (interaction t); the backward block of t - 1 (g_y)
sn_status mlp_bx_bo(int N, int F, const float *gx, PackRef W_int, PackRef Wo2t, const float *o_prev, PackRef Wo1t,
                    float *gh, float *gy, float *gymax, hipStream_t s);

// verlet (api.hip)

}  // namespace sn
