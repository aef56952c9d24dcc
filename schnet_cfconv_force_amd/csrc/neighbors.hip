// Cell-list CSR neighbour builder.
//
// Produces the full, directed neighbour list ("How", flash message passing:
// cutoff masking; flash aggregation: CSR -- FlashSchNet summary page) of
// every replica: row i lists, in ascending order, every atom j != i of the
// same replica with fp32 squared distance strictly below r_list^2.  The
// predicate is evaluated with one rounding per operation and no fused
// multiply-add, so the list is bit-for-bit reproducible from the positions.
//
// Pipeline (all on the caller's stream):
//   grid    ~256 blocks in all: cleared cell table, partial bounding boxes;
//           then one wavefront per replica: its cell grid
//   bin     one thread per atom: cell index, atomic cell histogram
//   scan    cell histogram -> cell start offsets
//   place   one thread per atom: atom copied into its cell's slot range
//   count   one wavefront per atom: candidates of the 27 surrounding cells,
//           exact predicate (survivors compacted by ballot), row length;
//           rows of up to kRowKeep entries are kept in the workspace
//   scan    row lengths -> row_ptr, total read back by the host
//   fill    one wavefront per atom: the kept row (or, for a longer row, the
//           candidates tested again) in LDS, rank-sorted into col_idx
//   rev     one wavefront per row: binary search of i in row j
// The order of atoms inside a cell depends on atomic arrival order; the
// sorted rows do not, so the output is deterministic.
#pragma clang fp contract(off)

#include <algorithm>
#include <vector>

#include "sn_internal.h"

namespace sn {

namespace {

constexpr int kWave = 64;
constexpr int kNbWaves = 4;   // wavefronts per block in the per-atom kernels

struct PredParams {
    float rl2;
    float L[3];
    float invL[3];
    int periodic;
};

// Device-driven MD steps rebuild the list only some of the time: every
// kernel of the build then returns at once unless the step's flag is set.
__device__ inline bool skipped(const int *run_flag) { return run_flag && *run_flag == 0; }

__global__ void fill_int_kernel(int *p, int v, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// The cell grid of one replica of n atoms from its bounding box lo..hi
// (`bad`: some coordinate of the replica is not finite; the box is then
// ignored).  At most 8 n + 64 cells, each edge at least cell_edge.
__device__ inline CellGrid make_grid(const float (&lo)[3], const float (&hi)[3], bool bad, int n,
                                     const PredParams &pp, float cell_edge, int offset) {
    const long cap = 8L * n + 64;
    CellGrid g;
    if (pp.periodic) {
        int m[3];
        for (int c = 0; c < 3; ++c) m[c] = (int)floorf(pp.L[c] / cell_edge);
        while ((long)m[0] * m[1] * m[2] > cap) {           // coarser cells for sparse replicas
            int c = (m[0] >= m[1] && m[0] >= m[2]) ? 0 : (m[1] >= m[2] ? 1 : 2);
            if (m[c] <= 3) break;
            m[c] = max(3, (m[c] * 4) / 5);
        }
        for (int c = 0; c < 3; ++c) {
            g.lo[c] = 0.0f;
            g.n[c] = m[c];
            g.inv[c] = (float)m[c] / pp.L[c];
        }
    } else {
        const bool use = n > 0 && !bad;
        float ext[3];
        for (int c = 0; c < 3; ++c) {
            ext[c] = use ? hi[c] - lo[c] : 0.0f;
            if (!(ext[c] >= 0.0f && ext[c] <= 1.0e30f)) ext[c] = 0.0f;   // overflowed extent: one cell
        }
        float ce = cell_edge;
        int m[3];
        for (;;) {                       // ends: the extents are finite, and ce grows
            for (int c = 0; c < 3; ++c) m[c] = (int)fminf(floorf(ext[c] / ce) + 1.0f, 1048576.0f);
            if ((double)m[0] * m[1] * m[2] <= (double)cap) break;
            ce *= 1.25f;
        }
        for (int c = 0; c < 3; ++c) {
            g.lo[c] = use ? lo[c] : 0.0f;
            g.n[c] = m[c];
            g.inv[c] = 1.0f / ce;
        }
    }
    g.offset = offset;
    return g;
}

// Bounding box of atoms [s, e) over a block of NT threads: the result in
// lo / hi of thread 0; the return value (every thread) tells whether any
// coordinate is not finite.  red: 6 x (NT / 64) floats of LDS.
template <int NT>
__device__ inline bool block_bbox(const float *pos, int s, int e, float (*red)[NT / 64], float (&lo)[3],
                                  float (&hi)[3]) {
    const int lane = threadIdx.x % 64, wv = threadIdx.x / 64;
    bool bad = false;
    for (int c = 0; c < 3; ++c) { lo[c] = INFINITY; hi[c] = -INFINITY; }
    for (int i = s + threadIdx.x; i < e; i += NT)
        for (int c = 0; c < 3; ++c) {
            const float v = pos[3 * i + c];
            if (!isfinite(v)) bad = true;
            lo[c] = fminf(lo[c], v);
            hi[c] = fmaxf(hi[c], v);
        }
    for (int c = 0; c < 3; ++c)
        for (int o = 32; o > 0; o >>= 1) {
            lo[c] = fminf(lo[c], __shfl_xor(lo[c], o, 64));
            hi[c] = fmaxf(hi[c], __shfl_xor(hi[c], o, 64));
        }
    if (lane == 0)
        for (int c = 0; c < 3; ++c) { red[c][wv] = lo[c]; red[3 + c][wv] = hi[c]; }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0)
        for (int w = 1; w < NT / 64; ++w)
            for (int c = 0; c < 3; ++c) { lo[c] = fminf(lo[c], red[c][w]); hi[c] = fmaxf(hi[c], red[3 + c][w]); }
    return bad;
}

// The cell grid in two launches, so that a large replica is spread over
// many compute units.  grid_part_kernel: R blocks per replica, block (b,
// part) takes a 1/R slice of replica b's atoms (atom -> replica map and a
// partial bounding box with its non-finite flag, written to part[8 (b R +
// part) ..]) and of its cells (the counters are cleared: cells [8 s + 64 b,
// 8 e + 64 (b + 1)) belong to replica b; the last block clears the final
// entry); block 0 also resets the builder's status slots.  grid_make_kernel
// (one wavefront per replica) combines the R partial boxes into the
// replica's grid (min / max: the result does not depend on the order).
__global__ __launch_bounds__(256) void grid_part_kernel(const float *pos, const int32_t *rptr, int R, float *part,
                                                        int *rep_of, int *cell_cnt, int *cell_fill, int64_t n_cells,
                                                        int step_mark, int *status, const int *run_flag) {
    __shared__ float red[6][4];
    if (skipped(run_flag)) return;
    const int b = blockIdx.x / R, k = blockIdx.x % R;
    const int s = rptr[b], e = rptr[b + 1];
    const int64_t c0 = 8 * (int64_t)s + 64 * b, c1 = 8 * (int64_t)e + 64 * (b + 1);
    const int64_t cper = (c1 - c0 + R - 1) / R;
    const int64_t cs = c0 + k * cper, ce = min(c1, cs + cper);
    for (int64_t c = cs + threadIdx.x; c < ce; c += blockDim.x) {
        cell_cnt[c] = 0;
        cell_fill[c] = 0;
    }
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) {
        cell_cnt[n_cells] = 0;
        cell_fill[n_cells] = 0;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        status[kMaxRow] = 0;
        status[kEdgeTotal] = 0;
        if (step_mark >= 0 && *status == 0) status[kStepsDone] = step_mark;
    }
    const int aper = (e - s + R - 1) / R;
    const int as = min(e, s + k * aper), ae = min(e, as + aper);
    for (int i = as + threadIdx.x; i < ae; i += 256) rep_of[i] = b;
    float lo[3], hi[3];
    const bool bad = block_bbox<256>(pos, as, ae, red, lo, hi);
    if (threadIdx.x != 0) return;
    float *o = part + 8 * (int64_t)blockIdx.x;
    for (int c = 0; c < 3; ++c) {
        o[c] = lo[c];
        o[3 + c] = hi[c];
    }
    o[6] = bad ? 1.0f : 0.0f;
}

__global__ __launch_bounds__(64) void grid_make_kernel(const int32_t *rptr, int R, const float *part, PredParams pp,
                                                       float cell_edge, CellGrid *grid, int *status,
                                                       const int *run_flag) {
    if (skipped(run_flag)) return;
    const int b = blockIdx.x, lane = threadIdx.x;
    float lo[3] = {INFINITY, INFINITY, INFINITY}, hi[3] = {-INFINITY, -INFINITY, -INFINITY};
    bool bad = false;
    for (int k = lane; k < R; k += 64) {
        const float *o = part + 8 * ((int64_t)b * R + k);
        for (int c = 0; c < 3; ++c) {
            lo[c] = fminf(lo[c], o[c]);
            hi[c] = fmaxf(hi[c], o[3 + c]);
        }
        bad |= o[6] != 0.0f;
    }
    for (int c = 0; c < 3; ++c)
        for (int o = 32; o > 0; o >>= 1) {
            lo[c] = fminf(lo[c], __shfl_xor(lo[c], o, 64));
            hi[c] = fmaxf(hi[c], __shfl_xor(hi[c], o, 64));
        }
    bad = __any(bad);
    if (lane != 0) return;
    if (bad) flag_status(status, SN_ERR_NONFINITE);
    const int s = rptr[b], e = rptr[b + 1];
    grid[b] = make_grid(lo, hi, bad, e - s, pp, cell_edge, 8 * s + 64 * b);
}

__device__ inline int cell_coord(float x, int c, const CellGrid &g, const PredParams &pp) {
    float t;
    if (pp.periodic) {
        float xw = x - pp.L[c] * floorf(x * pp.invL[c]);
        t = floorf(xw * g.inv[c]);
    } else {
        t = floorf((x - g.lo[c]) * g.inv[c]);
    }
    int k = (t != t) ? 0 : (int)fminf(fmaxf(t, 0.0f), (float)(g.n[c] - 1));
    return k;
}

__global__ void bin_kernel(const float *pos, int n_atoms, const CellGrid *grid, const int *rep_of, PredParams pp,
                           int *cell_of, int *cell_cnt, const int *run_flag) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_atoms || skipped(run_flag)) return;
    const CellGrid g = grid[rep_of[i]];
    int c0 = cell_coord(pos[3 * i + 0], 0, g, pp);
    int c1 = cell_coord(pos[3 * i + 1], 1, g, pp);
    int c2 = cell_coord(pos[3 * i + 2], 2, g, pp);
    int cell = g.offset + (c2 * g.n[1] + c1) * g.n[0] + c0;
    cell_of[i] = cell;
    atomicAdd(&cell_cnt[cell], 1);
}

__global__ void place_kernel(const float *pos, int n_atoms, const int *cell_of, const int *cell_start,
                             int *cell_fill, float4 *spos, const int *run_flag) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_atoms || skipped(run_flag)) return;
    int cell = cell_of[i];
    int slot = atomicAdd(&cell_fill[cell], 1);
    spos[cell_start[cell] + slot] = make_float4(pos[3 * i], pos[3 * i + 1], pos[3 * i + 2], __int_as_float(i));
}

// Order this wavefront's LDS writes before its later LDS reads (LDS requests
// of one wavefront complete in issue order; this also stops the compiler
// from moving the reads up).
__device__ inline void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The exact fp32 neighbour predicate (contraction is off in this file).
__device__ inline bool within(float xi, float yi, float zi, float4 q, const PredParams &pp) {
    float dx = q.x - xi, dy = q.y - yi, dz = q.z - zi;
    if (pp.periodic) {
        dx = dx - pp.L[0] * rintf(dx * pp.invL[0]);
        dy = dy - pp.L[1] * rintf(dy * pp.invL[1]);
        dz = dz - pp.L[2] * rintf(dz * pp.invL[2]);
    }
    float r2 = (dx * dx + dy * dy) + dz * dz;
    return r2 < pp.rl2;
}

// One wavefront per atom.  FILL = false: write the row length into cnt[i]
// and, for rows of at most kRowKeep entries, the row's columns in candidate
// order into keep[i kRowKeep ...].  FILL = true: write the sorted row into
// col[row_ptr[i] ...], from keep when the row fitted there, else by testing
// the candidates again.
constexpr int kRowKeep = 256;
template <bool FILL>
__global__ __launch_bounds__(kWave * kNbWaves) void rows_kernel(const float *pos, int n_atoms, const CellGrid *grid,
                                                               const int *rep_of, const int *cell_start,
                                                               const float4 *spos, PredParams pp, int *cnt,
                                                               int32_t *keep, const int32_t *row_ptr, int32_t *col,
                                                               int64_t capacity, int *status, const int *run_flag) {
    __shared__ int s_start[kNbWaves][28];
    __shared__ int s_pre[kNbWaves][28];
    __shared__ int s_buf[FILL ? kNbWaves : 1][FILL ? SN_MAX_ROW : 1];
    const int wv = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int i = blockIdx.x * kNbWaves + wv;
    if (i >= n_atoms || skipped(run_flag)) return;   // whole wavefront exits together
    if (FILL) {
        // a row kept by the count pass: its columns, unsorted, into LDS
        const int r0 = row_ptr[i];
        const int n = row_ptr[i + 1] - r0;
        if (n <= kRowKeep && (int64_t)row_ptr[n_atoms] <= capacity) {
            for (int k = lane; k < n; k += kWave) s_buf[FILL ? wv : 0][FILL ? k : 0] = keep[(int64_t)i * kRowKeep + k];
            wave_sync();
            for (int k = lane; k < n; k += kWave) {
                const int v = s_buf[FILL ? wv : 0][FILL ? k : 0];
                int rank = 0;
                for (int m = 0; m < n; ++m) rank += (s_buf[FILL ? wv : 0][FILL ? m : 0] < v);
                col[r0 + rank] = v;
            }
            return;
        }
    }
    const CellGrid g = grid[rep_of[i]];
    const float xi = pos[3 * i], yi = pos[3 * i + 1], zi = pos[3 * i + 2];
    const int ci[3] = {cell_coord(xi, 0, g, pp), cell_coord(yi, 1, g, pp), cell_coord(zi, 2, g, pp)};

    int len = 0, start = 0;
    if (lane < 27) {
        int d[3] = {lane % 3 - 1, (lane / 3) % 3 - 1, lane / 9 - 1};
        int cc[3];
        bool ok = true;
        for (int c = 0; c < 3; ++c) {
            int v = ci[c] + d[c];
            if (pp.periodic) {
                v = (v + g.n[c]) % g.n[c];
            } else if (v < 0 || v >= g.n[c]) {
                ok = false;
            }
            cc[c] = v;
        }
        if (ok) {
            int cell = g.offset + (cc[2] * g.n[1] + cc[1]) * g.n[0] + cc[0];
            start = cell_start[cell];
            len = cell_start[cell + 1] - start;
        }
    }
    // inclusive prefix of the 27 lengths across the wavefront
    int incl = len;
    for (int o = 1; o < 32; o <<= 1) {
        int t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
    }
    const int total = __shfl(incl, 26, kWave);
    if (lane < 27) {
        s_start[wv][lane] = start;
        s_pre[wv][lane] = incl - len;
    }
    if (lane == 27) s_pre[wv][27] = total;
    wave_sync();                    // only this wavefront touches its LDS slice

    int base = 0;
    for (int k0 = 0; k0 < total; k0 += kWave) {
        const int k = k0 + lane;
        bool pass = false;
        int j = -1;
        if (k < total) {
            int lo = 0, hi = 26;                    // largest r with pre[r] <= k
            while (lo < hi) {
                int mid = (lo + hi + 1) >> 1;
                if (s_pre[wv][mid] <= k) lo = mid; else hi = mid - 1;
            }
            float4 q = spos[s_start[wv][lo] + (k - s_pre[wv][lo])];
            j = __float_as_int(q.w);
            pass = (j != i) && within(xi, yi, zi, q, pp);
        }
        uint64_t mask = __ballot(pass);
        const int off = base + __popcll(mask & ((1ull << lane) - 1ull));
        if (FILL) {
            if (pass && off < SN_MAX_ROW) s_buf[FILL ? wv : 0][FILL ? off : 0] = j;
        } else if (pass && off < kRowKeep) {
            keep[(int64_t)i * kRowKeep + off] = j;
        }
        base += __popcll(mask);
    }
    if (!FILL) {
        if (lane == 0) cnt[i] = base;
        return;
    }
    const int r0 = row_ptr[i];
    const int n = row_ptr[i + 1] - r0;
    if ((int64_t)row_ptr[n_atoms] > capacity || n > SN_MAX_ROW || n != base) {
        if (lane == 0)
            flag_status(status, (int64_t)row_ptr[n_atoms] > capacity ? SN_ERR_CAPACITY
                                : n > SN_MAX_ROW                    ? SN_ERR_ROW
                                                                    : SN_ERR_INVALID);
        return;
    }
    wave_sync();
    for (int k = lane; k < n; k += kWave) {
        int v = s_buf[FILL ? wv : 0][FILL ? k : 0];
        int rank = 0;
        for (int m = 0; m < n; ++m) rank += (s_buf[FILL ? wv : 0][FILL ? m : 0] < v);
        col[r0 + rank] = v;
    }
}

// One wavefront per row: rev[e] = index of (j, i) in row j.
__global__ __launch_bounds__(256) void rev_kernel(int n_atoms, const int32_t *row_ptr, const int32_t *col,
                                                  int32_t *rev, int *status, const int *run_flag) {
    const int wv = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int i = blockIdx.x * 4 + wv;
    // after an error the rows may not be filled
    if (i >= n_atoms || *status != 0 || skipped(run_flag)) return;
    const int e0 = row_ptr[i], e1 = row_ptr[i + 1];
    for (int e = e0 + lane; e < e1; e += kWave) {
        const int j = col[e];
        int lo = row_ptr[j], hi = row_ptr[j + 1] - 1, found = -1;
        while (lo <= hi) {
            int mid = (lo + hi) >> 1;
            int v = col[mid];
            if (v == i) { found = mid; break; }
            if (v < i) lo = mid + 1; else hi = mid - 1;
        }
        if (found < 0) flag_status(status, SN_ERR_INVALID);
        rev[e] = found;
    }
}

// ------------------------------------------------------------------ scan
// Exclusive prefix sum in three passes over tiles of 4096 values (1024
// threads x 4): tile sums (and maxima), a scan of the tile sums in one
// block, then each tile's own scan plus its offset.  out may alias in.

constexpr int kScanThreads = 1024;
constexpr int kScanTile = 4 * kScanThreads;

// block-wide exclusive scan of one value per thread; *total receives the sum
__device__ inline int block_exclusive(int v, int *s_w, int *total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int x = v;
    for (int o = 1; o < 64; o <<= 1) {
        int t = __shfl_up(x, o, 64);
        if (lane >= o) x += t;
    }
    if (lane == 63) s_w[wv] = x;
    __syncthreads();
    if (wv == 0) {
        int w = (lane < kScanThreads / 64) ? s_w[lane] : 0;
        for (int o = 1; o < 16; o <<= 1) {
            int t = __shfl_up(w, o, 64);
            if (lane >= o) w += t;
        }
        if (lane < kScanThreads / 64) s_w[lane] = w;
    }
    __syncthreads();
    const int base = wv > 0 ? s_w[wv - 1] : 0;
    *total = s_w[kScanThreads / 64 - 1];
    __syncthreads();
    return base + x - v;
}

__device__ inline int block_max(int v, int *s_w) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
    if (lane == 0) s_w[wv] = v;
    __syncthreads();
    int m = s_w[0];
    for (int k = 1; k < kScanThreads / 64; ++k) m = max(m, s_w[k]);
    __syncthreads();
    return m;
}

__device__ inline void load4(const int32_t *in, int n, int64_t b, int v[4]) {
    for (int r = 0; r < 4; ++r) v[r] = (b + r < n) ? in[b + r] : 0;
}

// Exclusive scan in one launch.  Block b scans tile b (kScanTile values) and
// finds the sum of all earlier tiles by reading them itself: at the sizes
// used here (up to a few hundred thousand values) that redundant read from
// L2 costs less than the launches of a multi-pass scan.  The last block also
// writes out[n] (the total) and the optional total and maximum slots.  in and
// out must not overlap; in must be 16-byte aligned.
__global__ __launch_bounds__(kScanThreads) void scan_kernel(const int32_t *in, int32_t *out, int n,
                                                            int32_t *total_slot, int32_t *max_slot,
                                                            PairCountCheck chk, const int *run_flag) {
    __shared__ int s_w[kScanThreads / 64];
    if (skipped(run_flag)) return;
    const int64_t t0 = (int64_t)blockIdx.x * kScanTile;   // a multiple of 4 * kScanThreads
    const bool last = blockIdx.x == gridDim.x - 1;
    int pre = 0, mx = 0;
#pragma unroll 4
    for (int64_t b = 4 * (int64_t)threadIdx.x; b < t0; b += 4 * kScanThreads) {
        const int4 v = *reinterpret_cast<const int4 *>(in + b);
        pre += (v.x + v.y) + (v.z + v.w);
        mx = max(mx, max(max(v.x, v.y), max(v.z, v.w)));
    }
    int before;
    block_exclusive(pre, s_w, &before);   // the block-wide sum of the earlier tiles
    int v[4];
    load4(in, n, t0 + 4 * threadIdx.x, v);
    int tot;
    int run = before + block_exclusive(v[0] + v[1] + v[2] + v[3], s_w, &tot);
    for (int r = 0; r < 4; ++r) {
        if (t0 + 4 * threadIdx.x + r < n) out[t0 + 4 * threadIdx.x + r] = run;
        run += v[r];
    }
    if (last) {
        const int m = block_max(max(mx, max(max(v[0], v[1]), max(v[2], v[3]))), s_w);
        if (threadIdx.x == 0) {
            out[n] = before + tot;
            if (total_slot) *total_slot = before + tot;
            if (max_slot) *max_slot = m;
            if (chk.status) {
                const int64_t P = (chk.E >= 0 ? chk.E : (int64_t)chk.row_ptr[chk.N]) / 2;
                const bool flagged = chk.guard && chk.status[kStatusWord] != 0;
                const bool ok = !flagged && before + tot == P;
                if (!ok && !flagged) flag_status(chk.status, SN_ERR_INVALID);
                chk.status[kPairTotal] = ok ? (int)P : 0;
            }
        }
    }
}

// ------------------------------------------------------------- tile build
// Replicas of at most kRepMaxAtoms atoms: each block holds its replica's
// positions in LDS and tests every ordered pair of its rows, 64 columns (one
// wavefront ballot) at a time, so that each row's neighbours form a bit mask
// over the replica's atoms.  A replica this small spans about three cells of
// r_list per dimension, so cells would not thin out the candidates much; the
// masks instead give everything else by population counts: a bit's position
// in its row (sorted order for free), the reverse edge (the position of i in
// row j), the first upper edge of a row and the pair numbers.  R blocks per
// replica (R = split) share its rows; two launches:
//   count  row masks -> mask; per block, edge count and longest row -> rep
//   fill   offsets of the earlier blocks (from rep), row_ptr, col, rev and
//          optionally the pair arrays (one pair per upper edge, numbered
//          replica by replica and row by row, as the pair setup numbers them)
// Each fill block reads the masks of its whole replica.  A system of one
// replica of at most kTileOneMax atoms takes one launch instead (every block
// evaluates all of the replica's masks itself).  The predicate is the
// cell-list path's, so all of them give the same CSR.

constexpr int kTileThreads = kScanThreads;   // the block size block_exclusive assumes
constexpr int kTileWaves = kTileThreads / kWave;
constexpr int kTileWords = kRepMaxAtoms / 64;

struct TileArgs {
    const float *pos;
    const int32_t *rptr;
    int B, N;
    int Rc, R;                   // blocks per replica: count pass, fill pass
    PredParams pp;
    uint64_t *mask;              // [N][kTileWords] row masks
    int32_t *rep;                // [2 B R]: edge count, then longest row, per block
    int32_t *row_ptr, *col, *rev;
    int64_t capacity;
    int flag;                    // flag SN_ERR_ROW / SN_ERR_CAPACITY in the status word
    NbPairOut pr;                // pr.edge_pair null: no pair arrays
    int step_mark;               // >= 0: to status slot kStepsDone unless an error is flagged
    int *status;
    const int *run_flag;         // (may be null) nothing is done unless *run_flag is non-zero
};

__device__ inline uint64_t below_mask(int bit) { return (1ull << bit) - 1ull; }

// The replica's positions into LDS (sp[3 q + c]); returns whether any is not
// finite (block-wide, after a barrier).
__device__ inline bool tile_positions(const float *pos, int s, int n, float *sp) {
    bool bad = false;
    for (int k = threadIdx.x; k < 3 * n; k += kTileThreads) {
        const float v = pos[3 * (int64_t)s + k];
        bad |= !isfinite(v);
        sp[k] = v;
    }
    return __syncthreads_or(bad);
}

__global__ __launch_bounds__(kTileThreads) void tile_count_kernel(TileArgs a) {
    __shared__ float sp[3 * kRepMaxAtoms];
    __shared__ int s_sum, s_max;
    if (skipped(a.run_flag)) return;
    const int b = blockIdx.x / a.Rc, part = blockIdx.x % a.Rc;
    const int s = a.rptr[b], e = a.rptr[b + 1], n = e - s;
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    if (threadIdx.x == 0) {
        s_sum = 0;
        s_max = 0;
        if (blockIdx.x == 0 && a.step_mark >= 0 && *a.status == 0) a.status[kStepsDone] = a.step_mark;
    }
    if (tile_positions(a.pos, s, n, sp)) {       // the fill pass sees the flag and writes nothing
        if (threadIdx.x == 0) flag_status(a.status, SN_ERR_NONFINITE);
        return;
    }
    const int W = (n + kWave - 1) / kWave;
    const int per = (n + a.Rc - 1) / a.Rc, q0 = part * per, q1 = min(n, q0 + per);
    int sum = 0, mx = 0;
    for (int q = q0 + wv; q < q1; q += kTileWaves) {
        const float xi = sp[3 * q], yi = sp[3 * q + 1], zi = sp[3 * q + 2];
        uint64_t mine = 0;
        int cnt = 0;
#pragma unroll
        for (int w = 0; w < kTileWords; ++w) {
            if (w >= W) break;
            const int j = kWave * w + lane, jj = j < n ? j : 0;
            const float4 pj = make_float4(sp[3 * jj], sp[3 * jj + 1], sp[3 * jj + 2], 0.0f);
            const bool pass = j < n && j != q && within(xi, yi, zi, pj, a.pp);
            const uint64_t m = __ballot(pass);
            cnt += __popcll(m);
            if (lane == w) mine = m;
        }
        if (lane < W) a.mask[(int64_t)(s + q) * kTileWords + lane] = mine;
        sum += cnt;
        mx = max(mx, cnt);
    }
    if (lane == 0) {
        atomicAdd(&s_sum, sum);
        atomicMax(&s_max, mx);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        a.rep[blockIdx.x] = s_sum;
        a.rep[a.B * a.Rc + blockIdx.x] = s_max;
    }
}

// LDS of a fill block: the replica's row masks and positions, and per row
// the prefix counts of its words, its edge offset, its first upper edge and
// its pair offset.
struct TileSmem {
    uint64_t sm[kRepMaxAtoms][kTileWords];
    int wpre[kRepMaxAtoms][kTileWords];          // set bits of the row's earlier words
    int rptr[kRepMaxAtoms + 1], upf[kRepMaxAtoms], upp[kRepMaxAtoms];
    float sp[3 * kRepMaxAtoms];
    int sw[kTileWaves];
};

// Row offsets of the replica (masks in LDS): thread q takes row q.  Returns
// the replica's edge and upper-edge totals and, with LONGEST, its longest
// row; the row offsets, first upper edges and pair offsets go to LDS.  Holds
// barriers.
struct RowTotals {
    int edges, upper, longest;
};
template <bool LONGEST>
__device__ inline RowTotals tile_row_offsets(TileSmem &t, int n) {
    const int W = (n + kWave - 1) / kWave;
    const int q = threadIdx.x;
    int cnt = 0, upf = 0;
    if (q < n) {
        for (int w = 0; w < W; ++w) {
            t.wpre[q][w] = cnt;
            cnt += __popcll(t.sm[q][w]);
        }
        upf = t.wpre[q][q / kWave] + __popcll(t.sm[q][q / kWave] & below_mask(q % kWave));
        t.upf[q] = upf;
    }
    RowTotals r;
    const int pre = block_exclusive(cnt, t.sw, &r.edges);
    const int pup = block_exclusive(cnt - upf, t.sw, &r.upper);
    r.longest = LONGEST ? block_max(cnt, t.sw) : 0;
    if (q < n) {
        t.rptr[q] = pre;
        t.upp[q] = pup;
    }
    if (q == 0) t.rptr[n] = r.edges;
    return r;
}

// The totals of the build into the status words (block 0) and the error
// flags; returns whether the build failed (capacity or row length).
__device__ inline bool tile_publish_totals(const TileArgs &a, int64_t total, int max_row) {
    const bool fail = max_row > SN_MAX_ROW || total > a.capacity || total > INT32_MAX;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        a.status[kEdgeTotal] = (int)min(total, (int64_t)INT32_MAX);
        a.status[kMaxRow] = max_row;
        if (a.flag && fail) flag_status(a.status, max_row > SN_MAX_ROW ? SN_ERR_ROW : SN_ERR_CAPACITY);
        if (a.pr.edge_pair) a.status[kPairTotal] = fail ? 0 : (int)(total / 2);
    }
    return fail;
}

// Position of the j-th set bit (from 0) of m, which has more than j set bits.
__device__ inline int select_bit(uint64_t m, int j) {
    int pos = 0;
    int c = __popc((uint32_t)m);
    uint32_t x = (uint32_t)m;
    if (j >= c) {
        j -= c;
        x = (uint32_t)(m >> 32);
        pos = 32;
    }
#pragma unroll
    for (int sh = 16; sh >= 2; sh >>= 1) {
        c = __popc(x & ((1u << sh) - 1u));
        if (j >= c) {
            j -= c;
            x >>= sh;
            pos += sh;
        }
    }
    return pos + (j >= (int)(x & 1u) ? 1 : 0);
}

// Rows [q0, q1) of replica b (first atom s, n atoms; masks, positions and row
// offsets in LDS; `before` edges in earlier replicas): columns, reverse
// edges and, when asked for, the pair arrays.  One wavefront per row, one
// lane per edge: lane k finds the row's k-th set bit (the mask word from the
// word prefix counts, the bit by halving popcounts), so every lane has work
// instead of the few whose column bit is set in each word.
__device__ inline void tile_fill_rows(const TileArgs &a, const TileSmem &t, int s, int n, int q0, int q1,
                                      int64_t before) {
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    const int W = (n + kWave - 1) / kWave;
    const int64_t pbase = before / 2;           // pairs of the earlier replicas
    for (int r = q0 + wv; r < q1; r += kTileWaves) {
        const int i = s + r;
        const int len = t.rptr[r + 1] - t.rptr[r];
        const int64_t rbase = before + t.rptr[r];
        for (int k = lane; k < len; k += kWave) {
            int w = 0;                            // the word of the k-th set bit
            for (int u = 1; u < W; ++u)
                if (t.wpre[r][u] <= k) w = u;
            const int c = kWave * w + select_bit(t.sm[r][w], k - t.wpre[r][w]);   // column, local index
            const int64_t ed = rbase + k;
            a.col[ed] = s + c;
            // position of r in row c (present when the predicate is symmetric)
            const uint64_t mc = t.sm[c][r / kWave];
            const int kc = t.wpre[c][r / kWave] + __popcll(mc & below_mask(r % kWave));
            const bool sym = (mc >> (r % kWave)) & 1ull;
            if (!sym) flag_status(a.status, SN_ERR_INVALID);
            a.rev[ed] = sym ? (int)(before + t.rptr[c] + kc) : -1;
            if (!a.pr.edge_pair) continue;
            if (c > r) {
                const int64_t p = pbase + t.upp[r] + (k - t.upf[r]);
                a.pr.edge_pair[ed] = (int)p;
                a.pr.pair_ij[p] = make_int2(i, s + c);
                float4 g;
                float fc, lfc;
                pair_geometry(t.sp + 3 * r, t.sp + 3 * c, a.pp.periodic, a.pp.L, a.pp.invL, a.pr.cutoff, g, fc, lfc);
                a.pr.pgeo[p] = g;
                a.pr.pfc[p] = fc;
                a.pr.plfc[p] = lfc;
            } else {
                a.pr.edge_pair[ed] = sym ? (int)(pbase + t.upp[c] + (kc - t.upf[c])) : 0;
            }
        }
    }
}

__global__ __launch_bounds__(kTileThreads, 8) void tile_fill_kernel(TileArgs a) {
    __shared__ TileSmem t;
    __shared__ unsigned long long s_before, s_total;
    __shared__ int s_max, s_st;
    if (skipped(a.run_flag)) return;
    const int b = blockIdx.x / a.R, part = blockIdx.x % a.R;
    const int s = a.rptr[b], e = a.rptr[b + 1], n = e - s;
    const int lane = threadIdx.x % kWave;
    if (threadIdx.x == 0) {
        s_before = 0;
        s_total = 0;
        s_max = 0;
        s_st = *a.status;                         // read before this kernel flags anything
    }
    __syncthreads();
    {
        const int first = b * a.Rc;               // this replica's first count block: "before" = earlier replicas
        unsigned long long before = 0, total = 0;
        int mx = 0;
        for (int r = threadIdx.x; r < a.B * a.Rc; r += kTileThreads) {
            const unsigned long long v = (unsigned)a.rep[r];
            total += v;
            if (r < first) before += v;
            mx = max(mx, a.rep[a.B * a.Rc + r]);
        }
        // wavefront sums first: one LDS atomic per wavefront and value
        for (int o = 32; o > 0; o >>= 1) {
            total += __shfl_xor(total, o, kWave);
            before += __shfl_xor(before, o, kWave);
            mx = max(mx, __shfl_xor(mx, o, kWave));
        }
        if (lane == 0) {
            if (total) atomicAdd(&s_total, total);
            if (before) atomicAdd(&s_before, before);
            if (mx) atomicMax(&s_max, mx);
        }
    }
    __syncthreads();
    if (s_st != 0) return;                        // uniform: nothing is written after an error
    const int64_t before = (int64_t)s_before, total = (int64_t)s_total;
    const bool fail = tile_publish_totals(a, total, s_max);
    for (int k = threadIdx.x; k < n * kTileWords; k += kTileThreads)
        (&t.sm[0][0])[k] = a.mask[(int64_t)s * kTileWords + k];
    for (int k = threadIdx.x; k < 3 * n; k += kTileThreads) t.sp[k] = a.pos[3 * (int64_t)s + k];
    __syncthreads();
    const RowTotals rt = tile_row_offsets<false>(t, n);
    const int per = (n + a.R - 1) / a.R, q0 = part * per, q1 = min(n, q0 + per);
    const int q = threadIdx.x;
    if (q >= q0 && q < q1) a.row_ptr[s + q] = (int)(before + t.rptr[q]);
    if (blockIdx.x == gridDim.x - 1 && q == 0) a.row_ptr[a.N] = (int)min(total, (int64_t)INT32_MAX);
    if (fail) return;                             // uniform
    if (2 * rt.upper != rt.edges) {               // not symmetric: the pair numbering would not fit
        if (q == 0) flag_status(a.status, SN_ERR_INVALID);
        return;                                   // uniform
    }
    __syncthreads();
    tile_fill_rows(a, t, s, n, q0, q1, before);
}

// A system of one small replica (n <= kTileOneMax): count and fill in one
// launch.  Each block evaluates every row mask of the replica itself (n^2
// predicate tests, a few per thread at this size) into LDS, so no masks or
// counts go through global memory, then writes its share of the rows as the
// fill pass does.
__global__ __launch_bounds__(kTileThreads, 8) void tile_one_kernel(TileArgs a) {
    __shared__ TileSmem t;
    __shared__ int s_st;
    if (skipped(a.run_flag)) return;
    const int s = a.rptr[0], n = a.rptr[1] - s;
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    if (threadIdx.x == 0) {
        s_st = *a.status;                         // read before this kernel flags anything
        if (blockIdx.x == 0 && a.step_mark >= 0 && s_st == 0) a.status[kStepsDone] = a.step_mark;
    }
    if (tile_positions(a.pos, s, n, t.sp)) {      // (holds a barrier, so s_st is visible below)
        if (blockIdx.x == 0 && threadIdx.x == 0) flag_status(a.status, SN_ERR_NONFINITE);
        return;                                   // uniform
    }
    if (s_st != 0) return;                        // uniform: nothing is written after an error
    const int W = (n + kWave - 1) / kWave;
    for (int q = wv; q < n; q += kTileWaves) {
        const float xi = t.sp[3 * q], yi = t.sp[3 * q + 1], zi = t.sp[3 * q + 2];
#pragma unroll
        for (int w = 0; w < kTileWords; ++w) {
            if (w >= W) break;
            const int j = kWave * w + lane, jj = j < n ? j : 0;
            const float4 pj = make_float4(t.sp[3 * jj], t.sp[3 * jj + 1], t.sp[3 * jj + 2], 0.0f);
            const bool pass = j < n && j != q && within(xi, yi, zi, pj, a.pp);
            const uint64_t m = __ballot(pass);
            if (lane == 0) t.sm[q][w] = m;
        }
    }
    __syncthreads();
    const RowTotals rt = tile_row_offsets<true>(t, n);
    const bool fail = tile_publish_totals(a, rt.edges, rt.longest);
    const int per = (n + gridDim.x - 1) / gridDim.x, q0 = blockIdx.x * per, q1 = min(n, q0 + per);
    const int q = threadIdx.x;
    if (q >= q0 && q < q1) a.row_ptr[s + q] = t.rptr[q];
    if (blockIdx.x == gridDim.x - 1 && q == 0) a.row_ptr[a.N] = rt.edges;
    if (fail) return;                             // uniform
    if (2 * rt.upper != rt.edges) {               // not symmetric: the pair numbering would not fit
        if (q == 0) flag_status(a.status, SN_ERR_INVALID);
        return;                                   // uniform
    }
    __syncthreads();
    tile_fill_rows(a, t, s, n, q0, q1, 0);
}
}  // namespace

sn_status scan_exclusive(const int32_t *in, int32_t *out, int n, int32_t *total_slot, int32_t *max_slot,
                         hipStream_t s, PairCountCheck chk, const int *run_flag) {
    ProfScope ps(K_NB_SCAN, s);
    if (n < 0 || in == out) return SN_ERR_INVALID;
    const int ntiles = n > 0 ? (n + kScanTile - 1) / kScanTile : 1;
    scan_kernel<<<ntiles, kScanThreads, 0, s>>>(in, out, n, total_slot, max_slot, chk, run_flag);
    return launch_status();
}

static sn_status fill_int(int *p, int v, int64_t n, hipStream_t s) {
    if (n <= 0) return SN_OK;
    fill_int_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p, v, n);
    return launch_status();
}

// Blocks per replica of the cell-grid set-up: about 256 in all.
static int grid_parts(int B) { return B >= 256 ? 1 : (256 + B - 1) / B; }

NbLayout nb_layout(const sn_system &sys, size_t base) {
    NbLayout L;
    const int64_t N = sys.n_atoms, B = sys.n_replicas;
    L.n_cells = 8 * N + 64 * B;
    size_t o = base;
    L.grid = o;       o = align256(o + sizeof(CellGrid) * B);
    L.gpart = o;      o = align256(o + 4 * 8 * (int64_t)B * grid_parts((int)B));
    L.rep_of = o;     o = align256(o + 4 * N);
    L.cell_of = o;    o = align256(o + 4 * N);
    L.cell_cnt = o;   o = align256(o + 4 * (L.n_cells + 1));
    L.cell_start = o; o = align256(o + 4 * (L.n_cells + 1));
    L.cell_fill = o;  o = align256(o + 4 * (L.n_cells + 1));
    L.spos = o;       o = align256(o + 16 * N);
    L.row_cnt = o;    o = align256(o + 4 * N);
    L.keep = o;       o = align256(o + 4 * (int64_t)kRowKeep * N);
    L.rep = o;        o = align256(o + 8 * kTileMaxSplit * B);
    L.mask = o;       o = align256(o + 8 * kTileWords * N);
    L.total = o;
    return L;
}

int max_replica_atoms(const sn_system &sys, hipStream_t s) {
    const int B = sys.n_replicas;
    std::vector<int32_t> h((size_t)B + 1);
    if (hipMemcpyAsync(h.data(), sys.replica_ptr, 4 * ((size_t)B + 1), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return -1;
    if (h[0] != 0 || h[B] != sys.n_atoms) return -1;
    int m = 0;
    for (int b = 0; b < B; ++b) {
        if (h[b + 1] < h[b]) return -1;
        m = std::max(m, h[b + 1] - h[b]);
    }
    return m;
}

// The build's counters (status, longest row, edge total), read back into
// host memory of the caller's thread: a copy into pageable memory, then the
// stream is synchronised (no library-wide host buffer, so calls on other
// streams or threads cannot overwrite each other's counters).
static sn_status read_counters(const int *status, int (&host)[4], hipStream_t s) {
    SN_HIP(hipMemcpyAsync(host, status, sizeof(host), hipMemcpyDeviceToHost, s));
    SN_HIP(hipStreamSynchronize(s));
    return SN_OK;
}

sn_status nb_build(const sn_system &sys, const float *pos, float r_list, int32_t *row_ptr, int32_t *col,
                   int32_t *rev, int64_t capacity, int64_t *n_edges, char *ws, hipStream_t s, bool sync,
                   int max_rep, const NbPairOut *pairs, bool *pairs_done, int step_mark, const int *run_flag) {
    if (pairs_done) *pairs_done = false;
    const int N = sys.n_atoms, B = sys.n_replicas;
    int *status = reinterpret_cast<int *>(ws);
    PredParams pp;
    pp.rl2 = r_list * r_list;
    pp.periodic = sys.periodic ? 1 : 0;
    for (int c = 0; c < 3; ++c) {
        pp.L[c] = sys.periodic ? sys.box[c] : 1.0f;
        pp.invL[c] = (float)(1.0 / (double)pp.L[c]);
    }
    // cell edge with a margin above r_list: rounding in the cell index can never
    // hide a pair that passes the fp32 predicate
    const float cell_edge = r_list * 1.001f + 0.01f;
    if (sys.periodic)
        for (int c = 0; c < 3; ++c)
            if (!(sys.box[c] > 0.0f) || (int)floorf(sys.box[c] / cell_edge) < 3) return SN_ERR_BOX;

    NbLayout L = nb_layout(sys, kWsBase);
    CellGrid *grid = reinterpret_cast<CellGrid *>(ws + L.grid);
    int *rep_of = reinterpret_cast<int *>(ws + L.rep_of);
    int *cell_of = reinterpret_cast<int *>(ws + L.cell_of);
    int *cell_cnt = reinterpret_cast<int *>(ws + L.cell_cnt);
    int *cell_start = reinterpret_cast<int *>(ws + L.cell_start);
    int *cell_fill = reinterpret_cast<int *>(ws + L.cell_fill);
    float4 *spos = reinterpret_cast<float4 *>(ws + L.spos);
    int *row_cnt = reinterpret_cast<int *>(ws + L.row_cnt);

    // reset the counters but keep the status word: an error flagged by earlier
    // work on this workspace (e.g. a non-finite force) is reported below
    if (N == 0) {
        SN_TRY(fill_int(row_ptr, 0, 1, s));
        *n_edges = 0;
        return SN_OK;
    }
    if (max_rep >= 0 && max_rep <= kRepMaxAtoms && B <= kRepMaxReplicas) {
        TileArgs a;
        a.pos = pos;
        a.rptr = sys.replica_ptr;
        a.B = B;
        a.N = N;
        // blocks per replica: about one per CU for the count pass and two for
        // the fill pass (measured best on 64 replicas)
        a.Rc = std::min(kTileMaxSplit, std::max(1, (256 + B - 1) / B));
        a.R = std::min(kTileMaxSplit, std::max(1, (512 + B - 1) / B));
        a.pp = pp;
        a.mask = pairs ? pairs->mask : reinterpret_cast<uint64_t *>(ws + L.mask);
        a.rep = pairs ? pairs->rep : reinterpret_cast<int32_t *>(ws + L.rep);
        a.row_ptr = row_ptr;
        a.col = col;
        a.rev = rev;
        a.capacity = capacity;
        a.flag = sync ? 0 : 1;
        a.pr = pairs ? *pairs : NbPairOut{};
        a.step_mark = step_mark;
        a.status = status;
        a.run_flag = run_flag;
        if (B == 1 && max_rep <= kTileOneMax) {
            // one small replica: a block per 16 rows (one per wavefront)
            ProfScope ps(K_NB_FILL, s);
            const int R = std::max(1, (max_rep + kTileWaves - 1) / kTileWaves);
            tile_one_kernel<<<R, kTileThreads, 0, s>>>(a);
            SN_TRY(launch_status());
        } else {
            {
                ProfScope ps(K_NB_COUNT, s);
                tile_count_kernel<<<B * a.Rc, kTileThreads, 0, s>>>(a);
                SN_TRY(launch_status());
            }
            {
                ProfScope ps(K_NB_FILL, s);
                tile_fill_kernel<<<B * a.R, kTileThreads, 0, s>>>(a);
                SN_TRY(launch_status());
            }
        }
        if (pairs_done) *pairs_done = pairs != nullptr;
        if (sync) {
            int host[4];
            SN_TRY(read_counters(status, host, s));
            const int st = host[kStatusWord], max_row = host[kMaxRow];
            *n_edges = host[kEdgeTotal];
            if (st != 0) return st;
            if (max_row > SN_MAX_ROW) return SN_ERR_ROW;
            if (*n_edges > capacity) return SN_ERR_CAPACITY;
        }
        return SN_OK;
    }
    {
        ProfScope ps(K_NB_GRID, s);
        const int R = grid_parts(B);
        float *part = reinterpret_cast<float *>(ws + L.gpart);
        grid_part_kernel<<<B * R, 256, 0, s>>>(pos, sys.replica_ptr, R, part, rep_of, cell_cnt, cell_fill,
                                               L.n_cells, step_mark, status, run_flag);
        SN_TRY(launch_status());
        grid_make_kernel<<<B, 64, 0, s>>>(sys.replica_ptr, R, part, pp, cell_edge, grid, status, run_flag);
        SN_TRY(launch_status());
    }
    {
        ProfScope ps(K_NB_BIN, s);
        bin_kernel<<<(N + 255) / 256, 256, 0, s>>>(pos, N, grid, rep_of, pp, cell_of, cell_cnt, run_flag);
        SN_TRY(launch_status());
    }
    SN_TRY(scan_exclusive(cell_cnt, cell_start, (int)L.n_cells, nullptr, nullptr, s, PairCountCheck{}, run_flag));
    {
        ProfScope ps(K_NB_BIN, s);
        place_kernel<<<(N + 255) / 256, 256, 0, s>>>(pos, N, cell_of, cell_start, cell_fill, spos, run_flag);
        SN_TRY(launch_status());
    }
    const int blocks = (N + kNbWaves - 1) / kNbWaves;
    int32_t *keep = reinterpret_cast<int32_t *>(ws + L.keep);
    {
        ProfScope ps(K_NB_COUNT, s);
        rows_kernel<false><<<blocks, kWave * kNbWaves, 0, s>>>(pos, N, grid, rep_of, cell_start, spos, pp,
                                                               row_cnt, keep, nullptr, nullptr, capacity, status,
                                                               run_flag);
        SN_TRY(launch_status());
    }
    SN_TRY(scan_exclusive(row_cnt, row_ptr, N, status + kEdgeTotal, status + kMaxRow, s, PairCountCheck{},
                          run_flag));
    if (sync) {
        int host[4];
        SN_TRY(read_counters(status, host, s));
        const int st = host[kStatusWord], max_row = host[kMaxRow];
        const int64_t E = host[kEdgeTotal];
        *n_edges = E;
        if (st != 0) return st;
        if (max_row > SN_MAX_ROW) return SN_ERR_ROW;
        if (E > capacity) return SN_ERR_CAPACITY;
    }
    {
        ProfScope ps(K_NB_FILL, s);
        rows_kernel<true><<<blocks, kWave * kNbWaves, 0, s>>>(pos, N, grid, rep_of, cell_start, spos, pp, nullptr,
                                                              keep, row_ptr, col, capacity, status, run_flag);
        SN_TRY(launch_status());
    }
    {
        ProfScope ps(K_NB_REV, s);
        rev_kernel<<<(N + 3) / 4, 256, 0, s>>>(N, row_ptr, col, rev, status, run_flag);
        SN_TRY(launch_status());
    }
    return SN_OK;
}

}  // namespace sn
