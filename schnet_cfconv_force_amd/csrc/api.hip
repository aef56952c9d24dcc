// C-ABI entry points of libsn.so: argument checks, workspace carving, the
// energy/force pipeline, the velocity-Verlet driver and per-kernel timing.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "sn_internal.h"

namespace sn {

// --------------------------------------------------------------- timing
//
// The per-kernel timer is the library's only process-wide state: a switch
// and the lists of recorded events, all behind one mutex (the switch is an
// atomic).  It is a measuring aid, off unless sn_profile_enable() turns it
// on; launches recorded into a HIP graph are never timed.

namespace {
struct ProfRecord {
    int cls;
    hipEvent_t start, stop;
};
std::atomic<bool> g_prof_on{false};
thread_local bool t_capturing = false;   // this thread is recording a HIP graph
std::mutex g_prof_mu;
std::vector<ProfRecord> g_prof_open;   // started, not yet stopped (stack per class)
std::vector<ProfRecord> g_prof_done;
std::vector<hipEvent_t> g_event_pool;  // reused events (creating events is slow)
const char *kClassNames[K_NUM_CLASSES] = {
    "nb_grid", "nb_bin", "nb_scan", "nb_count", "nb_fill", "nb_rev", "pairs", "mlp",
    "filter_fwd", "cfconv", "filter_bwd", "forces", "verlet", "kinetic", "pack"};
}  // namespace

static hipEvent_t pooled_event() {
    if (!g_event_pool.empty()) {
        hipEvent_t e = g_event_pool.back();
        g_event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

void prof_begin(int cls, hipStream_t s) {
    if (!g_prof_on.load(std::memory_order_relaxed) || t_capturing) return;
    std::lock_guard<std::mutex> g(g_prof_mu);
    ProfRecord r{cls, pooled_event(), pooled_event()};
    if (!r.start || !r.stop) return;
    hipEventRecord(r.start, s);
    g_prof_open.push_back(r);
}

void prof_end(int cls, hipStream_t s) {
    if (!g_prof_on.load(std::memory_order_relaxed) || t_capturing) return;
    std::lock_guard<std::mutex> g(g_prof_mu);
    for (size_t k = g_prof_open.size(); k-- > 0;) {
        if (g_prof_open[k].cls == cls) {
            ProfRecord r = g_prof_open[k];
            g_prof_open.erase(g_prof_open.begin() + k);
            hipEventRecord(r.stop, s);
            g_prof_done.push_back(r);
            return;
        }
    }
}

// --------------------------------------------------------------- layout

EfLayout ef_layout(const sn_model &m, const sn_system &sys, int64_t E, size_t base) {
    EfLayout L;
    const int64_t N = sys.n_atoms, P = E / 2, F = m.n_features, I = m.n_interactions;
    const int64_t B = sys.n_replicas;
    size_t o = base;
    auto take = [&](size_t bytes) { size_t r = o; o = align256(o + bytes); return r; };
    L.up_first = take(4 * N);
    L.up_cnt = take(4 * N);
    L.up_ptr = take(4 * (N + 1));
    L.edge_pair = take(4 * E);
    L.pair_ij = take(8 * P);
    L.pgeo = take(16 * P);
    L.pfc = take(4 * P);
    L.plfc = take(4 * P);
    L.phi = take(4 * I * P * fp24_words((int)F));   // 24-bit filter rows
    L.x = take(4 * I * N * F);
    L.o = take(4 * I * N * F);
    L.gy = take(4 * I * N * F);
    L.h = take(4 * N * F);
    L.y = take(4 * N * F);
    L.gh = take(4 * N * F);
    L.eps = take(4 * N + 4 * B);   // eps[N], then an energy scratch [B]
    L.S = take(4 * P * I);   // one slice per interaction (small systems; otherwise slice 0 accumulates)
    L.xmax = take(4 * I * N);
    L.gmax = take(4 * I * N);
    L.pack = take(pack_bytes((int)I));
    L.rep = take(8 * kTileMaxSplit * B);   // the tile neighbour build's per-block counts
    L.mask = take(8 * (kRepMaxAtoms / 64) * N);   // and its row masks
    L.h0 = take(4 * N * F);                // the embedding rows (kept across MD steps)
    L.ref_pos = take(12 * N);              // positions at the last neighbour build (skin)
    L.total = o;
    return L;
}

namespace {

__global__ void clear_status_kernel(int *status) {
    if (threadIdx.x < kStatusSlots) status[threadIdx.x] = 0;
}

sn_status clear_status(void *ws, hipStream_t s) {
    clear_status_kernel<<<1, 64, 0, s>>>(reinterpret_cast<int *>(ws));
    return launch_status();
}

// A step's opening half kick v += dt/2 c F / m and drift r += dt v (the
// closing kick runs in the force assembly).  Nothing moves once an error is
// flagged.  Device-driven steps (n_total >= 0): only when the current step
// (status slot kMdStep minus one) is not the call's last; with ref_pos set,
// an atom that ends more than sqrt(half_skin2) from it sets kDisplaced.
__global__ void open_step_kernel(int N, float *pos, float *vel, const float *forces, const float *inv_mass,
                                 float half_dt_c, float dt, int *status, int n_total, const float *ref_pos,
                                 float half_skin2) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= N || status[kStatusWord] != 0) return;
    if (n_total >= 0 && status[kMdStep] >= n_total) return;
    float r2 = 0.0f;
    for (int c = 0; c < 3; ++c) {
        // explicit fused multiply-adds, as in the force assembly's kicks
        const float v = fmaf(half_dt_c * forces[3 * i + c], inv_mass[i], vel[3 * i + c]);
        const float r = fmaf(dt, v, pos[3 * i + c]);
        pos[3 * i + c] = r;
        vel[3 * i + c] = v;
        if (ref_pos) {
            const float dr = r - ref_pos[3 * i + c];
            r2 = fmaf(dr, dr, r2);
        }
    }
    if (ref_pos && !(r2 <= half_skin2))
        __hip_atomic_store(status + kDisplaced, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The first launch of a device-driven MD step (one thread): advances the
// step counter, records the step as begun while no error is flagged, and
// decides whether the step rebuilds the neighbour list: at the call's first
// step, when an atom left half the skin during the last drift, and every
// rebuild_every steps (0: only on displacement).
__global__ void md_begin_kernel(int *status, int rebuild_every) {
    if (threadIdx.x != 0) return;
    const int step = status[kMdStep];
    status[kMdStep] = step + 1;
    if (status[kStatusWord] == 0) status[kStepsDone] = step;
    const bool build = step == 0 || status[kDisplaced] != 0 ||
                       (rebuild_every > 0 && step - status[kLastBuild] >= rebuild_every);
    status[kBuildFlag] = build ? 1 : 0;
    status[kDisplaced] = 0;
    if (build) status[kLastBuild] = step;
}

// out[b] = sum over replica b of m v^2 / (2 c), in fp64; step_status (may be
// null): device-driven steps, out[(status[kMdStep] - 1) B + b]
__global__ __launch_bounds__(256) void kinetic_kernel(const int32_t *rptr, const float *vel, const float *inv_mass,
                                                      double inv_2c, double *out, const int *step_status) {
    __shared__ double red[256];
    const int b = blockIdx.x;
    if (step_status) out += (int64_t)(step_status[kMdStep] - 1) * gridDim.x;
    double s = 0.0;
    for (int i = rptr[b] + threadIdx.x; i < rptr[b + 1]; i += 256) {
        double v2 = (double)vel[3 * i] * vel[3 * i] + (double)vel[3 * i + 1] * vel[3 * i + 1] +
                    (double)vel[3 * i + 2] * vel[3 * i + 2];
        s += v2 / (double)inv_mass[i];
    }
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[b] = red[0] * inv_2c;
}

sn_status check_system(const sn_system *sys) {
    if (!sys || sys->n_atoms < 0 || sys->n_replicas < 1 || !sys->replica_ptr) return SN_ERR_INVALID;
    if (sys->n_atoms > 0 && !sys->types) return SN_ERR_INVALID;
    if (sys->periodic)
        for (int c = 0; c < 3; ++c)
            if (!(sys->box[c] > 0.0f) || !std::isfinite(sys->box[c])) return SN_ERR_BOX;
    return SN_OK;
}

sn_status check_model(const sn_model *m) {
    if (!m || !m->params || (reinterpret_cast<uintptr_t>(m->params) & 15) != 0) return SN_ERR_INVALID;
    const int F = m->n_features;
    if (F != 32 && F != 64 && F != 128) return SN_ERR_INVALID;
    if (m->n_rbf < 2 || m->n_rbf > 64 || m->n_interactions < 1 || m->n_interactions > 16 || m->n_types < 1)
        return SN_ERR_INVALID;
    if (!(m->cutoff > 0.0f) || !(m->rbf_gamma > 0.0f) || !std::isfinite(m->rbf_lo) || !std::isfinite(m->rbf_hi))
        return SN_ERR_INVALID;
    if (m->filter_format != 0 && m->filter_format != 1) return SN_ERR_INVALID;
    if (m->filter_format == 1 && (!m->qweights || !m->qscales)) return SN_ERR_INVALID;
    if (m->filter_math != 0 && m->filter_math != 1) return SN_ERR_INVALID;
    return SN_OK;
}

sn_status check_ws(void *ws, size_t ws_bytes, size_t need) {
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255) != 0 || ws_bytes < need) return SN_ERR_WORKSPACE;
    return SN_OK;
}

size_t bytes_needed(const sn_model *m, const sn_system *s, int64_t E) {
    size_t nb = nb_layout(*s, kWsBase).total;
    size_t ef = m ? ef_layout(*m, *s, E, kWsBase).total : kWsBase;
    return std::max(nb, ef);
}

// The pipeline itself; arguments already checked, status not cleared.
// device_edges: E is only the edge capacity (workspace layout and launch
// sizes); the edge and pair counts are taken on the device (row_ptr[N]), so
// nothing is read back to the host, and the kernels that read the CSR do
// nothing once an error is flagged (the neighbour build may then have left
// the rows unfilled).  packed: the weight pack in the workspace is current
// (written by filter_pack and mlp_pack since the weights last changed).
// pairs_ready: the neighbour build has written the pair arrays and count.
// vf: the integrator's part applied with the forces (MD steps).
// embedded: h0, x_0 and its row maxima are current (the types do not change
// during an MD call).
// build_flag (may be null): the pair setup runs only when *build_flag is set
// (device-driven MD steps; on the others the pair arrays are kept and their
// geometry refreshed).  elog (may be null): the replica energies in fp64,
// at elog[step B + b] with elog_by_step (device-driven steps).  energy may be
// null when elog is set.
sn_status energy_forces_impl(const sn_model &m, const sn_system &sys, const float *pos, const int32_t *row_ptr,
                             const int32_t *col, const int32_t *rev, int64_t E, float *energy, float *forces,
                             char *ws, hipStream_t s, bool device_edges = false, bool packed = false,
                             bool pairs_ready = false, const VerletFuse *vf = nullptr, bool embedded = false,
                             const int *build_flag = nullptr, double *elog = nullptr, int elog_by_step = 0) {
    const int N = sys.n_atoms, B = sys.n_replicas, F = m.n_features, I = m.n_interactions;
    const int64_t P = E / 2;
    int *status = reinterpret_cast<int *>(ws);
    const EfLayout L = ef_layout(m, sys, E, kWsBase);
    float *eps = reinterpret_cast<float *>(ws + L.eps);
    if (N == 0)
        return forces_rows(0, B, sys.replica_ptr, eps, energy, row_ptr, col, nullptr, nullptr, nullptr, 1, 0, forces,
                           status, nullptr, vf, s, elog, elog_by_step);

    int64_t off[9 * 16 + 6];
    sn_param_offsets(m.n_types, I, F, m.n_rbf, off, (int32_t)(sizeof(off) / sizeof(off[0])));
    const float *prm = m.params;
    auto blk = [&](int t, int k) { return prm + off[1 + 9 * t + k]; };
    enum { W_IN = 0, A1, B1, A2, B2, WO1, BO1, WO2, BO2 };
    const float *R1 = prm + off[1 + 9 * I], *c1 = prm + off[2 + 9 * I], *R2 = prm + off[3 + 9 * I],
                *c2 = prm + off[4 + 9 * I];

    auto F32 = [&](size_t o) { return reinterpret_cast<float *>(ws + o); };
    const int32_t *edge_pair = reinterpret_cast<const int32_t *>(ws + L.edge_pair);
    const int2 *pair_ij = reinterpret_cast<const int2 *>(ws + L.pair_ij);
    const float4 *pgeo = reinterpret_cast<const float4 *>(ws + L.pgeo);
    const float *pfc = F32(L.pfc);
    const float *plfc = F32(L.plfc);
    float *h = F32(L.h), *y = F32(L.y), *gh = F32(L.gh), *h0 = F32(L.h0);
    float *S = F32(L.S);
    const int64_t NF = (int64_t)N * F;
    auto phi_t = [&](int t) { return reinterpret_cast<uint32_t *>(ws + L.phi) + P * fp24_words(F) * t; };
    auto x_t = [&](int t) { return F32(L.x) + NF * t; };
    auto o_t = [&](int t) { return F32(L.o) + NF * t; };
    auto gy_t = [&](int t) { return F32(L.gy) + NF * t; };
    auto xmax_t = [&](int t) { return F32(L.xmax) + (int64_t)N * t; };
    auto gmax_t = [&](int t) { return F32(L.gmax) + (int64_t)N * t; };

    char *pack = ws + L.pack;
    const int *p_dev = status + kPairTotal;   // the pair count, written by the pair setup
    const int *guard = device_edges ? status : nullptr;
    auto pk = [&](int t, int kind) { return pack_ref(pack, I, pack_slot(t, kind)); };
    auto pr = [&](int k) { return pack_ref(pack, I, pack_readout_slot(I, k)); };

    // Every kernel on the caller's stream, in this order.  The filter network
    // depends only on the pair distances and could run beside the atom-wise
    // chain on a second stream, but its persistent blocks fill every CU, so
    // little overlaps, while each cross-stream hand-off leaves the GPU idle
    // for about 12 us; one stream measured 3 % faster per MD step.
    if (!packed) {
        SN_TRY(filter_pack(m, pack, s));
        SN_TRY(mlp_pack(m, pack, s));
    }
    if (!pairs_ready)
        SN_TRY(pairs_setup(sys, pos, row_ptr, col, rev, device_edges ? -1 : E, m.cutoff, ws, L, status, guard, s,
                           build_flag));
    // few pairs: every interaction's rows in one launch (they are small, so
    // the cache argument below does not apply)
    const bool fused = filter_forward_fused(m, P);
    if (fused) {
        uint32_t *rows[16];
        for (int t = 0; t < I; ++t) rows[t] = phi_t(t);
        SN_TRY(filter_forward_all(m, pgeo, pfc, P, rows, pack, p_dev, guard, s));
    } else {
        SN_TRY(filter_forward(m, 0, pgeo, pfc, P, phi_t(0), pack, p_dev, guard, s));
    }
    if (!embedded)
        SN_TRY(mlp_embed_x(N, F, m.n_types, sys.types, prm + off[0], pk(0, PK_XW), h0, x_t(0), xmax_t(0), status, s));
    for (int t = 0; t < I; ++t) {
        SN_TRY(cfconv(F, N, row_ptr, col, edge_pair, phi_t(t), x_t(t), y, guard, s));
        if (t + 1 < I) {
            SN_TRY(mlp_out_x(N, F, y, pk(t, PK_OW1), blk(t, BO1), pk(t, PK_OW2), blk(t, BO2), pk(t + 1, PK_XW),
                             o_t(t), t == 0 ? h0 : h, h, x_t(t + 1), xmax_t(t + 1), s));
            // the next interaction's rows are written right before their
            // CFConv: the rows a kernel writes are not kept in the Infinity
            // Cache, but the part written last is still in L2 when it starts
            if (!fused) SN_TRY(filter_forward(m, t + 1, pgeo, pfc, P, phi_t(t + 1), pack, p_dev, guard, s));
        } else {   // the last interaction, the readout and the first backward block
            SN_TRY(mlp_tail(N, F, y, pk(t, PK_OW1), blk(t, BO1), pk(t, PK_OW2), blk(t, BO2), t == 0 ? h0 : h, pr(0),
                            c1, pr(1), R2, c2, pk(t, PK_BOW1), pk(t, PK_BOW2), eps, gh, gy_t(t), gmax_t(t), s));
        }
    }
    // backward through the interactions in reverse (g_y of t is ready).  The
    // input-gradient CFConv (not needed below the first block) goes first:
    // for the last interaction its rows are still in the Infinity Cache,
    // where the forward CFConv's reads left them; the filter backward does
    // not read them.
    // With few pairs the filter backward of every interaction runs as one
    // launch after the chain (each g_y_t is kept), each interaction into its
    // own S slice; the force assembly adds the slices in the order of the
    // per-interaction accumulation.
    for (int t = I - 1; t >= 0; --t) {
        if (t > 0) SN_TRY(cfconv(F, N, row_ptr, col, edge_pair, phi_t(t), gy_t(t), y, guard, s));
        if (!fused)
            SN_TRY(filter_backward(m, t, pgeo, pfc, plfc, pair_ij, P, N, x_t(t), gy_t(t), xmax_t(t), gmax_t(t), S,
                                   t != I - 1, pack, p_dev, guard, s));
        if (t > 0) {
            SN_TRY(mlp_bx_bo(N, F, y, pk(t, PK_BXW), pk(t - 1, PK_BOW1), o_t(t - 1), pk(t - 1, PK_BOW2), gh,
                             gy_t(t - 1), gmax_t(t - 1), s));
        }
    }
    if (fused) {
        const float *xs[16], *gys[16], *xm[16], *gm[16];
        for (int t = 0; t < I; ++t) {
            xs[t] = x_t(t);
            gys[t] = gy_t(t);
            xm[t] = xmax_t(t);
            gm[t] = gmax_t(t);
        }
        SN_TRY(filter_backward_all(m, pgeo, pfc, plfc, pair_ij, P, xs, gys, xm, gm, S, pack, p_dev, guard, s));
    }
    return forces_rows(N, B, sys.replica_ptr, eps, energy, row_ptr, col, edge_pair, pgeo, S, fused ? I : 1, P, forces,
                       status, guard, vf, s, elog, elog_by_step);
}

// Ends a stream capture that an error interrupted and frees what it made.
struct CaptureGuard {
    hipStream_t cs = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    bool open = false;
    ~CaptureGuard() {
        t_capturing = false;
        if (open) {
            hipGraph_t g = nullptr;
            (void)hipStreamEndCapture(cs, &g);
            if (g) (void)hipGraphDestroy(g);
        }
        if (exec) (void)hipGraphExecDestroy(exec);
        if (graph) (void)hipGraphDestroy(graph);
        if (cs) (void)hipStreamDestroy(cs);
    }
};

}  // namespace
}  // namespace sn

// --------------------------------------------------------------- no-allocation variant
//
// sn_energy_forces_static runs the energy/force pipeline with its scratch in
// `scratch`, a file-scope device array of a fixed size, instead of a
// caller's workspace, for callers that cannot allocate.  In host code the
// array's name only stands in for the symbol: its device address (one per
// GPU, each GPU holding its own copy from module load until the process
// ends) is looked up with hipGetSymbolAddress on the first call on each
// device, with that device current, and kept in a per-device table; only
// that address is ever passed to kernels.
namespace sn {
constexpr size_t kStaticScratchBytes = size_t(64) << 20;   // 64 MiB per GPU
constexpr int kStaticScratchDevices = 64;
}  // namespace sn

static __device__ __align__(256) char scratch[sn::kStaticScratchBytes];

namespace sn {
namespace {
std::mutex g_scratch_mu;
char *g_scratch_ptr[kStaticScratchDevices] = {};

// The device address of `scratch` on the current device (looked up once per device).
sn_status static_scratch(char **out) {
    int dev = -1;
    SN_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kStaticScratchDevices) return SN_ERR_INVALID;
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SN_ERR_HIP;
        g_scratch_ptr[dev] = static_cast<char *>(p);
    }
    *out = g_scratch_ptr[dev];
    return SN_OK;
}

__global__ void copy_status_kernel(const int *status, int32_t *out) {
    if (threadIdx.x == 0) *out = status[kStatusWord];
}
}  // namespace
}  // namespace sn

using namespace sn;

extern "C" {

int32_t sn_version(void) { return 3; }

const char *sn_status_string(sn_status st) {
    switch (st) {
        case SN_OK: return "ok";
        case SN_ERR_INVALID: return "invalid argument";
        case SN_ERR_CAPACITY: return "edge capacity too small";
        case SN_ERR_BOX: return "periodic box too small for the neighbour cutoff";
        case SN_ERR_HIP: return "HIP runtime error";
        case SN_ERR_NONFINITE: return "non-finite value";
        case SN_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case SN_ERR_ROW: return "neighbour row longer than SN_MAX_ROW";
        default: return "unknown status";
    }
}

int32_t sn_param_offsets(int32_t T, int32_t I, int32_t F, int32_t K, int64_t *offsets, int32_t max_offsets) {
    if (T < 1 || I < 1 || F < 2 || (F % 2) || K < 1) return -1;
    const int32_t n = 9 * I + 6;
    const int64_t H = F / 2;
    std::vector<int64_t> tab;
    tab.reserve(n);
    int64_t o = 0;
    tab.push_back(o); o += (int64_t)T * F;                          // Emb
    for (int t = 0; t < I; ++t) {
        const int64_t sizes[9] = {(int64_t)F * F, (int64_t)K * F, F, (int64_t)F * F, F,
                                  (int64_t)F * F, F, (int64_t)F * F, F};
        for (int k = 0; k < 9; ++k) { tab.push_back(o); o += sizes[k]; }
    }
    tab.push_back(o); o += F * H;     // R1
    tab.push_back(o); o += H;         // c1
    tab.push_back(o); o += H;         // R2
    tab.push_back(o); o += 1;         // c2
    tab.push_back(o);                 // total
    if (offsets)
        for (int32_t k = 0; k < std::min(n, max_offsets); ++k) offsets[k] = tab[k];
    return n;
}

int64_t sn_param_count(int32_t T, int32_t I, int32_t F, int32_t K) {
    int64_t off[9 * 16 + 6];
    if (I > 16) {
        std::vector<int64_t> v(9 * I + 6);
        if (sn_param_offsets(T, I, F, K, v.data(), (int32_t)v.size()) < 0) return -1;
        return v.back();
    }
    int32_t n = sn_param_offsets(T, I, F, K, off, 9 * 16 + 6);
    return n < 0 ? -1 : off[n - 1];
}

sn_status sn_quantize_filter_weights(int32_t T, int32_t I, int32_t F, int32_t K, const float *params_host,
                                     int16_t *q_host, float *s_host) {
    if (!params_host || !q_host || !s_host) return SN_ERR_INVALID;
    std::vector<int64_t> off(9 * (size_t)std::max(I, 1) + 6);
    if (sn_param_offsets(T, I, F, K, off.data(), (int32_t)off.size()) < 0) return SN_ERR_INVALID;
    for (int t = 0; t < I; ++t) {
        for (int which = 0; which < 2; ++which) {
            const int rows = which == 0 ? K : F;
            const float *w = params_host + off[1 + 9 * t + (which == 0 ? 1 : 3)];
            int16_t *q = q_host + ((int64_t)K * F + (int64_t)F * F) * t + (which == 0 ? 0 : (int64_t)K * F);
            float *sc = s_host + (int64_t)2 * F * t + (which == 0 ? 0 : F);
            for (int f = 0; f < F; ++f) {
                float amax = 0.0f;
                for (int k = 0; k < rows; ++k) amax = std::max(amax, std::fabs(w[(int64_t)k * F + f]));
                const float s = (float)((double)amax / 32767.0);
                sc[f] = s;
                for (int k = 0; k < rows; ++k) {
                    double r = s > 0.0f ? (double)w[(int64_t)k * F + f] / (double)s : 0.0;
                    r = std::nearbyint(r);   // default rounding mode: to nearest, ties to even
                    r = std::min(32767.0, std::max(-32767.0, r));
                    q[(int64_t)k * F + f] = (int16_t)r;
                }
            }
        }
    }
    return SN_OK;
}

size_t sn_workspace_bytes(const sn_model *model, const sn_system *sys, int64_t max_edges) {
    if (!sys || max_edges < 0) return 0;
    return bytes_needed(model, sys, max_edges);
}

sn_status sn_build_csr_neighbors(const sn_system *sys, const float *pos, float r_list, int32_t *row_ptr,
                                 int32_t *col_idx, int32_t *rev_idx, int64_t capacity, int64_t *n_edges, void *ws,
                                 size_t ws_bytes, void *stream) {
    SN_TRY(check_system(sys));
    if (!n_edges || !row_ptr || capacity < 0 || !(r_list > 0.0f) || !std::isfinite(r_list)) return SN_ERR_INVALID;
    if (sys->n_atoms > 0 && (!pos || (capacity > 0 && (!col_idx || !rev_idx)))) return SN_ERR_INVALID;
    SN_TRY(check_ws(ws, ws_bytes, nb_layout(*sys, kWsBase).total));
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    SN_TRY(clear_status(ws, s));
    const int max_rep = sys->n_atoms > 0 ? max_replica_atoms(*sys, s) : -1;
    return nb_build(*sys, pos, r_list, row_ptr, col_idx, rev_idx, capacity, n_edges, reinterpret_cast<char *>(ws), s,
                    true, max_rep);
}

sn_status sn_energy_forces(const sn_model *model, const sn_system *sys, const float *pos, const int32_t *row_ptr,
                           const int32_t *col_idx, const int32_t *rev_idx, int64_t n_edges, float *energy,
                           float *forces, void *ws, size_t ws_bytes, void *stream) {
    SN_TRY(check_system(sys));
    SN_TRY(check_model(model));
    if (n_edges < 0 || (n_edges & 1) || n_edges > INT32_MAX || !energy) return SN_ERR_INVALID;
    if (sys->n_atoms > 0 && (!pos || !row_ptr || !forces)) return SN_ERR_INVALID;
    if (n_edges > 0 && (!col_idx || !rev_idx)) return SN_ERR_INVALID;
    SN_TRY(check_ws(ws, ws_bytes, bytes_needed(model, sys, n_edges)));
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    SN_TRY(clear_status(ws, s));
    return energy_forces_impl(*model, *sys, pos, row_ptr, col_idx, rev_idx, n_edges, energy, forces,
                              reinterpret_cast<char *>(ws), s);
}

sn_status sn_verlet_step(const sn_model *model, const sn_system *sys, float *pos, float *vel, float *forces,
                         const float *inv_mass, float dt, float force_to_accel, int32_t n_steps,
                         int32_t rebuild_every, float r_list, int32_t *row_ptr, int32_t *col_idx, int32_t *rev_idx,
                         int64_t capacity, int64_t *n_edges, double *epot_log, double *ekin_log, int32_t *edge_log,
                         int32_t *n_steps_done, uint32_t flags, void *ws, size_t ws_bytes, void *stream) {
    if (n_steps_done) *n_steps_done = 0;
    SN_TRY(check_system(sys));
    SN_TRY(check_model(model));
    if (n_steps < 0 || rebuild_every < 0 || (flags & ~uint32_t(SN_MD_GRAPH)) != 0 || !n_edges || !row_ptr ||
        !(r_list > 0.0f) || !std::isfinite(r_list) || !std::isfinite(dt) || !std::isfinite(force_to_accel))
        return SN_ERR_INVALID;
    const int N = sys->n_atoms, B = sys->n_replicas;
    if (N > 0 && (!pos || !vel || !forces || !inv_mass || !col_idx || !rev_idx)) return SN_ERR_INVALID;
    SN_TRY(check_ws(ws, ws_bytes, bytes_needed(model, sys, capacity)));
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char *w = reinterpret_cast<char *>(ws);
    SN_TRY(clear_status(ws, s));
    int *status = reinterpret_cast<int *>(w);
    const float half = 0.5f * dt * force_to_accel;
    // Steps are either host-driven (the list rebuilt every step, each step's
    // log slots passed as arguments) or device-driven: a neighbour skin
    // (rebuild_every != 1) or graph replay needs every step's launches to be
    // identical, so the step index, the rebuild decision and the log slots
    // then live in the status words (md_begin_kernel).
    const bool skin = rebuild_every != 1;
    const bool device_steps = skin || (flags & SN_MD_GRAPH);
    const float half_skin = 0.5f * (r_list - model->cutoff);
    const float half_skin2 = half_skin > 0.0f ? half_skin * half_skin : 0.0f;
    // no host synchronisation inside the loop: the neighbour build and the
    // pipeline take the edge and pair counts on the device, errors are
    // flagged in the status word (after which nothing moves and the kernels
    // that read the neighbour list do nothing), and the counters are read
    // once at the end
    const EfLayout L = ef_layout(*model, *sys, capacity, kWsBase);
    float *ref_pos = skin ? reinterpret_cast<float *>(w + L.ref_pos) : nullptr;
    // the weights do not change during the call: one weight pack serves every
    // step, unless the neighbour build's scratch reaches into it
    const size_t nb_end = nb_layout(*sys, kWsBase).total;
    const bool pack_once = nb_end <= L.pack;
    if (pack_once) {
        SN_TRY(filter_pack(*model, w + L.pack, s));
        SN_TRY(mlp_pack(*model, w + L.pack, s));
    }
    // nor do the types: the embedding rows and the first interaction's x are
    // computed once (where no neighbour scratch overlaps them)
    const bool embed_once = pack_once && nb_end <= L.x && N > 0;
    if (embed_once) {
        int64_t off[9 * 16 + 6];
        sn_param_offsets(model->n_types, model->n_interactions, model->n_features, model->n_rbf, off,
                         (int32_t)(sizeof(off) / sizeof(off[0])));
        SN_TRY(mlp_embed_x(N, model->n_features, model->n_types, sys->types, model->params + off[0],
                           pack_ref(w + L.pack, model->n_interactions, pack_slot(0, PK_XW)),
                           reinterpret_cast<float *>(w + L.h0), reinterpret_cast<float *>(w + L.x),
                           reinterpret_cast<float *>(w + L.xmax), status, s));
    }
    // small replicas: the neighbour build also writes the pair arrays
    const int max_rep = N > 0 && n_steps > 0 ? max_replica_atoms(*sys, s) : -1;
    NbPairOut pairs;
    pairs.edge_pair = reinterpret_cast<int32_t *>(w + L.edge_pair);
    pairs.pair_ij = reinterpret_cast<int2 *>(w + L.pair_ij);
    pairs.pgeo = reinterpret_cast<float4 *>(w + L.pgeo);
    pairs.pfc = reinterpret_cast<float *>(w + L.pfc);
    pairs.plfc = reinterpret_cast<float *>(w + L.plfc);
    pairs.cutoff = model->cutoff;
    pairs.mask = reinterpret_cast<uint64_t *>(w + L.mask);
    pairs.rep = reinterpret_cast<int32_t *>(w + L.rep);
    // the opening half kick and drift: host-driven steps pass n_total = -1
    // (always), device-driven ones let the kernel skip it after the last step
    auto open_step = [&](hipStream_t st, int n_total, const float *ref) -> sn_status {
        if (N == 0) return SN_OK;
        ProfScope ps(K_VERLET, st);
        open_step_kernel<<<(N + 255) / 256, 256, 0, st>>>(N, pos, vel, forces, inv_mass, half, dt, status, n_total,
                                                          ref, half_skin2);
        return launch_status();
    };
    // one step; `step` is only used by host-driven steps
    const int *build_flag = device_steps ? status + kBuildFlag : nullptr;
    auto one_step = [&](hipStream_t st, int32_t step) -> sn_status {
        if (device_steps) {
            ProfScope ps(K_VERLET, st);
            md_begin_kernel<<<1, 64, 0, st>>>(status, rebuild_every);
            SN_TRY(launch_status());
        }
        int64_t E_unused = 0;
        bool pairs_done = false;
        // host-driven: the build marks the step as begun without error (the steps completed)
        SN_TRY(nb_build(*sys, pos, r_list, row_ptr, col_idx, rev_idx, capacity, &E_unused, w, st, false, max_rep,
                        &pairs, &pairs_done, device_steps ? -1 : step, build_flag));
        if (skin) SN_TRY(pairs_refresh(*sys, pos, model->cutoff, w, L, status, capacity / 2, st));
        double *elog = epot_log ? (device_steps ? epot_log : epot_log + (int64_t)step * B) : nullptr;
        // the force assembly closes this step and opens the next (unless the
        // kinetic energy is logged between the two)
        VerletFuse vf{};
        vf.pos = pos;
        vf.vel = vel;
        vf.inv_mass = inv_mass;
        vf.half = half;
        vf.dt = dt;
        vf.close = 1;
        vf.ref_pos = ref_pos;
        vf.half_skin2 = half_skin2;
        if (device_steps) {
            vf.open = !ekin_log;
            vf.n_total = n_steps;
            vf.edge_log = edge_log;
        } else {
            vf.open = step + 1 < n_steps && !ekin_log;
            vf.n_total = -1;
            vf.edge_slot = edge_log ? edge_log + step : nullptr;
        }
        SN_TRY(energy_forces_impl(*model, *sys, pos, row_ptr, col_idx, rev_idx, capacity, nullptr, forces, w, st,
                                  true, pack_once, pairs_done, &vf, embed_once, build_flag, elog,
                                  device_steps ? 1 : 0));
        if (ekin_log) {
            {
                ProfScope ps(K_KINETIC, st);
                kinetic_kernel<<<B, 256, 0, st>>>(sys->replica_ptr, vel, inv_mass, 0.5 / (double)force_to_accel,
                                                  device_steps ? ekin_log : ekin_log + (int64_t)step * B,
                                                  device_steps ? status : nullptr);
                SN_TRY(launch_status());
            }
            if (device_steps) SN_TRY(open_step(st, n_steps, ref_pos));
            else if (step + 1 < n_steps) SN_TRY(open_step(st, -1, nullptr));
        }
        return SN_OK;
    };
    // the first step's opening kick and drift; each later one runs in the
    // previous step's force assembly (unless the kinetic energy is logged between)
    if (n_steps > 0) SN_TRY(open_step(s, -1, nullptr));
    int32_t done = 0;
    if ((flags & SN_MD_GRAPH) && n_steps > 0) {
        // one rebuild interval recorded as a HIP graph (on a private stream;
        // nothing runs while recording) and replayed on the caller's stream
        const int32_t G = std::max(1, std::min(n_steps, rebuild_every > 1 ? rebuild_every : 10));
        CaptureGuard cg;
        SN_HIP(hipStreamCreateWithFlags(&cg.cs, hipStreamNonBlocking));
        SN_HIP(hipStreamBeginCapture(cg.cs, hipStreamCaptureModeThreadLocal));
        cg.open = true;
        t_capturing = true;
        for (int32_t g = 0; g < G; ++g) SN_TRY(one_step(cg.cs, -1));
        t_capturing = false;
        cg.open = false;
        SN_HIP(hipStreamEndCapture(cg.cs, &cg.graph));
        SN_HIP(hipGraphInstantiate(&cg.exec, cg.graph, nullptr, nullptr, 0));
        for (; done + G <= n_steps; done += G) SN_HIP(hipGraphLaunch(cg.exec, s));
        for (; done < n_steps; ++done) SN_TRY(one_step(s, done));
        SN_HIP(hipStreamSynchronize(s));
    } else {
        for (; done < n_steps; ++done) SN_TRY(one_step(s, done));
    }
    int host[kStepsDone + 1] = {};
    SN_HIP(hipMemcpyAsync(host, status, sizeof(host), hipMemcpyDeviceToHost, s));
    SN_HIP(hipStreamSynchronize(s));
    *n_edges = host[kEdgeTotal];
    if (n_steps_done) *n_steps_done = host[kStatusWord] == 0 ? n_steps : host[kStepsDone];
    SN_TRY(clear_status(ws, s));
    return host[kStatusWord];
}

sn_status sn_filter_forward(const sn_model *model, int32_t interaction, const float *d, int64_t n, float *phi,
                            void *ws, size_t ws_bytes, void *stream) {
    SN_TRY(check_model(model));
    if (interaction < 0 || interaction >= model->n_interactions || n < 0 || (n > 0 && (!d || !phi)))
        return SN_ERR_INVALID;
    SN_TRY(check_ws(ws, ws_bytes, kWsBase + pack_bytes(model->n_interactions)));
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char *pack = reinterpret_cast<char *>(ws) + kWsBase;
    SN_TRY(filter_pack(*model, pack, s));
    return filter_forward_plain(*model, interaction, d, n, phi, pack, s);
}

sn_status sn_read_status(void *ws, void *stream) {
    if (!ws) return SN_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int v = 0;
    SN_HIP(hipMemcpyAsync(&v, ws, sizeof(int), hipMemcpyDeviceToHost, s));
    SN_HIP(hipStreamSynchronize(s));
    SN_TRY(clear_status(ws, s));
    return v;
}

sn_status sn_energy_forces_static(const sn_model *model, const sn_system *sys, const float *pos,
                                  const int32_t *row_ptr, const int32_t *col_idx, const int32_t *rev_idx,
                                  int64_t n_edges, float *energy, float *forces, int32_t *status_out,
                                  void *stream) {
    SN_TRY(check_system(sys));
    SN_TRY(check_model(model));
    if (n_edges < 0 || (n_edges & 1) || n_edges > INT32_MAX || !energy) return SN_ERR_INVALID;
    if (sys->n_atoms > 0 && (!pos || !row_ptr || !forces)) return SN_ERR_INVALID;
    if (n_edges > 0 && (!col_idx || !rev_idx)) return SN_ERR_INVALID;
    if (bytes_needed(model, sys, n_edges) > kStaticScratchBytes) return SN_ERR_WORKSPACE;
    char *ws = nullptr;
    SN_TRY(static_scratch(&ws));
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    SN_TRY(clear_status(ws, s));   // a kernel: the array keeps the previous call's contents
    SN_TRY(energy_forces_impl(*model, *sys, pos, row_ptr, col_idx, rev_idx, n_edges, energy, forces, ws, s));
    if (status_out) {
        copy_status_kernel<<<1, 64, 0, s>>>(reinterpret_cast<const int *>(ws), status_out);
        SN_TRY(launch_status());
    }
    return SN_OK;
}

void sn_profile_enable(int32_t on) { g_prof_on.store(on != 0); }

int32_t sn_profile_classes(void) { return K_NUM_CLASSES; }

const char *sn_profile_name(int32_t id) { return (id >= 0 && id < K_NUM_CLASSES) ? kClassNames[id] : ""; }

sn_status sn_profile_collect(double *ms_total, int64_t *launches) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    sn_status st = SN_OK;
    for (auto &r : g_prof_done) {
        float ms = 0.0f;
        if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
            st = SN_ERR_HIP;
        if (ms_total) ms_total[r.cls] += ms;
        if (launches) launches[r.cls] += 1;
        g_event_pool.push_back(r.start);
        g_event_pool.push_back(r.stop);
    }
    g_prof_done.clear();
    return st;
}

}  // extern "C"
