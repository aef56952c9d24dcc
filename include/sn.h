/*
 * sn.h -- C ABI of the MI355X SchNet continuous-filter-convolution
 * energy/force library (libsn.so).
 *
 * What it computes.  One energy-plus-force evaluation of a SchNet-style
 * coarse-grained potential over a cutoff neighbour graph, for a batch of
 * independent replicas, plus the neighbour-list build and a velocity-Verlet
 * driver around it.  The stages follow the FlashSchNet pages:
 *   - "FlashSchNet: Fast and Accurate Coarse-Grained Neural Network Molecular
 *     Dynamics" (paper-curation summary), section "How": flash radial basis
 *     (distance, Gaussian expansion and cosine envelope in one pass), flash
 *     message passing (cutoff masking, neighbour gather, filter multiply and
 *     reduction in one kernel, no E x F edge tensor in HBM), flash
 *     aggregation (scatter-add recast as a CSR segment reduce, contention
 *     free in forward and backward), channel-wise 16-bit quantisation of the
 *     filter network's weights;
 *   - the OpenAlex record of the same paper, abstract, techniques (1)-(4);
 *   - section "Achievement" item 1 of the summary: MD throughput aggregated
 *     over parallel replicas of one protein on one GPU.
 * The pages print no equations; the model is plain SchNet:
 *     h0_i = Emb[type_i]
 *     per interaction t:  x = h W_in
 *                         W_ij = fc(d_ij) * (ssp(rbf(d_ij) A1 + b1) A2 + b2)
 *                         y_i  = sum_{j in N(i)} W_ij (.) x_j
 *                         h   += ssp(y Wo1 + bo1) Wo2 + bo2
 *     eps_i = ssp(h_i R1 + c1) . R2 + c2,   E_b = sum_{i in replica b} eps_i
 *     F_i = -dE/dr_i  (analytic backward through the same stages)
 * with rbf_k(d) = exp(-gamma (d - mu_k)^2), mu_k = lo + k (hi - lo)/(K - 1),
 * fc(d) = (cos(pi d / rc) + 1)/2 for d < rc else 0, ssp(x) = ln(e^x/2 + 1/2).
 *
 * Conventions.
 *   - Units are the caller's; the library never converts (Å, fs, Da and
 *     kcal/mol are the intended set).
 *   - Unless marked "host", every pointer is a device pointer (HIP global
 *     memory) that the caller allocated and owns.  The library allocates no
 *     device memory in any call below; scratch comes from `ws`, a caller-
 *     owned device buffer of at least sn_workspace_bytes() bytes, aligned to
 *     256 bytes.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  All
 *     work is enqueued on it in order; only the calls documented as
 *     synchronising wait for it.
 *   - Matrices are row-major; a layer maps a row vector x[in] to
 *     x @ W[in][out] + b[out].
 *   - On any non-zero status the outputs are undefined.
 */
#ifndef SN_H
#define SN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sn_status;
#define SN_OK 0
#define SN_ERR_INVALID -1   /* null pointer, bad size, unsupported shape or inconsistent CSR */
#define SN_ERR_CAPACITY -2  /* edge capacity too small; the required count is reported */
#define SN_ERR_BOX -3       /* periodic box shorter than 3 neighbour cells along a side */
#define SN_ERR_HIP -4       /* a HIP runtime call or kernel launch failed */
#define SN_ERR_NONFINITE -5 /* a non-finite position, energy or force was produced */
#define SN_ERR_WORKSPACE -6 /* ws is NULL, misaligned or smaller than sn_workspace_bytes() */
#define SN_ERR_ROW -7       /* an atom has more than SN_MAX_ROW neighbours */

/* Largest neighbour count of a single atom that the list builder accepts. */
#define SN_MAX_ROW 2048

/* Batched system: the atoms of replica b are [replica_ptr[b], replica_ptr[b+1]);
 * neighbours are only ever searched within one replica. */
typedef struct sn_system {
    int32_t n_atoms;             /* N >= 0 */
    int32_t n_replicas;          /* B >= 1 */
    const int32_t *replica_ptr;  /* device [B+1], replica_ptr[0] = 0, non-decreasing, [B] = N */
    const int32_t *types;        /* device [N], each in [0, n_types) */
    int32_t periodic;            /* 0 = open boundaries, 1 = orthorhombic periodic box */
    float box[3];                /* box edge lengths (host values), used when periodic */
} sn_system;

/* Model.  `params` is one packed fp32 buffer laid out as sn_param_offsets()
 * reports: Emb[T][F]; for each interaction W_in[F][F], A1[K][F], b1[F],
 * A2[F][F], b2[F], Wo1[F][F], bo1[F], Wo2[F][F], bo2[F]; then R1[F][F/2],
 * c1[F/2], R2[F/2], c2[1].
 * filter_format 1 replaces every A1 and A2 (the filter network's weights)
 * by symmetric int16 codes with one fp32 scale per output column:
 * qweights holds, per interaction, qA1[K][F] then qA2[F][F]; qscales holds,
 * per interaction, sA1[F] then sA2[F]; the weight used is float(q) * s
 * (an fp32 multiply).  The fp32 A1/A2 slots of `params` are then ignored.
 * filter_math selects the arithmetic of the filter network's two matrix
 * products (and of their recomputation in the force pass): 0 (the default)
 * forms each fp32 product from three fp16 matrix-core products (hi.hi +
 * hi.lo + lo.hi of each operand split into two fp16 halves), which matches
 * an fp32 evaluation; 1 uses one fp16 product of the rounded operands with
 * fp32 accumulation, the reduced-precision tensor-core arithmetic that the
 * FlashSchNet summary page measures its filter network in ("How", the
 * TF32/MFU bullet), about three times cheaper in matrix instructions and
 * roughly 10-bit accurate per product.  Everything else is unchanged.
 * Supported shapes: n_features in {32, 64, 128}, 2 <= n_rbf <= 64,
 * n_interactions in [1, 16]. */
typedef struct sn_model {
    int32_t n_types;          /* T >= 1 */
    int32_t n_interactions;   /* I */
    int32_t n_features;       /* F */
    int32_t n_rbf;            /* K */
    float cutoff;             /* rc of the envelope (> 0) */
    float rbf_lo, rbf_hi;     /* first and last Gaussian centre */
    float rbf_gamma;          /* Gaussian width gamma (> 0) */
    int32_t filter_format;    /* 0 = fp32 filter weights, 1 = int16 per-output-channel */
    const float *params;      /* device, packed fp32 (see above), 16-byte aligned */
    const int16_t *qweights;  /* device, int16 codes (filter_format 1), else NULL */
    const float *qscales;     /* device, fp32 scales (filter_format 1), else NULL */
    int32_t filter_math;      /* 0 = fp32-accurate split products, 1 = one fp16 product */
} sn_model;

/* ---------------------------------------------------------------- host helpers */

/* Number of fp32 values in the packed parameter buffer (host, no GPU). */
int64_t sn_param_count(int32_t n_types, int32_t n_interactions, int32_t n_features, int32_t n_rbf);

/* Offsets (in floats) of every array of the packed buffer, in the order
 * Emb, {W_in, A1, b1, A2, b2, Wo1, bo1, Wo2, bo2} per interaction, R1, c1,
 * R2, c2, and finally the total count (9 I + 6 entries).  Writes at most
 * `max_offsets` entries into the host array `offsets` and returns the
 * number of entries of the full table, or -1 on a bad shape. */
int32_t sn_param_offsets(int32_t n_types, int32_t n_interactions, int32_t n_features, int32_t n_rbf,
                         int64_t *offsets, int32_t max_offsets);

/* Channel-wise 16-bit quantisation of the filter weights ("How", bullet
 * channel-wise 16-bit quantization, of the FlashSchNet summary page).
 * Host only.  For each interaction and each of A1, A2 (read from the host
 * copy of the packed buffer `params_host`): per output column f,
 * s_f = float(max_k |w_kf| / 32767) (ratio in double) and
 * q_kf = clamp(round_half_even(w_kf / s_f), -32767, 32767) (ratio in
 * double), q = 0 where s_f = 0.  Writes host arrays qweights_host
 * [I * (K*F + F*F)] and qscales_host [I * 2F] in the layout described at
 * sn_model.  Returns SN_ERR_INVALID on null pointers or a bad shape. */
sn_status sn_quantize_filter_weights(int32_t n_types, int32_t n_interactions, int32_t n_features,
                                     int32_t n_rbf, const float *params_host, int16_t *qweights_host,
                                     float *qscales_host);

/* Bytes of device workspace needed by the calls below for this model and
 * system with at most `max_edges` directed edges (host, no GPU).  One
 * workspace serves every entry point. */
size_t sn_workspace_bytes(const sn_model *model, const sn_system *sys, int64_t max_edges);

/* Human-readable name of a status code (static string). */
const char *sn_status_string(sn_status status);

/* Library ABI version (incremented on any signature or layout change). */
int32_t sn_version(void);

/* ---------------------------------------------------------------- entry points */

/* Neighbour list.  ("How", flash message passing -- cutoff masking -- and
 * flash aggregation -- CSR --, FlashSchNet summary page; the full, directed
 * list a machine-learned potential needs, section 1 of the GROMACS/DeePMD
 * slide summary.)
 * Builds, with a cell list, the CSR of all ordered pairs (i, j), i != j, of
 * the same replica whose squared distance, evaluated in fp32 as
 *     dx = x_j - x_i;  periodic: dx = dx - L * rint(dx * invL), invL = float(1/L)
 *     r2 = (dx*dx + dy*dy) + dz*dz      (no fused multiply-add)
 * is strictly below float(r_list) * float(r_list).
 * Outputs (device): row_ptr[N+1]; col_idx[E], ascending within each row;
 * rev_idx[E], the index of edge (j, i) for edge (i, j).
 * capacity = length of col_idx and rev_idx.  *n_edges (host) receives E.
 * Synchronises `stream` once (to read E).  Errors: SN_ERR_CAPACITY when
 * E > capacity (then *n_edges = E and only row_ptr is valid), SN_ERR_BOX
 * when a periodic side holds fewer than 3 cells of edge r_list,
 * SN_ERR_ROW when a row exceeds SN_MAX_ROW, SN_ERR_NONFINITE for a
 * non-finite position. */
sn_status sn_build_csr_neighbors(const sn_system *sys, const float *pos /* [N][3] */, float r_list,
                                 int32_t *row_ptr, int32_t *col_idx, int32_t *rev_idx, int64_t capacity,
                                 int64_t *n_edges, void *ws, size_t ws_bytes, void *stream);

/* Energy and forces.  ("How", all four bullets, FlashSchNet summary page;
 * OpenAlex abstract techniques (1)-(4).)
 * Inputs: positions pos[N][3], a symmetric CSR as built above (rev_idx
 * must be the reverse-edge index; n_edges = E, even).  Edges at distance
 * >= cutoff contribute nothing (the envelope is 0 there).
 * Outputs: energy[B] (one per replica) and forces[N][3] = -dE/dr.
 * Atomic-free and deterministic: repeated calls give identical bits.
 * Does not synchronise; a non-finite force sets the device status read by
 * sn_read_status().  Every kernel runs on `stream`, in order. */
sn_status sn_energy_forces(const sn_model *model, const sn_system *sys, const float *pos,
                           const int32_t *row_ptr, const int32_t *col_idx, const int32_t *rev_idx,
                           int64_t n_edges, float *energy /* [B] */, float *forces /* [N][3] */,
                           void *ws, size_t ws_bytes, void *stream);

/* Flags of sn_verlet_step. */
#define SN_MD_GRAPH 1u  /* record one rebuild interval of steps as a HIP graph and replay it */

/* Velocity Verlet over all replicas ("Achievement" item 1, FlashSchNet
 * summary page: aggregate MD throughput of parallel replicas; the neighbour
 * skin and the replay of each rebuild interval as one graph follow the
 * abstract of "Ab Initio Accuracy Beyond the Cutoff ..." (Tessera), which
 * keeps the list topology across updates with a conservative skin).
 * Per step, with a = force_to_accel * F * inv_mass:
 *     v += dt/2 a;  r += dt v;  (re)build the neighbour list at r_list;
 *     F = F(r);  v += dt/2 a
 * On entry `forces` must hold F(r) for the entry positions (call
 * sn_energy_forces once before the first step); on return it holds F at the
 * final positions.  pos, vel, forces [N][3] are updated in place;
 * inv_mass[N].
 *
 * Neighbour list.  rebuild_every = 1 rebuilds it at r_list every step (exact
 * for r_list >= cutoff).  Any other value keeps a list built at r_list =
 * cutoff + skin across steps: it is rebuilt at the call's first step, every
 * rebuild_every steps (0: never on a schedule), and at the step after any
 * atom has drifted more than skin/2 from where it was at the last build
 * (checked on the device during the drift; no host synchronisation).  Every
 * pair within the cutoff is then always in the list (two atoms close in by
 * at most skin), and the kept pairs get their geometry from the current
 * positions each step; pairs beyond the cutoff have a zero envelope and
 * contribute exactly nothing, so results equal those of a per-step rebuild
 * up to summation order.  With skin <= 0 any motion triggers a rebuild.
 * The list is still built in full when it is rebuilt; skin pairs cost filter
 * work (about ((cutoff + skin)/cutoff)^3 - 1 more pairs).
 *
 * flags: 0 or SN_MD_GRAPH.  With SN_MD_GRAPH the launches of one rebuild
 * interval (rebuild_every steps when it is above 1, else 10 steps; at most
 * n_steps) are recorded once, on a private stream, as a HIP graph that is
 * replayed on `stream`; the steps left over run as ordinary launches.  The
 * results are bit-identical to the same call without the flag.
 *
 * row_ptr/col_idx/rev_idx (capacity as above) receive the last neighbour
 * list built (at r_list) and *n_edges its size (host).  epot_log and
 * ekin_log, if not NULL, receive per step and replica the potential energy
 * and 0.5 sum m v^2 / force_to_accel ([n_steps][B] doubles, device; both are
 * sums over the replica's atoms taken in fp64, so that the drift of their
 * sum is resolved below fp32 rounding); edge_log, if not
 * NULL, the edge count of each step's neighbour list ([n_steps], device).
 * The steps run without host synchronisation: the edge and pair counts stay
 * on the device, the capacity and row-length checks run there, and the
 * call synchronises once, at its end.  After the first error (for example
 * SN_ERR_CAPACITY, SN_ERR_ROW or SN_ERR_NONFINITE) no atom moves again and
 * the kernels that read a neighbour list do nothing; the call returns that
 * error, with *n_steps_done (host, may be NULL) = the steps completed before
 * it; pos, vel, forces and the neighbour-list outputs then hold the state of
 * the failing step, not a valid one.  SN_ERR_INVALID also for
 * rebuild_every < 0 or an unknown flag; SN_ERR_HIP if recording or
 * replaying the graph fails. */
sn_status sn_verlet_step(const sn_model *model, const sn_system *sys, float *pos, float *vel, float *forces,
                         const float *inv_mass, float dt, float force_to_accel, int32_t n_steps,
                         int32_t rebuild_every, float r_list, int32_t *row_ptr, int32_t *col_idx, int32_t *rev_idx,
                         int64_t capacity, int64_t *n_edges, double *epot_log, double *ekin_log, int32_t *edge_log,
                         int32_t *n_steps_done, uint32_t flags, void *ws, size_t ws_bytes, void *stream);

/* Filter network alone ("How", flash radial basis and the filter network,
 * FlashSchNet summary page): phi[p][F] = ssp(rbf(d_p) A1 + b1) A2 + b2 of
 * interaction `interaction` for n distances d[p] (no envelope), in fp32.
 * It writes the filter part of the weight pack into ws (a workspace as for
 * the calls above; it needs at least 256 bytes plus the weight pack) and
 * runs the same kernel and weight pack as sn_energy_forces, which stores
 * fc phi in the 24-bit row format instead.  For testing and benchmarking. */
sn_status sn_filter_forward(const sn_model *model, int32_t interaction, const float *d, int64_t n,
                            float *phi, void *ws, size_t ws_bytes, void *stream);

/* Energy and forces without allocation, for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  The same computation as
 * sn_energy_forces (same kernels, same bits), with its scratch in a static
 * device array of SN_STATIC_SCRATCH_BYTES that the library holds on every GPU
 * it runs on until the process ends.  It allocates nothing, calls no
 * allocating routine and does not synchronise.
 * Limits and errors: SN_ERR_WORKSPACE when sn_workspace_bytes(model, sys,
 * n_edges) exceeds SN_STATIC_SCRATCH_BYTES (checked on the host, before any
 * GPU work); otherwise as sn_energy_forces.  `stream` must belong to the
 * current device.  status_out (device int32, may be NULL) receives, in
 * stream order, the call's device status (SN_OK, or for example
 * SN_ERR_NONFINITE).  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (other streams or host threads) race and give
 * undefined results; calls ordered on one stream are safe. */
#define SN_STATIC_SCRATCH_BYTES (64u << 20)
sn_status sn_energy_forces_static(const sn_model *model, const sn_system *sys, const float *pos,
                                  const int32_t *row_ptr, const int32_t *col_idx, const int32_t *rev_idx,
                                  int64_t n_edges, float *energy /* [B] */, float *forces /* [N][3] */,
                                  int32_t *status_out, void *stream);

/* Synchronise `stream`, return the device status word of workspace `ws`
 * (SN_OK or the first error a kernel flagged) and clear it. */
sn_status sn_read_status(void *ws, void *stream);

/* ---------------------------------------------------------------- timing */

/* Per-kernel timing with HIP events recorded around every launch on the
 * launch stream.  Enabling it adds two event records per launch. */
void sn_profile_enable(int32_t on);
/* Number of kernel classes and the name of class `id` (static string). */
int32_t sn_profile_classes(void);
const char *sn_profile_name(int32_t id);
/* Synchronise on the recorded events and add their durations, per class, to
 * ms_total[id] and launch counts to launches[id] (host arrays of
 * sn_profile_classes() entries); then forget them. */
sn_status sn_profile_collect(double *ms_total, int64_t *launches);

#ifdef __cplusplus
}
#endif
#endif /* SN_H */
