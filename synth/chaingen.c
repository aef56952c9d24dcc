/*
 * Seeded synthetic coordinate generators for coarse-grained test systems.
 *
 * These build inputs only: bead chains with fixed bond length and a
 * hard-core exclusion between non-bonded beads, Monte Carlo compaction of
 * such chains towards a target radius of gyration, and random sequential
 * addition of particles into a periodic cubic box.  None of the potential's
 * arithmetic lives here.
 *
 * Random numbers: xoshiro256** (Blackman & Vigna, 2018) seeded through
 * splitmix64, so a 64-bit seed fixes every draw.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct { uint64_t s[4]; } rng_t;

static uint64_t splitmix64(uint64_t *x) {
    uint64_t z = (*x += 0x9E3779B97F4A7C15ULL);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}
static void rng_seed(rng_t *r, uint64_t seed) {
    for (int i = 0; i < 4; ++i) r->s[i] = splitmix64(&seed);
}
static inline uint64_t rotl(uint64_t x, int k) { return (x << k) | (x >> (64 - k)); }
static uint64_t rng_next(rng_t *r) {
    uint64_t *s = r->s;
    uint64_t out = rotl(s[1] * 5, 7) * 9;
    uint64_t t = s[1] << 17;
    s[2] ^= s[0]; s[3] ^= s[1]; s[1] ^= s[2]; s[0] ^= s[3];
    s[2] ^= t; s[3] = rotl(s[3], 45);
    return out;
}
/* uniform in [0,1) with 53 random bits */
static double rng_unif(rng_t *r) { return (double)(rng_next(r) >> 11) * 0x1.0p-53; }

/* uniform direction on the unit sphere (Archimedes: z uniform in [-1,1]) */
static void rng_dir(rng_t *r, double v[3]) {
    double z = 2.0 * rng_unif(r) - 1.0;
    double phi = 2.0 * M_PI * rng_unif(r);
    double s = sqrt(fmax(0.0, 1.0 - z * z));
    v[0] = s * cos(phi); v[1] = s * sin(phi); v[2] = z;
}

static double dist2(const double *a, const double *b) {
    double dx = a[0] - b[0], dy = a[1] - b[1], dz = a[2] - b[2];
    return dx * dx + dy * dy + dz * dz;
}

/* true if point p keeps >= excl from every bead j in [0, upto) with |j-k| >= 2 */
static int clear_of(const double *pos, int upto, int k, const double *p, double excl2, int skip_hi) {
    for (int j = 0; j < upto; ++j) {
        if (j >= k - 1 && j <= k + 1) continue;
        if (skip_hi >= 0 && j > skip_hi) break;
        if (dist2(pos + 3 * j, p) < excl2) return 0;
    }
    return 1;
}

/*
 * Grow an n-bead chain bead by bead: each new bead sits at `bond` from the
 * previous one in a uniformly random direction; a draw is rejected when the
 * bead comes closer than `excl` to any non-bonded earlier bead or, if
 * r_conf > 0, leaves the sphere of radius r_conf about the origin.  After
 * `tries` rejected draws in a row the last `backtrack` beads are removed.
 * Returns 0 on success, -1 if the total draw budget ran out.
 */
int synth_grow_chain(int n, double bond, double excl, double r_conf, uint64_t seed,
                     int tries, int backtrack, int64_t max_draws, double *pos) {
    rng_t r; rng_seed(&r, seed);
    double excl2 = excl * excl;
    if (n <= 0) return 0;
    pos[0] = pos[1] = pos[2] = 0.0;
    int i = 1, fails = 0;
    int64_t draws = 0;
    while (i < n) {
        if (++draws > max_draws) return -1;
        double v[3], p[3];
        rng_dir(&r, v);
        for (int c = 0; c < 3; ++c) p[c] = pos[3 * (i - 1) + c] + bond * v[c];
        int ok = 1;
        if (r_conf > 0.0 && p[0] * p[0] + p[1] * p[1] + p[2] * p[2] > r_conf * r_conf) ok = 0;
        if (ok) ok = clear_of(pos, i, i, p, excl2, -1);
        if (ok) {
            memcpy(pos + 3 * i, p, sizeof p);
            ++i; fails = 0;
        } else if (++fails >= tries) {
            i = i - backtrack; if (i < 1) i = 1;
            fails = 0;
        }
    }
    return 0;
}

static double rg2_of(const double *pos, int n, double s1[3], double *s2) {
    s1[0] = s1[1] = s1[2] = 0.0; *s2 = 0.0;
    for (int i = 0; i < n; ++i) {
        for (int c = 0; c < 3; ++c) s1[c] += pos[3 * i + c];
        *s2 += pos[3 * i] * pos[3 * i] + pos[3 * i + 1] * pos[3 * i + 1] + pos[3 * i + 2] * pos[3 * i + 2];
    }
    return *s2 / n - (s1[0] * s1[0] + s1[1] * s1[1] + s1[2] * s1[2]) / ((double)n * n);
}

/*
 * Monte Carlo compaction of a valid chain.  A move picks a bead uniformly:
 * an end bead is re-placed at `bond` from its neighbour in a uniform
 * direction; an interior bead is rotated by a uniform angle about the axis
 * through its two neighbours (both bond lengths kept).  A move is accepted
 * only if it keeps every non-bonded pair >= excl apart and does not raise
 * the radius of gyration.  Stops when Rg <= rg_target or after max_moves.
 * Writes the final Rg to *rg_out and returns the number of moves made.
 */
int64_t synth_compact_chain(int n, double bond, double excl, double rg_target, int64_t max_moves,
                            uint64_t seed, double *pos, double *rg_out) {
    rng_t r; rng_seed(&r, seed);
    double excl2 = excl * excl;
    double s1[3], s2;
    double rg2 = rg2_of(pos, n, s1, &s2);
    double tgt2 = rg_target * rg_target;
    int64_t m = 0, acc = 0;
    if (n < 3) { *rg_out = sqrt(fmax(rg2, 0.0)); return 0; }
    for (; m < max_moves && rg2 > tgt2; ++m) {
        int k = (int)(rng_unif(&r) * n);
        if (k >= n) k = n - 1;
        double p[3];
        const double *old = pos + 3 * k;
        if (k == 0 || k == n - 1) {
            const double *nb = pos + 3 * (k == 0 ? 1 : n - 2);
            double v[3]; rng_dir(&r, v);
            for (int c = 0; c < 3; ++c) p[c] = nb[c] + bond * v[c];
        } else {
            const double *a = pos + 3 * (k - 1), *b = pos + 3 * (k + 1);
            double ax[3] = {b[0] - a[0], b[1] - a[1], b[2] - a[2]};
            double al = sqrt(ax[0] * ax[0] + ax[1] * ax[1] + ax[2] * ax[2]);
            double th = (2.0 * rng_unif(&r) - 1.0) * M_PI;
            if (al < 1e-12) continue;
            for (int c = 0; c < 3; ++c) ax[c] /= al;
            double v[3] = {old[0] - a[0], old[1] - a[1], old[2] - a[2]};
            double vp = v[0] * ax[0] + v[1] * ax[1] + v[2] * ax[2];
            double par[3], perp[3], w[3];
            for (int c = 0; c < 3; ++c) { par[c] = vp * ax[c]; perp[c] = v[c] - par[c]; }
            w[0] = ax[1] * perp[2] - ax[2] * perp[1];
            w[1] = ax[2] * perp[0] - ax[0] * perp[2];
            w[2] = ax[0] * perp[1] - ax[1] * perp[0];
            double cs = cos(th), sn = sin(th);
            for (int c = 0; c < 3; ++c) p[c] = a[c] + par[c] + cs * perp[c] + sn * w[c];
        }
        double ns1[3], ns2;
        for (int c = 0; c < 3; ++c) ns1[c] = s1[c] - old[c] + p[c];
        ns2 = s2 - (old[0] * old[0] + old[1] * old[1] + old[2] * old[2]) + (p[0] * p[0] + p[1] * p[1] + p[2] * p[2]);
        double nrg2 = ns2 / n - (ns1[0] * ns1[0] + ns1[1] * ns1[1] + ns1[2] * ns1[2]) / ((double)n * n);
        if (nrg2 > rg2) continue;
        if (!clear_of(pos, n, k, p, excl2, -1)) continue;
        memcpy(pos + 3 * k, p, sizeof p);
        s1[0] = ns1[0]; s1[1] = ns1[1]; s1[2] = ns1[2]; s2 = ns2; rg2 = nrg2;
        if ((++acc & 4095) == 0) rg2 = rg2_of(pos, n, s1, &s2);
    }
    rg2 = rg2_of(pos, n, s1, &s2);
    *rg_out = sqrt(fmax(rg2, 0.0));
    return m;
}

/*
 * Random sequential addition of n points into the periodic cube [0,L)^3:
 * each trial point is uniform in the cube and is kept only if its
 * minimum-image distance to every kept point is >= dmin.  A cell grid with
 * cells of edge >= dmin limits each test to the 27 surrounding cells.
 * Returns 0 on success, -1 if max_trials ran out.
 */
int synth_box_rsa(int n, double L, double dmin, uint64_t seed, int64_t max_trials, double *pos) {
    rng_t r; rng_seed(&r, seed);
    int nc = (int)floor(L / dmin);
    if (nc < 3) nc = 3;
    double cell = L / nc;
    int ncell = nc * nc * nc;
    int *head = (int *)malloc(sizeof(int) * ncell);
    int *next = (int *)malloc(sizeof(int) * (n > 0 ? n : 1));
    if (!head || !next) { free(head); free(next); return -2; }
    for (int c = 0; c < ncell; ++c) head[c] = -1;
    double d2min = dmin * dmin;
    int placed = 0;
    int64_t trials = 0;
    while (placed < n) {
        if (++trials > max_trials) { free(head); free(next); return -1; }
        double p[3];
        int ci[3];
        for (int c = 0; c < 3; ++c) {
            p[c] = rng_unif(&r) * L;
            ci[c] = (int)(p[c] / cell);
            if (ci[c] >= nc) ci[c] = nc - 1;
        }
        int ok = 1;
        for (int dz = -1; dz <= 1 && ok; ++dz)
            for (int dy = -1; dy <= 1 && ok; ++dy)
                for (int dx = -1; dx <= 1 && ok; ++dx) {
                    int cx = (ci[0] + dx + nc) % nc, cy = (ci[1] + dy + nc) % nc, cz = (ci[2] + dz + nc) % nc;
                    for (int j = head[(cz * nc + cy) * nc + cx]; j >= 0; j = next[j]) {
                        double d[3];
                        for (int c = 0; c < 3; ++c) {
                            d[c] = pos[3 * j + c] - p[c];
                            d[c] -= L * nearbyint(d[c] / L);
                        }
                        if (d[0] * d[0] + d[1] * d[1] + d[2] * d[2] < d2min) { ok = 0; break; }
                    }
                }
        if (!ok) continue;
        memcpy(pos + 3 * placed, p, sizeof p);
        int c = (ci[2] * nc + ci[1]) * nc + ci[0];
        next[placed] = head[c]; head[c] = placed;
        ++placed;
    }
    free(head); free(next);
    return 0;
}
