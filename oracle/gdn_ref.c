/*
 * gdn_ref.c -- the CPU oracle of the gated delta rule forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
 * bench's CPU-baseline leg load this library.  It shares no code, header,
 * table or helper with the HIP library and never calls it.
 *
 * What it computes: the sequential recurrence that the ferrox-core
 * gdn_chunk.rs page states as the definition of the rule ("The algebra",
 * and the test comment that the sequential step IS the definition), with the
 * decay taken as the value that multiplies the state and the output scaled
 * by 1/sqrt(Dk):
 *
 *     d_t = beta_t * (v_t - g_t * S_{t-1} k_t)        (vector over rows j)
 *     S_t = g_t * S_{t-1} + d_t k_t^T                  (rank one)
 *     y_t = S_t q_t / sqrt(Dk)                         (post-update state)
 *
 * Layouts as on the metaltile-std gated_delta_wy.rs page ("Layouts"):
 * q,k [B,T,Hk,Dk]; v,y [B,T,Hv,Dv]; g,beta [B,T,Hv]; state [B,Hv,Dv,Dk],
 * state row j (value index) holding Dk contiguous key-index entries.
 * Key head of value head hv: grouped as on that page, hk = hv / (Hv / Hk)
 * (head_map 0), or tiled, hk = hv mod Hk (head_map 1): the two head maps
 * the ferrox-core page's host body chooses between when it picks the key
 * head of a value head.
 * Gate input: the decay itself (log_gate 0), or its natural logarithm
 * (log_gate 1), which the ferrox-core page's host body turns into the decay
 * with exp before use.
 * Gate shape: one decay per (token, value head), g [B,T,Hv] (vector_gate 0),
 * or one per key dimension, g [B,T,Hv,Dk] (vector_gate 1): the 4-D gate the
 * MLX pull request page names ("Out of scope": a vector gate of shape
 * [B, T, Hv, Dk]).  Read as a decay of each key column of the state:
 *     S_t = S_{t-1} diag(g_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 * i.e. S[j][i] is multiplied by g_t[i] before the prediction, exactly where
 * the scalar gate multiplies the whole state.
 *
 * Everything is float64 with plain loops in token order.  Slots (b, hv) are
 * independent (ferrox-core page: "Heads are independent") and run on an
 * OpenMP thread pool.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Returns 0 on success, -1 on bad arguments, -2 on allocation failure.
 * state_in may be NULL (zero initial state).  slot_mask may be NULL (all
 * slots); otherwise slots with slot_mask[b*Hv+hv]==0 are skipped and their
 * y / state_out entries are left untouched.  nthreads <= 0 means the
 * OpenMP default. */
int gdn_ref_forward(const double *q, const double *k, const double *v,
                    const double *g, const double *beta,
                    const double *state_in, double *state_out, double *y,
                    long B, long T, long Hk, long Hv, long Dk, long Dv,
                    int head_map, int log_gate, int vector_gate,
                    const unsigned char *slot_mask, int nthreads)
{
    if (B < 0 || T < 0 || Hk <= 0 || Hv <= 0 || Dk <= 0 || Dv <= 0) return -1;
    if (Hv % Hk != 0) return -1;
    if ((head_map != 0 && head_map != 1) || (log_gate != 0 && log_gate != 1) ||
        (vector_gate != 0 && vector_gate != 1)) return -1;
    const long gdim = vector_gate ? Dk : 1;      /* decays per (token, head) */
    if (!state_out) return -1;
    if (T > 0 && (!q || !k || !v || !g || !beta || !y)) return -1;
    const long group = Hv / Hk;
    const double scale = 1.0 / sqrt((double)Dk);
    const long nslots = B * Hv;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (long slot = 0; slot < nslots; ++slot) {
        if (slot_mask && !slot_mask[slot]) continue;
        const long b = slot / Hv, hv = slot % Hv;
        const long hk = head_map == 1 ? hv % Hk : hv / group;
        double *S = (double *)malloc(sizeof(double) * (size_t)(Dv * Dk));
        double *pred = (double *)malloc(sizeof(double) * (size_t)Dv);
        double *gv = (double *)malloc(sizeof(double) * (size_t)Dk);
        if (!S || !pred || !gv) {
            free(S); free(pred); free(gv);
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
            continue;
        }
        const double *s0 = state_in ? state_in + slot * Dv * Dk : NULL;
        for (long e = 0; e < Dv * Dk; ++e) S[e] = s0 ? s0[e] : 0.0;
        for (long t = 0; t < T; ++t) {
            const double *kt = k + ((b * T + t) * Hk + hk) * Dk;
            const double *qt = q + ((b * T + t) * Hk + hk) * Dk;
            const double *vt = v + ((b * T + t) * Hv + hv) * Dv;
            /* the decay of every key column i of the state */
            const double *gin = g + ((b * T + t) * Hv + hv) * gdim;
            for (long i = 0; i < Dk; ++i) {
                const double x = gin[vector_gate ? i : 0];
                gv[i] = log_gate ? exp(x) : x;
            }
            const double bt = beta[(b * T + t) * Hv + hv];
            double *yt = y + ((b * T + t) * Hv + hv) * Dv;
            /* the decayed previous state, g_t S_{t-1} (column i by gv[i]) */
            for (long j = 0; j < Dv; ++j)
                for (long i = 0; i < Dk; ++i) S[j * Dk + i] *= gv[i];
            /* prediction from the decayed state */
            for (long j = 0; j < Dv; ++j) {
                double acc = 0.0;
                for (long i = 0; i < Dk; ++i) acc += S[j * Dk + i] * kt[i];
                pred[j] = acc;
            }
            /* d_t and the rank-one update of the decayed state */
            for (long j = 0; j < Dv; ++j) {
                const double dj = bt * (vt[j] - pred[j]);
                for (long i = 0; i < Dk; ++i) S[j * Dk + i] += dj * kt[i];
            }
            /* read-out of the updated state */
            for (long j = 0; j < Dv; ++j) {
                double acc = 0.0;
                for (long i = 0; i < Dk; ++i) acc += S[j * Dk + i] * qt[i];
                yt[j] = acc * scale;
            }
        }
        memcpy(state_out + slot * Dv * Dk, S, sizeof(double) * (size_t)(Dv * Dk));
        free(S);
        free(pred);
        free(gv);
    }
    return failed ? -2 : 0;
}

/* Number of threads the OpenMP runtime would use by default. */
int gdn_ref_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
