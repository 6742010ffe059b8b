/*
 * gdn.h -- C ABI of the gated delta rule (gated DeltaNet) forward pass on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation.  Per batch b and value head hv, with k-head hk = hv / (Hv/Hk)
 * (the grouped head map of the metaltile-std gated_delta_wy.rs page,
 * "Layouts"), a state S of Dv x Dk float32 advances over tokens t:
 *
 *     d_t = beta_t * (v_t - g_t * S_{t-1} k_t)
 *     S_t = g_t * S_{t-1} + d_t k_t^T
 *     y_t = S_t q_t / sqrt(Dk)
 *
 * (the rule as stated on the ferrox-core gdn_chunk.rs page, "The algebra",
 * with g_t the decay that multiplies the state -- not its logarithm -- and
 * the output read from the updated state and scaled by 1/sqrt(Dk)).
 *
 * Layouts (dense, contiguous, row-major; metaltile-std page, "Layouts"):
 *     q, k      [B, T, Hk, Dk]     dtype
 *     v, y      [B, T, Hv, Dv]     dtype
 *     g, beta   [B, T, Hv]         float32
 *     state     [B, Hv, Dv, Dk]    float32 (row j = value index j)
 *
 * Ownership and execution.  Every pointer is device memory owned by the
 * caller (for example from torch on ROCm).  The library allocates nothing,
 * keeps no state between calls and is thread-safe.  Work is enqueued on
 * `stream` (NULL = the default stream) without host synchronisation; the
 * outputs are valid once the stream reaches that point.
 *
 * Errors.  All arguments are checked on the host before anything is
 * enqueued; on any GDN_ERR_* other than GDN_ERR_HIP nothing is launched and
 * no output is touched.  GDN_ERR_HIP means a launch failed; the outputs are
 * then undefined.  There is no host fallback.
 */
#ifndef GDN_H
#define GDN_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of q, k, v and y.  g, beta and the state are always float32. */
typedef enum gdn_dtype {
    GDN_F32 = 0,
    GDN_BF16 = 1,
    GDN_F16 = 2
} gdn_dtype;

enum {
    GDN_OK = 0,
    GDN_ERR_NULL = -1,        /* a required pointer is NULL                  */
    GDN_ERR_SHAPE = -2,       /* negative size, or Hv not a multiple of Hk   */
    GDN_ERR_UNSUPPORTED = -3, /* Dk, Dv, C or flags outside the supported set */
    GDN_ERR_ALIAS = -4,       /* an output overlaps another buffer           */
    GDN_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned (4 for beta and a scalar g) */
    GDN_ERR_HIP = -6,         /* a HIP launch failed                         */
    GDN_ERR_DTYPE = -7        /* dtype is not a gdn_dtype value              */
};

/*
 * gdn_chunk_fwd -- T tokens of the rule, processed in chunks of C tokens,
 * with the state read once from state_in and written once to state_out.
 *
 * The chunked computation is the one the metaltile-std gated_delta_wy.rs page
 * describes ("Algorithm": gates, K K^T, the unit lower triangular system,
 * the chunk's outputs and the chunk-end state) and the ferrox-core
 * gdn_chunk.rs page derives ("The algebra": every decay ratio a product of
 * decays, never a quotient).  It equals the sequential rule above up to
 * float association; C changes speed, not the result.
 *
 *   q, k        [B,T,Hk,Dk] dtype, 16-byte aligned.
 *   v           [B,T,Hv,Dv] dtype, 16-byte aligned.
 *   g, beta     [B,T,Hv] float32, 4-byte aligned.  g is the decay value.
 *   state_in    [B,Hv,Dv,Dk] float32, 16-byte aligned, or NULL for a zero
 *               initial state.
 *   state_out   [B,Hv,Dv,Dk] float32, 16-byte aligned.  May equal state_in
 *               (in-place update); any other overlap is GDN_ERR_ALIAS.
 *   y           [B,T,Hv,Dv] dtype, 16-byte aligned; must not overlap any
 *               other buffer.
 *   B, T        batch and tokens; B = 0 is a no-op, T = 0 copies the initial
 *               state (or zeros) to state_out and writes no y (q, k, v, g,
 *               beta and y may then be NULL).
 *   Hk, Hv      key and value heads, Hv % Hk == 0.
 *   Dk, Dv      head dimensions, each one of 32, 64, 128.
 *   C           chunk length, one of 16, 32, 64 (the tail chunk of
 *               T - C*floor(T/C) tokens is handled inside the kernel), or 0:
 *               let the library choose, for this shape and T, between the
 *               sequential kernel of gdn_seq_fwd (short T) and the chunked
 *               kernel with a chunk length of its own choice.  float32
 *               inputs run chunks of at most 32 tokens: C = 64 is served as
 *               C = 32 (same result, as C never changes it beyond float
 *               association; the chunk's products run at the float32 MFMA
 *               rate, where 64-token chunks do not pay).
 *   dtype       storage type of q, k, v, y.
 *   stream      HIP stream (NULL = default stream).
 * Returns GDN_OK or a GDN_ERR_* code.
 */
int gdn_chunk_fwd(const void *q, const void *k, const void *v,
                  const float *g, const float *beta,
                  const float *state_in, float *state_out, void *y,
                  int B, int T, int Hk, int Hv, int Dk, int Dv, int C,
                  gdn_dtype dtype, hipStream_t stream);

/*
 * gdn_seq_fwd -- T tokens of the rule, token by token, with the state read
 * once from state_in and written once to state_out: the sequential rule
 * itself (the ferrox-core gdn_chunk.rs page, "The algebra", takes it as the
 * definition the chunked form must match), each state row held in registers
 * across the tokens.  Faster than gdn_chunk_fwd for short T (a few tokens of
 * decode or speculation), where the chunk's triangular solve does not pay.
 *   The gates are applied through a running per-slot scale that is folded
 *   into the state when it leaves [2^-24, 2^24]; results equal those of T
 *   calls of gdn_step up to float32 rounding.
 *   Arguments, layouts, alignment, aliasing and errors as for gdn_chunk_fwd
 *   (without C); Dk and Dv each one of 32, 64, 128; T = 0 copies the initial
 *   state (or zeros) to state_out.
 */
int gdn_seq_fwd(const void *q, const void *k, const void *v,
                const float *g, const float *beta,
                const float *state_in, float *state_out, void *y,
                int B, int T, int Hk, int Hv, int Dk, int Dv,
                gdn_dtype dtype, hipStream_t stream);

/*
 * gdn_step -- one token of the rule (decode): each state row is read once
 * and written once (the sequential step of the ferrox-core gdn_chunk.rs
 * page, "Why": the step is bound by the state traffic).
 *
 *   q, k        [B,Hk,Dk] dtype (the T = 1 case of the layouts above).
 *   v, y        [B,Hv,Dv] dtype.
 *   g, beta     [B,Hv] float32.
 *   state_in    [B,Hv,Dv,Dk] float32 or NULL (zero state).
 *   state_out   [B,Hv,Dv,Dk] float32; may equal state_in (in place).
 *   Other arguments, alignment and errors as for gdn_chunk_fwd; Dk and Dv
 *   each one of 32, 64, 128.
 */
int gdn_step(const void *q, const void *k, const void *v,
             const float *g, const float *beta,
             const float *state_in, float *state_out, void *y,
             int B, int Hk, int Hv, int Dk, int Dv,
             gdn_dtype dtype, hipStream_t stream);

/*
 * Conventions of the ferrox-core gdn_chunk.rs page's host body, which takes
 * the same rule with a choice of head map and with the gate given as the
 * logarithm of the decay (it exponentiates the gate before use).  The _ex
 * entry points take them as bits of `flags`:
 *
 *   GDN_HEADS_TILED   key head of value head hv is hv mod Hk (the tiled map:
 *                     the Hk key heads repeat across the value heads)
 *                     instead of hv / (Hv/Hk) (the grouped map).
 *   GDN_GATE_LOG      g holds log(decay); the decay used is exp(g), so g = 0
 *                     keeps the state and g = -inf forgets it.
 *   GDN_GATE_VECTOR   g holds one decay per key dimension: [B,T,Hv,Dk]
 *                     float32 ([B,Hv,Dk] for gdn_step_ex), 16-byte aligned.
 *                     Key column i of the state decays by g_t[i]:
 *                       S_t = S_{t-1} diag(g_t) (I - beta_t k_t k_t^T)
 *                             + beta_t v_t k_t^T
 *                     (the 4-D "vector" gate the MLX pull request page names
 *                     as a shape its kernels would misread).  The chunked
 *                     path then uses chunks of at most 32 tokens (16 for
 *                     float32 inputs) whatever C asks for.
 *
 * flags = 0 is exactly gdn_chunk_fwd / gdn_seq_fwd / gdn_step; the bits
 * combine freely.  Any other bit is GDN_ERR_UNSUPPORTED.  All other arguments, layouts, alignment,
 * aliasing and errors as for the entry points without _ex.
 */
enum {
    GDN_HEADS_TILED = 1,
    GDN_GATE_LOG = 2,
    GDN_GATE_VECTOR = 4
};

int gdn_chunk_fwd_ex(const void *q, const void *k, const void *v,
                     const float *g, const float *beta,
                     const float *state_in, float *state_out, void *y,
                     int B, int T, int Hk, int Hv, int Dk, int Dv, int C, int flags,
                     gdn_dtype dtype, hipStream_t stream);

int gdn_seq_fwd_ex(const void *q, const void *k, const void *v,
                   const float *g, const float *beta,
                   const float *state_in, float *state_out, void *y,
                   int B, int T, int Hk, int Hv, int Dk, int Dv, int flags,
                   gdn_dtype dtype, hipStream_t stream);

int gdn_step_ex(const void *q, const void *k, const void *v,
                const float *g, const float *beta,
                const float *state_in, float *state_out, void *y,
                int B, int Hk, int Hv, int Dk, int Dv, int flags,
                gdn_dtype dtype, hipStream_t stream);

/* Static description of a status code (never NULL). */
const char *gdn_status_string(int status);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
