// gdn_api.cpp -- the C ABI of libgdn: argument checks, then one launch.
//
// Every check runs on the host before anything touches the device, so an
// invalid call returns its error code with no output written (the ferrox-core
// gdn_chunk.rs page's convention that a failed call leaves the state
// untouched, without that page's host fallback).
#include <math.h>
#include <stdint.h>

#include "gdn.h"
#include "gdn_internal.h"

namespace {

static_assert(GDN_HEADS_TILED == gdn::kTiledHeads && GDN_GATE_LOG == gdn::kLogGate &&
              GDN_GATE_VECTOR == gdn::kVectorGate, "flag values of the ABI and the kernels");
constexpr int kKnownFlags = GDN_HEADS_TILED | GDN_GATE_LOG | GDN_GATE_VECTOR;

struct Range {
    uintptr_t lo, hi;                 // [lo, hi); empty when lo == hi
};

Range range_of(const void *p, uint64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, p ? a + (uintptr_t)bytes : a};
}

bool overlap(Range a, Range b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

bool supported_dim(int d) { return d == 32 || d == 64 || d == 128; }

int elem_size(int dtype) { return dtype == GDN_F32 ? 4 : 2; }

// Shared checks of the entry points; T = 1 for the step.
int check(const void *q, const void *k, const void *v, const float *g,
          const float *beta, const float *state_in, const float *state_out,
          const void *y, long B, long T, long Hk, long Hv, long Dk, long Dv,
          int dtype, int flags = 0)
{
    const bool vg = (flags & GDN_GATE_VECTOR) != 0;
    if (B < 0 || T < 0 || Hk <= 0 || Hv <= 0 || Dk <= 0 || Dv <= 0) return GDN_ERR_SHAPE;
    if (Hv % Hk != 0) return GDN_ERR_SHAPE;
    if (B * Hv * (Dv / 32 > 0 ? Dv / 32 : 1) > INT32_MAX) return GDN_ERR_SHAPE;
    if (dtype != GDN_F32 && dtype != GDN_BF16 && dtype != GDN_F16) return GDN_ERR_DTYPE;
    if (!supported_dim((int)Dk) || !supported_dim((int)Dv)) return GDN_ERR_UNSUPPORTED;
    if (B == 0) return GDN_OK;
    if (!state_out) return GDN_ERR_NULL;
    if (T > 0 && (!q || !k || !v || !g || !beta || !y)) return GDN_ERR_NULL;
    const void *p16[] = {q, k, v, y, state_in, state_out};
    for (const void *p : p16)
        if (p && !aligned(p, 16)) return GDN_ERR_ALIGN;
    if ((g && !aligned(g, vg ? 16 : 4)) || (beta && !aligned(beta, 4))) return GDN_ERR_ALIGN;

    const uint64_t es = (uint64_t)elem_size(dtype);
    const uint64_t nqk = (uint64_t)B * T * Hk * Dk, nv = (uint64_t)B * T * Hv * Dv;
    const uint64_t ngb = (uint64_t)B * T * Hv, ns = (uint64_t)B * Hv * Dv * Dk;
    const Range rq = range_of(T ? q : nullptr, nqk * es), rk = range_of(T ? k : nullptr, nqk * es);
    const Range rv = range_of(T ? v : nullptr, nv * es), ry = range_of(T ? y : nullptr, nv * es);
    const Range rg = range_of(T ? g : nullptr, ngb * (vg ? (uint64_t)Dk : 1) * 4);
    const Range rb = range_of(T ? beta : nullptr, ngb * 4);
    const Range rsi = range_of(state_in, ns * 4), rso = range_of(state_out, ns * 4);
    // y overlaps nothing; state_out overlaps nothing but (exactly) state_in
    const Range others_y[] = {rq, rk, rv, rg, rb, rsi, rso};
    for (const Range &r : others_y)
        if (overlap(ry, r)) return GDN_ERR_ALIAS;
    const Range others_s[] = {rq, rk, rv, rg, rb};
    for (const Range &r : others_s)
        if (overlap(rso, r)) return GDN_ERR_ALIAS;
    if (state_in && state_in != state_out && overlap(rsi, rso)) return GDN_ERR_ALIAS;
    return GDN_OK;
}

// The automatic choice of gdn_chunk_fwd (C = 0), from launch timings on the
// MI355X.  The sequential kernel costs one read and one write of the state
// plus a few microseconds per token at the largest grids; the chunked kernel
// has a higher fixed cost and a far smaller one per token, so the sequential
// kernel wins up to a handful of tokens (more for float32 inputs, whose
// chunked kernel runs its products at the float32 MFMA rate).  Against the
// per-wave chunk kernel (16-bit inputs, Dk = 128, Dv a multiple of 64; GPU
// time of graph replays with the state read from HBM, 64..2048 slots) the
// sequential kernel keeps only the shortest calls: up to 3 tokens on 64
// slots, 2 up to 256, 4 up to 1024 (where the per-wave kernel's grid fills
// the chip in two or three rounds), 1 beyond.
bool seq_for(int dtype, int Dk, int Dv, long slots, int T, int flags) {
    if (dtype != GDN_F32 && Dk == 128 && Dv % 64 == 0 && !(flags & gdn::kVectorGate))
        return T <= (slots <= 64 ? 3 : slots <= 256 ? 2 : slots <= 1024 ? 4 : 1);
    return T <= (dtype == GDN_F32 ? 12 : 6);
}

// Chunk length, from timed sweeps of GPU time (launches replayed from a HIP
// graph) over B Hv = 2..1024, T = 2..1111, Dk/Dv in {32, 64, 128}, all
// dtypes.  16 keeps the most work in flight per token and wins on grids of
// many (batch, head) slots and on short sequences; 32 wins from 32 tokens on
// grids of up to 256 slots (the generic kernel then runs several value
// slices per slot).  For 16-bit inputs with 128-dimensional heads the
// pipelined 64-token kernel wins from 48 tokens on up to 64 slots (where it
// runs four workgroups per slot) and on 129..256 slots, and from 128 tokens
// on other grids.  float32 inputs run their products at the f32 MFMA rate:
// 16 for 128-dimensional heads, 32 from 32 tokens for smaller ones.
int chunk_for(int dtype, int Dk, int Dv, long slots, int T) {
    if (dtype == GDN_F32) return (Dk <= 64 && Dv <= 64 && T >= 32) ? 32 : 16;
    if (Dk == 128 && Dv == 128) {
        if (T < 32) return 16;
        if (slots <= 64 || (slots > 128 && slots <= 256)) return T < 48 ? 32 : 64;
        if (slots <= 128) return T < 128 ? 32 : 64;
        return T < 128 ? 16 : 64;
    }
    return (T >= 64 || (T >= 32 && slots <= 256)) ? 32 : 16;
}

int launch(const gdn::FwdArgs &a, int dtype, bool seq, hipStream_t stream) {
    hipError_t e;
    if (seq) e = gdn::launch_seq(dtype, a, stream);
    else if (a.flags & gdn::kVectorGate)
        e = dtype == GDN_F32 ? gdn::launch_chunk_vg_f32(a, stream)
          : dtype == GDN_BF16 ? gdn::launch_chunk_vg_bf16(a, stream)
          : gdn::launch_chunk_vg_f16(a, stream);
    else if (dtype == GDN_F32) e = gdn::launch_chunk_f32(a, stream);
    else if (dtype == GDN_BF16) e = gdn::launch_chunk_bf16(a, stream);
    else e = gdn::launch_chunk_f16(a, stream);
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // namespace

extern "C" {

int gdn_chunk_fwd_ex(const void *q, const void *k, const void *v,
                     const float *g, const float *beta,
                     const float *state_in, float *state_out, void *y,
                     int B, int T, int Hk, int Hv, int Dk, int Dv, int C, int flags,
                     gdn_dtype dtype, hipStream_t stream)
{
    int rc = check(q, k, v, g, beta, state_in, state_out, y, B, T, Hk, Hv, Dk, Dv, (int)dtype, flags);
    if (rc != GDN_OK) return rc;
    if (C != 0 && C != 16 && C != 32 && C != 64) return GDN_ERR_UNSUPPORTED;
    if (flags & ~kKnownFlags) return GDN_ERR_UNSUPPORTED;
    if (B == 0) return GDN_OK;
    const bool seq = C == 0 && seq_for((int)dtype, Dk, Dv, (long)B * Hv, T, flags);
    if (C == 0) C = chunk_for((int)dtype, Dk, Dv, (long)B * Hv, T);
    gdn::FwdArgs a{q, k, v, g, beta, state_in, state_out, y,
                   B, T, Hk, Hv, Dk, Dv, C, (float)(1.0 / sqrt((double)Dk)), flags};
    return launch(a, (int)dtype, seq, stream);
}

int gdn_chunk_fwd(const void *q, const void *k, const void *v,
                  const float *g, const float *beta,
                  const float *state_in, float *state_out, void *y,
                  int B, int T, int Hk, int Hv, int Dk, int Dv, int C,
                  gdn_dtype dtype, hipStream_t stream)
{
    return gdn_chunk_fwd_ex(q, k, v, g, beta, state_in, state_out, y, B, T, Hk, Hv, Dk, Dv, C,
                            0, dtype, stream);
}

int gdn_seq_fwd_ex(const void *q, const void *k, const void *v,
                   const float *g, const float *beta,
                   const float *state_in, float *state_out, void *y,
                   int B, int T, int Hk, int Hv, int Dk, int Dv, int flags,
                   gdn_dtype dtype, hipStream_t stream)
{
    int rc = check(q, k, v, g, beta, state_in, state_out, y, B, T, Hk, Hv, Dk, Dv, (int)dtype, flags);
    if (rc != GDN_OK) return rc;
    if (flags & ~kKnownFlags) return GDN_ERR_UNSUPPORTED;
    if (B == 0) return GDN_OK;
    gdn::FwdArgs a{q, k, v, g, beta, state_in, state_out, y,
                   B, T, Hk, Hv, Dk, Dv, 0, (float)(1.0 / sqrt((double)Dk)), flags};
    return launch(a, (int)dtype, true, stream);
}

int gdn_seq_fwd(const void *q, const void *k, const void *v,
                const float *g, const float *beta,
                const float *state_in, float *state_out, void *y,
                int B, int T, int Hk, int Hv, int Dk, int Dv,
                gdn_dtype dtype, hipStream_t stream)
{
    return gdn_seq_fwd_ex(q, k, v, g, beta, state_in, state_out, y, B, T, Hk, Hv, Dk, Dv, 0,
                          dtype, stream);
}

int gdn_step_ex(const void *q, const void *k, const void *v,
                const float *g, const float *beta,
                const float *state_in, float *state_out, void *y,
                int B, int Hk, int Hv, int Dk, int Dv, int flags,
                gdn_dtype dtype, hipStream_t stream)
{
    int rc = check(q, k, v, g, beta, state_in, state_out, y, B, 1, Hk, Hv, Dk, Dv, (int)dtype, flags);
    if (rc != GDN_OK) return rc;
    if (flags & ~kKnownFlags) return GDN_ERR_UNSUPPORTED;
    if (B == 0) return GDN_OK;
    gdn::FwdArgs a{q, k, v, g, beta, state_in, state_out, y,
                   B, 1, Hk, Hv, Dk, Dv, 0, (float)(1.0 / sqrt((double)Dk)), flags};
    hipError_t e = gdn::launch_step((int)dtype, a, stream);
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_step(const void *q, const void *k, const void *v,
             const float *g, const float *beta,
             const float *state_in, float *state_out, void *y,
             int B, int Hk, int Hv, int Dk, int Dv,
             gdn_dtype dtype, hipStream_t stream)
{
    return gdn_step_ex(q, k, v, g, beta, state_in, state_out, y, B, Hk, Hv, Dk, Dv, 0, dtype,
                       stream);
}

const char *gdn_status_string(int status)
{
    switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "a required pointer is NULL";
    case GDN_ERR_SHAPE: return "invalid shape (negative size, or Hv not a multiple of Hk)";
    case GDN_ERR_UNSUPPORTED: return "unsupported size or flag (Dk, Dv must be 32, 64 or 128; C must be 0, 16, 32 or 64; flags only GDN_HEADS_TILED | GDN_GATE_LOG | GDN_GATE_VECTOR)";
    case GDN_ERR_ALIAS: return "an output overlaps another buffer";
    case GDN_ERR_ALIGN: return "misaligned pointer (16 bytes for q, k, v, y, state and a per-key-dimension g; 4 for a scalar g and beta)";
    case GDN_ERR_HIP: return "HIP launch failed";
    case GDN_ERR_DTYPE: return "unknown dtype";
    default: return "unknown status";
    }
}

int gdn_version(void) { return 10300; }

}  // extern "C"
