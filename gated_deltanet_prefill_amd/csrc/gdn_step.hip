// gdn_step.hip -- one token of the gated delta rule (decode) for gfx950.
//
// The step reads every state row once and writes it once; it is bound by
// that traffic (the ferrox-core gdn_chunk.rs page, "Why": nothing about the
// loop is slow, the traffic is the cost).  Eight lanes own one state row
// (8 value rows per wave, 32 per workgroup); lane i of a row holds the
// 16-byte pieces i, i+8, ... of the row so that each load or store
// instruction of the 8 lanes covers 128 contiguous bytes.  Per row j:
//     a_j = S_j . k,   b_j = S_j . q          (one pass over the row)
//     d_j = beta (v_j - g a_j)
//     S'_j = g S_j + d_j k
//     y_j = (g b_j + d_j (k . q)) / sqrt(Dk)  (= S'_j . q / sqrt(Dk))
// The three dot products finish with a butterfly over the row's 8 lanes.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kStepRowsPerBlock = 32;
constexpr int kStepLanesPerRow = 8;
// fewest waves (over the whole grid) for which the sequential kernel keeps
// four value rows per lane
constexpr long kSeqMinWaves = 2048;

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// sum over the eight lanes of an aligned group (every lane gets the sum):
// swap neighbours, swap pairs, then add the mirror lane of the half row
__device__ __forceinline__ float sum8(float x) {
    x += dpp_mov<0xb1>(x);      // quad_perm [1,0,3,2]
    x += dpp_mov<0x4e>(x);      // quad_perm [2,3,0,1]
    x += dpp_mov<0x141>(x);     // row_half_mirror
    return x;
}


// VG: g is [B,Hv,Dk], one decay per key dimension (column i of the state
// decays by g_i); else one decay per (batch, value head).
template <typename ET, int DK, bool VG>
__global__ __launch_bounds__(256)
void step_kernel(const ET *__restrict__ q, const ET *__restrict__ k,
                 const ET *__restrict__ v, const float *__restrict__ g,
                 const float *__restrict__ beta, const float *state_in,
                 float *state_out, ET *__restrict__ y,
                 int Hk, int Hv, int Dv, float scale, int flags)
{
    constexpr int LPR = kStepLanesPerRow;
    constexpr int NP = DK / (4 * LPR);            // 16-byte state pieces per lane
    const int tid = threadIdx.x;
    const int sub = tid & (LPR - 1);
    const int blocks_per_slot = Dv / kStepRowsPerBlock;
    const int slot = blockIdx.x / blocks_per_slot;
    const int j = (blockIdx.x - slot * blocks_per_slot) * kStepRowsPerBlock + tid / LPR;
    const int hv = slot % Hv, b = slot / Hv, hk = key_head(hv, Hk, Hv, flags);

    const ET *kp = k + ((size_t)b * Hk + hk) * DK;
    const ET *qp = q + ((size_t)b * Hk + hk) * DK;
    const size_t row = ((size_t)slot * Dv + j) * DK;
    gfloat *sin = state_in ? (gfloat *)state_in + row : (gfloat *)kZeroRow;

    f32x4 s[NP], kv[NP], qv[NP];
#pragma unroll
    for (int m = 0; m < NP; ++m) {
        const int e = 4 * (m * LPR + sub);
        kv[m] = to_f32x4<ET>(ld4<ET>(kp + e));
        qv[m] = to_f32x4<ET>(ld4<ET>(qp + e));
        s[m] = *reinterpret_cast<gf32x4 *>(sin + e);
    }
    if constexpr (VG) {             // decay each key column first: s <- s diag(g)
#pragma unroll
        for (int m = 0; m < NP; ++m) {
            f32x4 gv = *reinterpret_cast<const f32x4 *>(g + (size_t)slot * DK + 4 * (m * LPR + sub));
            if (flags & kLogGate) {            // uniform: exp only for log-space gates
#pragma unroll
                for (int i = 0; i < 4; ++i) gv[i] = expf(gv[i]);
            }
            s[m] *= gv;
        }
    }
    float a = 0.f, bq = 0.f, kq = 0.f;
#pragma unroll
    for (int m = 0; m < NP; ++m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a += s[m][i] * kv[m][i];
            bq += s[m][i] * qv[m][i];
            kq += kv[m][i] * qv[m][i];
        }
    }
    static_assert(LPR == 8, "sum8 reduces over aligned groups of eight lanes");
    a = sum8(a);
    bq = sum8(bq);
    kq = sum8(kq);
    const float gt = VG ? 1.f : decay_of(g[slot], flags), bt = beta[slot];
    const float vj = to_f32(v[(size_t)slot * Dv + j]);
    const float d = bt * (vj - gt * a);
#pragma unroll
    for (int m = 0; m < NP; ++m) {
        const int e = 4 * (m * LPR + sub);
        *reinterpret_cast<f32x4 *>(state_out + row + e) = gt * s[m] + d * kv[m];
    }
    if (sub == 0) y[(size_t)slot * Dv + j] = from_f32<ET>((gt * bq + d * kq) * scale);
}

template <typename ET, int DK, bool VG>
static hipError_t launch_step_vg(const FwdArgs &a, hipStream_t st) {
    const dim3 grid((unsigned)a.B * (unsigned)a.Hv * (unsigned)(a.Dv / kStepRowsPerBlock));
    const dim3 block(kStepRowsPerBlock * kStepLanesPerRow);
    hipLaunchKernelGGL((step_kernel<ET, DK, VG>), grid, block, 0, st,
                       static_cast<const ET *>(a.q), static_cast<const ET *>(a.k),
                       static_cast<const ET *>(a.v), a.g, a.beta, a.state_in, a.state_out,
                       static_cast<ET *>(a.y), a.Hk, a.Hv, a.Dv, a.scale, a.flags);
    return hipGetLastError();
}

template <typename ET, int DK>
static hipError_t launch_step_inst(const FwdArgs &a, hipStream_t st) {
    return (a.flags & kVectorGate) ? launch_step_vg<ET, DK, true>(a, st) : launch_step_vg<ET, DK, false>(a, st);
}

template <typename ET>
static hipError_t launch_step_typed(const FwdArgs &a, hipStream_t st) {
    switch (a.Dk) {
    case 32: return launch_step_inst<ET, 32>(a, st);
    case 64: return launch_step_inst<ET, 64>(a, st);
    case 128: return launch_step_inst<ET, 128>(a, st);
    default: return hipErrorInvalidValue;
    }
}

// T tokens with the state read once and written once: the sequential rule
// of the step above (the form the ferrox-core gdn_chunk.rs page takes as the
// definition, "The algebra"), looped over the tokens with the state held in
// registers.  Packing several value rows into one SIMD group for the
// token-by-token path follows the MLX pull request page "Pack
// gated_delta_seq: 8 value rows per SIMD-group" (Summary).  Here eight lanes
// share R value rows (R = 1, 2 or 4): lane i of the eight holds the 16-byte
// pieces i, i+8, ... of each of its rows, so that one conversion of k and q
// serves R rows and one butterfly finishes 2R + 1 dot products.
//
// The decay is kept outside the registers: the state is c * S' with a
// per-slot scalar c (the running product of the gates, reset to 1 whenever
// it leaves [2^-24, 2^24] by folding it into S').  A token then costs two
// dot products and one multiply-add per state element:
//     c <- c g,  a = c (S' . k),  b = c (S' . q),  d = beta (v - a)
//     S' <- S' + (d / c) k,  y = (b + d (k . q)) / sqrt(Dk)
// which is the step's arithmetic with g S applied lazily.  The next token's
// k, q, v, g and beta are loaded while the current one runs.
template <typename ET, int R> struct RowVec;
template <typename ET> struct RowVec<ET, 1> {
    using T = ET;
    static __device__ __forceinline__ T ld(const ET *p) { return *p; }
    static __device__ __forceinline__ float at(T v, int) { return to_f32(v); }
};
template <typename ET> struct RowVec<ET, 2> {
    using T = ET __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ T ld(const ET *p) { return *reinterpret_cast<const T *>(p); }
    static __device__ __forceinline__ float at(T v, int i) { return to_f32(v[i]); }
};
template <typename ET> struct RowVec<ET, 4> {
    using T = typename Vec<ET>::x4;
    static __device__ __forceinline__ T ld(const ET *p) { return ld4<ET>(p); }
    static __device__ __forceinline__ float at(T v, int i) { return to_f32(v[i]); }
};

// VG: g is [B,T,Hv,Dk]; each token first decays the state's key columns by
// their own factors (no deferred scale), then runs the same steps.
template <typename ET, int DK, int R, bool VG>
__global__ __launch_bounds__(256)
void seq_kernel(const ET *__restrict__ q, const ET *__restrict__ k,
                const ET *__restrict__ v, const float *__restrict__ g,
                const float *__restrict__ beta, const float *state_in,
                float *state_out, ET *__restrict__ y,
                int T, int Hk, int Hv, int Dv, float scale, int flags)
{
    constexpr int NP = DK / 32;                   // 16-byte pieces per lane and row
    constexpr int ROWS = 32 * R;                  // value rows per workgroup
    using RV = RowVec<ET, R>;
    const int tid = threadIdx.x;
    const int sub = tid & 7;
    const int blocks_per_slot = Dv / ROWS;
    const int slot = blockIdx.x / blocks_per_slot;
    const int j0 = (blockIdx.x - slot * blocks_per_slot) * ROWS + (tid >> 3) * R;
    const int hv = slot % Hv, b = slot / Hv, hk = key_head(hv, Hk, Hv, flags);
    const size_t qks = (size_t)Hk * DK, vs = (size_t)Hv * Dv;
    const ET *kp = k + ((size_t)b * T * Hk + hk) * DK + 4 * sub;
    const ET *qp = q + ((size_t)b * T * Hk + hk) * DK + 4 * sub;
    const ET *vp = v + ((size_t)b * T * Hv + hv) * Dv + j0;
    const float *gp = g + ((size_t)b * T * Hv + hv) * (VG ? DK : 1), *bp = beta + (size_t)b * T * Hv + hv;
    ET *yp = y + ((size_t)b * T * Hv + hv) * Dv + j0;
    const size_t row0 = ((size_t)slot * Dv + j0) * DK + 4 * sub;

    // rows of zeros (stride 0) when there is no initial state
    gfloat *sin = state_in ? (gfloat *)state_in + row0 : (gfloat *)kZeroRow + 4 * sub;
    const int sstride = state_in ? DK : 0;
    f32x4 s[R][NP];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < NP; ++m)
            s[r][m] = *reinterpret_cast<gf32x4 *>(sin + (size_t)r * sstride + 32 * m);
    typename Vec<ET>::x4 kn[NP], qn[NP];
    typename RV::T vn{};
    float gn = 0.f, bn = 0.f;
    f32x4 gvn[VG ? NP : 1];
    auto load = [&](int t) {
#pragma unroll
        for (int m = 0; m < NP; ++m) {
            kn[m] = ld4<ET>(kp + (size_t)t * qks + 32 * m);
            qn[m] = ld4<ET>(qp + (size_t)t * qks + 32 * m);
        }
        vn = RV::ld(vp + (size_t)t * vs);
        if constexpr (VG) {
#pragma unroll
            for (int m = 0; m < NP; ++m)
                gvn[m] = *reinterpret_cast<const f32x4 *>(gp + (size_t)t * Hv * DK + 4 * sub + 32 * m);
        } else {
            gn = gp[(size_t)t * Hv];
        }
        bn = bp[(size_t)t * Hv];
    };
    if (T > 0) load(0);
    float c = 1.f;
    for (int t = 0; t < T; ++t) {
        f32x4 kv[NP], qv[NP];
#pragma unroll
        for (int m = 0; m < NP; ++m) {
            kv[m] = to_f32x4<ET>(kn[m]);
            qv[m] = to_f32x4<ET>(qn[m]);
        }
        const typename RV::T vt = vn;
        f32x4 gvt[VG ? NP : 1];
        if constexpr (VG) {
#pragma unroll
            for (int m = 0; m < NP; ++m) gvt[m] = gvn[m];
        }
        float gt = VG ? 1.f : gn;
        if (!VG && (flags & kLogGate)) gt = expf(gt);   // uniform
        const float bt = bn;
        if (t + 1 < T) load(t + 1);
        if constexpr (VG) {
            if (flags & kLogGate) {            // uniform: exp only for log-space gates
#pragma unroll
                for (int m = 0; m < NP; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i) gvt[m][i] = expf(gvt[m][i]);
            }
#pragma unroll
            for (int m = 0; m < NP; ++m)
#pragma unroll
                for (int r = 0; r < R; ++r) s[r][m] *= gvt[m];
        } else {
            c *= gt;
            if (!(c >= 0x1p-24f && c <= 0x1p24f)) {   // uniform over the slot
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < NP; ++m) s[r][m] = c * s[r][m];
                c = 1.f;
            }
        }
        float kq = 0.f, a[R], bq[R];
#pragma unroll
        for (int r = 0; r < R; ++r) a[r] = bq[r] = 0.f;
#pragma unroll
        for (int m = 0; m < NP; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kq += kv[m][i] * qv[m][i];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    a[r] += s[r][m][i] * kv[m][i];
                    bq[r] += s[r][m][i] * qv[m][i];
                }
            }
        kq = sum8(kq);
        const float rc = VG ? 1.f : __builtin_amdgcn_rcpf(c);   // 1 ulp
        float yo[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float ar = sum8(a[r]), br = sum8(bq[r]);
            const float d = bt * (RV::at(vt, r) - c * ar);
            yo[r] = (c * br + d * kq) * scale;
            const float dc = d * rc;
#pragma unroll
            for (int m = 0; m < NP; ++m) s[r][m] += dc * kv[m];
        }
        if (sub == 0) {
            ET *yt = yp + (size_t)t * vs;
#pragma unroll
            for (int r = 0; r < R; ++r) yt[r] = from_f32<ET>(yo[r]);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < NP; ++m)
            *reinterpret_cast<f32x4 *>(state_out + row0 + (size_t)r * DK + 32 * m) = c * s[r][m];
}

template <typename ET, int DK, int R, bool VG>
static hipError_t launch_seq_vg(const FwdArgs &a, hipStream_t st) {
    const dim3 grid((unsigned)a.B * (unsigned)a.Hv * (unsigned)(a.Dv / (32 * R)));
    hipLaunchKernelGGL((seq_kernel<ET, DK, R, VG>), grid, dim3(256), 0, st,
                       static_cast<const ET *>(a.q), static_cast<const ET *>(a.k),
                       static_cast<const ET *>(a.v), a.g, a.beta, a.state_in, a.state_out,
                       static_cast<ET *>(a.y), a.T, a.Hk, a.Hv, a.Dv, a.scale, a.flags);
    return hipGetLastError();
}

template <typename ET, int DK, int R>
static hipError_t launch_seq_inst(const FwdArgs &a, hipStream_t st) {
    return (a.flags & kVectorGate) ? launch_seq_vg<ET, DK, R, true>(a, st) : launch_seq_vg<ET, DK, R, false>(a, st);
}

// rows per lane: R = 4 when the grid has enough waves to fill the chip,
// fewer rows (more waves, shorter token loops) when it has not; never more
// rows than one workgroup's share of Dv
template <typename ET, int DK>
static hipError_t launch_seq_dk(const FwdArgs &a, hipStream_t st) {
    const long slots = (long)a.B * a.Hv;
    int r = 4;
    while (r > 1 && (32 * r > a.Dv || slots * (a.Dv / (8 * r)) < kSeqMinWaves)) r >>= 1;
    switch (r) {
    case 4: return launch_seq_inst<ET, DK, 4>(a, st);
    case 2: return launch_seq_inst<ET, DK, 2>(a, st);
    default: return launch_seq_inst<ET, DK, 1>(a, st);
    }
}

template <typename ET>
static hipError_t launch_seq_typed(const FwdArgs &a, hipStream_t st) {
    switch (a.Dk) {
    case 32: return launch_seq_dk<ET, 32>(a, st);
    case 64: return launch_seq_dk<ET, 64>(a, st);
    case 128: return launch_seq_dk<ET, 128>(a, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_seq(int dtype, const FwdArgs &a, hipStream_t st) {
    switch (dtype) {
    case 0: return launch_seq_typed<float>(a, st);
    case 1: return launch_seq_typed<__bf16>(a, st);
    case 2: return launch_seq_typed<_Float16>(a, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_step(int dtype, const FwdArgs &a, hipStream_t st) {
    switch (dtype) {
    case 0: return launch_step_typed<float>(a, st);
    case 1: return launch_step_typed<__bf16>(a, st);
    case 2: return launch_step_typed<_Float16>(a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
