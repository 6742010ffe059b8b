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
// The state is read and written with non-temporal loads and stores: it is
// touched once per call, and a decode loop over many layers' states does
// not find it in the cache again; back to back over 8 state buffers in
// rotation (each state from HBM, each output written back) a step took
// 43.8 us with them against 46.6 us with ordinary accesses.
#include <algorithm>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kStepRowsPerBlock = 32;
constexpr int kStepLanesPerRow = 8;
// fewest waves (over the whole grid) for which the sequential kernel keeps
// four value rows per lane
constexpr long kSeqMinWaves = 2048;

// (bound_ctrl set: no lane of these permutations reads outside its row, so
// it changes nothing, and it lets the compiler fold each move into its add)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
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
        s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>((const float *)sin + e));
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
        __builtin_nontemporal_store(gt * s[m] + d * kv[m], reinterpret_cast<f32x4 *>(state_out + row + e));
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
    static __device__ __forceinline__ void set(T &v, int, ET x) { v = x; }
};
template <typename ET> struct RowVec<ET, 2> {
    using T = ET __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ T ld(const ET *p) { return *reinterpret_cast<const T *>(p); }
    static __device__ __forceinline__ float at(T v, int i) { return to_f32(v[i]); }
    static __device__ __forceinline__ void set(T &v, int i, ET x) { v[i] = x; }
};
template <typename ET> struct RowVec<ET, 4> {
    using T = typename Vec<ET>::x4;
    static __device__ __forceinline__ T ld(const ET *p) { return ld4<ET>(p); }
    static __device__ __forceinline__ float at(T v, int i) { return to_f32(v[i]); }
    static __device__ __forceinline__ void set(T &v, int i, ET x) { v[i] = x; }
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
            s[r][m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>((const float *)sin + (size_t)r * sstride + 32 * m));
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
            __builtin_nontemporal_store(c * s[r][m], reinterpret_cast<f32x4 *>(state_out + row0 + (size_t)r * DK + 32 * m));
}

// Persistent form of the sequential kernel (16-bit inputs, scalar gate, a
// few tokens per call).  Each workgroup walks tiles of 32 R value rows; while
// it runs the tokens of one tile, the inputs of its next tile (k, q, the
// tile's v columns, g and beta of every token) stream into the other half of
// a double buffer in LDS and the next tile's state rows into registers, so
// that the state traffic of one tile overlaps the arithmetic of another.
// Per token it is the arithmetic of seq_kernel above.
// (the longest call it takes: at 8 tokens it is still a few percent ahead
// of the kernel above, beyond that the arithmetic per token, not the state
// traffic, sets the time; at most 8, one token per group of eight lanes
// for k . q)
constexpr int kSeqPipeMaxT = 8;
static_assert(kSeqPipeMaxT <= 8, "k . q of one token per group of eight lanes");
// s_waitcnt vmcnt(0) as an immediate (gfx9 encoding: vmcnt 0, expcnt and
// lgkmcnt at their maxima), issued through the builtin so that the
// compiler's own wait bookkeeping sees it: otherwise it assumes the state
// registers loaded before the token loop are still in flight and waits for
// every outstanding load, the next tile's included, before the loop
constexpr int kVmcnt0 = 0x0F70;

template <typename ET, int DK, int R>
struct SeqPipeCfg {
    static constexpr int ROWS = 32 * R;                   // value rows per tile
    static constexpr int VPT = ROWS * 2 / 16;             // 16-byte pieces of v per token
    // bytes of one input buffer for Tp token rows (Tp a multiple of 8)
    static __host__ __device__ constexpr unsigned kq_bytes(int Tp) { return (unsigned)Tp * DK * sizeof(ET); }
    static __host__ __device__ constexpr unsigned v_bytes(int Tp) { return (unsigned)Tp * ROWS * sizeof(ET); }
    // (rounded up to 1 KB, the block of one load instruction)
    static __host__ __device__ constexpr unsigned buf_bytes(int Tp) {
        return (2 * kq_bytes(Tp) + v_bytes(Tp) + 2 * 64 * 4 + 1023) & ~1023u;
    }
};

template <typename ET, int DK, int R>
__global__ __launch_bounds__(256)
void seq_pipe_kernel(const ET *__restrict__ q, const ET *__restrict__ k,
                     const ET *__restrict__ v, const float *__restrict__ g,
                     const float *__restrict__ beta, const float *state_in,
                     float *state_out, ET *__restrict__ y,
                     int T, int Hk, int Hv, int Dv, float scale, int flags, int ntiles)
{
    static_assert(sizeof(ET) == 2, "16-bit inputs");
    using L = SeqPipeCfg<ET, DK, R>;
    using RV = RowVec<ET, R>;
    constexpr int NP = DK / 32;                   // 16-byte state pieces per lane and row
    constexpr int ROWS = L::ROWS;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int Tp = (T + 7) & ~7;
    const unsigned oQ = L::kq_bytes(Tp), oV = 2 * L::kq_bytes(Tp), oG = oV + L::v_bytes(Tp), oB = oG + 256;
    const unsigned bufb = L::buf_bytes(Tp);
    const int tid = threadIdx.x, lane = tid & 63, sub = tid & 7;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tiles_per_slot = Dv / ROWS;
    const size_t qks = (size_t)Hk * DK, vs = (size_t)Hv * Dv;
    const unsigned lds_base = (unsigned)(uintptr_t)((__attribute__((address_space(3))) char *)smem);
    const int sstride = state_in ? DK : 0;

    // inputs of tile ti into buffer bf: wave 0 the k rows, wave 1 the q rows,
    // wave 2 the v columns, wave 3 g and beta; rows past T repeat row T - 1
    auto issue_inputs = [&](int ti, int bf) {
        const int slot = ti / tiles_per_slot, jt = (ti - slot * tiles_per_slot) * ROWS;
        const int hv = slot % Hv, b = slot / Hv, hk = key_head(hv, Hk, Hv, flags);
        const unsigned base = lds_base + (unsigned)bf * bufb;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
        if (wave < 2) {
            const ET *src = (wave == 0 ? k : q) + ((size_t)b * T * Hk + hk) * DK;
            const unsigned dst = base + (wave == 0 ? 0u : oQ);
            for (int i = 0; i < Tp / 4; ++i) {
                const int tok = min(4 * i + (lane >> 4), T - 1);
                const unsigned off = (unsigned)((tok * qks + 8 * (lane & 15)) * sizeof(ET));
                const unsigned la = __builtin_amdgcn_readfirstlane(dst + 1024 * i);
                asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                             :: "v"(off), "s"(src), "s"(la) : "memory", "m0");
            }
        } else if (wave == 2) {
            const ET *src = v + ((size_t)b * T * Hv + hv) * Dv + jt;
            constexpr int TPI = 64 / L::VPT;      // tokens per instruction
            for (int i = 0; i < Tp / TPI; ++i) {
                const int tok = min(TPI * i + lane / L::VPT, T - 1);
                const unsigned off = (unsigned)((tok * vs + 8 * (lane % L::VPT)) * sizeof(ET));
                const unsigned la = __builtin_amdgcn_readfirstlane(base + oV + 1024 * i);
                asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                             :: "v"(off), "s"(src), "s"(la) : "memory", "m0");
            }
        } else {
            const float *gs = g + (size_t)b * T * Hv + hv, *bs = beta + (size_t)b * T * Hv + hv;
            const unsigned off = (unsigned)(min(lane, T - 1) * Hv * 4);
            const unsigned lg = __builtin_amdgcn_readfirstlane(base + oG), lb = __builtin_amdgcn_readfirstlane(base + oB);
            asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                         :: "v"(off), "s"(gs), "s"(lg) : "memory", "m0");
            asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                         :: "v"(off), "s"(bs), "s"(lb) : "memory", "m0");
        }
#pragma clang diagnostic pop
    };
    // first state row of this lane's group in tile ti
    auto row_of = [&](int ti) {
        const int slot = ti / tiles_per_slot, jt = (ti - slot * tiles_per_slot) * ROWS;
        return ((size_t)slot * Dv + jt + (tid >> 3) * R) * DK + 4 * sub;
    };
    auto load_state = [&](int ti, f32x4 (&st)[R][NP]) {
        gfloat *sin = state_in ? (gfloat *)state_in + row_of(ti) : (gfloat *)kZeroRow + 4 * sub;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < NP; ++m)
                st[r][m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>((const float *)sin + (size_t)r * sstride + 32 * m));
    };

    int ti = blockIdx.x;
    f32x4 s[R][NP], sn[R][NP];
    issue_inputs(ti, 0);
    load_state(ti, s);
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    __syncthreads();
    for (int it = 0;; ++it) {
        const int tn = ti + (int)gridDim.x;
        if (tn < ntiles) {
            issue_inputs(tn, (it + 1) & 1);
            load_state(tn, sn);
        }
        const int slot = ti / tiles_per_slot, jt = (ti - slot * tiles_per_slot) * ROWS;
        const int hv = slot % Hv, b = slot / Hv;
        ET *yp = y + ((size_t)b * T * Hv + hv) * Dv + jt + (tid >> 3) * R;
        const char *buf = smem + (it & 1) * bufb;
        // token t's inputs from LDS, read at the start of the token (reading
        // one token ahead cost a register copy of every fragment and a wave
        // per SIMD: 124 registers let four waves share a SIMD)
        typename Vec<ET>::x4 kn[NP], qn[NP];
        typename RV::T vn;
        // the decays and betas of the tile's tokens, lane t holding token t's
        // (one exp per token for log-space gates, not one per token and lane)
        const float dec_l = decay_of(reinterpret_cast<const float *>(buf + oG)[lane], flags);
        const float beta_l = reinterpret_cast<const float *>(buf + oB)[lane];
        // k . q of token t on the eight lanes of group t (T <= 8 groups),
        // read per token from lane 8 t
        float kq_l = 0.f;
        {
            const int tq = min(tid >> 3 & 7, T - 1);
#pragma unroll
            for (int m = 0; m < NP; ++m) {
                const f32x4 kk = to_f32x4<ET>(*reinterpret_cast<const typename Vec<ET>::x4 *>(buf + (tq * DK + 32 * m + 4 * sub) * sizeof(ET)));
                const f32x4 qq = to_f32x4<ET>(*reinterpret_cast<const typename Vec<ET>::x4 *>(buf + oQ + (tq * DK + 32 * m + 4 * sub) * sizeof(ET)));
#pragma unroll
                for (int i = 0; i < 4; ++i) kq_l += kk[i] * qq[i];
            }
            kq_l = sum8(kq_l);
        }
        auto lds_token = [&](int t) {
#pragma unroll
            for (int m = 0; m < NP; ++m) {
                kn[m] = *reinterpret_cast<const typename Vec<ET>::x4 *>(buf + (t * DK + 32 * m + 4 * sub) * sizeof(ET));
                qn[m] = *reinterpret_cast<const typename Vec<ET>::x4 *>(buf + oQ + (t * DK + 32 * m + 4 * sub) * sizeof(ET));
            }
            vn = *reinterpret_cast<const typename RV::T *>(buf + oV + (t * ROWS + (tid >> 3) * R) * sizeof(ET));
        };
        float c = 1.f;
        for (int t = 0; t < T; ++t) {
            lds_token(t);
            f32x4 kv[NP], qv[NP];
#pragma unroll
            for (int m = 0; m < NP; ++m) {
                kv[m] = to_f32x4<ET>(kn[m]);
                qv[m] = to_f32x4<ET>(qn[m]);
            }
            const typename RV::T vt = vn;
            const float gt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, dec_l), t));
            const float bt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, beta_l), t));
            c *= gt;
            if (!(c >= 0x1p-24f && c <= 0x1p24f)) {   // uniform over the tile
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int m = 0; m < NP; ++m) s[r][m] = c * s[r][m];
                c = 1.f;
            }
            float a[R], bq[R];
#pragma unroll
            for (int r = 0; r < R; ++r) a[r] = bq[r] = 0.f;
#pragma unroll
            for (int m = 0; m < NP; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        a[r] += s[r][m][i] * kv[m][i];
                        bq[r] += s[r][m][i] * qv[m][i];
                    }
                }
            const float kq = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, kq_l), 8 * t));
            const float rc = __builtin_amdgcn_rcpf(c);   // 1 ulp
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
                typename RV::T yv;
#pragma unroll
                for (int r = 0; r < R; ++r) RV::set(yv, r, from_f32<ET>(yo[r]));
                *reinterpret_cast<typename RV::T *>(yp + (size_t)t * vs) = yv;
            }
        }
        auto store_state = [&]() {
            const size_t row = row_of(ti);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < NP; ++m)
                    __builtin_nontemporal_store(c * s[r][m], reinterpret_cast<f32x4 *>(state_out + row + (size_t)r * DK + 32 * m));
        };
        if (tn >= ntiles) {
            store_state();
            break;
        }
        // the next tile's inputs (every wave's share) and state have landed;
        // this tile's state is stored after the wait, so that the wait does
        // not include the time its stores take to complete
        __builtin_amdgcn_s_waitcnt(kVmcnt0);
        __syncthreads();
        store_state();
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < NP; ++m) s[r][m] = sn[r][m];
        ti = tn;
    }
}

// Workgroups of seq_pipe_kernel resident on the current device at once
// (bound by registers: the input buffers for the longest token count allowed
// take a few percent of the LDS); 0 if the runtime cannot say.
template <typename ET, int DK, int R>
static long seq_pipe_resident() {
    using L = SeqPipeCfg<ET, DK, R>;
    static long per_dev[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (per_dev[dev] == 0) {
        int nb = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, seq_pipe_kernel<ET, DK, R>, 256,
                                                         2 * L::buf_bytes(kSeqPipeMaxT)) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        per_dev[dev] = (long)std::max(nb, 0) * std::max(cus, 0);
    }
    return per_dev[dev];
}

template <typename ET, int DK, int R>
static hipError_t launch_seq_pipe(const FwdArgs &a, hipStream_t st, long resident) {
    using L = SeqPipeCfg<ET, DK, R>;
    const long ntiles = (long)a.B * a.Hv * (a.Dv / L::ROWS);
    const int Tp = (a.T + 7) & ~7;
    const size_t lds = 2 * (size_t)L::buf_bytes(Tp);
    const long grid = std::min(ntiles, resident);
    hipLaunchKernelGGL((seq_pipe_kernel<ET, DK, R>), dim3((unsigned)grid), dim3(256), lds, st,
                       static_cast<const ET *>(a.q), static_cast<const ET *>(a.k),
                       static_cast<const ET *>(a.v), a.g, a.beta, a.state_in, a.state_out,
                       static_cast<ET *>(a.y), a.T, a.Hk, a.Hv, a.Dv, a.scale, a.flags, (int)ntiles);
    return hipGetLastError();
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
    // a few tokens on a grid of at least two tiles per resident workgroup:
    // the persistent kernel, whose state traffic for one tile overlaps the
    // arithmetic of another (two rows per lane: about 125 registers, four
    // waves per SIMD; four rows per lane need over 200 and run slower per
    // token, one row per lane is slower too)
    if constexpr (sizeof(ET) == 2 && DK == 128) {
        if (!(a.flags & kVectorGate) && a.T >= 1 && a.T <= kSeqPipeMaxT && a.Dv % 64 == 0) {
            const long res = seq_pipe_resident<ET, DK, 2>();
            if (res > 0 && slots * (a.Dv / 64) >= 2 * res) return launch_seq_pipe<ET, DK, 2>(a, st, res);
        }
    }
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
