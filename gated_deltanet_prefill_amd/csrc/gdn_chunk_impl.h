// gdn_chunk_impl.h -- the chunked gated-delta-rule forward kernel for gfx950.
//
// One workgroup owns one (batch, value head) slot and walks its T tokens in
// chunks of C, with the Dk x Dv state resident in registers (MFMA
// accumulator tiles of S^T) from the first chunk to the last; the state is
// read from HBM once and written once.
//
// Per chunk (c <= C tokens; rows past the end of the sequence are staged as
// k = q = v = 0, g = 1, beta = 0, which leaves the recurrence unchanged --
// the padding the metaltile-std gated_delta_wy.rs page asks its caller for):
//
//  stage    K, Q and this slice of V into LDS, row-major (transposed
//           operands are read from the same rows with gfx950's LDS transpose
//           load).
//  gates    chunk-local decay products, every one formed by multiplying
//           decays (ferrox-core gdn_chunk.rs page, "The algebra": a ratio is
//           a product, and an underflow is a state really forgotten):
//             G[t] = g_0 ... g_t,   R[t][j] = g_{j+1} ... g_t  (j <= t),
//           from 16-token blocks: in-block rows by running products, across
//           blocks (prefix in t's block) x (whole blocks between) x (suffix
//           in j's block).
//  X = K S0^T, Y^T = S0 Q^T and the C x C tiles K K^T, Q K^T (MFMA), all
//           from one pass over the K and Q fragments;
//           A[t][j] = beta_t R[t][j] k_t.k_j (j < t), QKR[t][j] = R[t][j] q_t.k_j (j <= t).
//  T_ii = (I + A_ii)^-1 for the 16x16 diagonal blocks, f32 forward
//           substitution (four lanes per column).
//  D = (I + A)^-1 beta (V - G X): the true per-token deltas
//           d_t = beta_t (v_t - g_t S_{t-1} k_t) of the whole chunk (the
//           ferrox-core page's per-row forward substitution, written for all
//           rows at once), by blocked forward substitution over 16-token
//           blocks: D_i = T_ii (RHS_i - sum_{j<i} A_ij D_j), in float32
//           throughout (-A, T_ii and the solved blocks float32, float32
//           matrix-core products, v_mfma_f32_16x16x4_f32).
//           This is the unit lower triangular system of the metaltile-std
//           page's steps 4-5.
//  y_t = (G_t S0 q_t + sum_{j<=t} R[t][j] (q_t.k_j) d_j) / sqrt(Dk)   (MFMA)
//  S  <- G_{c-1} S0 + sum_t R[c-1][t] d_t k_t^T                        (MFMA)
//
// Work split: wave w owns 16*NB value columns of the slice and holds
// S^T[0:Dk, its columns] as NBK x NB accumulator tiles; it computes X, D, y
// and the update for its columns alone (a state row's update needs only that
// row, k and the shared C x C matrices).  The C x C work is shared through
// LDS; wave w computes the tile columns tb = w, w + NW, ...

#pragma once

#include "gdn_device.h"

namespace gdn {

template <typename ET, int DK_, int DVS_, int C_, int NB_>
struct ChunkCfg {
    static constexpr int DK = DK_, DVS = DVS_, C = C_, NB = NB_;
    static constexpr int NW = DVS / (16 * NB);        // waves per workgroup
    static constexpr int NT = 64 * NW;                // threads per workgroup
    static constexpr int NBT = C / 16;                // 16-token blocks per chunk
    static constexpr int NBK = DK / 16;               // 16-wide key blocks
    static constexpr int NTPW = (NBT + NW - 1) / NW;  // tile columns per wave
    static constexpr int ES = (int)sizeof(ET);
    static constexpr int EPU = 16 / ES;               // elements per 16-byte unit
    // Row padding of 16 bytes: sixteen rows read at one column offset fall in
    // sixteen different 4-bank groups.
    static constexpr int LDK = DK + EPU;              // sK, sQ
    static constexpr int LDV = DVS + EPU;             // sV
    static constexpr int LDC = C + EPU;               // sQKR (rows of C input-type elements)
    static constexpr int LDCF = C + 4;                // sAn (float32 rows of C)
    static constexpr int LDD = 16 + 4;                // sAd (f32 diagonal blocks)
    static constexpr int LDTF = 16 + 4;               // sTd (float32 diagonal inverses)
    static constexpr int oK = 0;
    static constexpr int oQ = oK + C * LDK * ES;
    static constexpr int oV = oQ + C * LDK * ES;
    static constexpr int oAn = oV + C * LDV * ES;
    static constexpr int oQKR = oAn + C * LDCF * 4;
    static constexpr int oAd = oQKR + C * LDC * ES;
    static constexpr int oTd = oAd + C * LDD * 4;
    static constexpr int oVec = oTd + C * LDTF * 4;   // beta, g, P, Sfx, G, Rlast, block totals
    static constexpr int BYTES = oVec + 7 * C * 4;
    // staging in 16-byte units
    static constexpr int UPK = DK / EPU;
    static constexpr int UPV = DVS / EPU;
    static constexpr int KIT = C * UPK, VIT = C * UPV;
    static constexpr int PERK = (KIT + NT - 1) / NT;
    static constexpr int PERV = (VIT + NT - 1) / NT;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(NW >= 1 && NW * 16 * NB == DVS, "value slice must split into whole waves");
    static_assert(LDK % 4 == 0 && LDV % 4 == 0, "transpose loads need 8-byte aligned rows");
};

// A fragment over one contraction step: two 16-blocks (16-bit types, one
// MFMA) or one 16-block (f32, four MFMAs).
template <typename ET> struct Step {
    static constexpr int BLK = 2;
    using frag = typename Vec<ET>::x8;
};
template <> struct Step<float> {
    static constexpr int BLK = 1;
    using frag = f32x4;
};

template <int NBLK, int BLK> struct Steps { static constexpr int n = (NBLK + BLK - 1) / BLK; };

// Fragment of contraction step s from per-block fetches fb(kb); blocks at or
// past `lim` read as zero.
template <typename ET, typename F>
__device__ __forceinline__ typename Step<ET>::frag make_frag(int s, int lim, F fb) {
    if constexpr (sizeof(ET) == 4) {
        return fb(s);
    } else {
        using X4 = typename Vec<ET>::x4;
        const int kb = 2 * s;
        X4 lo = fb(kb);
        X4 hi = (kb + 1 < lim) ? fb(kb + 1) : cvt4<ET>(zero4());
        return cat8<ET>(lo, hi);
    }
}

__device__ __forceinline__ f32x4 mfma_step(f32x4 a, f32x4 b, f32x4 c) {
    c = mfma(a[0], b[0], c);
    c = mfma(a[1], b[1], c);
    c = mfma(a[2], b[2], c);
    c = mfma(a[3], b[3], c);
    return c;
}
__device__ __forceinline__ f32x4 mfma_step(bf16x8 a, bf16x8 b, f32x4 c) { return mfma(a, b, c); }
__device__ __forceinline__ f32x4 mfma_step(f16x8 a, f16x8 b, f32x4 c) { return mfma(a, b, c); }

// Row fragment of a row-major matrix: lane (x, qd) holds row r0 + x,
// columns c0 + 16 kb + 4 qd + (0..3).
template <typename ET>
__device__ __forceinline__ typename Vec<ET>::x4 frag_row(const ET *m, int ld, int r0, int c0, int kb, int x, int qd) {
    return ld4<ET>(m + (r0 + x) * ld + c0 + 16 * kb + 4 * qd);
}

// Column fragment of a row-major matrix (the fragment of its transpose):
// lane (x, qd) holds column c0 + x, rows r0 + 16 kb + 4 qd + (0..3).  For
// 16-bit types one LDS transpose load does it: within each group of 16
// lanes, lane m receives element m%4 of the 8-byte pieces addressed by lanes
// m/4 + 4i (i = 0..3), so lane j points at row j/4, columns 4 (j%4) .. +3.
template <typename ET>
__device__ __forceinline__ typename Vec<ET>::x4 frag_col(const ET *m, int ld, int r0, int c0, int kb, int x, int qd) {
    const int rb = r0 + 16 * kb + 4 * qd;
    if constexpr (sizeof(ET) == 2) {
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        const ET *p = m + (rb + (x >> 2)) * ld + c0 + 4 * (x & 3);
        const s16x4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(p));
        return __builtin_bit_cast(typename Vec<ET>::x4, raw);
    } else {
        typename Vec<ET>::x4 r;
        r[0] = m[(rb + 0) * ld + c0 + x];
        r[1] = m[(rb + 1) * ld + c0 + x];
        r[2] = m[(rb + 2) * ld + c0 + x];
        r[3] = m[(rb + 3) * ld + c0 + x];
        return r;
    }
}

// Broadcast lane K of every group of four lanes to the group (DPP quad_perm).
template <int K>
__device__ __forceinline__ float quad_bcast(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), K * 0x55, 0xf, 0xf, true));
}

// Value of the lane S below / above within each row of 16 lanes (DPP
// row_shr / row_shl); lanes without one get 1.
template <int S>
__device__ __forceinline__ float dpp_row_shr(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        __builtin_bit_cast(int, 1.0f), __builtin_bit_cast(int, v), 0x110 + S, 0xf, 0xf, false));
}
template <int S>
__device__ __forceinline__ float dpp_row_shl(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        __builtin_bit_cast(int, 1.0f), __builtin_bit_cast(int, v), 0x100 + S, 0xf, 0xf, false));
}

__device__ __forceinline__ uint4 zero_u4() { return make_uint4(0u, 0u, 0u, 0u); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, then for every wave.  Unlike __syncthreads() it does not wait
// for outstanding global loads and stores, so the next chunk's loads and this
// chunk's y stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// y rows t0 .. t0 + cn - 1 of one slot from accumulator tiles Ya[vb][tb]
// (lane (x, qd): token 16 tb + x, values vloc + 16 vb + 4 qd + (0..3)),
// through a buffer resource that spans the cn valid rows: the hardware drops
// the stores of rows past the end, with no branch around them.  `ybase`
// points at row t0, `ld` is the row stride in elements.
template <typename ET, int NB, int NBT>
__device__ __forceinline__ void store_y(ET *ybase, int ld, int cn, int vloc, int x, int qd,
                                        const f32x4 (&Ya)[NB][NBT]) {
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    const unsigned rowb = (unsigned)ld * (unsigned)sizeof(ET);
    const __amdgpu_buffer_rsrc_t yr =
        __builtin_amdgcn_make_buffer_rsrc((void *)ybase, (short)0, (int)((unsigned)cn * rowb), 0x00020000);
#pragma unroll
    for (int tb = 0; tb < NBT; ++tb)
#pragma unroll
        for (int vb = 0; vb < NB; ++vb) {
            const int off = (int)((16 * tb + x) * rowb + (vloc + 16 * vb + 4 * qd) * sizeof(ET));
            if constexpr (sizeof(ET) == 2)
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, cvt4<ET>(Ya[vb][tb])), yr, off, 0, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, Ya[vb][tb]), yr, off, 0, 0);
        }
}

template <typename ET, int DK, int DVS, int C, int NB>
__global__ __launch_bounds__(4 * DVS / NB, 1)
void chunk_fwd_kernel(const ET *__restrict__ q, const ET *__restrict__ k,
                      const ET *__restrict__ v, const float *__restrict__ g,
                      const float *__restrict__ beta, const float *state_in,
                      float *state_out, ET *__restrict__ y,
                      int T, int Hk, int Hv, int Dv, int nsplit, int xcd_group, float scale,
                      int flags)
{
    using L = ChunkCfg<ET, DK, DVS, C, NB>;
    using X4 = typename Vec<ET>::x4;
    using FR = typename Step<ET>::frag;
    constexpr int BLK = Step<ET>::BLK;
    constexpr int NBT = L::NBT, NBK = L::NBK, NW = L::NW, NT = L::NT, NTPW = L::NTPW;
    constexpr int LDK = L::LDK, LDV = L::LDV, LDC = L::LDC, LDCF = L::LDCF, LDD = L::LDD,
                  LDTF = L::LDTF, EPU = L::EPU;
    constexpr int NSK = Steps<NBK, BLK>::n;            // contraction steps over Dk
    constexpr int NST = Steps<NBT, BLK>::n;            // contraction steps over C

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    ET *sK = reinterpret_cast<ET *>(smem + L::oK);
    ET *sQ = reinterpret_cast<ET *>(smem + L::oQ);
    ET *sV = reinterpret_cast<ET *>(smem + L::oV);
    float *sAn = reinterpret_cast<float *>(smem + L::oAn);  // -A (f32)
    ET *sQKR = reinterpret_cast<ET *>(smem + L::oQKR);
    float *sAd = reinterpret_cast<float *>(smem + L::oAd);  // diagonal blocks of A (f32)
    float *sTd = reinterpret_cast<float *>(smem + L::oTd);  // diagonal blocks of (I + A)^-1 (f32)
    float *sb = reinterpret_cast<float *>(smem + L::oVec);
    float *sg = sb + C;
    float *sP = sg + C;
    float *sSfx = sP + C;
    float *sG = sSfx + C;
    float *sRl = sG + C;
    float *sBT = sRl + C;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, x = lane & 15, qd = lane >> 4;
    // Workgroups are dealt round-robin over the 8 XCDs, so workgroups i and
    // i + 8 share an XCD and its L2.  With xcd_group = Hv/Hk > 1 they get
    // value heads of the same key head, whose q/k stream is then fetched
    // from HBM once per group instead of once per head.
    int bid = blockIdx.x;
    if (xcd_group > 1) {
        const int xcd = bid & 7, kk = bid >> 3;
        const int sib = kk % xcd_group, m = kk / xcd_group;
        bid = (m * 8 + xcd) * xcd_group + sib;
    }
    const int rank = bid / nsplit, vs = bid - rank * nsplit;
    const int b = rank / Hv, hv = value_head_of_rank(rank % Hv, Hk, Hv, flags);
    const int hk = key_head(hv, Hk, Hv, flags);
    const int slot = b * Hv + hv;
    const int vloc = wave * 16 * NB;               // first slice column of this wave

    // ---- the state, S^T tiles [key block][value block], f32 accumulators
    f32x4 S[NBK][NB];
    const size_t sbase = (size_t)slot * Dv * DK;
    {
        // rows of zeros (stride 0) when there is no initial state
        gfloat *sin = state_in ? (gfloat *)state_in + sbase : (gfloat *)kZeroRow;
        const size_t rstride = state_in ? DK : 0;
#pragma unroll
        for (int vb = 0; vb < NB; ++vb) {
            const size_t row = (size_t)(vs * DVS + vloc + 16 * vb + x) * rstride;
#pragma unroll
            for (int kb = 0; kb < NBK; ++kb)
                S[kb][vb] = *reinterpret_cast<gf32x4 *>(sin + row + 16 * kb + 4 * qd);
        }
    }

    // ---- -A and QKR above the diagonal blocks stay zero; clear them once
    for (int i = tid; i < (L::oAd - L::oAn) / 16; i += NT)
        reinterpret_cast<uint4 *>(smem + L::oAn)[i] = zero_u4();

    // ---- global -> register prefetch of one chunk.  Every load is issued
    // unconditionally from a clamped (always valid) row; rows past the end
    // of the sequence are zeroed when the registers are staged.
    const size_t kstride = (size_t)Hk * DK, vstride = (size_t)Hv * Dv;
    const ET *kbase = k + ((size_t)b * T * Hk + hk) * DK;
    const ET *qbase = q + ((size_t)b * T * Hk + hk) * DK;
    const ET *vbase = v + ((size_t)b * T * Hv + hv) * Dv + vs * DVS;
    const float *gbase = g + (size_t)b * T * Hv + hv;
    const float *bbase = beta + (size_t)b * T * Hv + hv;

    uint4 rk[L::PERK], rq[L::PERK], rv[L::PERV];
    float rg = 1.f, rb = 0.f;
    auto prefetch = [&](int t0) {
        const int last = min(C, T - t0) - 1;
#pragma unroll
        for (int i = 0; i < L::PERK; ++i) {
            const int it = min(tid + i * NT, L::KIT - 1);
            const int t = min(it / L::UPK, last), u = it % L::UPK;
            rk[i] = *reinterpret_cast<const uint4 *>(kbase + (size_t)(t0 + t) * kstride + u * EPU);
            rq[i] = *reinterpret_cast<const uint4 *>(qbase + (size_t)(t0 + t) * kstride + u * EPU);
        }
#pragma unroll
        for (int i = 0; i < L::PERV; ++i) {
            const int it = min(tid + i * NT, L::VIT - 1);
            const int t = min(it / L::UPV, last), u = it % L::UPV;
            rv[i] = *reinterpret_cast<const uint4 *>(vbase + (size_t)(t0 + t) * vstride + u * EPU);
        }
        const int tg = min(tid, last);
        rg = gbase[(size_t)(t0 + tg) * Hv];
        rb = bbase[(size_t)(t0 + tg) * Hv];
    };

    // Registers -> LDS (row-major K, Q, V; beta); rows t >= cn become zero,
    // g = 1, beta = 0.  The empty asm statements pin the point where the
    // prefetched values are first needed here, after the barrier.
    auto stage = [&](int cn) {
#pragma unroll
        for (int i = 0; i < L::PERK; ++i) {
            asm volatile("" : "+v"(rk[i].x), "+v"(rk[i].y), "+v"(rk[i].z), "+v"(rk[i].w));
            asm volatile("" : "+v"(rq[i].x), "+v"(rq[i].y), "+v"(rq[i].z), "+v"(rq[i].w));
        }
#pragma unroll
        for (int i = 0; i < L::PERV; ++i)
            asm volatile("" : "+v"(rv[i].x), "+v"(rv[i].y), "+v"(rv[i].z), "+v"(rv[i].w));
        asm volatile("" : "+v"(rg), "+v"(rb));
        if (cn < C) {                                  // tail chunk: zero the padded rows
#pragma unroll
            for (int i = 0; i < L::PERK; ++i) {
                const int t = (tid + i * NT) / L::UPK;
                if (t >= cn) { rk[i] = zero_u4(); rq[i] = zero_u4(); }
            }
#pragma unroll
            for (int i = 0; i < L::PERV; ++i)
                if ((tid + i * NT) / L::UPV >= cn) rv[i] = zero_u4();
        }
#pragma unroll
        for (int i = 0; i < L::PERK; ++i) {
            const int it = tid + i * NT;
            if (L::KIT % NT == 0 || it < L::KIT) {
                const int t = it / L::UPK, u = it - t * L::UPK;
                *reinterpret_cast<uint4 *>(sK + t * LDK + u * EPU) = rk[i];
                *reinterpret_cast<uint4 *>(sQ + t * LDK + u * EPU) = rq[i];
            }
        }
#pragma unroll
        for (int i = 0; i < L::PERV; ++i) {
            const int it = tid + i * NT;
            if (L::VIT % NT == 0 || it < L::VIT) {
                const int t = it / L::UPV, u = it - t * L::UPV;
                *reinterpret_cast<uint4 *>(sV + t * LDV + u * EPU) = rv[i];
            }
        }
        // Gate products (wave 0, lane t holds g_t; g = 1 past the end):
        // within each 16-token block (one DPP row) the inclusive prefix
        // products P and the exclusive suffix products Sfx by four
        // doubling steps; block totals BT; G[t] = P[t] * BT of earlier
        // blocks; Rl[t] = R[c-1][t] = Sfx[t] * BT of later blocks.
        if (wave == 0) {
            const float gt = (tid < cn) ? decay_of(rg, flags) : 1.f;
            float p = gt, sx = gt;
            p *= dpp_row_shr<1>(p);
            p *= dpp_row_shr<2>(p);
            p *= dpp_row_shr<4>(p);
            p *= dpp_row_shr<8>(p);
            sx *= dpp_row_shl<1>(sx);
            sx *= dpp_row_shl<2>(sx);
            sx *= dpp_row_shl<4>(sx);
            sx *= dpp_row_shl<8>(sx);
            const float sfx = dpp_row_shl<1>(sx);
            const int bt = lane >> 4;
            float gpre = p, rl = sfx;
#pragma unroll
            for (int bb = 0; bb < NBT; ++bb) {
                const float tot = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), 16 * bb + 15));
                if (bb < bt) gpre *= tot;
                if (bb > bt) rl *= tot;
                if (lane == bb) sBT[bb] = tot;
            }
            if (lane < C) {
                sb[lane] = (lane < cn) ? rb : 0.f;
                sg[lane] = gt;
                sP[lane] = p;
                sSfx[lane] = sfx;
                sG[lane] = gpre;
                sRl[lane] = rl;
            }
        }
    };

    const int nchunks = (T + C - 1) / C;
    // chunk 0 is staged before the loop; inside, chunk n+1 is loaded into
    // registers at the top of iteration n and staged into LDS at its bottom,
    // once chunk n is done with LDS.
    // chunk 0's loads are issued while the state is still in flight; then
    // the loaded state is consumed here, before the chunk loop, so that no
    // load is still pending at the loop header (where a wait would otherwise
    // be placed on every iteration)
    if (nchunks > 0) prefetch(0);
#pragma unroll
    for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
        for (int vb = 0; vb < NB; ++vb) asm volatile("" : "+v"(S[kb][vb]));
    if (nchunks > 0) stage(min(C, T));

    for (int n = 0; n < nchunks; ++n) {
        const int t0 = n * C;
        const int cn = min(C, T - t0);
        if (n + 1 < nchunks) prefetch(t0 + C);
        lds_barrier();                     // chunk n staged

        // ---- one pass over the K and Q fragments:
        //   X = K S0^T (tiles [t][v]), Y^T = S0 Q^T (tiles [v][t]) for this
        //   wave's columns, and the C x C tile columns tb = wave + i*NW of
        //   K K^T and Q K^T: tile (jb, tb) has rows j and columns t, so lane
        //   x holds row t = 16 tb + x along j = 16 jb + 4 qd + r.
        X4 Sf[NBK][NB];
#pragma unroll
        for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) Sf[kb][vb] = cvt4<ET>(S[kb][vb]);
        f32x4 Xa[NBT][NB], Ya[NB][NBT];
        f32x4 tkk[NTPW][NBT], tqk[NTPW][NBT];
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb)
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) { Xa[tb][vb] = zero4(); Ya[vb][tb] = zero4(); }
#pragma unroll
        for (int i = 0; i < NTPW; ++i)
#pragma unroll
            for (int jb = 0; jb < NBT; ++jb) { tkk[i][jb] = zero4(); tqk[i][jb] = zero4(); }
#pragma unroll
        for (int s = 0; s < NSK; ++s) {
            FR fk[NBT], fq[NBT];
#pragma unroll
            for (int tb = 0; tb < NBT; ++tb) {
                fk[tb] = make_frag<ET>(s, NBK, [&](int kb) { return frag_row<ET>(sK, LDK, 16 * tb, 0, kb, x, qd); });
                fq[tb] = make_frag<ET>(s, NBK, [&](int kb) { return frag_row<ET>(sQ, LDK, 16 * tb, 0, kb, x, qd); });
            }
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) {
                FR fs = make_frag<ET>(s, NBK, [&](int kb) { return Sf[kb][vb]; });
#pragma unroll
                for (int tb = 0; tb < NBT; ++tb) {
                    Xa[tb][vb] = mfma_step(fk[tb], fs, Xa[tb][vb]);
                    Ya[vb][tb] = mfma_step(fs, fq[tb], Ya[vb][tb]);
                }
            }
#pragma unroll
            for (int i = 0; i < NTPW; ++i) {
                const int tbw = wave + i * NW;             // this wave's tile column
                FR bk = fk[0], bq = fq[0];
#pragma unroll
                for (int tb = 1; tb < NBT; ++tb)
                    if (tb == tbw) { bk = fk[tb]; bq = fq[tb]; }
#pragma unroll
                for (int jb = 0; jb < NBT; ++jb) {
                    tkk[i][jb] = mfma_step(fk[jb], bk, tkk[i][jb]);
                    tqk[i][jb] = mfma_step(fk[jb], bq, tqk[i][jb]);
                }
            }
        }
        lds_barrier();

        // ---- A = beta R (K K^T) strictly lower (stored as -A, 16-bit, and
        // its diagonal blocks in f32); QKR = R (Q K^T) / sqrt(Dk), lower incl.
        // the diagonal.  R[t][j] for j in an earlier block: P[t] x BT of the
        // blocks between x Sfx[j]; in t's own block: g_{j+1} ... g_t by a
        // running product.  Blocks above the diagonal keep their zeros.
#pragma unroll
        for (int i = 0; i < NTPW; ++i) {
            const int tb = wave + i * NW;
            if (NBT % NW == 0 || tb < NBT) {
                const int t = 16 * tb + x;
                const float bt = sb[t], pt = sP[t];
#pragma unroll
                for (int jb = 0; jb < NBT; ++jb) {
                    const int j0 = 16 * jb + 4 * qd;
                    const f32x4 zk = tkk[i][jb], zq = tqk[i][jb];
                    if (jb < tb) {
                        float m = pt;
                        for (int bb = jb + 1; bb < tb; ++bb) m *= sBT[bb];
                        const f32x4 R = *reinterpret_cast<const f32x4 *>(sSfx + j0) * m;
                        *reinterpret_cast<f32x4 *>(sAn + t * LDCF + j0) = R * zk * (-bt);
                        st4<ET>(sQKR + t * LDC + j0, cvt4<ET>(R * zq * scale));
                    } else if (jb == tb) {
                        const float *gblk = sg + 16 * tb;
                        float acc = 1.f;                    // g over [4 qd + 4, x]
#pragma unroll
                        for (int ii = 1; ii < 16; ++ii)
                            acc *= (ii >= 4 * qd + 4 && ii <= x) ? gblk[ii] : 1.f;
                        const f32x4 g4 = *reinterpret_cast<const f32x4 *>(gblk + 4 * qd);
                        f32x4 R;
                        R[3] = acc;
                        R[2] = (4 * qd + 3 <= x) ? R[3] * g4[3] : 1.f;
                        R[1] = (4 * qd + 2 <= x) ? R[2] * g4[2] : 1.f;
                        R[0] = (4 * qd + 1 <= x) ? R[1] * g4[1] : 1.f;
                        f32x4 a, o;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            a[r] = (4 * qd + r < x) ? bt * (R[r] * zk[r]) : 0.f;
                            o[r] = (4 * qd + r <= x) ? scale * (R[r] * zq[r]) : 0.f;
                        }
                        *reinterpret_cast<f32x4 *>(sAn + t * LDCF + j0) = -a;
                        st4<ET>(sQKR + t * LDC + j0, cvt4<ET>(o));
                        *reinterpret_cast<f32x4 *>(sAd + t * LDD + 4 * qd) = a;
                    }
                }
            }
        }
        lds_barrier();

        // ---- T_bb = (I + A_bb)^-1 for the 16x16 diagonal blocks: wave w
        // solves blocks w, w + NW, ...; four lanes per column c, lane part p
        // holding rows p, p+4, p+8, p+12.  Column sweep: once x_j is final
        // (it sits in part j%4), every later row subtracts A[i][j] x_j.
#pragma unroll
        for (int i = 0; i < NTPW; ++i) {
            const int bb = wave + i * NW;
            if (NBT % NW == 0 || bb < NBT) {
                const int base = 16 * bb;
                const int p = lane & 3, c = ((lane >> 4) << 2) | ((lane >> 2) & 3);
                f32x4 arow[4][4];
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int j4 = 0; j4 < 4; ++j4)
                        arow[m][j4] = *reinterpret_cast<const f32x4 *>(sAd + (base + p + 4 * m) * LDD + 4 * j4);
                float s[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) s[m] = (p + 4 * m == c) ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < 15; ++j) {
                    float xj;
                    switch (j & 3) {
                    case 0: xj = quad_bcast<0>(s[j >> 2]); break;
                    case 1: xj = quad_bcast<1>(s[j >> 2]); break;
                    case 2: xj = quad_bcast<2>(s[j >> 2]); break;
                    default: xj = quad_bcast<3>(s[j >> 2]); break;
                    }
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        if (4 * m + 3 > j) s[m] -= arow[m][j >> 2][j & 3] * xj;   // A[i][j] = 0 for j >= i
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) sTd[(base + p + 4 * m) * LDTF + c] = s[m];
            }
        }
        lds_barrier();

        // ---- D by blocked forward substitution (per wave, its columns), in
        // float32: RHS = beta (V - G X); D_i = T_ii (RHS_i + sum_{j<i} (-A_ij) D_j),
        // with -A, T_ii and every solved block D_j float32 and every product a
        // float32 matrix-core product; D is rounded to the input type only
        // afterwards, as an operand of the output and state products.
        // Fragments over rows t: lane x holds column v, rows 16 i + 4 qd + r.
        f32x4 Da[NBT][NB];
        X4 Df[NBT][NB];
#pragma unroll
        for (int ib = 0; ib < NBT; ++ib) {
            const f32x4 bv = *reinterpret_cast<const f32x4 *>(sb + 16 * ib + 4 * qd);
            const f32x4 gv = *reinterpret_cast<const f32x4 *>(sG + 16 * ib + 4 * qd);
            f32x4 Z[NB];
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) {
                const f32x4 vv = to_f32x4<ET>(frag_col<ET>(sV, LDV, 0, vloc + 16 * vb, ib, x, qd));
                Z[vb] = bv * (vv - gv * Xa[ib][vb]);
            }
#pragma unroll
            for (int jb = 0; jb < ib; ++jb) {
                const f32x4 fa = ld4<float>(sAn + (16 * ib + x) * LDCF + 16 * jb + 4 * qd);
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) Z[vb] = mfma_step(fa, Da[jb][vb], Z[vb]);
            }
            const f32x4 ft = ld4<float>(sTd + (16 * ib + x) * LDTF + 4 * qd);
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) {
                Da[ib][vb] = mfma_step(ft, Z[vb], zero4());
                Df[ib][vb] = cvt4<ET>(Da[ib][vb]);
            }
        }

        // ---- Y^T = G (S0 Q^T) / sqrt(Dk) + D^T QKR^T  (intra-chunk term; QKR carries 1/sqrt(Dk))
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb) {
            const float gt = sG[16 * tb + x] * scale;
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) Ya[vb][tb] *= gt;
            FR fr[NST];
#pragma unroll
            for (int s = 0; s < NST; ++s) {
                if (s * BLK > tb) continue;
                fr[s] = make_frag<ET>(s, NBT, [&](int jb) { return frag_row<ET>(sQKR, LDC, 16 * tb, 0, jb, x, qd); });
            }
#pragma unroll
            for (int s = 0; s < NST; ++s) {
                if (s * BLK > tb) continue;
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) {
                    FR fd = make_frag<ET>(s, NBT, [&](int jb) { return Df[jb][vb]; });
                    Ya[vb][tb] = mfma_step(fd, fr[s], Ya[vb][tb]);
                }
            }
        }

        // ---- y store: lane holds token t = 16 tb + x, values 16 vb + 4 qd + (0..3)
        store_y(y + (((size_t)b * T + t0) * Hv + hv) * Dv + vs * DVS, Hv * Dv, cn, vloc, x, qd, Ya);

        // ---- S^T <- G_last S^T + K^T diag(R[c-1][:]) D
        X4 Dpf[NBT][NB];
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb) {
            const f32x4 rl = *reinterpret_cast<const f32x4 *>(sRl + 16 * tb + 4 * qd);
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) Dpf[tb][vb] = cvt4<ET>(Da[tb][vb] * rl);
        }
        const float glast = sG[C - 1];
#pragma unroll
        for (int kb = 0; kb < NBK; ++kb) {
            FR fk[NST];
#pragma unroll
            for (int s = 0; s < NST; ++s)
                fk[s] = make_frag<ET>(s, NBT, [&](int tb) { return frag_col<ET>(sK, LDK, 0, 16 * kb, tb, x, qd); });
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) S[kb][vb] *= glast;
#pragma unroll
            for (int s = 0; s < NST; ++s) {
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) {
                    FR fd = make_frag<ET>(s, NBT, [&](int tb) { return Dpf[tb][vb]; });
                    S[kb][vb] = mfma_step(fk[s], fd, S[kb][vb]);
                }
            }
        }
        if (n + 1 < nchunks) {
            lds_barrier();                 // chunk n is done with LDS
            stage(min(C, T - t0 - C));
        }
    }

    // ---- the state, written once
#pragma unroll
    for (int vb = 0; vb < NB; ++vb) {
        const size_t row = sbase + (size_t)(vs * DVS + vloc + 16 * vb + x) * DK;
#pragma unroll
        for (int kb = 0; kb < NBK; ++kb)
            *reinterpret_cast<f32x4 *>(state_out + row + 16 * kb + 4 * qd) = S[kb][vb];
    }
}

}  // namespace gdn
