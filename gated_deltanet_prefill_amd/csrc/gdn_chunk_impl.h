// gdn_chunk_impl.h -- the chunked gated-delta-rule forward kernel for gfx950.
//
// One workgroup owns one (batch, value head) slot -- or a slice of its value
// rows -- and walks the slot's T tokens in chunks of C, with the Dk x Dv
// state resident in registers (as MFMA accumulator tiles of S^T) from the
// first chunk to the last; the state is read from HBM once and written once.
//
// Per chunk (c <= C tokens; rows past the end of the sequence are staged as
// k = q = v = 0, g = 1, beta = 0, which leaves the recurrence unchanged --
// the padding the metaltile-std gated_delta_wy.rs page asks its caller for):
//
//  stage    K, K^T, Q and this slice's V^T into LDS (16-bit or f32), g, beta.
//  gates    chunk-local decay products, all formed by multiplying decays
//           (ferrox-core gdn_chunk.rs page, "The algebra": ratios are
//           products, an underflow is a state really forgotten):
//             G[t]    = g_0 ... g_t,
//             R[t][j] = g_{j+1} ... g_t  (j <= t),
//           built from 16-token blocks: in-block rows by running products,
//           across blocks as (prefix in t's block) x (whole blocks between)
//           x (suffix in j's block).
//  K K^T, Q K^T     (MFMA)  ->  A[t][j] = beta_t R[t][j] k_t.k_j  (j < t),
//                               QKR[t][j] = R[t][j] q_t.k_j      (j <= t).
//  T = (I + A)^-1   (f32 in LDS): 16x16 diagonal blocks by forward
//           substitution, off-diagonal blocks by the block recurrence
//           T_ij = -T_ii A_ij T_jj (two levels, MFMA).  This is the unit lower
//           triangular system of the metaltile-std page's steps 4-5, solved
//           once for every right-hand side of the chunk.
//  X = K S0^T                          (MFMA, state-dependent)
//  D = T diag(beta) V - T diag(beta G) X      -- the true per-token deltas
//           d_t = beta_t (v_t - g_t S_{t-1} k_t) of all c tokens at once
//           (ferrox-core page: the predictions written in S0 and the earlier
//           deltas; one forward substitution for the whole chunk).
//  y_t = (G_t S0 q_t + sum_{j<=t} R[t][j] (q_t.k_j) d_j) / sqrt(Dk)   (MFMA)
//  S  <- G_{c-1} S0 + sum_t R[c-1][t] d_t k_t^T                        (MFMA)
//
// Work split: wave w of the workgroup owns 16*NB value columns of the
// slice; it holds S^T[0:Dk, its columns] as NBK x NB accumulator tiles and
// computes X, y and the update for its columns alone (each state row's
// update needs only that row, k and the shared C x C matrices).  The C x C
// work (gates, K K^T, Q K^T, T) is shared through LDS.

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
    static constexpr int EPU = 16 / (int)sizeof(ET);  // elements per 16-byte unit
    static constexpr int LDK = DK + EPU;              // row stride of sK, sQ
    static constexpr int LDC = C + 4;                 // row stride of sKt, sVt, sT1, sT2, sQKR
                                                      // (odd multiple of 8 bytes / bank group)
    static constexpr int LDF = C + 4;                 // row stride of f32 C x C matrices
    static constexpr int ES = (int)sizeof(ET);
    static constexpr int oK = 0;
    static constexpr int oQ = oK + C * LDK * ES;
    static constexpr int oKt = oQ + C * LDK * ES;
    static constexpr int oVt = oKt + DK * LDC * ES;
    static constexpr int oT1 = oVt + DVS * LDC * ES;  // T1..Tt: cleared once per launch
    static constexpr int oT2 = oT1 + C * LDC * ES;
    static constexpr int oQKR = oT2 + C * LDC * ES;
    static constexpr int oA = oQKR + C * LDC * ES;
    static constexpr int oT = oA + C * LDF * 4;
    static constexpr int oTt = oT + C * LDF * 4;
    static constexpr int oRin = oTt + C * LDF * 4;    // [C][16] in-block decay ratios
    static constexpr int oVec = oRin + C * 16 * 4;    // g, beta, P, Sfx, G, Rlast, BT
    static constexpr int BYTES = oVec + 8 * C * 4;
    static constexpr int NPAIR = NBT * (NBT + 1) / 2;   // lower block tiles of C x C
    static constexpr int NTILE = 2 * NPAIR;             // K K^T and Q K^T tiles
    // staging: 16-byte units
    static constexpr int UPK = DK / EPU;                // units per K / Q row
    static constexpr int UPV = DVS / EPU;               // units per V row (slice)
    static constexpr int KIT = (C / 4) * UPK;           // (4-row group, unit) items of K
    static constexpr int QIT = C * UPK;
    static constexpr int VIT = (C / 4) * UPV;
    static constexpr int PERK = (KIT + NT - 1) / NT;
    static constexpr int PERQ = (QIT + NT - 1) / NT;
    static constexpr int PERV = (VIT + NT - 1) / NT;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(NW >= 1 && NW * 16 * NB == DVS, "value slice must split into whole waves");
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

template <int NBLK, int BLK> struct Steps { static constexpr int n = (NBLK + BLK - 1) / BLK; };

template <typename ET> union Unit16 {
    uint4 u;
    ET e[16 / sizeof(ET)];
};

__device__ __forceinline__ uint4 zero_u4() { return make_uint4(0u, 0u, 0u, 0u); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, then for every wave.  Unlike __syncthreads() it does not wait
// for outstanding global loads and stores, so the next chunk's prefetch and
// this chunk's y stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <typename ET, int DK, int DVS, int C, int NB>
__global__ __launch_bounds__(4 * DVS / NB, 1)
void chunk_fwd_kernel(const ET *__restrict__ q, const ET *__restrict__ k,
                      const ET *__restrict__ v, const float *__restrict__ g,
                      const float *__restrict__ beta, const float *state_in,
                      float *state_out, ET *__restrict__ y,
                      int T, int Hk, int Hv, int Dv, int nsplit, int xcd_group, float scale)
{
    using L = ChunkCfg<ET, DK, DVS, C, NB>;
    using X4 = typename Vec<ET>::x4;
    using FR = typename Step<ET>::frag;
    constexpr int BLK = Step<ET>::BLK;
    constexpr int NBT = L::NBT, NBK = L::NBK, NW = L::NW, NT = L::NT;
    constexpr int LDK = L::LDK, LDC = L::LDC, LDF = L::LDF, EPU = L::EPU;

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    ET *sK = reinterpret_cast<ET *>(smem + L::oK);
    ET *sQ = reinterpret_cast<ET *>(smem + L::oQ);
    ET *sKt = reinterpret_cast<ET *>(smem + L::oKt);
    ET *sVt = reinterpret_cast<ET *>(smem + L::oVt);
    ET *sT1 = reinterpret_cast<ET *>(smem + L::oT1);
    ET *sT2 = reinterpret_cast<ET *>(smem + L::oT2);
    ET *sQKR = reinterpret_cast<ET *>(smem + L::oQKR);
    float *sA = reinterpret_cast<float *>(smem + L::oA);
    float *sT = reinterpret_cast<float *>(smem + L::oT);
    float *sTt = reinterpret_cast<float *>(smem + L::oTt);
    float *sRin = reinterpret_cast<float *>(smem + L::oRin);
    float *sg = reinterpret_cast<float *>(smem + L::oVec);
    float *sb = sg + C;
    float *sP = sb + C;
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
    const int slot = bid / nsplit, vs = bid - slot * nsplit;
    const int hv = slot % Hv, b = slot / Hv, hk = hv / (Hv / Hk);
    const int vloc = wave * 16 * NB;               // first slice column of this wave

    // ---- the state, S^T tiles [key block][value block], f32 accumulators
    f32x4 S[NBK][NB];
    const size_t sbase = (size_t)slot * Dv * DK;
#pragma unroll
    for (int vb = 0; vb < NB; ++vb) {
        const size_t row = sbase + (size_t)(vs * DVS + vloc + 16 * vb + x) * DK;
#pragma unroll
        for (int kb = 0; kb < NBK; ++kb)
            S[kb][vb] = state_in ? *reinterpret_cast<const f32x4 *>(state_in + row + 16 * kb + 4 * qd)
                                 : zero4();
    }
    // Consume the loaded state here, before the chunk loop, so that no load
    // is still pending at the loop header (where a wait would otherwise be
    // placed on every iteration).
#pragma unroll
    for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
        for (int vb = 0; vb < NB; ++vb) asm volatile("" : "+v"(S[kb][vb]));

    // ---- structural zeros of the C x C matrices (upper triangles never written)
    for (int i = tid; i < (L::oRin - L::oT1) / 16; i += NT)
        reinterpret_cast<uint4 *>(smem + L::oT1)[i] = zero_u4();

    // ---- global -> register prefetch of one chunk.  Every load is issued
    // unconditionally from a clamped (always valid) row; rows past the end
    // of the sequence are zeroed when the registers are staged, so nothing
    // consumes the loaded values before the next chunk's staging point.
    const size_t kstride = (size_t)Hk * DK, vstride = (size_t)Hv * Dv;
    const ET *kbase = k + ((size_t)b * T * Hk + hk) * DK;
    const ET *qbase = q + ((size_t)b * T * Hk + hk) * DK;
    const ET *vbase = v + ((size_t)b * T * Hv + hv) * Dv + vs * DVS;
    const float *gbase = g + (size_t)b * T * Hv + hv;
    const float *bbase = beta + (size_t)b * T * Hv + hv;

    uint4 rk[L::PERK][4], rq[L::PERQ], rv[L::PERV][4];
    float rg = 1.f, rb = 0.f;
    auto prefetch = [&](int t0) {
        const int last = min(C, T - t0) - 1;
#pragma unroll
        for (int i = 0; i < L::PERK; ++i) {
            const int it = min(tid + i * NT, L::KIT - 1);
            const int rgp = it / L::UPK, u = it - rgp * L::UPK;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = min(4 * rgp + r, last);
                rk[i][r] = *reinterpret_cast<const uint4 *>(kbase + (size_t)(t0 + t) * kstride + u * EPU);
            }
        }
#pragma unroll
        for (int i = 0; i < L::PERQ; ++i) {
            const int it = min(tid + i * NT, L::QIT - 1);
            const int t = min(it / L::UPK, last), u = it % L::UPK;
            rq[i] = *reinterpret_cast<const uint4 *>(qbase + (size_t)(t0 + t) * kstride + u * EPU);
        }
#pragma unroll
        for (int i = 0; i < L::PERV; ++i) {
            const int it = min(tid + i * NT, L::VIT - 1);
            const int rgp = it / L::UPV, u = it - rgp * L::UPV;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = min(4 * rgp + r, last);
                rv[i][r] = *reinterpret_cast<const uint4 *>(vbase + (size_t)(t0 + t) * vstride + u * EPU);
            }
        }
        const int tg = min(tid, last);
        rg = gbase[(size_t)(t0 + tg) * Hv];
        rb = bbase[(size_t)(t0 + tg) * Hv];
    };

    // Registers -> LDS: K row-major and transposed, Q, the V slice
    // transposed, g and beta; rows t >= cn become k = q = v = 0, g = 1,
    // beta = 0.  The empty asm statements pin the point where the prefetched
    // values are first needed here, after the barrier.
    auto stage = [&](int cn, float &gcur, float &bcur) {
#pragma unroll
        for (int i = 0; i < L::PERK; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                asm volatile("" : "+v"(rk[i][r].x), "+v"(rk[i][r].y), "+v"(rk[i][r].z), "+v"(rk[i][r].w));
#pragma unroll
        for (int i = 0; i < L::PERQ; ++i)
            asm volatile("" : "+v"(rq[i].x), "+v"(rq[i].y), "+v"(rq[i].z), "+v"(rq[i].w));
#pragma unroll
        for (int i = 0; i < L::PERV; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                asm volatile("" : "+v"(rv[i][r].x), "+v"(rv[i][r].y), "+v"(rv[i][r].z), "+v"(rv[i][r].w));
        asm volatile("" : "+v"(rg), "+v"(rb));
#pragma unroll
        for (int i = 0; i < L::PERK; ++i) {
            const int it = tid + i * NT;
            if (L::KIT % NT == 0 || it < L::KIT) {
                const int rgp = it / L::UPK, u = it - rgp * L::UPK;
                Unit16<ET> w[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    w[r].u = (4 * rgp + r < cn) ? rk[i][r] : zero_u4();
                    *reinterpret_cast<uint4 *>(sK + (4 * rgp + r) * LDK + u * EPU) = w[r].u;
                }
#pragma unroll
                for (int e = 0; e < EPU; ++e) {
                    X4 col;
                    col[0] = w[0].e[e]; col[1] = w[1].e[e]; col[2] = w[2].e[e]; col[3] = w[3].e[e];
                    st4<ET>(sKt + (u * EPU + e) * LDC + 4 * rgp, col);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < L::PERQ; ++i) {
            const int it = tid + i * NT;
            if (L::QIT % NT == 0 || it < L::QIT) {
                const int t = it / L::UPK, u = it - t * L::UPK;
                *reinterpret_cast<uint4 *>(sQ + t * LDK + u * EPU) = (t < cn) ? rq[i] : zero_u4();
            }
        }
#pragma unroll
        for (int i = 0; i < L::PERV; ++i) {
            const int it = tid + i * NT;
            if (L::VIT % NT == 0 || it < L::VIT) {
                const int rgp = it / L::UPV, u = it - rgp * L::UPV;
                Unit16<ET> w[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) w[r].u = (4 * rgp + r < cn) ? rv[i][r] : zero_u4();
#pragma unroll
                for (int e = 0; e < EPU; ++e) {
                    X4 col;
                    col[0] = w[0].e[e]; col[1] = w[1].e[e]; col[2] = w[2].e[e]; col[3] = w[3].e[e];
                    st4<ET>(sVt + (u * EPU + e) * LDC + 4 * rgp, col);
                }
            }
        }
        gcur = (tid < cn) ? rg : 1.f;
        bcur = (tid < cn) ? rb : 0.f;
        if (tid < C) sb[tid] = bcur;
    };

    // Which wave computes shared K K^T / Q K^T tile number cnt: with four or
    // more waves, wave 0 (which also forms the gate products) is skipped.
    constexpr int TW0 = NW >= 4 ? 1 : 0, TWN = NW - TW0;
    constexpr int MAXT = (L::NTILE + TWN - 1) / TWN;

    const int nchunks = (T + C - 1) / C;
    // chunk 0 is staged before the loop; inside, chunk n+1 is loaded into
    // registers at the top of iteration n and staged into LDS at its bottom,
    // once chunk n is done with LDS.
    float gcur = 1.f, bcur = 0.f;
    if (nchunks > 0) {
        prefetch(0);
        stage(min(C, T), gcur, bcur);
    }

    for (int n = 0; n < nchunks; ++n) {
        const int t0 = n * C;
        const int cn = min(C, T - t0);
        if (n + 1 < nchunks) prefetch(t0 + C);
        lds_barrier();                     // chunk n staged

        // ---- gates (wave 0, lane t holds g_t): products of decays only.
        // P[t]: g over [block start, t]; Sfx[t]: over (t, block end];
        // Rin[t][j']: over (block start + j', t]; block totals BT;
        // G[t] = P[t] * BT of earlier blocks; Rl[t] = Sfx[t] * BT of later ones.
        if (wave == 0) {
            const int t = lane, bt = t >> 4, ti = t & 15, base = bt << 4;
            const float gt = (t < C) ? gcur : 1.f;
            float gb[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) gb[i] = __shfl(gt, base + i);
            float p = 1.f, sx = 1.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (i <= ti) p *= gb[i];
                if (i > ti) sx *= gb[i];
            }
            f32x4 rin[4];
            float r = 1.f;
#pragma unroll
            for (int jj = 15; jj >= 0; --jj) {
                if (jj < ti) r *= gb[jj + 1];
                rin[jj >> 2][jj & 3] = (jj <= ti) ? r : 0.f;
            }
            float btot[NBT];
#pragma unroll
            for (int bb = 0; bb < NBT; ++bb) btot[bb] = __shfl(p, 16 * bb + 15);
            float gpre = p, rl = sx;
#pragma unroll
            for (int bb = 0; bb < NBT; ++bb) {
                if (bb < bt) gpre *= btot[bb];
                if (bb > bt) rl *= btot[bb];
            }
            if (t < C) {
                sP[t] = p;
                sSfx[t] = sx;
                sG[t] = gpre;
                sRl[t] = rl;
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4)
                    *reinterpret_cast<f32x4 *>(sRin + t * 16 + 4 * i4) = rin[i4];
                if (t < NBT) sBT[t] = btot[t];
            }
        }

        // ---- K K^T and Q K^T lower block tiles, kept in registers.
        // Tile (jb, tb) has rows j (keys) and columns t, so lane x holds
        // row t = 16 tb + x of the result along j = 16 jb + 4 qd + r.
        f32x4 tacc[MAXT];
#pragma unroll
        for (int i = 0; i < MAXT; ++i) tacc[i] = zero4();
        {
            int cnt = 0;
#pragma unroll
            for (int kind = 0; kind < 2; ++kind) {
#pragma unroll
                for (int tb = 0; tb < NBT; ++tb) {
#pragma unroll
                    for (int jb = 0; jb <= tb; ++jb, ++cnt) {
                        if (TW0 + cnt % TWN != wave) continue;
                        const ET *bsrc = kind ? sQ : sK;
                        f32x4 acc = zero4();
#pragma unroll
                        for (int s = 0; s < Steps<NBK, BLK>::n; ++s) {
                            FR fa = make_frag<ET>(s, NBK, [&](int kb) {
                                return ld4<ET>(sK + (16 * jb + x) * LDK + 16 * kb + 4 * qd); });
                            FR fb = make_frag<ET>(s, NBK, [&](int kb) {
                                return ld4<ET>(bsrc + (16 * tb + x) * LDK + 16 * kb + 4 * qd); });
                            acc = mfma_step(fa, fb, acc);
                        }
                        tacc[cnt / TWN] = acc;
                    }
                }
            }
        }

        // ---- state products that need no C x C matrix:
        // X = K S0^T (tiles [t][v]) and Y^T = S0 Q^T (tiles [v][t])
        X4 Sf[NBK][NB];
#pragma unroll
        for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) Sf[kb][vb] = cvt4<ET>(S[kb][vb]);
        f32x4 Xa[NBT][NB], Ya[NB][NBT];
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb) {
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) { Xa[tb][vb] = zero4(); Ya[vb][tb] = zero4(); }
#pragma unroll
            for (int s = 0; s < Steps<NBK, BLK>::n; ++s) {
                FR fk = make_frag<ET>(s, NBK, [&](int kb) {
                    return ld4<ET>(sK + (16 * tb + x) * LDK + 16 * kb + 4 * qd); });
                FR fq = make_frag<ET>(s, NBK, [&](int kb) {
                    return ld4<ET>(sQ + (16 * tb + x) * LDK + 16 * kb + 4 * qd); });
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) {
                    FR fs = make_frag<ET>(s, NBK, [&](int kb) { return Sf[kb][vb]; });
                    Xa[tb][vb] = mfma_step(fk, fs, Xa[tb][vb]);
                    Ya[vb][tb] = mfma_step(fs, fq, Ya[vb][tb]);
                }
            }
        }
        lds_barrier();

        // ---- A = beta R (K K^T) strictly lower; QKR = R (Q K^T) lower
        {
            int cnt = 0;
#pragma unroll
            for (int kind = 0; kind < 2; ++kind) {
#pragma unroll
                for (int tb = 0; tb < NBT; ++tb) {
#pragma unroll
                    for (int jb = 0; jb <= tb; ++jb, ++cnt) {
                        if (TW0 + cnt % TWN != wave) continue;
                        const int t = 16 * tb + x, j0 = 16 * jb + 4 * qd;
                        f32x4 R;
                        if (jb == tb) {
                            R = *reinterpret_cast<const f32x4 *>(sRin + t * 16 + 4 * qd);
                        } else {
                            float m = sP[t];
#pragma unroll
                            for (int bb = jb + 1; bb < tb; ++bb) m *= sBT[bb];
                            const f32x4 sf = *reinterpret_cast<const f32x4 *>(sSfx + j0);
                            R = sf * m;
                        }
                        const f32x4 z = tacc[cnt / TWN];
                        f32x4 o;
                        if (kind == 0) {
                            const float bt = sb[t];
#pragma unroll
                            for (int r = 0; r < 4; ++r) o[r] = (j0 + r < t) ? bt * (R[r] * z[r]) : 0.f;
                            *reinterpret_cast<f32x4 *>(sA + t * LDF + j0) = o;
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r) o[r] = (j0 + r <= t) ? R[r] * z[r] : 0.f;
                            st4<ET>(sQKR + t * LDC + j0, cvt4<ET>(o));
                        }
                    }
                }
            }
        }
        lds_barrier();

        // ---- T = (I + A)^-1: 16x16 diagonal blocks by forward substitution
        if (wave == 0 && lane < 16 * NBT) {
            const int bb = lane >> 4, c = lane & 15, base = 16 * bb;
            float xv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float *arow = sA + (base + i) * LDF + base;
                f32x4 a4[4];
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    if (4 * m < i) a4[m] = *reinterpret_cast<const f32x4 *>(arow + 4 * m);
                float a0 = (i == c) ? 1.f : 0.f, a1 = 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) {
                    if (j & 1) a1 -= a4[j >> 2][j & 3] * xv[j];
                    else a0 -= a4[j >> 2][j & 3] * xv[j];
                }
                xv[i] = a0 + a1;
            }
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
                *reinterpret_cast<f32x4 *>(sTt + (base + c) * LDF + base + 4 * i4) =
                    f32x4{xv[4 * i4], xv[4 * i4 + 1], xv[4 * i4 + 2], xv[4 * i4 + 3]};
#pragma unroll
            for (int i = 0; i < 16; ++i) sT[(base + i) * LDF + base + c] = xv[i];
        }
        lds_barrier();

        // ---- first off-diagonal level: T[2p+1][2p] = -T[2p+1][2p+1] A[2p+1][2p] T[2p][2p]
        if constexpr (NBT >= 2) {
#pragma unroll
            for (int p = 0; p < NBT / 2; ++p) {
                if (p % NW != wave) continue;
                const int r0 = 32 * p;
                f32x4 P = zero4();
#pragma unroll
                for (int s = 0; s < Steps<1, BLK>::n; ++s) {
                    FR fa = make_frag<ET>(s, 1, [&](int) {
                        return cvt4<ET>(*reinterpret_cast<const f32x4 *>(sA + (r0 + 16 + x) * LDF + r0 + 4 * qd)); });
                    FR fb = make_frag<ET>(s, 1, [&](int) {
                        return cvt4<ET>(*reinterpret_cast<const f32x4 *>(sTt + (r0 + x) * LDF + r0 + 4 * qd)); });
                    P = mfma_step(fa, fb, P);
                }
                const X4 Pf = cvt4<ET>(P);
                f32x4 X = zero4();
#pragma unroll
                for (int s = 0; s < Steps<1, BLK>::n; ++s) {
                    FR fa = make_frag<ET>(s, 1, [&](int) {
                        return cvt4<ET>(-*reinterpret_cast<const f32x4 *>(sT + (r0 + 16 + x) * LDF + r0 + 16 + 4 * qd)); });
                    FR fb = make_frag<ET>(s, 1, [&](int) { return Pf; });
                    X = mfma_step(fa, fb, X);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) sT[(r0 + 16 + 4 * qd + r) * LDF + r0 + x] = X[r];
                *reinterpret_cast<f32x4 *>(sTt + (r0 + x) * LDF + r0 + 16 + 4 * qd) = X;
            }
            lds_barrier();
        }

        // ---- second level (C = 64): T[32:64][0:32] = -T_b (A[32:64][0:32] T_a)
        if constexpr (NBT == 4) {
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                if (jb % NW != wave) continue;
                X4 Pf[2];
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    f32x4 P = zero4();
#pragma unroll
                    for (int s = 0; s < Steps<2, BLK>::n; ++s) {
                        FR fa = make_frag<ET>(s, 2, [&](int kb) {
                            return cvt4<ET>(*reinterpret_cast<const f32x4 *>(sA + (32 + 16 * ib + x) * LDF + 16 * kb + 4 * qd)); });
                        FR fb = make_frag<ET>(s, 2, [&](int kb) {
                            return cvt4<ET>(*reinterpret_cast<const f32x4 *>(sTt + (16 * jb + x) * LDF + 16 * kb + 4 * qd)); });
                        P = mfma_step(fa, fb, P);
                    }
                    Pf[ib] = cvt4<ET>(P);
                }
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) {
                    f32x4 X = zero4();
#pragma unroll
                    for (int s = 0; s < Steps<2, BLK>::n; ++s) {
                        FR fa = make_frag<ET>(s, 2, [&](int kb) {
                            return cvt4<ET>(-*reinterpret_cast<const f32x4 *>(sT + (32 + 16 * ib + x) * LDF + 32 + 16 * kb + 4 * qd)); });
                        FR fb = make_frag<ET>(s, 2, [&](int kb) { return Pf[kb]; });
                        X = mfma_step(fa, fb, X);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) sT[(32 + 16 * ib + 4 * qd + r) * LDF + 16 * jb + x] = X[r];
                    *reinterpret_cast<f32x4 *>(sTt + (16 * jb + x) * LDF + 32 + 16 * ib + 4 * qd) = X;
                }
            }
            lds_barrier();
        }

        // ---- T1 = T diag(beta), T2 = -T diag(beta G), as MFMA operands
        {
            constexpr int ITEMS = C * C / 4, PER = (ITEMS + NT - 1) / NT;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                const int e = tid + i * NT;
                if (ITEMS % NT == 0 || e < ITEMS) {
                    const int t = e / (C / 4), c4 = (e - t * (C / 4)) * 4;
                    const f32x4 tv = *reinterpret_cast<const f32x4 *>(sT + t * LDF + c4);
                    const f32x4 bv = *reinterpret_cast<const f32x4 *>(sb + c4);
                    const f32x4 gv = *reinterpret_cast<const f32x4 *>(sG + c4);
                    const f32x4 t1 = tv * bv;
                    st4<ET>(sT1 + t * LDC + c4, cvt4<ET>(t1));
                    st4<ET>(sT2 + t * LDC + c4, cvt4<ET>(-(t1 * gv)));
                }
            }
        }
        lds_barrier();

        // ---- G_t S0 q_t
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb) {
            const float gt = sG[16 * tb + x];
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) Ya[vb][tb] *= gt;
        }

        // D = T1 V + T2 X  (T2 holds -T diag(beta G))
        X4 Xf[NBT][NB];
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb)
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) Xf[tb][vb] = cvt4<ET>(Xa[tb][vb]);
        f32x4 Da[NBT][NB];
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb) {
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) Da[tb][vb] = zero4();
#pragma unroll
            for (int s = 0; s < Steps<NBT, BLK>::n; ++s) {
                if (s * BLK > tb) continue;          // T is lower triangular
                FR f1 = make_frag<ET>(s, NBT, [&](int jb) {
                    return ld4<ET>(sT1 + (16 * tb + x) * LDC + 16 * jb + 4 * qd); });
                FR f2 = make_frag<ET>(s, NBT, [&](int jb) {
                    return ld4<ET>(sT2 + (16 * tb + x) * LDC + 16 * jb + 4 * qd); });
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) {
                    FR fv = make_frag<ET>(s, NBT, [&](int jb) {
                        return ld4<ET>(sVt + (vloc + 16 * vb + x) * LDC + 16 * jb + 4 * qd); });
                    FR fx = make_frag<ET>(s, NBT, [&](int jb) { return Xf[jb][vb]; });
                    Da[tb][vb] = mfma_step(f1, fv, Da[tb][vb]);
                    Da[tb][vb] = mfma_step(f2, fx, Da[tb][vb]);
                }
            }
        }

        // Y^T += D^T QKR^T  (intra-chunk term)
        X4 Df[NBT][NB];
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb)
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) Df[tb][vb] = cvt4<ET>(Da[tb][vb]);
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb) {
#pragma unroll
            for (int s = 0; s < Steps<NBT, BLK>::n; ++s) {
                if (s * BLK > tb) continue;
                FR fr = make_frag<ET>(s, NBT, [&](int jb) {
                    return ld4<ET>(sQKR + (16 * tb + x) * LDC + 16 * jb + 4 * qd); });
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) {
                    FR fd = make_frag<ET>(s, NBT, [&](int jb) { return Df[jb][vb]; });
                    Ya[vb][tb] = mfma_step(fd, fr, Ya[vb][tb]);
                }
            }
        }

        // y store: lane holds token t = 16 tb + x, values 16 vb + 4 qd + (0..3)
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb) {
            const int t = 16 * tb + x;
            if (t < cn) {
                ET *yrow = y + (((size_t)b * T + t0 + t) * Hv + hv) * Dv + vs * DVS + vloc + 4 * qd;
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) st4<ET>(yrow + 16 * vb, cvt4<ET>(Ya[vb][tb] * scale));
            }
        }

        // S^T <- G_last S^T + K^T diag(R[c-1][:]) D
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
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) S[kb][vb] *= glast;
#pragma unroll
            for (int s = 0; s < Steps<NBT, BLK>::n; ++s) {
                FR fk = make_frag<ET>(s, NBT, [&](int tb) {
                    return ld4<ET>(sKt + (16 * kb + x) * LDC + 16 * tb + 4 * qd); });
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) {
                    FR fd = make_frag<ET>(s, NBT, [&](int tb) { return Dpf[tb][vb]; });
                    S[kb][vb] = mfma_step(fk, fd, S[kb][vb]);
                }
            }
        }
        if (n + 1 < nchunks) {
            lds_barrier();                 // chunk n is done with LDS
            stage(min(C, T - t0 - C), gcur, bcur);
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
