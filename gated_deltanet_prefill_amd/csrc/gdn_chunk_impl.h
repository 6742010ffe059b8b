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
    static constexpr int LDC = C + EPU;               // row stride of sKt, sVt, sT1, sT2, sQKR
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
    static constexpr int MAXT = (NTILE + NW - 1) / NW;  // tiles per wave
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

template <typename ET, int DK, int DVS, int C, int NB>
__global__ __launch_bounds__(4 * DVS / NB, 1)
void chunk_fwd_kernel(const ET *__restrict__ q, const ET *__restrict__ k,
                      const ET *__restrict__ v, const float *__restrict__ g,
                      const float *__restrict__ beta, const float *state_in,
                      float *state_out, ET *__restrict__ y,
                      int T, int Hk, int Hv, int Dv, int nsplit, float scale)
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
    const int slot = blockIdx.x / nsplit, vs = blockIdx.x - slot * nsplit;
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

    // ---- structural zeros of the C x C matrices (upper triangles never written)
    for (int i = tid; i < (L::oRin - L::oT1) / 16; i += NT)
        reinterpret_cast<uint4 *>(smem + L::oT1)[i] = zero_u4();

    // ---- global -> register prefetch of one chunk
    const size_t kstride = (size_t)Hk * DK, vstride = (size_t)Hv * Dv;
    const ET *kbase = k + ((size_t)b * T * Hk + hk) * DK;
    const ET *qbase = q + ((size_t)b * T * Hk + hk) * DK;
    const ET *vbase = v + ((size_t)b * T * Hv + hv) * Dv + vs * DVS;
    const float *gbase = g + (size_t)b * T * Hv + hv;
    const float *bbase = beta + (size_t)b * T * Hv + hv;

    uint4 rk[L::PERK][4], rq[L::PERQ], rv[L::PERV][4];
    float rg = 1.f, rb = 0.f;
    auto prefetch = [&](int t0) {
        const int cn = min(C, T - t0);
#pragma unroll
        for (int i = 0; i < L::PERK; ++i) {
            const int it = tid + i * NT;
            const int rgp = it / L::UPK, u = it - rgp * L::UPK;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * rgp + r;
                rk[i][r] = (it < L::KIT && t < cn)
                    ? *reinterpret_cast<const uint4 *>(kbase + (size_t)(t0 + t) * kstride + u * EPU)
                    : zero_u4();
            }
        }
#pragma unroll
        for (int i = 0; i < L::PERQ; ++i) {
            const int it = tid + i * NT;
            const int t = it / L::UPK, u = it - t * L::UPK;
            rq[i] = (it < L::QIT && t < cn)
                ? *reinterpret_cast<const uint4 *>(qbase + (size_t)(t0 + t) * kstride + u * EPU)
                : zero_u4();
        }
#pragma unroll
        for (int i = 0; i < L::PERV; ++i) {
            const int it = tid + i * NT;
            const int rgp = it / L::UPV, u = it - rgp * L::UPV;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * rgp + r;
                rv[i][r] = (it < L::VIT && t < cn)
                    ? *reinterpret_cast<const uint4 *>(vbase + (size_t)(t0 + t) * vstride + u * EPU)
                    : zero_u4();
            }
        }
        if (tid < C) {
            const bool in = tid < cn;
            rg = in ? gbase[(size_t)(t0 + tid) * Hv] : 1.f;
            rb = in ? bbase[(size_t)(t0 + tid) * Hv] : 0.f;
        }
    };

    auto stage = [&]() {
#pragma unroll
        for (int i = 0; i < L::PERK; ++i) {
            const int it = tid + i * NT;
            if (it < L::KIT) {
                const int rgp = it / L::UPK, u = it - rgp * L::UPK;
                Unit16<ET> w[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    w[r].u = rk[i][r];
                    *reinterpret_cast<uint4 *>(sK + (4 * rgp + r) * LDK + u * EPU) = rk[i][r];
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
            if (it < L::QIT) {
                const int t = it / L::UPK, u = it - t * L::UPK;
                *reinterpret_cast<uint4 *>(sQ + t * LDK + u * EPU) = rq[i];
            }
        }
#pragma unroll
        for (int i = 0; i < L::PERV; ++i) {
            const int it = tid + i * NT;
            if (it < L::VIT) {
                const int rgp = it / L::UPV, u = it - rgp * L::UPV;
                Unit16<ET> w[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) w[r].u = rv[i][r];
#pragma unroll
                for (int e = 0; e < EPU; ++e) {
                    X4 col;
                    col[0] = w[0].e[e]; col[1] = w[1].e[e]; col[2] = w[2].e[e]; col[3] = w[3].e[e];
                    st4<ET>(sVt + (u * EPU + e) * LDC + 4 * rgp, col);
                }
            }
        }
        if (tid < C) {
            sg[tid] = rg;
            sb[tid] = rb;
        }
    };

    const int nchunks = (T + C - 1) / C;
    if (nchunks > 0) prefetch(0);

    for (int n = 0; n < nchunks; ++n) {
        const int t0 = n * C;
        const int cn = min(C, T - t0);
        __syncthreads();                     // the previous chunk is done with LDS
        stage();
        if (n + 1 < nchunks) prefetch(t0 + C);
        __syncthreads();

        // ---- gates (wave 0): products of decays only
        if (wave == 0) {
            const int t = lane;
            const int bt = t >> 4, ti = t & 15, base = bt << 4;
            float p = 1.f, s = 1.f;
            if (t < C) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float gi = sg[base + i];
                    if (i <= ti) p *= gi;
                    if (i > ti) s *= gi;
                }
                float r = 1.f;
#pragma unroll
                for (int jj = 15; jj >= 0; --jj) {
                    if (jj < ti) r *= sg[base + jj + 1];
                    sRin[t * 16 + jj] = (jj <= ti) ? r : 0.f;
                }
            }
            float bt_[NBT];
#pragma unroll
            for (int bb = 0; bb < NBT; ++bb) bt_[bb] = __shfl(p, 16 * bb + 15);
            if (t < C) {
                float gpre = p, rl = s;
#pragma unroll
                for (int bb = 0; bb < NBT; ++bb) {
                    if (bb < bt) gpre *= bt_[bb];
                    if (bb > bt) rl *= bt_[bb];
                }
                sP[t] = p;
                sSfx[t] = s;
                sG[t] = gpre;
                sRl[t] = rl;
                if (ti == 15) sBT[bt] = p;
            }
        }

        // ---- K K^T and Q K^T lower block tiles, kept in registers.
        // Tile (jb, tb) has rows j (keys) and columns t, so lane x holds
        // row t = 16 tb + x of the result along j = 16 jb + 4 qd + r.
        f32x4 tacc[L::MAXT];
#pragma unroll
        for (int i = 0; i < L::MAXT; ++i) tacc[i] = zero4();
        {
            int cnt = 0;
#pragma unroll
            for (int kind = 0; kind < 2; ++kind) {
#pragma unroll
                for (int tb = 0; tb < NBT; ++tb) {
#pragma unroll
                    for (int jb = 0; jb <= tb; ++jb, ++cnt) {
                        if (cnt % NW != wave) continue;
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
                        tacc[cnt / NW] = acc;
                    }
                }
            }
        }
        __syncthreads();

        // ---- A = beta R (K K^T) strictly lower; QKR = R (Q K^T) lower
        {
            int cnt = 0;
#pragma unroll
            for (int kind = 0; kind < 2; ++kind) {
#pragma unroll
                for (int tb = 0; tb < NBT; ++tb) {
#pragma unroll
                    for (int jb = 0; jb <= tb; ++jb, ++cnt) {
                        if (cnt % NW != wave) continue;
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
                        const f32x4 z = tacc[cnt / NW];
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
        __syncthreads();

        // ---- T = (I + A)^-1: 16x16 diagonal blocks by forward substitution
        if (wave == 0 && lane < 16 * NBT) {
            const int bb = lane >> 4, c = lane & 15, base = 16 * bb;
            float xv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float *arow = sA + (base + i) * LDF + base;
                float a0 = (i == c) ? 1.f : 0.f, a1 = 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) {
                    if (j & 1) a1 -= arow[j] * xv[j];
                    else a0 -= arow[j] * xv[j];
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
        __syncthreads();

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
            __syncthreads();
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
            __syncthreads();
        }

        // ---- T1 = T diag(beta), T2 = -T diag(beta G), as MFMA operands
        for (int e = tid; e < C * C / 4; e += NT) {
            const int t = e / (C / 4), c4 = (e - t * (C / 4)) * 4;
            const f32x4 tv = *reinterpret_cast<const f32x4 *>(sT + t * LDF + c4);
            const f32x4 bv = *reinterpret_cast<const f32x4 *>(sb + c4);
            const f32x4 gv = *reinterpret_cast<const f32x4 *>(sG + c4);
            const f32x4 t1 = tv * bv;
            st4<ET>(sT1 + t * LDC + c4, cvt4<ET>(t1));
            st4<ET>(sT2 + t * LDC + c4, cvt4<ET>(-(t1 * gv)));
        }
        __syncthreads();

        // ---- state-dependent part, per wave over its value columns
        X4 Sf[NBK][NB];
#pragma unroll
        for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) Sf[kb][vb] = cvt4<ET>(S[kb][vb]);

        // X = K S0^T  (tiles [t][v]);  Y^T = S0 Q^T  (tiles [v][t])
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
        // G_t S0 q_t
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
