// gdn_chunk_vgp.h -- the pipelined chunk kernel for a decay per key dimension
// (16-bit inputs, Dk = Dv = 128, chunks of 32 tokens, one workgroup per
// slot).
//
// The algebra is that of gdn_chunk_vg.h: every decay ratio is a product of
// decays, formed per key dimension from segment scans over each 16-token
// block (the within-block pairs split at the highest differing bit of their
// in-block indices, four levels; the pairs across the two blocks as
// P16_t S16_j), the chunk's triangular system solved in float32, and the
// state products on operands scaled per key dimension:
//     D = (I + A)^-1 beta (V - (K diag G) S0^T),
//     y = ((Q diag G) S0^T) / sqrt(Dk) + QKR D,
//     S <- S0 diag(G_last) + D^T (K diag(G_last / G)).
//
// The segment scans are vector-ALU work and the state products matrix-core
// work, so they run on different waves, a chunk apart (the arrangement of
// the scalar-gate kernel in gdn_chunk_wy.h):
//   * 4 state waves, 32 value columns each, keep S^T in accumulators and
//     run chunk n: X = (K diag G) S0^T and Y^T = S0 (Q diag G)^T; the float32
//     blocked substitution for D, y; the update.
//   * 8 prep waves run chunk n+1: wave (block b, key quarter) scans its 16
//     tokens over its 32 keys, forms the four levels' scaled operands and
//     their partial K K^T / Q K^T tiles, the scaled K and Q of its block, and
//     its part of the cross-block tile; two waves sum the partial tiles and
//     invert the diagonal blocks.  Their inputs (k, q, g, beta) are loaded
//     straight into registers, a chunk ahead.
// Everything the state waves read from the prep waves is double-buffered by
// chunk parity.  An iteration has two phases, each ending in a workgroup
// barrier; the prep waves finish a chunk (diagonal inverses, cross-block
// tile) in the first phase of the next iteration, beside the next chunk's
// scans, and the state waves run that chunk one iteration later.

#pragma once

#include "gdn_chunk_vg.h"
#include "gdn_chunk_wy.h"

namespace gdn {

// DPP move that writes zero where a lane has no source: unlike a move that
// keeps an old value, the compiler folds it into the consuming multiply.
template <int CTRL>
__device__ __forceinline__ float dppz(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}

// Per-lane decay scales of the four within-block levels, for lane x of a
// 16-token block (the decays g of token x, four key dimensions).  Level l
// pairs a token j in the lower half of a 2^(l+1)-token segment with a token t
// in its upper half; their decay product over (j, t] is e_l(j) p_l(t), where
// p_l(t) runs from the start of t's 2^l-token segment to t and e_l(j) from
// j + 1 to the end of j's.  A lane is only ever the t side (upper half) or
// the j side (lower half) of a level, so one scale serves both MFMA
// operands: s[l] = p_l on the upper half, e_l on the lower.  Also the
// block's prefix P16 (tokens 0..x) and suffix S16 (x + 1..15).  Lanes
// without a DPP source read zero, and only where the select discards it.
struct VgScales {
    f32x4 s[4];
    f32x4 p16, s16;
};

__device__ __forceinline__ VgScales vg_scales(f32x4 g, int x) {
    const f32x4 one = {1.f, 1.f, 1.f, 1.f};
    auto sel = [](bool c, f32x4 a, f32x4 b) { return c ? a : b; };
    // 0x111 row_shr:1, 0x101 row_shl:1, 0x55 / 0xaa / 0xff / 0x00 quad lane
    // 1 / 2 / 3 / 0, 0x114 / 0x104 row_shr:4 / row_shl:4, 0x15N row_newbcast:N
    f32x4 t, u;
#pragma unroll
    for (int c = 0; c < 4; ++c) t[c] = g[c] * dppz<0x111>(g[c]);
    const f32x4 p1 = sel(x & 1, t, g);
#pragma unroll
    for (int c = 0; c < 4; ++c) t[c] = p1[c] * dppz<0x55>(p1[c]);
    const f32x4 p2 = sel(x & 2, t, p1);
#pragma unroll
    for (int c = 0; c < 4; ++c) { u[c] = dppz<0xff>(p2[c]); t[c] = p2[c] * dppz<0x114>(u[c]); }
    const f32x4 p3 = sel(x & 4, t, p2);
#pragma unroll
    for (int c = 0; c < 4; ++c) t[c] = p3[c] * dppz<0x157>(p3[c]);
    const f32x4 p4 = sel(x & 8, t, p3);
#pragma unroll
    for (int c = 0; c < 4; ++c) t[c] = dppz<0x101>(g[c]);
    const f32x4 e1 = sel(x & 1, one, t);
    f32x4 sg = g * e1;
#pragma unroll
    for (int c = 0; c < 4; ++c) t[c] = e1[c] * dppz<0xaa>(sg[c]);
    const f32x4 e2 = sel(x & 2, e1, t);
    sg = g * e2;
#pragma unroll
    for (int c = 0; c < 4; ++c) { u[c] = dppz<0x00>(sg[c]); t[c] = e2[c] * dppz<0x104>(u[c]); }
    const f32x4 e3 = sel(x & 4, e2, t);
    sg = g * e3;
#pragma unroll
    for (int c = 0; c < 4; ++c) t[c] = e3[c] * dppz<0x158>(sg[c]);
    const f32x4 e4 = sel(x & 8, e3, t);
    VgScales r;
    r.s[0] = sel(x & 1, g, one);
    r.s[1] = sel(x & 2, p1, e1);
    r.s[2] = sel(x & 4, p2, e2);
    r.s[3] = sel(x & 8, p3, e3);
    r.p16 = p4;
    r.s16 = e4;
    return r;
}

template <typename ET>
struct VgpCfg {
    static constexpr int DK = 128, DV = 128, C = 32, NB = 2, NBT = 2, NBK = 8;
    static constexpr int NSW = 4, NPW = 8, NW = NSW + NPW, NT = 64 * NW;
    static constexpr int ES = 2, EPU = 8;
    static constexpr int LDK = DK + EPU;          // rows of K diag(G), Q diag(G), K diag(G_last/G)
    static constexpr int LDC = C + EPU;           // rows of QKR
    static constexpr int LDCF = C + 4;            // rows of -A (float32)
    static constexpr int LDD = 16 + 4;            // rows of the diagonal blocks of A (float32)
    static constexpr int LDTF = 16 + 4;           // rows of their inverses (float32)
    static constexpr int VRB = 16 * NB * ES;      // bytes of a row of one state wave's V slice
    static constexpr int VSL = C * VRB;           // one state wave's V slice
    // per chunk parity
    static constexpr int pAn = 0;
    static constexpr int pQKR = pAn + C * LDCF * 4;
    static constexpr int pTd = pQKR + C * LDC * ES;
    static constexpr int pKg = pTd + C * LDTF * 4;
    static constexpr int pQg = pKg + C * LDK * ES;
    static constexpr int pKr = pQg + C * LDK * ES;
    static constexpr int pGl = pKr + C * LDK * ES;
    static constexpr int pB = pGl + DK * 4;
    static constexpr int pV = pB + C * 4;
    static constexpr int PAR = pV + NSW * VSL;
    // prep scratch, rewritten every iteration
    static constexpr int oPd = 2 * PAR;                     // partial diagonal tiles: wave x {A, QKR} x 64 lanes
    static constexpr int oPx = oPd + NPW * 2 * 1024;        // partial cross-block tiles: key quarter x {A, QKR}
    static constexpr int oKS = oPx + 4 * 2 * 1024;          // K diag(S16) of block 0 [16][LDK]
    static constexpr int oBT = oKS + 16 * LDK * ES;         // block totals [2][DK]
    static constexpr int oAd = oBT + 2 * DK * 4;            // diagonal blocks of A [C][LDD]
    static constexpr int BYTES = oAd + C * LDD * 4;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(PAR % 16 == 0 && pV % 16 == 0 && pKg % 16 == 0, "16-byte aligned blocks");
};

template <typename ET>
__global__ __launch_bounds__(768, 1)
void chunk_vgp_kernel(const ET *__restrict__ q, const ET *__restrict__ k,
                      const ET *__restrict__ v, const float *__restrict__ g,
                      const float *__restrict__ beta, const float *state_in,
                      float *state_out, ET *__restrict__ y,
                      int T, int Hk, int Hv, int xcd_group, float scale, int flags)
{
    using L = VgpCfg<ET>;
    using X4 = typename Vec<ET>::x4;
    using X8 = typename Vec<ET>::x8;
    constexpr int C = L::C, DK = L::DK, DV = L::DV, NBK = L::NBK, NB = L::NB, NBT = L::NBT, NSW = L::NSW;
    constexpr int LDK = L::LDK, LDC = L::LDC, LDCF = L::LDCF, LDD = L::LDD, LDTF = L::LDTF;
    constexpr int NSK = DK / 32;                   // 32-key contraction steps
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, x = lane & 15, qd = lane >> 4;
    // XCD-grouped slot order, as in the other chunk kernels
    int bid = blockIdx.x;
    if (xcd_group > 1) {
        const int xcd = bid & 7, kk = bid >> 3;
        const int sib = kk % xcd_group, m = kk / xcd_group;
        bid = (m * 8 + xcd) * xcd_group + sib;
    }
    const int b = bid / Hv, hv = value_head_of_rank(bid % Hv, Hk, Hv, flags);
    const int hk = key_head(hv, Hk, Hv, flags);
    const int slot = b * Hv + hv;
    const size_t kstride = (size_t)Hk * DK, vstride = (size_t)Hv * DV, gstride = (size_t)Hv * DK;
    const ET *kbase = k + ((size_t)b * T * Hk + hk) * DK;
    const ET *qbase = q + ((size_t)b * T * Hk + hk) * DK;
    const ET *vbase = v + ((size_t)b * T * Hv + hv) * DV;
    const float *gbase = g + ((size_t)b * T * Hv + hv) * DK;
    const float *bbase = beta + (size_t)b * T * Hv + hv;
    const int nchunks = (T + C - 1) / C;
    const unsigned lds_base = (unsigned)(uintptr_t)((__attribute__((address_space(3))) char *)smem);
    auto parity = [](int c) { return (unsigned)((c & 1) * L::PAR); };

    // -A and QKR of both parities: the block above the diagonal is never
    // written and stays zero
    for (int i = tid; i < 2 * (L::pTd / 16); i += L::NT) {
        const int par = i / (L::pTd / 16), u = i - par * (L::pTd / 16);
        reinterpret_cast<uint4 *>(smem + par * L::PAR)[u] = zero_u4();
    }
    lds_barrier();

    if (w < NSW) {
        // ================= state waves =================
        const int vloc = 32 * w;                   // this wave's 32 value columns
        f32x4 S[NBK][NB];
        const size_t sbase = (size_t)slot * DV * DK;
        {
            gfloat *sin = state_in ? (gfloat *)state_in + sbase : (gfloat *)kZeroRow;
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) {
                const size_t row = (size_t)(vloc + 16 * vb + x) * (state_in ? DK : 0);
#pragma unroll
                for (int kb = 0; kb < NBK; ++kb)
                    S[kb][vb] = *reinterpret_cast<gf32x4 *>(sin + row + 16 * kb + 4 * qd);
            }
        }
        // this wave's V columns of chunk c into its slice of the parity buffer
        // (global -> LDS, lane l: row l / 4 of a 16-row load, 8 values at 8 (l % 4));
        // rows past the end read the last row (beta = 0 there)
        auto issue_v = [&](int c) {
            const int t0 = c * C, cn = min(C, T - t0);
            const ET *src = vbase + (size_t)t0 * vstride + vloc;
            const unsigned dst = parity(c) + L::pV + w * L::VSL;
#pragma unroll
            for (int i = 0; i < C / 16; ++i) {
                const int r = min(16 * i + (lane >> 2), cn - 1);
                const unsigned off = (unsigned)((r * vstride + 8 * (lane & 3)) * sizeof(ET));
                const unsigned la = __builtin_amdgcn_readfirstlane(lds_base + dst + 1024 * i);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
                asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                             :: "v"(off), "s"(src), "s"(la) : "memory", "m0");
#pragma clang diagnostic pop
            }
        };
        // V column fragment: lane (x, qd) gets rows 16 ib + 4 qd + (0..3) of
        // value column 16 vb + x of the slice (transpose read)
        const unsigned lV = (unsigned)(L::pV + w * L::VSL + (4 * qd + (x >> 2)) * L::VRB + 8 * (x & 3));
        // iteration it: chunk it - 1 (the prep waves are a chunk ahead); V of
        // chunk it is loaded for the next iteration
        for (int it = 0; it <= nchunks; ++it) {
            const int n = it - 1;
            const bool more = it < nchunks;
            if (more) issue_v(it);
            if (n < 0) {
                lds_barrier();
                lds_barrier();
                continue;
            }
            const int t0 = n * C, cn = min(C, T - t0);
            const unsigned P = parity(n);
            const ET *sKg = reinterpret_cast<const ET *>(smem + P + L::pKg);
            const ET *sQg = reinterpret_cast<const ET *>(smem + P + L::pQg);
            // ---------------- phase a: X = (K diag G) S0^T, Y^T = S0 (Q diag G)^T
            f32x4 Xa[NBT][NB], Ya[NB][NBT];
#pragma unroll
            for (int tb = 0; tb < NBT; ++tb)
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) { Xa[tb][vb] = zero4(); Ya[vb][tb] = zero4(); }
#pragma unroll
            for (int s = 0; s < NSK; ++s) {
                X8 fk[NBT], fq[NBT];
#pragma unroll
                for (int tb = 0; tb < NBT; ++tb) {
                    fk[tb] = cat8<ET>(frag_row<ET>(sKg, LDK, 16 * tb, 0, 2 * s, x, qd),
                                      frag_row<ET>(sKg, LDK, 16 * tb, 0, 2 * s + 1, x, qd));
                    fq[tb] = cat8<ET>(frag_row<ET>(sQg, LDK, 16 * tb, 0, 2 * s, x, qd),
                                      frag_row<ET>(sQg, LDK, 16 * tb, 0, 2 * s + 1, x, qd));
                }
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) {
                    const X8 fs = cat8<ET>(cvt4<ET>(S[2 * s][vb]), cvt4<ET>(S[2 * s + 1][vb]));
#pragma unroll
                    for (int tb = 0; tb < NBT; ++tb) {
                        Xa[tb][vb] = mfma(fk[tb], fs, Xa[tb][vb]);
                        Ya[vb][tb] = mfma(fs, fq[tb], Ya[vb][tb]);
                    }
                }
            }
            lds_barrier();
            // ---------------- phase b: D by blocked substitution in float32, y, update
            if (more) __builtin_amdgcn_s_waitcnt(0x0F72);   // vmcnt(2): V of this chunk has landed
            else __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0)
            asm volatile("" ::: "memory");
            const float *sAn = reinterpret_cast<const float *>(smem + P + L::pAn);
            const float *sTd = reinterpret_cast<const float *>(smem + P + L::pTd);
            const float *sB = reinterpret_cast<const float *>(smem + P + L::pB);
            const ET *sQKR = reinterpret_cast<const ET *>(smem + P + L::pQKR);
            f32x4 Da[NBT][NB];
            X4 Df[NBT][NB];
#pragma unroll
            for (int ib = 0; ib < NBT; ++ib) {
                const f32x4 bv = *reinterpret_cast<const f32x4 *>(sB + 16 * ib + 4 * qd);
                f32x4 Z[NB];
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) {
                    const f32x4 vv = to_f32x4<ET>(ld_tr<ET>(smem, P + lV + 32 * vb + 1024 * ib));
                    Z[vb] = bv * (vv - Xa[ib][vb]);
                }
#pragma unroll
                for (int jb = 0; jb < ib; ++jb) {
                    const f32x4 fa = ld4<float>(sAn + (16 * ib + x) * LDCF + 16 * jb + 4 * qd);
#pragma unroll
                    for (int vb = 0; vb < NB; ++vb) Z[vb] = mma_f32(fa, Da[jb][vb], Z[vb]);
                }
                const f32x4 ft = ld4<float>(sTd + (16 * ib + x) * LDTF + 4 * qd);
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) {
                    Da[ib][vb] = mma_f32(ft, Z[vb], zero4());
                    Df[ib][vb] = cvt4<ET>(Da[ib][vb]);
                }
            }
            // Y^T = (S0 (Q diag G)^T) / sqrt(Dk) + D^T QKR^T
#pragma unroll
            for (int tb = 0; tb < NBT; ++tb) {
                const X8 fr = cat8<ET>(frag_row<ET>(sQKR, LDC, 16 * tb, 0, 0, x, qd),
                                       frag_row<ET>(sQKR, LDC, 16 * tb, 0, 1, x, qd));
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) {
                    Ya[vb][tb] *= scale;
                    Ya[vb][tb] = mfma(cat8<ET>(Df[0][vb], Df[1][vb]), fr, Ya[vb][tb]);
                }
            }
            store_y(y + (((size_t)b * T + t0) * Hv + hv) * DV, Hv * DV, cn, vloc, x, qd, Ya);
            // S^T <- diag(G_last) S^T + (K diag(G_last / G))^T D
            {
                const ET *sKr = reinterpret_cast<const ET *>(smem + P + L::pKr);
                const float *sGl = reinterpret_cast<const float *>(smem + P + L::pGl);
#pragma unroll
                for (int kb = 0; kb < NBK; ++kb) {
                    const f32x4 gl = *reinterpret_cast<const f32x4 *>(sGl + 16 * kb + 4 * qd);
                    const X8 fk = cat8<ET>(frag_col<ET>(sKr, LDK, 0, 16 * kb, 0, x, qd),
                                           frag_col<ET>(sKr, LDK, 0, 16 * kb, 1, x, qd));
#pragma unroll
                    for (int vb = 0; vb < NB; ++vb) {
                        S[kb][vb] *= gl;
                        S[kb][vb] = mfma(fk, cat8<ET>(Df[0][vb], Df[1][vb]), S[kb][vb]);
                    }
                }
            }
            lds_barrier();
        }
#pragma unroll
        for (int vb = 0; vb < NB; ++vb) {
            const size_t row = sbase + (size_t)(vloc + 16 * vb + x) * DK;
#pragma unroll
            for (int kb = 0; kb < NBK; ++kb)
                *reinterpret_cast<f32x4 *>(state_out + row + 16 * kb + 4 * qd) = S[kb][vb];
        }
    } else {
        // ================= prep waves =================
        // wave (bt, kq): tokens 16 bt .. + 15 over keys 32 kq .. + 31; lane
        // (x, qd) holds token 16 bt + x, keys 16 kb + 4 qd .. + 3 of the key
        // blocks kb = 2 kq + h
        const int pw = w - NSW, bt = pw >> 2, kq = pw & 3;
        const X4 z4 = cvt4<ET>(zero4());
        const int tok = 16 * bt + x;
        struct In {
            f32x4 g[2];
            X4 kk[2], qq[2];
            float be;
        };
        auto load_in = [&](int c, In &r) {
            const int t0 = c * C, cn = min(C, T - t0);
            const size_t t = (size_t)(t0 + min(tok, cn - 1));
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int i0 = 16 * (2 * kq + h) + 4 * qd;
                r.g[h] = *reinterpret_cast<const f32x4 *>(gbase + t * gstride + i0);
                r.kk[h] = ld4<ET>(kbase + t * kstride + i0);
                r.qq[h] = ld4<ET>(qbase + t * kstride + i0);
            }
            r.be = bbase[t * Hv];
        };
        In cur, nxt;
        if (nchunks > 0) load_in(0, cur);
        nxt = cur;
        // iteration it: the scans and tiles of chunk it, and the last steps of
        // chunk it - 1 (its diagonal inverses and cross-block tile)
        for (int it = 0; it <= nchunks; ++it) {
            const bool work = it < nchunks;
            const bool fin = it >= 1;
            if (it + 1 < nchunks) load_in(it + 1, nxt);
            const int cn = work ? min(C, T - it * C) : 0;
            const bool valid = tok < cn;
            const unsigned P = parity(it);
            ET *sKg = reinterpret_cast<ET *>(smem + P + L::pKg);
            ET *sQg = reinterpret_cast<ET *>(smem + P + L::pQg);
            ET *sKr = reinterpret_cast<ET *>(smem + P + L::pKr);
            float *sAn = reinterpret_cast<float *>(smem + P + L::pAn);
            ET *sQKR = reinterpret_cast<ET *>(smem + P + L::pQKR);
            float *sBT = reinterpret_cast<float *>(smem + L::oBT);
            ET *sKS = reinterpret_cast<ET *>(smem + L::oKS);
            float *sAd = reinterpret_cast<float *>(smem + L::oAd);
            X4 kx[2], qx[2];                       // k and q of this lane, zero past the end
            f32x4 P16[2], S16[2];
            // ---------------- phase a: scans, level products, partial tiles of chunk it
            if (work) {
                f32x4 kk[4], qk[4], q0 = zero4();
#pragma unroll
                for (int lv = 0; lv < 4; ++lv) { kk[lv] = zero4(); qk[lv] = zero4(); }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int i0 = 16 * (2 * kq + h) + 4 * qd;
                    f32x4 g4 = cur.g[h];
                    if (flags & kLogGate) {            // uniform: exp only for log-space gates
#pragma unroll
                        for (int e = 0; e < 4; ++e) g4[e] = expf(g4[e]);
                    }
                    const f32x4 one = {1.f, 1.f, 1.f, 1.f};
                    g4 = valid ? g4 : one;
                    kx[h] = valid ? cur.kk[h] : z4;
                    qx[h] = valid ? cur.qq[h] : z4;
                    const f32x4 kf = to_f32x4<ET>(kx[h]), qf = to_f32x4<ET>(qx[h]);
                    const VgScales sc = vg_scales(g4, x);
#pragma unroll
                    for (int lv = 0; lv < 4; ++lv) {
                        const X4 ku = cvt4<ET>(kf * sc.s[lv]);
                        kk[lv] = mfma(ku, ku, kk[lv]);
                        qk[lv] = mfma(ku, cvt4<ET>(qf * sc.s[lv]), qk[lv]);
                    }
                    q0 = mfma(kx[h], qx[h], q0);
                    P16[h] = sc.p16;
                    S16[h] = sc.s16;
                    if (x == 15) *reinterpret_cast<f32x4 *>(sBT + bt * DK + i0) = P16[h];
                    if (bt == 0) {
                        // block 0: G = P16; K diag(S16) for the cross-block tile
                        st4<ET>(sKg + x * LDK + i0, cvt4<ET>(kf * P16[h]));
                        st4<ET>(sQg + x * LDK + i0, cvt4<ET>(qf * P16[h]));
                        st4<ET>(sKS + x * LDK + i0, cvt4<ET>(kf * S16[h]));
                    } else {
                        // block 1: G_last / G = S16
                        st4<ET>(sKr + (16 + x) * LDK + i0, cvt4<ET>(kf * S16[h]));
                    }
                }
                // keep each entry's own level (the highest bit in which the
                // in-block indices of t and j differ); zero above the diagonal
                f32x4 za, zo;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int jl = 4 * qd + r, d = jl ^ x;
                    float zk = kk[0][r], zq = qk[0][r];
                    zk = d >= 2 ? kk[1][r] : zk;
                    zq = d >= 2 ? qk[1][r] : zq;
                    zk = d >= 4 ? kk[2][r] : zk;
                    zq = d >= 4 ? qk[2][r] : zq;
                    zk = d >= 8 ? kk[3][r] : zk;
                    zq = d >= 8 ? qk[3][r] : zq;
                    za[r] = jl < x ? zk : 0.f;
                    zo[r] = jl < x ? zq : (jl == x ? q0[r] : 0.f);
                }
                f32x4 *part = reinterpret_cast<f32x4 *>(smem + L::oPd) + (pw * 2) * 64 + lane;
                part[0] = za;
                part[64] = zo;
                if (kq == 0 && qd == 0)
                    reinterpret_cast<float *>(smem + P + L::pB)[tok] = valid ? cur.be : 0.f;
            }
            // the last steps of chunk it - 1: its cross-block tile (from the
            // partials its phase b left), its diagonal inverses.  The waves of
            // block 0 finish their scans first (the older wave of each SIMD
            // issues first), so they take this work, one piece per SIMD.
            if (fin) {
                const unsigned PP = parity(it - 1);
                if (pw == 3) {
                    f32x4 zk = zero4(), zq = zero4();
#pragma unroll
                    for (int pp = 0; pp < 4; ++pp) {
                        const f32x4 *px = reinterpret_cast<const f32x4 *>(smem + L::oPx) + (pp * 2) * 64 + lane;
                        zk += px[0];
                        zq += px[64];
                    }
                    const int t1 = 16 + x;
                    const float bv = reinterpret_cast<const float *>(smem + PP + L::pB)[t1];
                    *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(smem + PP + L::pAn) + t1 * LDCF + 4 * qd) =
                        zk * (-bv);
                    st4<ET>(reinterpret_cast<ET *>(smem + PP + L::pQKR) + t1 * LDC + 4 * qd, cvt4<ET>(zq * scale));
                }
                if (pw == 0 || pw == 2) {
                    // T_bb = (I + A_bb)^-1 of block pw / 2: four lanes per column
                    // c, lane part pt holding rows pt, pt + 4, pt + 8, pt + 12;
                    // once x_j is final (in part j % 4), every later row
                    // subtracts A[i][j] x_j
                    const int base = 8 * pw;
                    const int pt = lane & 3, c = ((lane >> 4) << 2) | ((lane >> 2) & 3);
                    f32x4 arow[4][4];
#pragma unroll
                    for (int mm = 0; mm < 4; ++mm)
#pragma unroll
                        for (int j4 = 0; j4 <= mm; ++j4)
                            arow[mm][j4] = *reinterpret_cast<const f32x4 *>(sAd + (base + pt + 4 * mm) * LDD + 4 * j4);
                    float sv[4];
#pragma unroll
                    for (int mm = 0; mm < 4; ++mm) sv[mm] = (pt + 4 * mm == c) ? 1.f : 0.f;
#pragma unroll
                    for (int j = 0; j < 15; ++j) {
                        float xj;
                        switch (j & 3) {
                        case 0: xj = quad_bcast<0>(sv[j >> 2]); break;
                        case 1: xj = quad_bcast<1>(sv[j >> 2]); break;
                        case 2: xj = quad_bcast<2>(sv[j >> 2]); break;
                        default: xj = quad_bcast<3>(sv[j >> 2]); break;
                        }
#pragma unroll
                        for (int mm = 0; mm < 4; ++mm)
                            if (4 * mm + 3 > j) sv[mm] -= arow[mm][j >> 2][j & 3] * xj;
                    }
                    float *td = reinterpret_cast<float *>(smem + PP + L::pTd);
#pragma unroll
                    for (int mm = 0; mm < 4; ++mm) td[(base + pt + 4 * mm) * LDTF + c] = sv[mm];
                }
            }
            lds_barrier();
            // ---------------- phase b: diagonal tiles of chunk it, cross-block
            // partials, the scaled K and Q that need the other block's totals
            if (work) {
                if (pw == 1 || pw == 3) {
                    // the diagonal tile of block db = pw / 2: partial sums of
                    // its four key quarters, rows scaled by beta (zero past
                    // the end)
                    const int db = pw >> 1, tb = 16 * db + x;
                    f32x4 a = zero4(), o = zero4();
#pragma unroll
                    for (int pp = 0; pp < 4; ++pp) {
                        const f32x4 *pin = reinterpret_cast<const f32x4 *>(smem + L::oPd) + ((4 * db + pp) * 2) * 64 + lane;
                        a += pin[0];
                        o += pin[64];
                    }
                    a *= reinterpret_cast<const float *>(smem + P + L::pB)[tb];
                    o *= scale;
                    const int j0 = 16 * db + 4 * qd;
                    *reinterpret_cast<f32x4 *>(sAn + tb * LDCF + j0) = -a;
                    st4<ET>(sQKR + tb * LDC + j0, cvt4<ET>(o));
                    *reinterpret_cast<f32x4 *>(sAd + tb * LDD + 4 * qd) = a;
                }
                if (bt == 1) {
                    // cross-block tile (j in block 0, t = this wave's token):
                    // R = P16_t S16_j, over this wave's keys
                    f32x4 zk = zero4(), zq = zero4();
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int i0 = 16 * (2 * kq + h) + 4 * qd;
                        const f32x4 kf = to_f32x4<ET>(kx[h]), qf = to_f32x4<ET>(qx[h]);
                        const X4 ks = ld4<ET>(sKS + x * LDK + i0);
                        zk = mfma(ks, cvt4<ET>(kf * P16[h]), zk);
                        zq = mfma(ks, cvt4<ET>(qf * P16[h]), zq);
                        const f32x4 bt0 = *reinterpret_cast<const f32x4 *>(sBT + i0);
                        const f32x4 G = P16[h] * bt0;
                        st4<ET>(sKg + (16 + x) * LDK + i0, cvt4<ET>(kf * G));
                        st4<ET>(sQg + (16 + x) * LDK + i0, cvt4<ET>(qf * G));
                    }
                    f32x4 *px = reinterpret_cast<f32x4 *>(smem + L::oPx) + (kq * 2) * 64 + lane;
                    px[0] = zk;
                    px[64] = zq;
                } else {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int i0 = 16 * (2 * kq + h) + 4 * qd;
                        const f32x4 bt0 = *reinterpret_cast<const f32x4 *>(sBT + i0);
                        const f32x4 bt1 = *reinterpret_cast<const f32x4 *>(sBT + DK + i0);
                        st4<ET>(sKr + x * LDK + i0, cvt4<ET>(to_f32x4<ET>(kx[h]) * (S16[h] * bt1)));
                        if (x == 0)
                            *reinterpret_cast<f32x4 *>(smem + P + L::pGl + 4 * i0) = bt0 * bt1;
                    }
                }
            }
            lds_barrier();
            cur = nxt;
        }
    }
}

#ifndef GDN_VG_PIPELINED
#define GDN_VG_PIPELINED 1
#endif

// The per-key-dimension gate: the pipelined kernel for 16-bit inputs with
// Dk = Dv = 128 on grids that need no value split (more than 128 slots) at
// the default chunk of 32 tokens; gdn_chunk_vg.h's kernel otherwise.
template <typename ET>
hipError_t launch_chunk_vg_any(const FwdArgs &a, hipStream_t st) {
    if constexpr (sizeof(ET) == 2 && GDN_VG_PIPELINED) {
        const long nslots = (long)a.B * a.Hv;
        if (a.Dk == 128 && a.Dv == 128 && a.C != 16 && vg_split(a.Dv, nslots) == 1) {
            const int group = a.Hv / a.Hk;
            const int xcd_group = (group > 1 && nslots % (8L * group) == 0) ? group : 1;
            hipLaunchKernelGGL(chunk_vgp_kernel<ET>, dim3((unsigned)nslots), dim3(VgpCfg<ET>::NT), 0, st,
                               static_cast<const ET *>(a.q), static_cast<const ET *>(a.k),
                               static_cast<const ET *>(a.v), a.g, a.beta, a.state_in, a.state_out,
                               static_cast<ET *>(a.y), a.T, a.Hk, a.Hv, xcd_group, a.scale, a.flags);
            return hipGetLastError();
        }
    }
    return launch_chunk_vg_typed<ET>(a, st);
}

}  // namespace gdn
