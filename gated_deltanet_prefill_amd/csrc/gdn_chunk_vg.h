// gdn_chunk_vg.h -- the chunked forward kernel for a decay per key dimension.
//
// The gate g [B,T,Hv,Dk] decays each key column of the state on its own:
//     S_t = S_{t-1} diag(g_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
// (the 4-D gate the MLX pull request page "Pack gated_delta_seq" names as a
// shape its kernels would misread).  Within a chunk the decay ratio between
// tokens j <= t becomes a vector over key dimensions,
//     R_i[t][j] = g_{j+1,i} ... g_{t,i},
// so it no longer factors out of K K^T: every product that carries a ratio
// is formed from operands scaled per key dimension, with each scale a
// product of decays (never a quotient; the ferrox-core gdn_chunk.rs page,
// "The algebra") and therefore at most 1 for decays in [0, 1]:
//
//  * tokens in different 16-token blocks (j in block 0, t in block 1):
//        R[t][j] = P_t S_j,  P_t = prefix product of t's block up to t,
//                            S_j = product over j's block after j;
//  * tokens in one 16-token block: with m the highest bit in which their
//    in-block indices differ, t lies in the upper and j in the lower half of
//    an aligned segment of 2^(m+1) tokens, and
//        R[t][j] = L^m_t E^m_j,  L^m_t = product over t's half up to t,
//                                E^m_j = product over j's half after j;
//    the block's K K^T and Q K^T are then four products, one per level m,
//    each kept where its level applies.  The segment products come from
//    cross-lane scans (DPP) over the block's sixteen tokens, one per lane.
//
// With G_t = prod_{s<=t} g_s and G_last = G_{c-1} (per key dimension):
//     A[t][j] = beta_t sum_i k_ti k_ji R_i[t][j]  (j < t),
//     QKR[t][j] = sum_i q_ti k_ji R_i[t][j] / sqrt(Dk)  (j <= t),
//     D = (I + A)^-1 beta (V - (K diag G) S0^T),
//     y = ((Q diag G) S0^T) / sqrt(Dk) + QKR D,
//     S <- S0 diag(G_last) + D^T (K diag(G_last / G)),
// where G_last / G_t = prod_{s>t} g_s is again a product of decays.
//
// The layout and the substitution follow the generic chunk kernel
// (gdn_chunk_impl.h); chunks are at most 32 tokens (two 16-token blocks)
// so that the gate tiles fit in LDS, 16 for float32 inputs.

#pragma once

#include "gdn_chunk_impl.h"

namespace gdn {

template <typename ET, int DK_, int DVS_, int C_, int NB_>
struct VgCfg : ChunkCfg<ET, DK_, DVS_, C_, NB_> {
    using Base = ChunkCfg<ET, DK_, DVS_, C_, NB_>;
    static constexpr int LDG = DK_ + 4;                   // f32 rows of decays / scans
    static constexpr int oGv = Base::BYTES;               // decays [C][LDG]
    static constexpr int oP16 = oGv + C_ * LDG * 4;       // in-block prefix products
    static constexpr int oS16 = oP16 + C_ * LDG * 4;      // in-block products after t
    static constexpr int oBT = oS16 + C_ * LDG * 4;       // block totals [NBT][DK]
    static constexpr int oGl = oBT + Base::NBT * DK_ * 4; // chunk totals [DK]
    static constexpr int oKg = oGl + DK_ * 4;             // K diag(G)       [C][LDK]
    static constexpr int oQg = oKg + C_ * Base::LDK * Base::ES;   // Q diag(G)
    static constexpr int oKr = oQg + C_ * Base::LDK * Base::ES;   // K diag(G_last / G)
    static constexpr int oPart = oKr + C_ * Base::LDK * Base::ES;  // per-wave partial tiles
    static constexpr int oPartX = oPart + Base::NW * 2 * 64 * 16;  // partials of the cross-block tile
    static constexpr int VBYTES = oPartX + Base::NW * 2 * 64 * 16;
    // the diagonal tiles of one block are summed over NPART waves, each
    // taking an equal share of the key steps
    static constexpr int NPART_ = Base::NW / Base::NBT;
    static constexpr int GUNITS = C_ * DK_ / 4;           // 16-byte units of a chunk's gates
    static constexpr int PERG = (GUNITS + Base::NT - 1) / Base::NT;
    static_assert(VBYTES <= 160 * 1024, "LDS budget");
    static_assert(Base::NBT <= 2 && Base::NBT <= Base::NW, "one wave per 16-token block");
};

// Products over aligned segments of the sixteen tokens of a block, one token
// per lane of a DPP row (x = lane index in the row), for the four key
// dimensions a lane holds.  p[m]: product over the lane's aligned 2^m-token
// segment up to and including the lane; e[m]: product over that segment
// after the lane (m = 0..4; p[0] = g, e[0] = 1).
struct SegScan {
    f32x4 p[5];
    f32x4 e[5];
};

template <int CTRL>
__device__ __forceinline__ float dpp_keep(float v) {   // DPP move, 1 where no source
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        __builtin_bit_cast(int, 1.0f), __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// The same DPP move on each of the four components (independent chains).
template <typename F>
__device__ __forceinline__ f32x4 each4(f32x4 v, F f) {
    return f32x4{f(v[0]), f(v[1]), f(v[2]), f(v[3])};
}

// Every cross-lane move below is issued by all sixteen lanes before any
// lane-dependent choice: a DPP move inside a branch would read lanes the
// branch has switched off.
__device__ __forceinline__ SegScan seg_scan(f32x4 g, int x) {
    const f32x4 one = {1.f, 1.f, 1.f, 1.f};
    auto sel = [](bool c, f32x4 a, f32x4 b) { return c ? a : b; };
    SegScan r;
    // prefix: the upper half of each segment multiplies by its lower half's total
    const f32x4 p0 = g;
    const f32x4 a1 = each4(p0, [](float v) { return dpp_row_shr<1>(v); });
    const f32x4 p1 = sel(x & 1, p0 * a1, p0);
    const f32x4 a2 = each4(p1, [](float v) { return quad_bcast<1>(v); });
    const f32x4 p2 = sel(x & 2, p1 * a2, p1);
    const f32x4 a3 = each4(p2, [](float v) { return dpp_row_shr<4>(quad_bcast<3>(v)); });
    const f32x4 p3 = sel(x & 4, p2 * a3, p2);
    const f32x4 w3a = each4(p3, [](float v) { return dpp_row_shr<4>(quad_bcast<3>(v)); });
    const f32x4 w3b = each4(w3a, [](float v) { return dpp_row_shr<4>(v); });   // lane 7's, two quads up
    const f32x4 p4 = sel(x & 8, p3 * sel(x & 4, w3b, w3a), p3);
    // after the lane: the lower half of each segment multiplies by its upper
    // half's total; s = g e is the product from the lane to the segment's end
    const f32x4 b1 = each4(g, [](float v) { return dpp_keep<0x101>(v); });      // next lane's g
    const f32x4 e1 = sel(x & 1, one, b1);
    const f32x4 b2 = each4(g * e1, [](float v) { return quad_bcast<2>(v); });
    const f32x4 e2 = sel(x & 2, e1, e1 * b2);
    const f32x4 b3 = each4(g * e2, [](float v) { return dpp_row_shl<4>(quad_bcast<0>(v)); });
    const f32x4 e3 = sel(x & 4, e2, e2 * b3);
    const f32x4 v3a = each4(g * e3, [](float v) { return dpp_row_shl<4>(quad_bcast<0>(v)); });
    const f32x4 v3b = each4(v3a, [](float v) { return dpp_row_shl<4>(v); });   // lane 8's, two quads down
    const f32x4 e4 = sel(x & 8, e3, e3 * sel(x & 4, v3a, v3b));
    r.p[0] = p0; r.p[1] = p1; r.p[2] = p2; r.p[3] = p3; r.p[4] = p4;
    r.e[0] = one; r.e[1] = e1; r.e[2] = e2; r.e[3] = e3; r.e[4] = e4;
    return r;
}

// 16-bit: two 4-element pieces make one 8-element operand; f32: one piece.
template <typename ET>
__device__ __forceinline__ typename Step<ET>::frag frag_of(const f32x4 *pc) {
    if constexpr (sizeof(ET) == 4) {
        return pc[0];
    } else {
        return cat8<ET>(cvt4<ET>(pc[0]), cvt4<ET>(pc[1]));
    }
}

template <typename ET, int DK, int DVS, int C, int NB>
__global__ __launch_bounds__(4 * DVS / NB, 1)
void chunk_vg_kernel(const ET *__restrict__ q, const ET *__restrict__ k,
                     const ET *__restrict__ v, const float *__restrict__ g,
                     const float *__restrict__ beta, const float *state_in,
                     float *state_out, ET *__restrict__ y,
                     int T, int Hk, int Hv, int Dv, int nsplit, int xcd_group, float scale, int flags)
{
    using L = VgCfg<ET, DK, DVS, C, NB>;
    using X4 = typename Vec<ET>::x4;
    using FR = typename Step<ET>::frag;
    constexpr int BLK = Step<ET>::BLK;
    constexpr int NBT = L::NBT, NBK = L::NBK, NW = L::NW, NT = L::NT;
    constexpr int LDK = L::LDK, LDV = L::LDV, LDC = L::LDC, LDCF = L::LDCF, LDD = L::LDD,
                  LDTF = L::LDTF, LDG = L::LDG, EPU = L::EPU;
    constexpr int NSK = Steps<NBK, BLK>::n;            // contraction steps over Dk
    constexpr int NST = Steps<NBT, BLK>::n;            // contraction steps over C
    constexpr int NPART_V = L::NPART_;
    static_assert(NBK % BLK == 0, "whole key steps");

    __shared__ __attribute__((aligned(16))) char smem[L::VBYTES];
    ET *sK = reinterpret_cast<ET *>(smem + L::oK);
    ET *sQ = reinterpret_cast<ET *>(smem + L::oQ);
    ET *sV = reinterpret_cast<ET *>(smem + L::oV);
    float *sAn = reinterpret_cast<float *>(smem + L::oAn);  // -A (f32)
    ET *sQKR = reinterpret_cast<ET *>(smem + L::oQKR);
    float *sAd = reinterpret_cast<float *>(smem + L::oAd);  // diagonal blocks of A (f32)
    float *sTd = reinterpret_cast<float *>(smem + L::oTd);  // diagonal blocks of (I + A)^-1 (f32)
    float *sb = reinterpret_cast<float *>(smem + L::oVec);
    float *sGv = reinterpret_cast<float *>(smem + L::oGv);
    float *sP16 = reinterpret_cast<float *>(smem + L::oP16);
    float *sS16 = reinterpret_cast<float *>(smem + L::oS16);
    float *sBT = reinterpret_cast<float *>(smem + L::oBT);
    float *sGl = reinterpret_cast<float *>(smem + L::oGl);
    ET *sKg = reinterpret_cast<ET *>(smem + L::oKg);
    ET *sQg = reinterpret_cast<ET *>(smem + L::oQg);
    ET *sKr = reinterpret_cast<ET *>(smem + L::oKr);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, x = lane & 15, qd = lane >> 4;
    // XCD-grouped slot order, as in the generic kernel
    int bid = blockIdx.x;
    if (xcd_group > 1) {
        const int xcd = bid & 7, kk = bid >> 3;
        const int sib = kk % xcd_group, m = kk / xcd_group;
        bid = (m * 8 + xcd) * xcd_group + sib;
    }
    // workgroup = (slot rank, value slice vs of DVS columns)
    const int rank = bid / nsplit, vs = bid - rank * nsplit;
    const int b = rank / Hv, hv = value_head_of_rank(rank % Hv, Hk, Hv, flags);
    const int hk = key_head(hv, Hk, Hv, flags);
    const int slot = b * Hv + hv;
    const int vloc = wave * 16 * NB;               // first slice column of this wave

    f32x4 S[NBK][NB];
    const size_t sbase = (size_t)slot * Dv * DK;
#pragma unroll
    for (int vb = 0; vb < NB; ++vb) {
        // rows of zeros (stride 0) when there is no initial state
        gfloat *sin = state_in ? (gfloat *)state_in + sbase : (gfloat *)kZeroRow;
        const size_t row = (size_t)(vs * DVS + vloc + 16 * vb + x) * (state_in ? DK : 0);
#pragma unroll
        for (int kb = 0; kb < NBK; ++kb)
            S[kb][vb] = *reinterpret_cast<gf32x4 *>(sin + row + 16 * kb + 4 * qd);
    }

    // -A and QKR above the diagonal blocks stay zero
    for (int i = tid; i < (L::oAd - L::oAn) / 16; i += NT)
        reinterpret_cast<uint4 *>(smem + L::oAn)[i] = zero_u4();

    const size_t kstride = (size_t)Hk * DK, vstride = (size_t)Hv * Dv, gstride = (size_t)Hv * DK;
    const ET *kbase = k + ((size_t)b * T * Hk + hk) * DK;
    const ET *qbase = q + ((size_t)b * T * Hk + hk) * DK;
    const ET *vbase = v + ((size_t)b * T * Hv + hv) * Dv + vs * DVS;
    const float *gbase = g + ((size_t)b * T * Hv + hv) * DK;
    const float *bbase = beta + (size_t)b * T * Hv + hv;

    uint4 rk[L::PERK], rq[L::PERK], rv[L::PERV], rg[L::PERG];
    float rb = 0.f;
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
#pragma unroll
        for (int i = 0; i < L::PERG; ++i) {
            const int it = min(tid + i * NT, L::GUNITS - 1);
            const int t = min(it / (DK / 4), last), u = it % (DK / 4);
            rg[i] = *reinterpret_cast<const uint4 *>(gbase + (size_t)(t0 + t) * gstride + 4 * u);
        }
        rb = bbase[(size_t)(t0 + min(tid, last)) * Hv];
    };

    // registers -> LDS; rows t >= cn: k = q = v = 0, g = 1, beta = 0
    auto stage = [&](int cn) {
#pragma unroll
        for (int i = 0; i < L::PERK; ++i) {
            asm volatile("" : "+v"(rk[i].x), "+v"(rk[i].y), "+v"(rk[i].z), "+v"(rk[i].w));
            asm volatile("" : "+v"(rq[i].x), "+v"(rq[i].y), "+v"(rq[i].z), "+v"(rq[i].w));
        }
#pragma unroll
        for (int i = 0; i < L::PERV; ++i)
            asm volatile("" : "+v"(rv[i].x), "+v"(rv[i].y), "+v"(rv[i].z), "+v"(rv[i].w));
#pragma unroll
        for (int i = 0; i < L::PERG; ++i)
            asm volatile("" : "+v"(rg[i].x), "+v"(rg[i].y), "+v"(rg[i].z), "+v"(rg[i].w));
        asm volatile("" : "+v"(rb));
#pragma unroll
        for (int i = 0; i < L::PERK; ++i) {
            const int it = tid + i * NT;
            if (L::KIT % NT == 0 || it < L::KIT) {
                const int t = it / L::UPK, u = it - t * L::UPK;
                const bool pad = t >= cn;
                *reinterpret_cast<uint4 *>(sK + t * LDK + u * EPU) = pad ? zero_u4() : rk[i];
                *reinterpret_cast<uint4 *>(sQ + t * LDK + u * EPU) = pad ? zero_u4() : rq[i];
            }
        }
#pragma unroll
        for (int i = 0; i < L::PERV; ++i) {
            const int it = tid + i * NT;
            if (L::VIT % NT == 0 || it < L::VIT) {
                const int t = it / L::UPV, u = it - t * L::UPV;
                *reinterpret_cast<uint4 *>(sV + t * LDV + u * EPU) = (t >= cn) ? zero_u4() : rv[i];
            }
        }
#pragma unroll
        for (int i = 0; i < L::PERG; ++i) {
            const int it = tid + i * NT;
            if (L::GUNITS % NT == 0 || it < L::GUNITS) {
                const int t = it / (DK / 4), u = it - t * (DK / 4);
                f32x4 gv = __builtin_bit_cast(f32x4, rg[i]);
                if (flags & kLogGate) {            // uniform: exp only for log-space gates
#pragma unroll
                    for (int e = 0; e < 4; ++e) gv[e] = expf(gv[e]);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) gv[e] = (t < cn) ? gv[e] : 1.f;
                *reinterpret_cast<f32x4 *>(sGv + t * LDG + 4 * u) = gv;
            }
        }
        if (tid < C) sb[tid] = (tid < cn) ? rb : 0.f;
    };

    const int nchunks = (T + C - 1) / C;
    // chunk 0's loads go out while the state is in flight; the state is then
    // consumed here, so that no load is pending at the loop header
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

        // ---- (a) wave w: block w % NBT over its share of the key steps:
        // the scans (P16, S16, block totals) and the partial diagonal tiles
        // of K K^T and Q K^T, one product per level, reduced to this lane's
        // entries (lane x of each DPP row is token 16 bt + x; the tile lane
        // (x, qd) holds column t = 16 bt + x, rows j = 16 bt + 4 qd + r).
        constexpr int NPART = NPART_V < NSK ? NPART_V : NSK;
        constexpr int SPP = NSK / NPART;                 // key steps per wave
        if (wave < NBT * NPART) {
            const int bt = wave % NBT, part = wave / NBT, t = 16 * bt + x;
            f32x4 kk[4], qk[4], q0 = zero4();
#pragma unroll
            for (int m = 0; m < 4; ++m) { kk[m] = zero4(); qk[m] = zero4(); }
#pragma unroll
            for (int ss = 0; ss < SPP; ++ss) {
                const int s = part * SPP + ss;
                f32x4 ka[4][BLK], kl[4][BLK], ql[4][BLK], k0[BLK], qq[BLK];
#pragma unroll
                for (int h = 0; h < BLK; ++h) {
                    const int kb = s * BLK + h, i0 = 16 * kb + 4 * qd;
                    const f32x4 g4 = *reinterpret_cast<const f32x4 *>(sGv + t * LDG + i0);
                    const f32x4 kf = to_f32x4<ET>(frag_row<ET>(sK, LDK, 16 * bt, 0, kb, x, qd));
                    const f32x4 qf = to_f32x4<ET>(frag_row<ET>(sQ, LDK, 16 * bt, 0, kb, x, qd));
                    const SegScan sc = seg_scan(g4, x);
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        ka[m][h] = kf * sc.e[m];
                        kl[m][h] = kf * sc.p[m];
                        ql[m][h] = qf * sc.p[m];
                    }
                    const f32x4 p16 = sc.p[4], s16 = sc.e[4];
                    k0[h] = kf;
                    qq[h] = qf;
                    *reinterpret_cast<f32x4 *>(sP16 + t * LDG + i0) = p16;
                    *reinterpret_cast<f32x4 *>(sS16 + t * LDG + i0) = s16;
                    if (x == 15) *reinterpret_cast<f32x4 *>(sBT + bt * DK + i0) = p16;
                    // the scaled K and Q that need no other block: G = P16 in
                    // the first block, G_last / G = S16 in the last
                    if (bt == 0) {
                        st4<ET>(sKg + t * LDK + i0, cvt4<ET>(kf * p16));
                        st4<ET>(sQg + t * LDK + i0, cvt4<ET>(qf * p16));
                    }
                    if (bt == NBT - 1) st4<ET>(sKr + t * LDK + i0, cvt4<ET>(kf * s16));
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const FR fa = frag_of<ET>(ka[m]);
                    kk[m] = mfma_step(fa, frag_of<ET>(kl[m]), kk[m]);
                    qk[m] = mfma_step(fa, frag_of<ET>(ql[m]), qk[m]);
                }
                q0 = mfma_step(frag_of<ET>(k0), frag_of<ET>(qq), q0);
            }
            // keep each entry's own level (the highest bit in which the
            // in-block indices of t and j differ): a weighted sum, no branches
            f32x4 za, zo;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int jl = 4 * qd + r, d = jl ^ x;
                const float w3 = d >= 8 ? 1.f : 0.f, w2 = (d >= 4 && d < 8) ? 1.f : 0.f,
                            w1 = (d >= 2 && d < 4) ? 1.f : 0.f, w0 = d == 1 ? 1.f : 0.f;
                const float lower = jl < x ? 1.f : 0.f, diag = jl == x ? 1.f : 0.f;
                za[r] = lower * (w0 * kk[0][r] + w1 * kk[1][r] + w2 * kk[2][r] + w3 * kk[3][r]);
                zo[r] = lower * (w0 * qk[0][r] + w1 * qk[1][r] + w2 * qk[2][r] + w3 * qk[3][r]) +
                        diag * q0[r];
            }
            f32x4 *part_out = reinterpret_cast<f32x4 *>(smem + L::oPart) + (wave * 2) * 64 + lane;
            part_out[0] = za;
            part_out[64] = zo;
        }
        lds_barrier();

        // ---- (b) waves w < NBT: the sum of block w's partial tiles, times
        // beta (A) and 1/sqrt(Dk) (QKR)
        if (wave < NBT) {
            const int bt = wave, t = 16 * bt + x;
            f32x4 a = zero4(), o = zero4();
#pragma unroll
            for (int pp = 0; pp < NPART; ++pp) {
                const f32x4 *pin = reinterpret_cast<const f32x4 *>(smem + L::oPart) + ((bt + NBT * pp) * 2) * 64 + lane;
                a += pin[0];
                o += pin[64];
            }
            a *= sb[t];
            o *= scale;
            const int j0 = 16 * bt + 4 * qd;
            *reinterpret_cast<f32x4 *>(sAn + t * LDCF + j0) = -a;
            st4<ET>(sQKR + t * LDC + j0, cvt4<ET>(o));
            *reinterpret_cast<f32x4 *>(sAd + t * LDD + 4 * qd) = a;
        }
        // tokens j in block 0, t in block 1: R = P16_t S16_j; every wave
        // takes a share of the key steps and leaves its partial tile in LDS
        constexpr int NPX = NW < NSK ? NW : NSK;         // waves sharing the cross-block tile
        constexpr int SPX = NSK / NPX;
        if constexpr (NBT == 2) {
            if (wave < NPX) {
                f32x4 zk = zero4(), zq = zero4();
#pragma unroll
                for (int ss = 0; ss < SPX; ++ss) {
                    const int s = wave * SPX + ss;
                    f32x4 ja[BLK], tk[BLK], tq[BLK];
#pragma unroll
                    for (int h = 0; h < BLK; ++h) {
                        const int kb = s * BLK + h, i0 = 16 * kb + 4 * qd;
                        const f32x4 sj = *reinterpret_cast<const f32x4 *>(sS16 + x * LDG + i0);
                        const f32x4 pt = *reinterpret_cast<const f32x4 *>(sP16 + (16 + x) * LDG + i0);
                        ja[h] = to_f32x4<ET>(frag_row<ET>(sK, LDK, 0, 0, kb, x, qd)) * sj;
                        tk[h] = to_f32x4<ET>(frag_row<ET>(sK, LDK, 16, 0, kb, x, qd)) * pt;
                        tq[h] = to_f32x4<ET>(frag_row<ET>(sQ, LDK, 16, 0, kb, x, qd)) * pt;
                    }
                    const FR fa = frag_of<ET>(ja);
                    zk = mfma_step(fa, frag_of<ET>(tk), zk);
                    zq = mfma_step(fa, frag_of<ET>(tq), zq);
                }
                f32x4 *px = reinterpret_cast<f32x4 *>(smem + L::oPartX) + (wave * 2) * 64 + lane;
                px[0] = zk;
                px[64] = zq;
            }
        }
        // the scaled K and Q that need the other block's totals: K diag(G)
        // and Q diag(G) of the second block (G = P16 x totals of the first),
        // K diag(G_last / G) of the first (S16 x totals of the second); and
        // G_last, elementwise
        if constexpr (NBT == 2) {
            constexpr int HU = 16 * DK / 4;                 // 16-byte units of one block
#pragma unroll
            for (int ii = 0; ii < (HU + NT - 1) / NT; ++ii) {
                const int it = tid + ii * NT;
                if (HU % NT != 0 && it >= HU) break;
                const int r = it / (DK / 4), i0 = 4 * (it - r * (DK / 4));
                const f32x4 bt0 = *reinterpret_cast<const f32x4 *>(sBT + i0);
                const f32x4 bt1 = *reinterpret_cast<const f32x4 *>(sBT + DK + i0);
                const int t1 = 16 + r;
                const f32x4 G = *reinterpret_cast<const f32x4 *>(sP16 + t1 * LDG + i0) * bt0;
                st4<ET>(sKg + t1 * LDK + i0, cvt4<ET>(to_f32x4<ET>(ld4<ET>(sK + t1 * LDK + i0)) * G));
                st4<ET>(sQg + t1 * LDK + i0, cvt4<ET>(to_f32x4<ET>(ld4<ET>(sQ + t1 * LDK + i0)) * G));
                const f32x4 Rl = *reinterpret_cast<const f32x4 *>(sS16 + r * LDG + i0) * bt1;
                st4<ET>(sKr + r * LDK + i0, cvt4<ET>(to_f32x4<ET>(ld4<ET>(sK + r * LDK + i0)) * Rl));
                if (r == 0) *reinterpret_cast<f32x4 *>(sGl + i0) = bt0 * bt1;
            }
        } else {
            for (int i0 = 4 * tid; i0 < DK; i0 += 4 * NT)
                *reinterpret_cast<f32x4 *>(sGl + i0) = *reinterpret_cast<const f32x4 *>(sBT + i0);
        }
        lds_barrier();

        // ---- (c) the cross-block tile of -A and QKR from its partials (last wave)
        if constexpr (NBT == 2) {
            if (wave == NW - 1) {
                f32x4 zk = zero4(), zq = zero4();
#pragma unroll
                for (int pp = 0; pp < NPX; ++pp) {
                    const f32x4 *px = reinterpret_cast<const f32x4 *>(smem + L::oPartX) + (pp * 2) * 64 + lane;
                    zk += px[0];
                    zq += px[64];
                }
                const int t = 16 + x;
                const float bv = sb[t];
                *reinterpret_cast<f32x4 *>(sAn + t * LDCF + 4 * qd) = zk * (-bv);
                st4<ET>(sQKR + t * LDC + 4 * qd, cvt4<ET>(zq * scale));
            }
        }
        // ---- (c) diagonal inverses (waves < NBT)
        if (wave < NBT) {
            const int base = 16 * wave;
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
                    if (4 * m + 3 > j) s[m] -= arow[m][j >> 2][j & 3] * xj;
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) sTd[(base + p + 4 * m) * LDTF + c] = s[m];
        }

        // ---- (c) X = (K diag G) S0^T and Y^T = S0 (Q diag G)^T for this wave's columns
        X4 Sf[NBK][NB];
#pragma unroll
        for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) Sf[kb][vb] = cvt4<ET>(S[kb][vb]);
        f32x4 Xa[NBT][NB], Ya[NB][NBT];
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb)
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) { Xa[tb][vb] = zero4(); Ya[vb][tb] = zero4(); }
#pragma unroll
        for (int s = 0; s < NSK; ++s) {
            FR fk[NBT], fq[NBT];
#pragma unroll
            for (int tb = 0; tb < NBT; ++tb) {
                fk[tb] = make_frag<ET>(s, NBK, [&](int kb) { return frag_row<ET>(sKg, LDK, 16 * tb, 0, kb, x, qd); });
                fq[tb] = make_frag<ET>(s, NBK, [&](int kb) { return frag_row<ET>(sQg, LDK, 16 * tb, 0, kb, x, qd); });
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
        }

        lds_barrier();                     // the inverses are in LDS

        // ---- (d) D = (I + A)^-1 beta (V - X), blocked forward substitution in
        // float32 (-A, T_ii and the solved blocks float32, float32 matrix-core
        // products); D is rounded to the input type only afterwards
        f32x4 Da[NBT][NB];
        X4 Df[NBT][NB];
#pragma unroll
        for (int ib = 0; ib < NBT; ++ib) {
            const f32x4 bv = *reinterpret_cast<const f32x4 *>(sb + 16 * ib + 4 * qd);
            f32x4 Z[NB];
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) {
                const f32x4 vv = to_f32x4<ET>(frag_col<ET>(sV, LDV, 0, vloc + 16 * vb, ib, x, qd));
                Z[vb] = bv * (vv - Xa[ib][vb]);
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

        // ---- (e) Y^T = (S0 (Q diag G)^T) / sqrt(Dk) + D^T QKR^T
#pragma unroll
        for (int tb = 0; tb < NBT; ++tb) {
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) Ya[vb][tb] *= scale;
#pragma unroll
            for (int s = 0; s < NST; ++s) {
                if (s * BLK > tb) continue;
                FR fr = make_frag<ET>(s, NBT, [&](int jb) { return frag_row<ET>(sQKR, LDC, 16 * tb, 0, jb, x, qd); });
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) {
                    FR fd = make_frag<ET>(s, NBT, [&](int jb) { return Df[jb][vb]; });
                    Ya[vb][tb] = mfma_step(fd, fr, Ya[vb][tb]);
                }
            }
        }
        store_y(y + (((size_t)b * T + t0) * Hv + hv) * Dv + vs * DVS, Hv * Dv, cn, vloc, x, qd, Ya);

        // ---- (f) S^T <- diag(G_last) S^T + (K diag(G_last / G))^T D
#pragma unroll
        for (int kb = 0; kb < NBK; ++kb) {
            const f32x4 gl = *reinterpret_cast<const f32x4 *>(sGl + 16 * kb + 4 * qd);
            FR fk[NST];
#pragma unroll
            for (int s = 0; s < NST; ++s)
                fk[s] = make_frag<ET>(s, NBT, [&](int tb) { return frag_col<ET>(sKr, LDK, 0, 16 * kb, tb, x, qd); });
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) S[kb][vb] *= gl;
#pragma unroll
            for (int s = 0; s < NST; ++s) {
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) {
                    FR fd = make_frag<ET>(s, NBT, [&](int tb) { return Df[tb][vb]; });
                    S[kb][vb] = mfma_step(fk[s], fd, S[kb][vb]);
                }
            }
        }
        if (n + 1 < nchunks) {
            lds_barrier();                 // chunk n is done with LDS
            stage(min(C, T - t0 - C));
        }
    }

#pragma unroll
    for (int vb = 0; vb < NB; ++vb) {
        const size_t row = sbase + (size_t)(vs * DVS + vloc + 16 * vb + x) * DK;
#pragma unroll
        for (int kb = 0; kb < NBK; ++kb)
            *reinterpret_cast<f32x4 *>(state_out + row + 16 * kb + 4 * qd) = S[kb][vb];
    }
}

// Value slices per slot: two slices of 64 columns for Dv = 128 while B Hv
// <= 128, each repeating the chunk's scans and C x C work for its half of
// the state (timed sweep over B Hv = 8..384, T = 128 and 512: 1.1-1.2x for
// 16-bit inputs, 1.3x for float32; slices of 32 columns leave two waves per
// workgroup and are slower, as is any split for Dv = 64).
inline int vg_split(int Dv, long nslots) { return (Dv == 128 && nslots <= 128) ? 2 : 1; }

// One slice of DVS value columns per workgroup, Dv / DVS workgroups per slot.
// Chunk length: 32 for 16-bit inputs, 16 for float32 (LDS budget).
template <typename ET, int DK, int DV, int DVS>
hipError_t launch_chunk_vg_slices(const FwdArgs &a, hipStream_t st) {
    constexpr int NB = DVS >= 128 ? 2 : 1;
    const long nslots = (long)a.B * a.Hv;
    const int group = a.Hv / a.Hk;
    const int nsplit = DV / DVS;
    const long nblocks = nslots * nsplit;
    const int xcd_group = (nsplit == 1 && group > 1 && nblocks % (8L * group) == 0) ? group : 1;
    auto go = [&](auto cc) -> hipError_t {
        constexpr int C = decltype(cc)::value;
        using L = VgCfg<ET, DK, DVS, C, NB>;
        hipLaunchKernelGGL((chunk_vg_kernel<ET, DK, DVS, C, NB>), dim3((unsigned)nblocks), dim3(L::NT), 0, st,
                           static_cast<const ET *>(a.q), static_cast<const ET *>(a.k),
                           static_cast<const ET *>(a.v), a.g, a.beta, a.state_in, a.state_out,
                           static_cast<ET *>(a.y), a.T, a.Hk, a.Hv, a.Dv, nsplit, xcd_group, a.scale, a.flags);
        return hipGetLastError();
    };
    if constexpr (sizeof(ET) == 4) {
        return go(std::integral_constant<int, 16>{});
    } else {
        if (a.C == 16) return go(std::integral_constant<int, 16>{});
        return go(std::integral_constant<int, 32>{});
    }
}

template <typename ET, int DK, int DV>
hipError_t launch_chunk_vg_dv(const FwdArgs &a, hipStream_t st) {
    if constexpr (DV == 128)
        if (vg_split(DV, (long)a.B * a.Hv) == 2) return launch_chunk_vg_slices<ET, DK, DV, 64>(a, st);
    return launch_chunk_vg_slices<ET, DK, DV, DV>(a, st);
}

template <typename ET, int DK>
hipError_t launch_chunk_vg_dk(const FwdArgs &a, hipStream_t st) {
    switch (a.Dv) {
    case 32: return launch_chunk_vg_dv<ET, DK, 32>(a, st);
    case 64: return launch_chunk_vg_dv<ET, DK, 64>(a, st);
    case 128: return launch_chunk_vg_dv<ET, DK, 128>(a, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename ET>
hipError_t launch_chunk_vg_typed(const FwdArgs &a, hipStream_t st) {
    switch (a.Dk) {
    case 32: return launch_chunk_vg_dk<ET, 32>(a, st);
    case 64: return launch_chunk_vg_dk<ET, 64>(a, st);
    case 128: return launch_chunk_vg_dk<ET, 128>(a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
