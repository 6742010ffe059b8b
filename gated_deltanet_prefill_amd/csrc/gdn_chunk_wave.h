// gdn_chunk_wave.h -- the chunked forward for a few tokens (1 <= T <= 16,
// one chunk) on grids of many (batch, head) slots: one wave per 16 value
// rows, four waves (64 value rows of one slot) per workgroup (16-bit
// inputs, Dk = 128, scalar gate).
//
// The chunk algebra is that of the ferrox-core gdn_chunk.rs page ("The
// algebra"), in the per-row form of the other chunk kernels:
//   A[t][j] = beta_t R[t][j] k_t.k_j (j < t),  T = (I + A)^-1 (float32),
//   M = K S0^T,  D = T (beta (V - G M)),
//   y_t = (G_t S0 q_t + sum_{j<=t} R[t][j] (q_t.k_j) d_j) / sqrt(Dk),
//   S <- G_last S0 + sum_t R[last][t] d_t k_t^T,
// with G[t] = g_0 ... g_t and every ratio R[t][j] = g_{j+1} ... g_t a product
// of decays (never a quotient).
//
// A call of a few tokens is bound by the state traffic (one read and one
// write of every state row), so the kernel is built around moving the state
// at full width:
//   * Each wave's 16 state rows (8 KB) go from HBM into a wave-private LDS
//     block with global_load_lds_dwordx4, eight lanes per 128-byte line, and
//     come back the same way through ordinary stores: the MFMA layout (a
//     lane per row) would make every lane of a load touch its own line.
//     The block is swizzled so that the MFMA-layout reads and writes are
//     free of bank conflicts; the state is in flight while the wave forms
//     the chunk's 16 x 16 matrices.
//   * K and Q of the chunk are staged once per workgroup, the same way.
//   * Each wave forms the chunk's 16 x 16 matrices (K K^T, K Q^T, the gate
//     ratios, the float32 inverse) itself, in a wave-private scratch: only
//     the K/Q staging is shared, so a workgroup synchronises once and its
//     waves otherwise run on their own.
//   * Transposed operands come from the matrix cores: the product X I of a
//     16-column block X with the identity lands X's rows on the
//     accumulator's rows, which is the operand layout of X^T (gdn_device.h),
//     exactly for 16-bit X.  V by tokens (for the right-hand side) and K^T
//     (for the update) are formed this way from their row fragments.

#pragma once

#include "gdn_chunk_impl.h"
#include "gdn_chunk_wy.h"

namespace gdn {

// Swizzle of a wave's state block: 16-byte unit u of each 128-byte piece of
// row r sits at u ^ wave_swz(r).  The MFMA-layout accesses (lane (x, qd) on
// unit 2 qd + h of row x) then put the 16 lanes of each bank group on 16
// different 16-byte bank slots.
__device__ __forceinline__ int wave_swz(int r) { return ((r >> 1) & 1) | (r & 4); }

template <typename ET>
__global__ __launch_bounds__(256)
void chunk_wave_kernel(const ET *__restrict__ q, const ET *__restrict__ k,
                       const ET *__restrict__ v, const float *__restrict__ g,
                       const float *__restrict__ beta, const float *state_in,
                       float *state_out, ET *__restrict__ y,
                       int T, int Hk, int Hv, int Dv, float scale, int flags)
{
    using X4 = typename Vec<ET>::x4;
    using X8 = typename Vec<ET>::x8;
    constexpr int DK = 128, C = 16;
    constexpr int NSK = DK / 32;                   // 32-key contraction steps
    constexpr int NBK = DK / 16;                   // key tiles of the state
    constexpr int LDA = 20;                        // f32 row stride of the scratch blocks
    constexpr int KQB = C * DK * 2;                // one chunk of K (or Q): 4 KB
    constexpr int STB = 16 * DK * 4;               // one wave's state rows: 8 KB
    constexpr int SCRB = (16 * LDA + 4 * 16) * 4;  // A (then T over it), then g, P, beta, R[last][t]
    constexpr int VB = 1024;                       // one wave's V columns (16 tokens x 16 values, twice)
    constexpr int WB = STB + SCRB + VB;
    constexpr int oQ = KQB, oGB = 2 * KQB, oW = oGB + 512;
    static_assert(KQB == 4 * 1024, "four 1 KB staging loads per chunk of K or Q");
    static_assert(STB == 8 * 1024, "eight 1 KB staging loads per state block");
    __shared__ __attribute__((aligned(16))) char smem[oW + 4 * WB];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, x = lane & 15, qd = lane >> 4;
    // Workgroups are dealt round-robin over the 8 XCDs.  The G workgroups
    // that read one q/k stream (the slot's value quarters, for each value
    // head of the key head) are renumbered onto one XCD, so that they share
    // its L2, while consecutive groups still go to consecutive XCDs: the
    // whole chip then streams the state from one narrow window of HBM.
    // (Giving each XCD one contiguous eighth of the grid instead, eight
    // windows far apart, made the state stream 10% slower.)
    int bid = blockIdx.x;
    {
        const int G = (Dv / 64) * (Hv / Hk);
        if (gridDim.x % (8 * G) == 0) {
            const int xcd = bid & 7, kk = bid >> 3;
            bid = ((kk / G) * 8 + xcd) * G + kk % G;
        }
    }
    const int nq = Dv / 64;                        // workgroups per slot
    const int rank = bid / nq;
    const int vblk = 4 * (bid - rank * nq) + wave;  // this wave's 16 value columns
    const int b = rank / Hv;
    const int hv = value_head_of_rank(rank % Hv, Hk, Hv, flags);
    const int hk = key_head(hv, Hk, Hv, flags);
    const size_t slot = (size_t)b * Hv + hv;

    char *wbuf = smem + oW + wave * WB;            // this wave's state block, scratch, V
    float *sA = reinterpret_cast<float *>(wbuf + STB);
    const unsigned oV = (unsigned)(oW + wave * WB + STB + SCRB);
    float *sT = sA, *sg = sA + 16 * LDA, *sP = sg + 16, *sb = sP + 16, *sRl = sb + 16;
    const unsigned lds_base = (unsigned)(uintptr_t)((__attribute__((address_space(3))) char *)smem);

    const size_t kstride = (size_t)Hk * DK, vstride = (size_t)Hv * Dv;
    const ET *kbase = k + ((size_t)b * T * Hk + hk) * DK;
    const ET *qbase = q + ((size_t)b * T * Hk + hk) * DK;
    const ET *vbase = v + ((size_t)b * T * Hv + hv) * Dv + 16 * vblk;
    const float *gbase = g + (size_t)b * T * Hv + hv;
    const float *bbase = beta + (size_t)b * T * Hv + hv;

    // global -> LDS, 16 bytes per lane at 16 lane of a 1 KB block (as inline
    // assembly, so that the compiler does not wait for it before this wave's
    // next LDS access; completion is awaited explicitly)
    auto g2lds = [&](const void *src, unsigned off, unsigned lds_byte) {
        const unsigned la = __builtin_amdgcn_readfirstlane(lds_base + lds_byte);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                     :: "v"(off), "s"(src), "s"(la) : "memory", "m0");
#pragma clang diagnostic pop
    };
    auto g2lds4 = [&](const void *src, unsigned off, unsigned lds_byte) {
        const unsigned la = __builtin_amdgcn_readfirstlane(lds_base + lds_byte);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                     :: "v"(off), "s"(src), "s"(la) : "memory", "m0");
#pragma clang diagnostic pop
    };
    auto wait_loads = [&]() {
        __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0)
        asm volatile("" ::: "memory");
    };

    // Identity fragments (16x16x32 operands, slot i of lane group qd):
    //   idK: contraction index 4 qd + i for i < 4 (zero slots above), the
    //        layout of half a K row fragment;
    //   idV: contraction index 8 qd + i for lane groups 0 and 1.
    X8 idK, idV;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        idK[i] = from_f32<ET>((i < 4 && 4 * qd + i == x) ? 1.f : 0.f);
        idV[i] = from_f32<ET>((qd < 2 && 8 * qd + i == x) ? 1.f : 0.f);
    }
    const X4 z4 = cvt4<ET>(zero4());

    // ---- the state block: load j (1 KB) holds rows 8 (j / 4) + lane / 8,
    // 128-byte piece j % 4, unit (lane % 8) ^ wave_swz(row).  In the MFMA
    // layout tile kb = 2 s + h has row 4 qd + r on key 32 s + 8 qd + 4 h + r
    // (so that a K or Q row fragment over a 32-key step is one 16-byte read)
    // and column x on value column 16 vblk + x: unit 2 qd + h of piece s of
    // row x.  A NULL state_in reads a row of zeros.
    const size_t srow0 = (slot * Dv + 16 * vblk) * DK;
    auto blk_row = [&](int j) { return 8 * (j >> 2) + (lane >> 3); };
    auto blk_unit = [&](int j) { return 8 * (j & 3) + ((lane & 7) ^ wave_swz(blk_row(j))); };
    auto tile_at = [&](int kb) {
        return (unsigned)(1024 * (4 * (x >> 3) + (kb >> 1)) + 16 * (8 * (x & 7) + ((2 * qd + (kb & 1)) ^ wave_swz(x))));
    };
    auto issue_state = [&]() {
        const float *src = state_in ? state_in + srow0 : kZeroRow;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const unsigned u = (unsigned)blk_unit(j);
            const unsigned off = state_in ? (unsigned)(blk_row(j) * DK * 4) + 16 * u : 16 * u;
            g2lds(src, off, (unsigned)(oW + wave * WB + 1024 * j));
        }
    };
    // K and Q of a chunk: load `wave` of each holds token rows 4 wave .. + 3,
    // unit u of row t at u ^ kq_swz(t); rows past the end read the last row
    auto issue_kq = [&](int t0, int cn) {
        const int t = 4 * wave + (lane >> 4);
        const unsigned u = (unsigned)((lane & 15) ^ kq_swz(t));
        const unsigned off = (unsigned)((min(t, cn - 1) * kstride + 8 * u) * sizeof(ET));
        g2lds(kbase + (size_t)t0 * kstride, off, (unsigned)(1024 * wave));
        g2lds(qbase + (size_t)t0 * kstride, off, (unsigned)(oQ + 1024 * wave));
    };
    // this wave's V columns: lane l holds token (l % 32) / 2, values
    // 8 (l % 2) .. + 7 (lanes 32..63 repeat them); rows past the end read the
    // last row
    auto issue_v = [&](int t0, int cn) {
        const int t = min((lane & 31) >> 1, cn - 1);
        g2lds(vbase + (size_t)t0 * vstride, (unsigned)((t * vstride + 8 * (lane & 1)) * sizeof(ET)), oV);
    };
    // the gates and betas of the chunk's tokens (lane l: token l % 16; lanes
    // past the 16th repeat them), by wave 0 for the workgroup
    auto issue_gb = [&](int t0, int cn) {
        const unsigned off = (unsigned)(min(lane & 15, cn - 1) * Hv * 4);
        g2lds4(gbase + (size_t)t0 * Hv, off, (unsigned)oGB);
        g2lds4(bbase + (size_t)t0 * Hv, off, (unsigned)(oGB + 256));
    };

    f32x4 S[NBK];
    {
        // the one chunk of 1 <= T <= 16 tokens
        constexpr int t0 = 0;
        const int cn = T;
        // Every load of the call is issued here, the state last; the wait
        // leaves the eight state loads in flight while the chunk's 16 x 16
        // work runs.
        issue_kq(t0, cn);
        issue_v(t0, cn);
        if (wave == 0) issue_gb(t0, cn);
        issue_state();
        __builtin_amdgcn_s_waitcnt(0x0F78);        // vmcnt(8): all but the state
        asm volatile("" ::: "memory");
        __syncthreads();                           // K, Q, g, beta of the chunk staged
        // V row fragment: lane groups 0 and 1 hold values 8 qd .. 8 qd + 7 of
        // token x (groups 2 and 3 are zeroed)
        X8 fv = lds8<ET>(smem, oV + 16 * (2 * x + (qd & 1)));
        const float graw = reinterpret_cast<const float *>(smem + oGB)[x];
        const float braw = reinterpret_cast<const float *>(smem + oGB + 256)[x];
        if (qd >= 2) fv = cat8<ET>(z4, z4);
        const unsigned lK = (unsigned)(x * 256 + ((qd ^ kq_swz(x)) << 4));
        X8 fk[NSK], fq[NSK];
#pragma unroll
        for (int s = 0; s < NSK; ++s) {
            fk[s] = lds8<ET>(smem, lK ^ (64 * s));
            fq[s] = lds8<ET>(smem, oQ + (lK ^ (64 * s)));
        }

        // ---- gates (lane x: token x; g = 1, beta = 0 past the end): inclusive
        // prefix products P (G of the chunk) and exclusive suffix products
        // (R[last][t]) by doubling steps within the row of 16 lanes
        const float gt = x < cn ? decay_of(graw, flags) : 1.f;
        const float bt = x < cn ? braw : 0.f;
        float p = gt, sx = gt;
        p *= dpp_row_shr<1>(p);
        p *= dpp_row_shr<2>(p);
        p *= dpp_row_shr<4>(p);
        p *= dpp_row_shr<8>(p);
        sx *= dpp_row_shl<1>(sx);
        sx *= dpp_row_shl<2>(sx);
        sx *= dpp_row_shl<4>(sx);
        sx *= dpp_row_shl<8>(sx);
        const float rlx = dpp_row_shl<1>(sx);      // g_{x+1} ... g_15
        const float glast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), 15));
        if (qd == 0) {
            sg[x] = gt;
            sP[x] = p;
            sb[x] = bt;
            sRl[x] = rlx;
        }

        // ---- K K^T (symmetric: lane (x, qd) holds k_x.k_{4qd+r}) and K Q^T
        // (lane (x, qd): k_{4qd+r}.q_x)
        f32x4 kk = zero4(), kq = zero4();
#pragma unroll
        for (int s = 0; s < NSK; ++s) {
            kk = mfma(fk[s], fk[s], kk);
            kq = mfma(fk[s], fq[s], kq);
        }
        // R[x][j] = g_{j+1} ... g_x for j = 4 qd + r <= x.  With E_x the
        // product over x's aligned quad up to x and Q_b the product over quad
        // b, g_{4qd+4} ... g_x = E_x Q_{qd+1} ... Q_{x/4-1}; the lower columns
        // follow by multiplying in g_{4qd+3}, g_{4qd+2}, g_{4qd+1}.
        f32x4 R;
        {
            const int xq = x & 3, xb = x >> 2;
            float e = gt;
            const float e1 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, e), 0x90, 0xf, 0xf, false));  // quad_perm [0,0,1,2]
            e = xq >= 1 ? e * e1 : e;
            const float e2 = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, e), 0x40, 0xf, 0xf, false));  // quad_perm [0,0,0,1]
            e = xq >= 2 ? e * e2 : e;
            const float q1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, e), 7));
            const float q2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, e), 11));
            float acc = xb > qd ? e : 1.f;          // g over [4 qd + 4, x]
            acc *= (qd < 1 && xb > 1) ? q1 : 1.f;
            acc *= (qd < 2 && xb > 2) ? q2 : 1.f;
            const f32x4 g4 = *reinterpret_cast<const f32x4 *>(sg + 4 * qd);
            R[3] = acc;
            R[2] = (4 * qd + 3 <= x) ? R[3] * g4[3] : 1.f;
            R[1] = (4 * qd + 2 <= x) ? R[2] * g4[2] : 1.f;
            R[0] = (4 * qd + 1 <= x) ? R[1] * g4[1] : 1.f;
        }
        // A (row x, columns 4 qd + r) into the scratch; QKR^T as the operand
        // of the output product: lane (x, qd) holds QKR[x][4 qd + r]
        X4 fqkr;
        {
            f32x4 a, o;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                a[r] = (4 * qd + r < x) ? bt * (R[r] * kk[r]) : 0.f;
                o[r] = (4 * qd + r <= x) ? scale * (R[r] * kq[r]) : 0.f;
            }
            *reinterpret_cast<f32x4 *>(sA + x * LDA + 4 * qd) = a;
            fqkr = cvt4<ET>(o);
        }
        // ---- T = (I + A)^-1 in float32: four lanes per column c, lane part p
        // holding rows p, p + 4, p + 8, p + 12; once x_j is final (in part
        // j % 4) every later row subtracts A[i][j] x_j.  The rows' entries are
        // read four columns at a time, as the sweep reaches them; T is
        // written over A once the sweep is done.
        {
            const int pp = lane & 3, c = ((lane >> 4) << 2) | ((lane >> 2) & 3);
            float sv[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) sv[m] = (pp + 4 * m == c) ? 1.f : 0.f;
#pragma unroll
            for (int j4 = 0; j4 < 4; ++j4) {
                f32x4 ar[4];
#pragma unroll
                for (int m = j4; m < 4; ++m)
                    ar[m] = *reinterpret_cast<const f32x4 *>(sA + (pp + 4 * m) * LDA + 4 * j4);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int j = 4 * j4 + jj;
                    if (j == 15) break;
                    float xj;
                    switch (jj) {
                    case 0: xj = quad_bcast<0>(sv[j4]); break;
                    case 1: xj = quad_bcast<1>(sv[j4]); break;
                    case 2: xj = quad_bcast<2>(sv[j4]); break;
                    default: xj = quad_bcast<3>(sv[j4]); break;
                    }
#pragma unroll
                    for (int m = j4; m < 4; ++m)
                        if (4 * m + 3 > j) sv[m] -= ar[m][jj] * xj;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) sT[(pp + 4 * m) * LDA + c] = sv[m];
        }

        // ---- the state part: M = K S0^T (tiles [token][value]) and
        // Y^T = S0 Q^T ([value][token]) from one 16-bit copy of S0
        wait_loads();                              // this wave's state block
#pragma unroll
        for (int kb = 0; kb < NBK; ++kb) S[kb] = *reinterpret_cast<const f32x4 *>(wbuf + tile_at(kb));
        f32x4 M = zero4(), Y = zero4();
#pragma unroll
        for (int s = 0; s < NSK; ++s) {
            const X8 fs = cat8<ET>(cvt4<ET>(S[2 * s]), cvt4<ET>(S[2 * s + 1]));
            M = mfma(fk[s], fs, M);
            Y = mfma(fs, fq[s], Y);
        }
        // V by tokens (lane (x, qd): tokens 4 qd + r of value column x), exact
        const f32x4 vt = mfma(fv, idV, zero4());
        // right-hand side beta (V - G M) and D = T RHS, float32 products
        const f32x4 G4 = *reinterpret_cast<const f32x4 *>(sP + 4 * qd);
        const f32x4 B4 = *reinterpret_cast<const f32x4 *>(sb + 4 * qd);
        const f32x4 rhs = B4 * (vt - G4 * M);
        const f32x4 D = mma_f32(*reinterpret_cast<const f32x4 *>(sT + x * LDA + 4 * qd), rhs, zero4());

        // ---- y^T = G (S0 Q^T) / sqrt(Dk) + D^T QKR^T; lane (x, qd) holds token
        // x, values 16 vblk + 4 qd .. + 3; the stores go through a buffer
        // resource spanning the chunk's cn valid rows (the rest are dropped)
        Y *= p * scale;
        Y = mfma(cat8<ET>(cvt4<ET>(D), z4), cat8<ET>(fqkr, z4), Y);
        {
            typedef int i32x2 __attribute__((ext_vector_type(2)));
            const unsigned rowb = (unsigned)(Hv * Dv) * (unsigned)sizeof(ET);
            const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(y + (((size_t)b * T + t0) * Hv + hv) * Dv + 16 * vblk), (short)0, (int)(cn * rowb), 0x00020000);
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, cvt4<ET>(Y)), yr,
                                                  (int)(x * rowb + 4 * qd * sizeof(ET)), 0, 0);
        }

        // ---- S^T <- G_last S^T + K^T diag(R[last][:]) D: K^T of key tile kb
        // from half of a K row fragment against the identity
        const X4 dp = cvt4<ET>(D * *reinterpret_cast<const f32x4 *>(sRl + 4 * qd));
#pragma unroll
        for (int kb = 0; kb < NBK; ++kb) {
            const X8 &f = fk[kb >> 1];
            X4 half;
#pragma unroll
            for (int i = 0; i < 4; ++i) half[i] = f[4 * (kb & 1) + i];
            const X4 kt = cvt4<ET>(mfma(cat8<ET>(half, z4), idK, zero4()));
            S[kb] = mfma(cat8<ET>(kt, z4), cat8<ET>(dp, z4), S[kb] * glast);
            if (kb & 1) __builtin_amdgcn_sched_barrier(0);   // two key tiles at a time
        }
    }
    // ---- the state, back through the block: MFMA layout in, full lines out
#pragma unroll
    for (int kb = 0; kb < NBK; ++kb) *reinterpret_cast<f32x4 *>(wbuf + tile_at(kb)) = S[kb];
    float *sout = state_out + srow0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const f32x4 val = *reinterpret_cast<const f32x4 *>(wbuf + 1024 * j + 16 * lane);
        __builtin_nontemporal_store(val, reinterpret_cast<f32x4 *>(sout + blk_row(j) * DK + 4 * blk_unit(j)));
    }
}

}  // namespace gdn
