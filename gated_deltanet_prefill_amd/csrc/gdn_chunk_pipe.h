// gdn_chunk_pipe.h -- the software-pipelined chunk kernel for gfx950:
// 16-bit q/k/v/y, Dk = Dv = 128, chunks of 64 tokens.
//
// The per-chunk work splits into a part that needs the running state and a
// part that does not.  In the compact WY form of a chunk (metaltile-std
// gated_delta_wy.rs page, module notes "Algorithm", steps 4-9: one unit lower
// triangular solve turns the chunk's keys and values into pseudo-keys and
// pseudo-values, and the state then enters only through products with them),
// with the decay products of the ferrox-core gdn_chunk.rs page ("The
// algebra": every ratio of decays is a product of decays):
//
//   A[t][j]   = beta_t R[t][j] k_t.k_j  (j < t),  T = (I + A)^-1
//   W         = T diag(beta G) K,   U = T diag(beta) V         (state free)
//   QKR[t][j] = R[t][j] q_t.k_j / sqrt(Dk)  (j <= t)            (state free)
//   D         = U - W S^T           the true deltas d_t of the chunk
//   y         = G (Q S^T) / sqrt(Dk) + QKR D
//   S        <- G_last S + (diag(Rl) D)^T K,   Rl[t] = R[c-1][t]
//
// One workgroup of eight waves owns one (batch, value head) slot.  Waves 0-3
// (state waves) keep the f32 state in registers, 32 value rows each.  Waves
// 4-7 (prep waves) build the state-free matrices one chunk ahead and stage
// the input two chunks ahead.  Each SIMD holds one wave of each kind, so the
// matrix-core work of one overlaps the vector and LDS work of the other.
// Iteration n has two phases, each closed by a workgroup barrier:
//
//   phase a   state: load V_{n+1}, K_{n+2}, g and beta of n+2; D = U_n +
//                    (-W_n) S^T, Y^T = S Q_n^T; gate products of chunk n+2
//             prep:  K K^T, Q K^T tiles of chunk n+1 -> -A, QKR; diagonal
//                    blocks T_ii
//   phase b   state: Y^T += D^T QKR^T, y, state update; U_{n+1} for its own
//                    value columns (kept in registers for the next chunk)
//             prep:  load Q_{n+2}; W_{n+1} (-W to LDS)
//
// U and W come from blocked forward substitution over 16-token blocks,
//   X_i = T_ii diag(d) B_i + T_ii sum_{j<i} (-A_ij) X_j,
// with B = V, d = beta for U and B = K, d = beta G for W: one 16x16x32
// product per block, [T_ii diag(d) | T_ii] times [B_i ; Z_i].
//
// LDS layouts are swizzled so that the fragment reads and writes of each
// buffer hit distinct banks: in the 256-byte rows of K, Q and -W (token rows,
// keys along the row) the 16-byte unit u of row t sits at u ^ (t % 16); in
// the 128-byte rows of QKR and -A at u ^ ((t / 2) % 8).  In QKR and -A,
// column j = 32 s + 16 h + 4 q + r sits at position 32 s + 8 q + 4 h + r, so
// that the 4-column pieces of blocks 2 s and 2 s + 1 that one lane holds
// are adjacent.
//
// Lane x of value tile vb of state wave w holds value column
//   32 w + 8 (x/4) + 4 vb + x%4,
// so that one lane stores eight consecutive values of a y row at once.  Row
// 4 qd + r of key tile kb = 2 s + h of the state holds key
//   32 s + 8 qd + 4 h + r,
// so that the two tiles of a 32-key step give each lane eight consecutive
// keys: the -W and Q operands of that step are then single 16-byte reads.
#pragma once

#include <type_traits>

#include "gdn_chunk_impl.h"

namespace gdn {

template <typename ET, int DK_, int DV_, int C_>
struct PipeCfg {
    static constexpr int DK = DK_, DV = DV_, C = C_;
    static_assert(sizeof(ET) == 2, "16-bit element types only");
    static_assert(DK == 128 && DV == 128 && C == 64, "the work split is written for this shape");
    static constexpr int NBT = C / 16;      // 16-token blocks
    static constexpr int NBK = DK / 16;     // 16-key blocks
    static constexpr int NSK = DK / 32;     // contraction steps over keys
    static constexpr int NB = 2;            // value tiles per state wave
    // byte offsets
    static constexpr unsigned KBUF = C * DK * 2;         // one chunk of K or Q
    static constexpr unsigned oK = 0;                    // 3 x K
    static constexpr unsigned oQ = oK + 3 * KBUF;        // 2 x Q
    static constexpr unsigned VSL = C * 32 * 2;          // one 32-column V slice
    static constexpr unsigned oV = oQ + 2 * KBUF;        // 4 x V slice [C][32]
    static constexpr unsigned oW = oV + 4 * VSL;         // -W [C][DK]
    static constexpr unsigned CBUF = C * C * 2;          // one C x C matrix
    static constexpr unsigned oQKR = oW + DK * C * 2;    // 2 x QKR [C][C]
    static constexpr unsigned oAn = oQKR + 2 * CBUF;     // -A [C][C]
    static constexpr unsigned LDD = 20;                  // floats per row of Ad
    static constexpr unsigned oAd = oAn + CBUF;          // A diagonal blocks [C][LDD] f32
    // Diagonal blocks of T with a scaled copy: row t holds, for q = 0..3,
    // [T_ii diag(d) columns 4q..4q+3 | T_ii columns 4q..4q+3], d = beta G (TW,
    // for W) or beta (TU, for U); 80-byte rows keep 16-byte reads conflict free.
    static constexpr unsigned LDTT = 40;                 // elements per row of TW / TU
    static constexpr unsigned oTW = oAd + C * LDD * 4;   // [C][LDTT]
    static constexpr unsigned oTU = oTW + C * LDTT * 2;  // [C][LDTT]
    static constexpr unsigned NV = 7 * C;                // floats per gate-vector set
    static constexpr unsigned oVec = oTU + C * LDTT * 2; // 3 x gate vectors
    static constexpr unsigned oGB = oVec + 3 * NV * 4;   // g, beta of two chunks, as loaded
    static constexpr unsigned BYTES = oGB + 2 * 2 * C * 4;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// Gate-vector set of one chunk (floats): beta, g, in-block inclusive prefix
// products P, in-block exclusive suffix products Sfx, G, Rl, block totals.
enum { kVb = 0, kVg = 1, kVP = 2, kVSfx = 3, kVG = 4, kVRl = 5, kVBT = 6 };

// Four 16-bit elements through gfx950's LDS transpose read: lane m of each
// 16-lane group receives element m%4 of the 8-byte pieces addressed by lanes
// m/4 + 4i, i = 0..3.  With lane j addressing row r0 + j/4 at column
// c(j%4) .. +3, lane m receives column c(m/4) + m%4 of rows r0 .. r0+3.
template <typename ET>
__device__ __forceinline__ typename Vec<ET>::x4 ld_tr(const char *smem, unsigned byte) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const s16x4 raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(smem + byte));
    return __builtin_bit_cast(typename Vec<ET>::x4, raw);
}
template <typename ET>
__device__ __forceinline__ typename Vec<ET>::x4 lds4(const char *smem, unsigned byte) {
    return *reinterpret_cast<const typename Vec<ET>::x4 *>(smem + byte);
}
template <typename ET>
__device__ __forceinline__ typename Vec<ET>::x8 lds8(const char *smem, unsigned byte) {
    return *reinterpret_cast<const typename Vec<ET>::x8 *>(smem + byte);
}
template <typename ET>
__device__ __forceinline__ void sts4(char *smem, unsigned byte, typename Vec<ET>::x4 v) {
    *reinterpret_cast<typename Vec<ET>::x4 *>(smem + byte) = v;
}

template <typename ET, int DK, int DV, int C>
__global__ __launch_bounds__(512, 1)
void chunk_pipe_kernel(const ET *__restrict__ q, const ET *__restrict__ k,
                       const ET *__restrict__ v, const float *__restrict__ g,
                       const float *__restrict__ beta, const float *state_in,
                       float *state_out, ET *__restrict__ y,
                       int T, int Hk, int Hv, int xcd_group, float scale, int flags)
{
    using L = PipeCfg<ET, DK, DV, C>;
    using X4 = typename Vec<ET>::x4;
    using X8 = typename Vec<ET>::x8;
    constexpr int NBT = L::NBT, NBK = L::NBK, NSK = L::NSK, NB = L::NB;

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    auto Gv = [&](int i) { return reinterpret_cast<float *>(smem + L::oVec + i * L::NV * 4); };

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int w = wave & 3;                      // state wave index, or prep wave index p
    const bool state_wave = wave < 4;
    // Lane coordinates.  They pass through an empty asm statement at the top
    // of every chunk, so the compiler forms lane-dependent addresses inside
    // the loop (one or two instructions each) instead of holding dozens of
    // precombined addresses in registers across it.
    int lane = tid & 63, x = lane & 15, qd = lane >> 4;

    // Workgroups are dealt round-robin over the 8 XCDs, so workgroups i and
    // i + 8 share an XCD and its L2; with xcd_group = Hv/Hk > 1 they get
    // value heads of the same key head, whose q/k stream is then fetched
    // from HBM once per group.  bid counts slots with the value heads of one
    // key head adjacent, under either head map.
    int bid = blockIdx.x;
    if (xcd_group > 1) {
        const int xcd = bid & 7, kk = bid >> 3;
        const int sib = kk % xcd_group, mm = kk / xcd_group;
        bid = (mm * 8 + xcd) * xcd_group + sib;
    }
    const int b = bid / Hv, hv = value_head_of_rank(bid % Hv, Hk, Hv, flags);
    const int hk = key_head(hv, Hk, Hv, flags);
    const int nchunks = (T + C - 1) / C;

    // ---- lane-dependent LDS byte offsets (see the layout notes above)
    // K/Q/-W row fragment (16 bytes at unit 4s + qd of row 16b + x): ^ 64 s, + 4096 b
    auto f_lKt = [&]() { return (unsigned)(x * 256 + (((qd ^ x) & 15) << 4)); };
    // K transpose read, rows r0 + r4, columns 16 kb + 4 (x%4) ..: ^ 32 kb, + 256 r0
    auto f_lKtr = [&]() {
        const int r4 = 4 * qd + (x >> 2);
        return (unsigned)(r4 * 256 + (((((x >> 1) & 1) ^ r4) & 15) << 4) + ((x & 1) << 3));
    };
    // K transpose read for the state update, rows r0 + r4, keys 32 s + 4 h +
    // 8 (x%4) .. +3 (lane x then receives key 32 s + 4 h + 8 (x/4) + x%4):
    // ^ 64 s, + 8 h, + 256 r0
    auto f_lKu = [&]() {
        const int r4 = 4 * qd + (x >> 2);
        return (unsigned)(r4 * 256 + ((((x & 3) ^ r4) & 15) << 4));
    };
    // -W, prep side: token 16 ib + x, keys 16 c + 4 qd .. + 3 (8 bytes) of
    // key tile c: ^ 32 c, + 4096 ib
    auto f_lWp = [&]() { return (unsigned)(x * 256 + ((((qd >> 1) ^ x) & 15) << 4) + 8 * (qd & 1)); };
    // QKR / -A rows 16 tb + x, the 4 columns 16 jb + 4 qd ..:
    //   (this ^ 64 (jb/2)) + 8 (jb%2) + 2048 tb;
    // the 8 columns of blocks 2 s, 2 s + 1 that lane (x, qd) holds: ^ 64 s
    auto f_lA = [&]() { return (unsigned)(x * 128 + (((qd ^ (x >> 1)) & 7) << 4)); };
    auto aoff = [](unsigned lA, int jb, int tb) { return (lA ^ (64 * (jb >> 1))) + 8 * (jb & 1) + 2048 * tb; };
    // V slice of state wave w: transpose read rows 16 ib + r4, permuted
    // columns 8 (m/4) + 4 vb + m%4: + 8 vb + 1024 ib
    auto f_lVs = [&]() { return (unsigned)((4 * qd + (x >> 2)) * 64 + (x & 3) * 16); };

    // ---------------- prep waves: global -> LDS loads ----------------
    // Chunks of K, Q and V go from global memory straight into LDS
    // (global_load_lds_dwordx4: lane l of the wave writes the 16 bytes at
    // 16 l of a 1 KB block), so no staging registers are held across the
    // loop.  The state waves load K and V in phase a, the prep waves Q in
    // phase b (when its buffer is free); wave w of either kind fills K/Q rows
    // 16 w .. 16 w + 15, state wave w the V columns 32 w .. 32 w + 31 that it
    // reads itself.  The swizzle of K and Q is applied on the source side: the lane
    // that fills position u' of row r fetches unit u' ^ (r % 16) of that row.
    // Rows past the end of the sequence fetch the last row again; with
    // g = 1 and beta = 0 there, those rows add nothing (A, W, U and D vanish
    // on them, and their y rows are not stored).
    const size_t kstride = (size_t)Hk * DK, vstride = (size_t)Hv * DV;
    const ET *kbase = k + ((size_t)b * T * Hk + hk) * DK;
    const ET *qbase = q + ((size_t)b * T * Hk + hk) * DK;
    const ET *vbase = v + ((size_t)b * T * Hv + hv) * DV + w * 32;
    const float *gbase = g + (size_t)b * T * Hv + hv;
    const float *bbase = beta + (size_t)b * T * Hv + hv;
    // K/Q: wave w fills rows r = 16 w + 4 i + l/16 (i = 0..3), lane l
    // fetching unit (l%16) ^ (r%16) = ((l%16) ^ (l/16)) ^ 4i; as an element
    // offset (kstride is a multiple of 128): (okq0 ^ 32 i) + 4 i kstride.
    // V: this wave's 32 columns, rows 16 i + l/4, 8 elements at 8 (l%4):
    // ov0 + 16 i vstride.
    auto f_okq0 = [&]() {
        return (unsigned)((16 * w + qd) * kstride + 8 * ((lane & 15) ^ qd));
    };
    auto f_ov0 = [&]() { return (unsigned)((lane >> 2) * vstride + 8 * (lane & 3)); };
    // One 1 KB block: lane l fetches the 16 bytes at src + off (off in
    // bytes, per lane; src uniform) into LDS at lds_byte + 16 l.  Written as
    // inline assembly: the compiler would otherwise make the wave wait for
    // the whole transfer before its next LDS read.  Completion is awaited
    // explicitly (s_waitcnt vmcnt) before the barrier that publishes it.
    const unsigned lds_base = (unsigned)(uintptr_t)((__attribute__((address_space(3))) char *)smem);
    auto g2lds = [&](const ET *src, unsigned off, unsigned lds_byte) {
        const unsigned la = __builtin_amdgcn_readfirstlane(lds_base + lds_byte);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                     :: "v"(off), "s"(src), "s"(la) : "memory", "m0");
#pragma clang diagnostic pop
    };
    // block i (rows 16 w + 4 i ..) of this wave's share of a K or Q chunk
    auto issue_kq_blk = [&](const ET *base, unsigned dst, int c, int i) {
        const int t0 = c * C;
        const ET *src = base + (size_t)t0 * kstride;
        if (t0 + C <= T) {
            g2lds(src, 2 * ((f_okq0() ^ (32 * i)) + 4 * i * (unsigned)kstride), dst + 4096 * w + 1024 * i);
        } else {
            const int r = 16 * w + 4 * i + (lane >> 4);
            g2lds(src, 2 * (unsigned)(min(r, T - t0 - 1) * kstride + 8 * ((lane & 15) ^ (r & 15))), dst + 4096 * w + 1024 * i);
        }
    };
    auto issue_kq = [&](const ET *base, unsigned dst, int c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) issue_kq_blk(base, dst, c, i);
    };
    auto issue_k = [&](int c) { issue_kq(kbase, L::oK + (c % 3) * L::KBUF, c); };
    auto issue_q = [&](int c) { issue_kq(qbase, L::oQ + (c & 1) * L::KBUF, c); };
    auto issue_v = [&](int c) {
        const int t0 = c * C;
        const ET *src = vbase + (size_t)t0 * vstride;
        const unsigned dst = L::oV + w * L::VSL;
        if (t0 + C <= T) {
            const unsigned o0 = f_ov0();
#pragma unroll
            for (int i = 0; i < 4; ++i) g2lds(src, 2 * (o0 + 16 * i * (unsigned)vstride), dst + 1024 * i);
        } else {
            const int last = T - t0 - 1;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                g2lds(src, 2 * (unsigned)(min(16 * i + (lane >> 2), last) * vstride + 8 * (lane & 3)), dst + 1024 * i);
        }
    };
    // g and beta of chunk c into LDS (wave 0 of a kind; lane = token, rows
    // past the end read the last row)
    auto load_gb = [&](int c) {
        if (w == 0) {
            const int t0 = c * C;
            const unsigned off = 4 * (unsigned)(min(lane, T - t0 - 1) * Hv);
            const float *gc = gbase + (size_t)t0 * Hv, *bc = bbase + (size_t)t0 * Hv;
            const unsigned gbo = L::oGB + (unsigned)(c & 1) * 2 * C * 4;
            const unsigned lg = __builtin_amdgcn_readfirstlane(lds_base + gbo);
            const unsigned lb = __builtin_amdgcn_readfirstlane(lds_base + gbo + C * 4);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
            asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                         :: "v"(off), "s"(gc), "s"(lg) : "memory", "m0");
            asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                         :: "v"(off), "s"(bc), "s"(lb) : "memory", "m0");
#pragma clang diagnostic pop
        }
    };
    // Gate products of chunk c (wave 0 of a kind, lane t holding g_t; g = 1 past
    // the end): within each 16-token block (one DPP row) the inclusive prefix
    // products P and the inclusive suffix products by four doubling steps;
    // the exclusive suffix Sfx; block totals; G[t] = P[t] x totals of the
    // earlier blocks; Rl[t] = Sfx[t] x totals of the later blocks.
    // `wait`: the loads of chunk c may still be in flight (else they were
    // awaited before an earlier barrier).
    auto scan_gates = [&](int c, bool wait) {
        if (w == 0) {
            if (wait) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            const float *gb = reinterpret_cast<const float *>(smem + L::oGB + (c & 1) * 2 * C * 4);
            const float rg = gb[lane];
            const float rb = gb[C + lane];
            const int cn = min(C, T - c * C);
            float *gv = Gv(c % 3);
            const float gt = lane < cn ? decay_of(rg, flags) : 1.f;
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
                if (lane == bb) gv[kVBT * C + bb] = tot;
            }
            gv[kVb * C + lane] = lane < cn ? rb : 0.f;
            gv[kVg * C + lane] = gt;
            gv[kVP * C + lane] = p;
            gv[kVSfx * C + lane] = sfx;
            gv[kVG * C + lane] = gpre;
            gv[kVRl * C + lane] = rl;
        }
    };
    static_assert(C == 64, "one lane per token in the gate scans");

    // Blocked forward substitution for two 16-column tiles of
    // X = T diag(d) B: bfrag(ib, cb) is the 16-bit fragment of B (lane x =
    // column, rows 16 ib + 4 qd + r), tbuf holds [T_ii diag(d) | T_ii].
    //   Z_i = sum_{j<i} (-A_ij) X_j,  X_i = [T_ii diag(d) | T_ii] [B_i ; Z_i];
    // emit(ib, cb, X_i f32, the two operands).  Returns the 16-bit blocks in Xf.
    auto substitute = [&](unsigned lA, unsigned tbuf, X4 (&Xf)[NBT][2], auto bfrag, auto emit) {
#pragma unroll
        for (int ib = 0; ib < NBT; ++ib) {
            f32x4 Z[2] = {zero4(), zero4()};
            // -A_ij X_j over j < ib, two blocks per 16x16x32 product; an odd
            // last block is paired with the diagonal block and a zero X.  Every
            // product into Z has the same shape: on gfx950 a 16x16x32 result
            // fed to a 16x16x16 accumulator (or back) needs five independent
            // issue slots in between, which the compiler does not always
            // insert; same-shape chains are interlocked by the hardware.
#pragma unroll
            for (int j = 0; j < ib; j += 2) {
                const X8 fa = lds8<ET>(smem, L::oAn + (lA ^ (32 * j)) + 2048 * ib);
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
                    Z[cb] = mfma(fa, cat8<ET>(Xf[j][cb], j + 1 < ib ? Xf[j + 1][cb] : X4{}), Z[cb]);
            }
            const X8 ft = lds8<ET>(smem, tbuf + (16 * ib + x) * L::LDTT * 2 + 16 * qd);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
                const X8 bz = cat8<ET>(bfrag(ib, cb), cvt4<ET>(Z[cb]));
                const f32x4 r = mfma(ft, bz, zero4());
                Xf[ib][cb] = cvt4<ET>(r);
                emit(ib, cb, r, ft, bz);
            }
        }
    };

    // ---------------- state waves: the state ----------------
    // S[kb][vb]: S^T tile, rows = keys kcol(kb, qd) + r, columns = values.
    f32x4 S[NBK][NB];
    X4 Uf[NBT][NB];                              // U of the next chunk (own value columns)
    const size_t sbase = ((size_t)b * Hv + hv) * DV * DK;
    auto vcol = [&](int vb, int xx) { return 32 * w + 8 * (xx >> 2) + 4 * vb + (xx & 3); };
    auto kcol = [&](int kb, int q4) { return 32 * (kb >> 1) + 8 * q4 + 4 * (kb & 1); };

    // QKR blocks above the diagonal are never written: zero both buffers once.
    auto zero_qkr = [&]() {
        for (int i = tid; i < (int)(2 * L::CBUF / 16); i += 512)
            reinterpret_cast<uint4 *>(smem + L::oQKR)[i] = zero_u4();
    };

    // The two kinds of waves run loops of their own with the same barriers
    // (two per chunk), so that each loop carries only its own registers; the
    // first chunk step of the state waves and the last of the prep waves,
    // which do only part of the work, are taken out of the loops.
    if (state_wave) {
        if (nchunks > 0) {
            issue_k(0);
            issue_q(0);
        }
        if (nchunks > 1) load_gb(1);                 // awaited before the first barrier
        {
            // rows of zeros (stride 0) when there is no initial state
            gfloat *sin = state_in ? (gfloat *)state_in + sbase : (gfloat *)kZeroRow;
            const size_t rstride = state_in ? DK : 0;
#pragma unroll
            for (int vb = 0; vb < NB; ++vb)
#pragma unroll
                for (int kb = 0; kb < NBK; ++kb)
                    S[kb][vb] = *reinterpret_cast<gf32x4 *>(sin + (size_t)vcol(vb, x) * rstride + kcol(kb, qd));
        }
#pragma unroll
        for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) asm volatile("" : "+v"(S[kb][vb]));
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        zero_qkr();
        lds_barrier();
        // K, g and beta of chunk n+2 and V of chunk n+1, all awaited before the
        // phase-a barrier (V is read in phase b, K and the gate products by the
        // prep waves next chunk)
        // The gates are loaded one chunk earlier than K (two buffers), so the
        // scan of chunk n+2 at the end of phase a reads loads that completed
        // before the previous barrier instead of waiting for this phase's.
        auto issue_inputs = [&](int n) {
            if (n + 2 < nchunks) issue_k(n + 2);
            if (n + 3 < nchunks) load_gb(n + 3);
            if (n + 1 < nchunks) issue_v(n + 1);
        };
        auto end_phase_a = [&](int n) {
            if (n + 2 < nchunks) scan_gates(n + 2, false);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_barrier();
        };
        // ---- U = T diag(beta) V of chunk n+1 for this wave's value columns,
        // V read with the permuted columns of the value tiles (after the last
        // chunk this reads stale LDS; its result is not used)
        auto compute_u = [&]() {
            const unsigned lA = f_lA(), vsl = L::oV + w * L::VSL + f_lVs();
            X4 Un[NBT][NB];
            substitute(lA, L::oTU, Un,
                [&](int ib, int vb) { return ld_tr<ET>(smem, vsl + 8 * vb + 1024 * ib); },
                [&](int, int, f32x4, X8, X8) {});
#pragma unroll
            for (int tb = 0; tb < NBT; ++tb)
#pragma unroll
                for (int vb = 0; vb < NB; ++vb) Uf[tb][vb] = Un[tb][vb];
        };
        // chunk step -1: inputs of chunks 0 (V) and 1 (K, gates), U of chunk 0
        issue_inputs(-1);
        end_phase_a(-1);
        compute_u();
        lds_barrier();
        for (int n = 0; n < nchunks; ++n) {
            asm volatile("" : "+v"(lane), "+v"(x), "+v"(qd));
            // ================= state waves =================
            const unsigned lKt = f_lKt(), lKu = f_lKu(), lA = f_lA();
            issue_inputs(n);
            f32x4 D[NBT][NB], Y[NB][NBT];
            {
                // ---- phase a: D = U + (-W) S^T, Y^T = S Q^T
                const unsigned qb = L::oQ + (n & 1) * L::KBUF;
                const float *gv = Gv(n % 3);
#pragma unroll
                for (int tb = 0; tb < NBT; ++tb)
#pragma unroll
                    for (int vb = 0; vb < NB; ++vb) {
                        D[tb][vb] = to_f32x4<ET>(Uf[tb][vb]);
                        Y[vb][tb] = zero4();
                    }
#pragma unroll
                for (int s = 0; s < NSK; ++s) {
                    // keys 32 s + 8 qd + (0..7) in lane (x, qd) of every operand
                    X8 fs[NB];
#pragma unroll
                    for (int vb = 0; vb < NB; ++vb)
                        fs[vb] = cat8<ET>(cvt4<ET>(S[2 * s][vb]), cvt4<ET>(S[2 * s + 1][vb]));
#pragma unroll
                    for (int tb = 0; tb < NBT; ++tb) {
                        const unsigned lo = (lKt ^ (64 * s)) + 4096 * tb;
                        const X8 fw = lds8<ET>(smem, L::oW + lo);
                        const X8 fq = lds8<ET>(smem, qb + lo);
#pragma unroll
                        for (int vb = 0; vb < NB; ++vb) {
                            D[tb][vb] = mfma(fw, fs[vb], D[tb][vb]);
                            Y[vb][tb] = mfma(fs[vb], fq, Y[vb][tb]);
                        }
                    }
                }
#pragma unroll
                for (int tb = 0; tb < NBT; ++tb) {
                    const float gt = gv[kVG * C + 16 * tb + x] * scale;
#pragma unroll
                    for (int vb = 0; vb < NB; ++vb) Y[vb][tb] *= gt;
                }
            }
            end_phase_a(n);
            {
                // ---- phase b: Y^T += D^T QKR^T, y, S^T <- G_last S^T + K^T diag(Rl) D
                const int t0 = n * C, cn = min(C, T - t0);
                const unsigned kb_ = L::oK + (n % 3) * L::KBUF, rb_ = L::oQKR + (n & 1) * L::CBUF;
                const float *gv = Gv(n % 3);
                X4 Df[NBT][NB];
#pragma unroll
                for (int tb = 0; tb < NBT; ++tb)
#pragma unroll
                    for (int vb = 0; vb < NB; ++vb) Df[tb][vb] = cvt4<ET>(D[tb][vb]);
#pragma unroll
                for (int tb = 0; tb < NBT; ++tb) {
                    // QKR is zero above the diagonal blocks: pair blocks (0,1), (2,3)
#pragma unroll
                    for (int s = 0; 2 * s <= tb; ++s) {
                        const X8 fr = lds8<ET>(smem, rb_ + (lA ^ (64 * s)) + 2048 * tb);
#pragma unroll
                        for (int vb = 0; vb < NB; ++vb)
                            Y[vb][tb] = mfma(cat8<ET>(Df[2 * s][vb], Df[2 * s + 1][vb]), fr, Y[vb][tb]);
                    }
                }
                // y: lane (x, qd) holds token 16 tb + x, values 32 w + 8 qd + (0..7).
                // The stores go through a buffer resource that spans the chunk's
                // cn valid token rows: the hardware drops those past the end of
                // the sequence, with no branch around the stores.
                {
                    typedef int i32x4 __attribute__((ext_vector_type(4)));
                    const unsigned rowb = (unsigned)(Hv * DV) * (unsigned)sizeof(ET);
                    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
                        (void *)(y + (((size_t)b * T + t0) * Hv + hv) * DV), (short)0, (int)(cn * rowb), 0x00020000);
#pragma unroll
                    for (int tb = 0; tb < NBT; ++tb)
                        __builtin_amdgcn_raw_buffer_store_b128(
                            __builtin_bit_cast(i32x4, cat8<ET>(cvt4<ET>(Y[0][tb]), cvt4<ET>(Y[1][tb]))), yr,
                            (int)((16 * tb + x) * rowb + (32 * w + 8 * qd) * sizeof(ET)), 0, 0);
                }
                X4 Dp[NBT][NB];
#pragma unroll
                for (int tb = 0; tb < NBT; ++tb) {
                    const f32x4 rl = *reinterpret_cast<const f32x4 *>(gv + kVRl * C + 16 * tb + 4 * qd);
#pragma unroll
                    for (int vb = 0; vb < NB; ++vb) Dp[tb][vb] = cvt4<ET>(D[tb][vb] * rl);
                }
                const float glast = gv[kVG * C + C - 1];
#pragma unroll
                for (int kb = 0; kb < NBK; ++kb) {
                    X8 fk[2];
#pragma unroll
                    for (int s = 0; s < 2; ++s) {
                        const unsigned ka = kb_ + (lKu ^ (64 * (kb >> 1))) + 8 * (kb & 1) + 256 * 32 * s;
                        fk[s] = cat8<ET>(ld_tr<ET>(smem, ka), ld_tr<ET>(smem, ka + 256 * 16));
                    }
#pragma unroll
                    for (int vb = 0; vb < NB; ++vb) S[kb][vb] *= glast;
#pragma unroll
                    for (int s = 0; s < 2; ++s)
#pragma unroll
                        for (int vb = 0; vb < NB; ++vb)
                            S[kb][vb] = mfma(fk[s], cat8<ET>(Dp[2 * s][vb], Dp[2 * s + 1][vb]), S[kb][vb]);
                }
                // in the same block as the work above, so that the scheduler can
                // interleave the chains
                compute_u();
            }
            lds_barrier();
        }
        // ---- the state, written once
#pragma unroll
        for (int vb = 0; vb < NB; ++vb)
#pragma unroll
            for (int kb = 0; kb < NBK; ++kb)
                *reinterpret_cast<f32x4 *>(state_out + sbase + (size_t)vcol(vb, x) * DK + kcol(kb, qd)) = S[kb][vb];
    } else {
        if (nchunks > 0) {
            // gates of chunk 0 (its V comes in the first iteration)
            load_gb(0);
            scan_gates(0, true);
        }
        zero_qkr();
        lds_barrier();
        // chunk m = n + 1 of every step but the last, which only keeps the two
        // barriers of the state waves' last chunk
        for (int n = -1; n + 1 < nchunks; ++n) {
            asm volatile("" : "+v"(lane), "+v"(x), "+v"(qd));
            // ================= prep waves =================
            const int m = n + 1, p = w;
            const unsigned lKt = f_lKt(), lKtr = f_lKtr(), lWp = f_lWp(), lA = f_lA();
            {
                // ---- tiles of K K^T and Q K^T of chunk m; tile (jb, tb) has rows
                // j = 16 jb + 4 qd + r and column t = 16 tb + x.  Prep wave p takes
                // the diagonal tiles of block p and three of the twelve below it,
                // chosen so that its own K_p (and Q_p) serve as operands:
                //   wave 0: QK(0,2) KK(0,3) QK(0,3)   wave 1: KK(0,1) QK(0,1) QK(1,3)
                //   wave 2: KK(1,2) QK(1,2) KK(0,2)   wave 3: KK(2,3) QK(2,3) KK(1,3)
                // (4, 4, 4 and 5 fragment reads per 32-key step instead of 8).
                const unsigned kbm = L::oK + (m % 3) * L::KBUF, qbm = L::oQ + (m & 1) * L::KBUF;
                const unsigned rbm = L::oQKR + (m & 1) * L::CBUF;
                const float *gv = Gv(m % 3);
                // tile i of wave p: block row jb, block column tb, from Q or K,
                // packed two bits per field at 6 p + 2 i (one bit at 3 p + i for Q)
                constexpr unsigned kJB = 0x685400u, kTB = 0xfead7eu, kQB = 0x4b5u;
                int tj[3], tt[3], tq[3];
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                    tj[i] = (kJB >> (6 * p + 2 * i)) & 3;
                    tt[i] = (kTB >> (6 * p + 2 * i)) & 3;
                    tq[i] = (kQB >> (3 * p + i)) & 1;
                }
                // gate values of the apply steps below, read before the tile
                // products so that their LDS latency overlaps them
                const int td = 16 * p + x;
                const float dg_b = gv[kVb * C + td];
                const float dg_g = gv[kVg * C + td];
                const f32x4 dg_g4 = *reinterpret_cast<const f32x4 *>(gv + kVg * C + 16 * p + 4 * qd);
                const f32x4 od_tot = *reinterpret_cast<const f32x4 *>(gv + kVBT * C);
                float od_P[3], od_b[3];
                f32x4 od_S[3];
#pragma unroll
                for (int i = 0; i < 3; ++i) {
                    const int t = 16 * tt[i] + x;
                    od_P[i] = gv[kVP * C + t];
                    od_b[i] = gv[kVb * C + t];
                    od_S[i] = *reinterpret_cast<const f32x4 *>(gv + kVSfx * C + 16 * tj[i] + 4 * qd);
                }
                f32x4 acc[5];
#pragma unroll
                for (int i = 0; i < 5; ++i) acc[i] = zero4();
                // acc[2 + i] = tile i: A operand K_jb, B operand K_tb or Q_tb
                auto tiles = [&](auto P) {
                    constexpr int pc = decltype(P)::value;
#pragma unroll
                    for (int s = 0; s < NSK; ++s) {
                        const unsigned lo = lKt ^ (64 * s);
                        const X8 kp = lds8<ET>(smem, kbm + lo + 4096 * pc);
                        const X8 qp = lds8<ET>(smem, qbm + lo + 4096 * pc);
                        acc[0] = mfma(kp, kp, acc[0]);
                        acc[1] = mfma(kp, qp, acc[1]);
                        if constexpr (pc == 0) {
                            const X8 q2 = lds8<ET>(smem, qbm + lo + 4096 * 2);
                            const X8 k3 = lds8<ET>(smem, kbm + lo + 4096 * 3);
                            const X8 q3 = lds8<ET>(smem, qbm + lo + 4096 * 3);
                            acc[2] = mfma(kp, q2, acc[2]);
                            acc[3] = mfma(kp, k3, acc[3]);
                            acc[4] = mfma(kp, q3, acc[4]);
                        } else if constexpr (pc == 1) {
                            const X8 k0 = lds8<ET>(smem, kbm + lo);
                            const X8 q3 = lds8<ET>(smem, qbm + lo + 4096 * 3);
                            acc[2] = mfma(k0, kp, acc[2]);
                            acc[3] = mfma(k0, qp, acc[3]);
                            acc[4] = mfma(kp, q3, acc[4]);
                        } else {
                            const X8 a1 = lds8<ET>(smem, kbm + lo + 4096 * (pc - 1));
                            const X8 a2 = lds8<ET>(smem, kbm + lo + 4096 * (pc - 2));
                            acc[2] = mfma(a1, kp, acc[2]);
                            acc[3] = mfma(a1, qp, acc[3]);
                            acc[4] = mfma(a2, kp, acc[4]);
                        }
                    }
                };
                switch (p) {
                case 0: tiles(std::integral_constant<int, 0>{}); break;
                case 1: tiles(std::integral_constant<int, 1>{}); break;
                case 2: tiles(std::integral_constant<int, 2>{}); break;
                default: tiles(std::integral_constant<int, 3>{}); break;
                }
                // ---- diagonal block p: R[t][j] = g_{j+1} ... g_t inside the block;
                // h = product of g over local indices [4 qd + 4, x] by an
                // inclusive scan along the 16 lanes x of a DPP row.
                {
                    const int t = td;
                    const float bt = dg_b;
                    float h = (x >= 4 * qd + 4) ? dg_g : 1.f;
                    h *= dpp_row_shr<1>(h);
                    h *= dpp_row_shr<2>(h);
                    h *= dpp_row_shr<4>(h);
                    h *= dpp_row_shr<8>(h);
                    const f32x4 g4 = dg_g4;
                    f32x4 R;
                    R[3] = h;
                    R[2] = (4 * qd + 3 <= x) ? R[3] * g4[3] : 1.f;
                    R[1] = (4 * qd + 2 <= x) ? R[2] * g4[2] : 1.f;
                    R[0] = (4 * qd + 1 <= x) ? R[1] * g4[1] : 1.f;
                    f32x4 a, o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        a[r] = (4 * qd + r < x) ? bt * (R[r] * acc[0][r]) : 0.f;
                        o[r] = (4 * qd + r <= x) ? scale * (R[r] * acc[1][r]) : 0.f;
                    }
                    const unsigned ao = aoff(lA, p, p);
                    sts4<ET>(smem, L::oAn + ao, cvt4<ET>(-a));
                    sts4<ET>(smem, rbm + ao, cvt4<ET>(o));
                    *reinterpret_cast<f32x4 *>(smem + L::oAd + (t * L::LDD + 4 * qd) * 4) = a;
                }
                // ---- tiles below the diagonal: R[t][j] = P[t] x (totals of the
                // blocks strictly between) x Sfx[j]
                {
                    const f32x4 tot = od_tot;
#pragma unroll
                    for (int i = 0; i < 3; ++i) {
                        const int jb = tj[i], tb = tt[i];
                        float mf = od_P[i];
#pragma unroll
                        for (int bb = 1; bb < NBT - 1; ++bb) mf *= (bb > jb && bb < tb) ? tot[bb] : 1.f;
                        const f32x4 R = od_S[i] * mf;
                        const unsigned ao = aoff(lA, jb, tb);
                        if (tq[i]) sts4<ET>(smem, rbm + ao, cvt4<ET>(R * acc[2 + i] * scale));
                        else sts4<ET>(smem, L::oAn + ao, cvt4<ET>(R * acc[2 + i] * (-od_b[i])));
                    }
                }
                // ---- T_pp = (I + A_pp)^-1 by f32 forward substitution: four
                // lanes per column c, lane part pt holding rows pt, pt+4, pt+8,
                // pt+12.  Column sweep: once x_j is final (it sits in part j%4),
                // every later row subtracts A[i][j] x_j.  The rows come from this
                // wave's own writes above (LDS keeps a wave's accesses in order).
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                {
                    const int base = 16 * p;
                    const int pt = lane & 3, c = ((lane >> 4) << 2) | ((lane >> 2) & 3);
                    const float *ad = reinterpret_cast<const float *>(smem + L::oAd);
                    f32x4 arow[4][4];
#pragma unroll
                    for (int mm = 0; mm < 4; ++mm)
#pragma unroll
                        for (int j4 = 0; j4 < 4; ++j4)
                            arow[mm][j4] = *reinterpret_cast<const f32x4 *>(ad + (base + pt + 4 * mm) * L::LDD + 4 * j4);
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
                    // column c of T_pp belongs to token 16 p + c: TW scales it by
                    // beta G, TU by beta
                    const float bc = gv[kVb * C + base + c], bgc = bc * gv[kVG * C + base + c];
                    ET *tw = reinterpret_cast<ET *>(smem + L::oTW), *tu = reinterpret_cast<ET *>(smem + L::oTU);
                    const int col = 8 * (c >> 2) + (c & 3);
#pragma unroll
                    for (int mm = 0; mm < 4; ++mm) {
                        const int o = (base + pt + 4 * mm) * L::LDTT + col;
                        const ET tv = from_f32<ET>(sv[mm]);
                        tw[o] = from_f32<ET>(sv[mm] * bgc);
                        tw[o + 4] = tv;
                        tu[o] = from_f32<ET>(sv[mm] * bc);
                        tu[o + 4] = tv;
                    }
                }
            }
            lds_barrier();
            // Q of chunk m + 1 (its buffer held Q of chunk m - 1, read in phase
            // a), issued at once: its transfer then has the whole phase
            if (m + 1 < nchunks) issue_q(m + 1);
            {
                // ---- W = T diag(beta G) K of chunk m, key columns 32 p + 16 cb + x
                const unsigned kbm = L::oK + (m % 3) * L::KBUF;
                const float *gv = Gv(m % 3);
                X4 Wf[NBT][2];
                substitute(lA, L::oTW, Wf,
                    [&](int ib, int cb) { return ld_tr<ET>(smem, kbm + (lKtr ^ (32 * (2 * p + cb))) + 4096 * ib); },
                    // the same product with the operands swapped gives the block
                    // transposed, lane (x, qd) holding keys 4 qd .. + 3 of token
                    // 16 ib + x: one 8-byte write into the token rows of -W
                    [&](int ib, int cb, f32x4, X8 ft, X8 bz) {
                        sts4<ET>(smem, L::oW + (lWp ^ (32 * (2 * p + cb))) + 4096 * ib, cvt4<ET>(-mfma(bz, ft, zero4())));
                    });
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_barrier();
        }
        lds_barrier();
        lds_barrier();
    }
}

}  // namespace gdn
