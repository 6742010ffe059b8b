// gdn_chunk_wy.h -- the pipelined chunk kernel for gfx950: 16-bit q/k/v/y,
// Dk = Dv = 128, chunks of 64 tokens, the chunk's triangular system inverted
// in float32.
//
// Per chunk, in the per-row form of the ferrox-core gdn_chunk.rs page ("The
// algebra": unrolled over a chunk, the state enters only through its
// products with the chunk's keys and queries, the deltas follow from a C x C
// triangular system, and every ratio of decays is a product of decays):
//
//   A[t][j]   = beta_t R[t][j] k_t.k_j  (j < t),   T = (I + A)^-1
//   M         = K S^T                 the state against the chunk's keys
//   E         = V - diag(G) M
//   D         = T diag(beta) E        the true deltas d_t of the chunk
//   QKR[t][j] = R[t][j] q_t.k_j / sqrt(Dk)  (j <= t)
//   y         = G (Q S^T) / sqrt(Dk) + QKR D
//   S        <- G_last S + (diag(Rl) D)^T K,   Rl[t] = R[c-1][t]
//
// (I + A) D = diag(beta) E is the same system that the compact WY form of
// the metaltile-std gated_delta_wy.rs page ("Algorithm", steps 4-9) solves
// for its pseudo-keys and pseudo-values; here its right-hand side carries the
// state, so the inverse T is applied once, to E.
//
// The triangular system is solved in float32 (the metaltile page's
// "Numerical precision": float32 is the floor for the solves):
//
//  * the 16x16 diagonal blocks T_ii = (I + A_ii)^-1 by float32 forward
//    substitution on the vector ALUs;
//  * the blocks below the diagonal column by column,
//      T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj,
//    every product a float32 matrix-core product (v_mfma_f32_16x16x4_f32:
//    float32 operands, products and accumulation);
//  * D as the product of T diag(beta), carried as a two-term expansion
//    T_h + T_l (16 significant bits, relative error <= 2^-17), with E
//    rounded once to 16 bits: [T_h | T_l] times [E ; E] is one 16x16x32 MFMA
//    per block.
//
// One workgroup of eight waves owns one (batch, value head) slot.  Waves 0-3
// (state waves) keep the float32 state in registers, 32 value rows each;
// waves 4-7 (prep waves) build T one chunk ahead and load the inputs.  Each
// SIMD holds one wave of each kind.  Iteration n has two phases, each closed
// by a workgroup barrier:
//
//   phase a  state: Y = Q_n S^T and M = K_n S^T from one 16-bit copy of the
//                   state, the Q K^T tiles of chunk n -> QKR, E = V - G M;
//                   load K_{n+2}
//            prep:  the last blocks of T_n below the diagonal; K K^T tiles
//                   of chunk n+1 -> A, the diagonal inverses T_ii
//   phase b  state: D = T_n diag(beta) E, y = G Y / sqrt(Dk) + QKR D, state
//                   update
//            prep:  the first blocks of T_{n+1} below the diagonal; gate
//                   products of chunk n+2; load Q_{n+1}, V_{n+1}
//
// The decay ratios of the four diagonal 16x16 tiles, which the prep waves
// form for their K K^T tiles, are kept in LDS (lane order, two chunks by
// parity) for the Q K^T diagonal tiles of the same chunk.
//
// LDS layouts.  K and Q have 256-byte token rows (keys along the row); the
// 16-byte unit u of row t sits at u ^ kq_swz(t).  QKR has 128-byte rows, unit
// u of row t at u ^ ((t / 2) % 8), and column j = 32 s + 16 h + 4 q + r at
// position 32 s + 8 q + 4 h + r.  Float32 16x16 blocks (A below the
// diagonal, T_ii by rows and by columns) have 64-byte rows, unit u of row r
// at u ^ ((r / 2) % 4).  The expansion of T diag(beta) is stored block by
// block transposed (row c holds column c of the block), 32-byte rows with
// the 8-byte piece s of row c at s ^ (2 (c / 8)), and read back as row
// fragments with gfx950's LDS transpose load.
//
// Lane x of value tile vb of state wave w holds value column
//   32 w + 8 (x/4) + 4 vb + x%4;
// row 4 qd + r of key tile kb = 2 s + h of the state holds key
//   32 s + 8 qd + 4 h + r,
// so that the K and Q row fragments of a 32-key step are single 16-byte
// reads of eight consecutive keys.
#pragma once

#include <type_traits>

#include "gdn_chunk_impl.h"

namespace gdn {

template <typename ET, int NSW_>
struct WyCfg {
    static_assert(sizeof(ET) == 2, "16-bit element types only");
    static_assert(NSW_ == 4 || NSW_ == 2, "four or two state waves");
    static constexpr int C = 64, DK = 128, DV = 128;
    static constexpr int NSW = NSW_;          // state waves
    static constexpr int NW = NSW == 4 ? 8 : 12;          // waves per workgroup
    static constexpr int NP = NW - NSW;       // prep waves
    static constexpr int NB = NSW == 4 ? 2 : 1;           // value tiles per state wave
    static constexpr int ROWS = 16 * NB * NSW;            // value rows per workgroup
    static constexpr int NSPLIT = DV / ROWS;              // workgroups per slot
    static constexpr int NBT = C / 16;        // 16-token blocks
    static constexpr int NBK = DK / 16;       // 16-key blocks
    static constexpr int NSK = DK / 32;       // contraction steps over keys
    static constexpr unsigned KBUF = C * DK * 2;          // one chunk of K or Q
    static constexpr unsigned oK = 0;                     // 3 x K
    static constexpr unsigned oQ = oK + 3 * KBUF;         // Q
    static constexpr unsigned VRB = 32 * NB;              // bytes per token row of a V slice
    static constexpr unsigned VSL = C * VRB;              // one state wave's V slice
    static constexpr unsigned oV = oQ + KBUF;             // NSW x V slice [C][16 NB]
    static constexpr unsigned oQKR = oV + NSW * VSL;      // QKR [C][C]
    static constexpr unsigned FBLK = 16 * 16 * 4;         // one float32 16x16 block
    // one chunk's float32 blocks: -A below the diagonal (6), T_ii by rows
    // (4) and by columns (4); two chunks, by parity
    static constexpr unsigned ABUF = 14 * FBLK, bTd = 6 * FBLK, bTdT = 10 * FBLK;
    static constexpr unsigned oA = oQKR + C * C * 2;
    static constexpr unsigned LDD = 20;                   // floats per row of Ad
    static constexpr unsigned oAd = oA + 2 * ABUF;        // A_ii [C][LDD]
    static constexpr unsigned oZ = oAd + C * LDD * 4;     // 2 float32 blocks between the solve's halves
    static constexpr unsigned HBLK = 16 * 16 * 2;         // one 16-bit 16x16 block
    static constexpr unsigned TBUF = 20 * HBLK;           // T diag(beta): 10 blocks x (hi, lo)
    static constexpr unsigned oTU = oZ + 2 * FBLK;        // two chunks, by parity
    static constexpr unsigned NV = 7 * C;                 // floats per gate-vector set
    static constexpr unsigned oVec = oTU + 2 * TBUF;      // 3 gate-vector sets
    static constexpr unsigned oGB = oVec + 3 * NV * 4;    // g, beta of two chunks, as loaded
    // decay ratios of the four diagonal tiles (lane order), two chunks
    static constexpr unsigned oRd = oGB + 2 * 2 * C * 4;
    static constexpr unsigned BYTES = oRd + 2 * NBT * 1024;
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
// Swizzle of the 16-byte units of the K and Q rows: t % 16 with bit 3
// flipped when bit 1 is set.  Both access kinds on these rows -- 16-byte row
// fragments (products with the state, the Q K^T and K K^T tiles) and the
// transpose reads of the state update (tokens along the contraction) -- are
// then free of LDS bank conflicts on gfx950, as timed on their exact lane
// addresses; with t % 16 alone the transpose reads take twice as long.  The
// same holds for the float32 blocks with their swizzle keyed on (r / 2) % 4
// rather than (r / 4) % 4.  kq_swz is linear over XOR: kq_swz(a ^ b) =
// kq_swz(a) ^ kq_swz(b), and kq_swz(4 i) = 4 i.
__device__ __forceinline__ int kq_swz(int t) { return (t ^ ((t & 2) << 2)) & 15; }
template <typename ET>
__device__ __forceinline__ typename Vec<ET>::x8 lds8(const char *smem, unsigned byte) {
    return *reinterpret_cast<const typename Vec<ET>::x8 *>(smem + byte);
}
template <typename ET>
__device__ __forceinline__ void sts4(char *smem, unsigned byte, typename Vec<ET>::x4 v) {
    *reinterpret_cast<typename Vec<ET>::x4 *>(smem + byte) = v;
}

// acc += a b for one 16x16x16 block in float32 (four v_mfma_f32_16x16x4_f32,
// float32 products and accumulation); a and b are float32 fragments (lane
// (x, qd) holds contraction indices 4 qd .. 4 qd + 3 of row / column x).
__device__ __forceinline__ f32x4 mma_f32(f32x4 a, f32x4 b, f32x4 acc) {
    acc = mfma(a[0], b[0], acc);
    acc = mfma(a[1], b[1], acc);
    acc = mfma(a[2], b[2], acc);
    acc = mfma(a[3], b[3], acc);
    return acc;
}

// Which wave computes which C x C tile of Q K^T and K K^T.  Tile (ib, jb)
// has token block ib (rows t of the result) and key block jb (columns j),
// ib >= jb.  Prep waves 0-3 hold the diagonal K K^T tile (p, p), whose
// inverse they form.  With four state and four prep waves:
//   Q K^T, state wave w = 0: (0,0) (1,0) (2,0)   w = 1: (1,1) (2,1) (3,1)
//                         w = 2: (2,2) (3,2)         w = 3: (3,3) (3,0)
//   K K^T, prep wave  p = 0: (0,0) (1,0) (2,0)   p = 1: (1,1) (2,1) (3,1)
//                         p = 2: (2,2) (3,2) (3,0)   p = 3: (3,3)
// (prep wave 3 finishes the longest column of T in the same phase).  With
// two state and ten prep waves:
//   Q K^T, state wave w = 0: (0,0) (1,0)   w = 1: (1,1) (2,1)
//          prep wave  p = 7: (2,0) (3,1)   p = 8: (2,2) (3,2)   p = 9: (3,3) (3,0)
//   K K^T, prep wave  p = 0..3: (p,p)   p = 4: (1,0) (2,0)   p = 5: (3,0) (2,1)
//                     p = 6: (3,1) (3,2)
// (prep wave 4 finishes the longest column of T, prep waves 5 and 6 load K).
struct Tile { int ib, jb; };
template <int N> struct Tiles { static constexpr int n = N; Tile t[N > 0 ? N : 1]; };
template <int NSW> constexpr auto qk_state(int w) {
    if (NSW == 4) {
        switch (w) {
        case 0: return Tiles<3>{{{0, 0}, {1, 0}, {2, 0}}};
        case 1: return Tiles<3>{{{1, 1}, {2, 1}, {3, 1}}};
        case 2: return Tiles<3>{{{2, 2}, {3, 2}, {-1, -1}}};
        default: return Tiles<3>{{{3, 3}, {3, 0}, {-1, -1}}};
        }
    }
    return w == 0 ? Tiles<3>{{{0, 0}, {1, 0}, {-1, -1}}} : Tiles<3>{{{1, 1}, {2, 1}, {-1, -1}}};
}
template <int NSW> constexpr auto qk_prep(int p) {
    if (NSW == 2 && p == 7) return Tiles<4>{{{2, 0}, {3, 1}, {-1, -1}, {-1, -1}}};
    if (NSW == 2 && p == 8) return Tiles<4>{{{2, 2}, {3, 2}, {-1, -1}, {-1, -1}}};
    if (NSW == 2 && p == 9) return Tiles<4>{{{3, 3}, {3, 0}, {-1, -1}, {-1, -1}}};
    return Tiles<4>{{{-1, -1}, {-1, -1}, {-1, -1}, {-1, -1}}};
}
template <int NSW> constexpr auto kk_prep(int p) {
    if (NSW == 4) {
        switch (p) {
        case 0: return Tiles<3>{{{0, 0}, {1, 0}, {2, 0}}};
        case 1: return Tiles<3>{{{1, 1}, {2, 1}, {3, 1}}};
        case 2: return Tiles<3>{{{2, 2}, {3, 2}, {3, 0}}};
        default: return Tiles<3>{{{3, 3}, {-1, -1}, {-1, -1}}};
        }
    }
    switch (p) {
    case 0: return Tiles<3>{{{0, 0}, {-1, -1}, {-1, -1}}};
    case 1: return Tiles<3>{{{1, 1}, {-1, -1}, {-1, -1}}};
    case 2: return Tiles<3>{{{2, 2}, {-1, -1}, {-1, -1}}};
    case 3: return Tiles<3>{{{3, 3}, {-1, -1}, {-1, -1}}};
    case 4: return Tiles<3>{{{1, 0}, {2, 0}, {-1, -1}}};
    case 5: return Tiles<3>{{{3, 0}, {2, 1}, {-1, -1}}};
    case 6: return Tiles<3>{{{3, 1}, {3, 2}, {-1, -1}}};
    default: return Tiles<3>{{{-1, -1}, {-1, -1}, {-1, -1}}};
    }
}
// f(std::integral_constant<int, p>) for the runtime wave index p < N
template <int N, typename F>
__device__ __forceinline__ void with_wave(int p, F &&f) {
    if constexpr (N > 0) {
        if (p == N - 1) f(std::integral_constant<int, N - 1>{});
        else with_wave<N - 1>(p, f);
    }
}
// number of real tiles (ib >= 0) in a list
template <typename TL> constexpr int ntiles(TL tl) {
    int c = 0;
    for (int i = 0; i < TL::n; ++i) c += tl.t[i].ib >= 0;
    return c;
}
// index of block (i, j), i > j, among the six blocks below the diagonal
constexpr int wy_aidx(int i, int j) { return i * (i - 1) / 2 + j; }
// index of block (i, j), i >= j, among the ten blocks of the lower triangle
constexpr int wy_tidx(int i, int j) { return i * (i + 1) / 2 + j; }

template <typename ET, int NSW>
__global__ __launch_bounds__(NSW == 4 ? 512 : 768, 1)
void chunk_wy_kernel(const ET *__restrict__ q, const ET *__restrict__ k,
                     const ET *__restrict__ v, const float *__restrict__ g,
                     const float *__restrict__ beta, const float *state_in,
                     float *state_out, ET *__restrict__ y,
                     int T, int Hk, int Hv, int xcd_group, float scale, int flags)
{
    using L = WyCfg<ET, NSW>;
    using X4 = typename Vec<ET>::x4;
    using X8 = typename Vec<ET>::x8;
    constexpr int C = L::C, DK = L::DK, DV = L::DV;
    constexpr int NBT = L::NBT, NBK = L::NBK, NSK = L::NSK, NB = L::NB, ROWS = L::ROWS;

    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    auto Gv = [&](int c) { return reinterpret_cast<float *>(smem + L::oVec + (c % 3) * L::NV * 4); };

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool state_wave = wave < NSW;
    const int w = state_wave ? wave : wave - NSW; // state wave index, or prep wave index
    // Lane coordinates.  With two state waves (twelve waves, at most 168
    // registers each) they pass through an empty asm statement at the top of
    // every chunk, so the compiler forms lane-dependent addresses inside the
    // loop instead of holding dozens of precombined addresses across it
    // (which spills there); the four-state-wave form keeps those addresses
    // in registers across chunks (256 registers, no spills, about 4% faster
    // on the long prefill).
    int lane = tid & 63, x = lane & 15, qd = lane >> 4;

    // Workgroups are dealt round-robin over the 8 XCDs, so workgroups i and
    // i + 8 share an XCD and its L2.  Workgroup r works on value rows
    // ROWS (r % NSPLIT) .. + ROWS - 1 of slot r / NSPLIT; with xcd_group > 1
    // the xcd_group workgroups that read the same q/k stream (the value
    // slices of a slot, the value heads of a key head) share an XCD, so that
    // the stream is fetched from HBM once per group.
    int bid = blockIdx.x;
    if (xcd_group > 1) {
        const int xcd = bid & 7, kk = bid >> 3;
        const int sib = kk % xcd_group, mm = kk / xcd_group;
        bid = (mm * 8 + xcd) * xcd_group + sib;
    }
    const int slot = bid / L::NSPLIT, row0 = ROWS * (bid % L::NSPLIT);
    const int b = slot / Hv, hv = value_head_of_rank(slot % Hv, Hk, Hv, flags);
    const int hk = key_head(hv, Hk, Hv, flags);
    const int nchunks = (T + C - 1) / C;

    // ---- lane-dependent LDS byte offsets
    // K/Q row fragment (16 bytes at unit 4 s + qd of row 16 b + x): ^ 64 s, + 4096 b
    auto f_lKt = [&]() { return (unsigned)(x * 256 + ((qd ^ kq_swz(x)) << 4)); };
    // K transpose read for the state update, rows r0 + r4, keys 32 s + 4 h +
    // 8 (x%4) .. +3 (lane x then receives key 32 s + 4 h + 8 (x/4) + x%4):
    // ^ 64 s, + 8 h, + 256 r0
    auto f_lKu = [&]() {
        const int r4 = 4 * qd + (x >> 2);
        return (unsigned)(r4 * 256 + (((x & 3) ^ kq_swz(r4)) << 4));
    };
    // QKR rows 16 tb + x, the 4 columns 16 jb + 4 qd ..: (this ^ 64 (jb/2)) +
    // 8 (jb%2) + 2048 tb; the 8 columns of blocks 2 s, 2 s + 1: ^ 64 s
    auto f_lA = [&]() { return (unsigned)(x * 128 + (((qd ^ (x >> 1)) & 7) << 4)); };
    auto aoff = [](unsigned lA, int jb, int tb) { return (lA ^ (64 * (jb >> 1))) + 8 * (jb & 1) + 2048 * tb; };
    // V slice: transpose read rows 16 jb + r4, permuted columns 4 NB (m/4) +
    // 4 vb + m%4: + 8 vb + 16 VRB jb
    auto f_lVs = [&]() { return (unsigned)((4 * qd + (x >> 2)) * L::VRB + (x & 3) * 8 * NB); };
    // float32 block, row fragment of row x (unit qd)
    auto f_lF = [&]() { return (unsigned)(x * 64 + ((qd ^ ((x >> 1) & 3)) << 4)); };
    // transposed 16-bit block of T: transpose read giving lane (x, qd) the
    // row-x entries of columns 4 qd .. 4 qd + 3
    auto f_lT = [&]() { return (unsigned)((4 * qd + (x >> 2)) * 32 + 8 * ((x & 3) ^ ((qd >> 1) << 1))); };

    // ---------------- input loads ----------------
    // Chunks of K, Q and V go from global memory straight into LDS
    // (global_load_lds_dwordx4: lane l of the wave writes the 16 bytes at
    // 16 l of a 1 KB block), written as inline assembly so that the compiler
    // does not wait for the transfer before the wave's next LDS access; the
    // issuing waves await them with s_waitcnt vmcnt(0) before the barrier
    // that closes the phase.  With four state waves, state wave w fills
    // rows 16 w .. 16 w + 15 of K and prep wave 3 all of Q; with two, prep
    // wave 5 fills K and prep waves 3 and 4 one half of Q each.  Prep wave 2
    // fills the V slices of all state waves.  The swizzle of K and Q
    // is applied on the source side.  Rows past the end of the sequence fetch
    // the last row again; with g = 1 and beta = 0 there, those rows add
    // nothing (their rows of A and columns of T diag(beta) vanish, so D is
    // zero on them, and their y rows are not stored).
    const size_t kstride = (size_t)Hk * DK, vstride = (size_t)Hv * DV;
    const ET *kbase = k + ((size_t)b * T * Hk + hk) * DK;
    const ET *qbase = q + ((size_t)b * T * Hk + hk) * DK;
    const ET *vbase = v + ((size_t)b * T * Hv + hv) * DV + row0;
    const float *gbase = g + (size_t)b * T * Hv + hv;
    const float *bbase = beta + (size_t)b * T * Hv + hv;
    auto f_okq0 = [&](int rg) { return (unsigned)((16 * rg + qd) * kstride + 8 * ((lane & 15) ^ kq_swz(qd))); };
    // V: 16-byte pieces of 8 values, 2 NB pieces per token row
    constexpr int VPR = 2 * NB, VRI = 64 / VPR;           // pieces per row, rows per load
    auto f_ov0 = [&]() { return (unsigned)((lane / VPR) * vstride + 8 * (lane % VPR)); };
    const unsigned lds_base = (unsigned)(uintptr_t)((__attribute__((address_space(3))) char *)smem);
    auto g2lds = [&](const ET *src, unsigned off, unsigned lds_byte) {
        const unsigned la = __builtin_amdgcn_readfirstlane(lds_base + lds_byte);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                     :: "v"(off), "s"(src), "s"(la) : "memory", "m0");
#pragma clang diagnostic pop
    };
    // rows 16 rg .. 16 rg + 15 of a K or Q chunk
    auto issue_kq = [&](const ET *base, unsigned dst, int c, int rg) {
        const int t0 = c * C;
        const ET *src = base + (size_t)t0 * kstride;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (t0 + C <= T) {
                g2lds(src, 2 * ((f_okq0(rg) ^ (32 * i)) + 4 * i * (unsigned)kstride), dst + 4096 * rg + 1024 * i);
            } else {
                const int r = 16 * rg + 4 * i + (lane >> 4);
                g2lds(src, 2 * (unsigned)(min(r, T - t0 - 1) * kstride + 8 * ((lane & 15) ^ kq_swz(r))),
                      dst + 4096 * rg + 1024 * i);
            }
        }
    };
    // the value columns of state wave sl (16 NB of them) of a V chunk
    auto issue_v = [&](int c, int sl) {
        const int t0 = c * C;
        const ET *src = vbase + (size_t)t0 * vstride + 16 * NB * sl;
        const unsigned dst = L::oV + sl * L::VSL;
        if (t0 + C <= T) {
            const unsigned o0 = f_ov0();
#pragma unroll
            for (int i = 0; i < C / VRI; ++i) g2lds(src, 2 * (o0 + VRI * i * (unsigned)vstride), dst + 1024 * i);
        } else {
            const int last = T - t0 - 1;
#pragma unroll
            for (int i = 0; i < C / VRI; ++i)
                g2lds(src, 2 * (unsigned)(min(VRI * i + lane / VPR, last) * vstride + 8 * (lane % VPR)), dst + 1024 * i);
        }
    };
    // g and beta of chunk c into the staging buffer c % 2 (one wave; lane =
    // token, rows past the end read the last row)
    auto load_gb = [&](int c) {
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
    };
    // Gate products of chunk c (one wave, lane t holding g_t; g = 1 and
    // beta = 0 past the end): within each 16-token block (one DPP row) the
    // inclusive prefix products P and the inclusive suffix products by four
    // doubling steps; the exclusive suffix Sfx; block totals; G[t] = P[t] x
    // totals of the earlier blocks; Rl[t] = Sfx[t] x totals of the later
    // blocks.  Every ratio of decays used later is a product of these.
    auto scan_gates = [&](int c) {
        const float *gb = reinterpret_cast<const float *>(smem + L::oGB + (c & 1) * 2 * C * 4);
        const float rg = gb[lane];
        const float rb = gb[C + lane];
        const int cn = min(C, T - c * C);
        float *gv = Gv(c);
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
    };
    static_assert(C == 64, "one lane per token in the gate scans");

    // ---- decay ratios of tile i of wave `wk` (token block ib, key block jb)
    // for lane (x, qd): t = 16 ib + x, j = 16 jb + 4 qd + r.
    // Diagonal tile: R[t][j] = g_{j+1} ... g_t (j <= t) by an inclusive scan
    // of g over the 16 lanes x of a DPP row, starting after 4 qd + 3.
    auto diag_ratio = [&](const float *gv, int blk) {
        const float gx = gv[kVg * C + 16 * blk + x];
        float h = (x >= 4 * qd + 4) ? gx : 1.f;
        h *= dpp_row_shr<1>(h);
        h *= dpp_row_shr<2>(h);
        h *= dpp_row_shr<4>(h);
        h *= dpp_row_shr<8>(h);
        const f32x4 g4 = *reinterpret_cast<const f32x4 *>(gv + kVg * C + 16 * blk + 4 * qd);
        f32x4 R;
        R[3] = h;
        R[2] = (4 * qd + 3 <= x) ? R[3] * g4[3] : 1.f;
        R[1] = (4 * qd + 2 <= x) ? R[2] * g4[2] : 1.f;
        R[0] = (4 * qd + 1 <= x) ? R[1] * g4[1] : 1.f;
        return R;
    };
    // Below the diagonal: R[t][j] = P[t] x (totals of the blocks strictly
    // between) x Sfx[j].
    auto off_ratio = [&](const float *gv, int ib, int jb) {
        float mf = gv[kVP * C + 16 * ib + x];
#pragma unroll
        for (int bb = 1; bb < NBT - 1; ++bb) mf *= (bb > jb && bb < ib) ? gv[kVBT * C + bb] : 1.f;
        return *reinterpret_cast<const f32x4 *>(gv + kVSfx * C + 16 * jb + 4 * qd) * mf;
    };

    // QKR = R (Q K^T) / sqrt(Dk), lower including the diagonal, from tile
    // (ib, jb) of Q K^T in registers (lane (x, qd): t = 16 ib + x, j = 16 jb
    // + 4 qd + r)
    auto store_qkr = [&](const float *gv, int c, int ib, int jb, f32x4 acc) {
        const unsigned lA = f_lA();
        if (ib == jb) {
            // the ratios the prep wave of this diagonal block formed for its
            // K K^T tile of the same chunk (same lanes, same values)
            const f32x4 R = *reinterpret_cast<const f32x4 *>(smem + L::oRd + (c & 1) * NBT * 1024 + ib * 1024 + 16 * lane);
            f32x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = (4 * qd + r <= x) ? scale * (R[r] * acc[r]) : 0.f;
            sts4<ET>(smem, L::oQKR + aoff(lA, ib, ib), cvt4<ET>(o));
        } else {
            const f32x4 R = off_ratio(gv, ib, jb);
            sts4<ET>(smem, L::oQKR + aoff(lA, jb, ib), cvt4<ET>(R * acc * scale));
        }
    };

    if (state_wave) {
        // ================= state waves =================
        f32x4 S[NBK][NB];                        // S^T tiles: rows = keys kcol, columns = values
        const size_t sbase = ((size_t)b * Hv + hv) * DV * DK;
        auto vcol = [&](int vb, int xx) { return row0 + 16 * NB * w + 4 * NB * (xx >> 2) + 4 * vb + (xx & 3); };
        auto kcol = [&](int kb, int q4) { return 32 * (kb >> 1) + 8 * q4 + 4 * (kb & 1); };
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
        // QKR blocks above the diagonal are never written: zero the buffer once.
        for (int i = tid; i < (int)(C * C * 2 / 16); i += 64 * NSW)
            reinterpret_cast<uint4 *>(smem + L::oQKR)[i] = zero_u4();
#pragma unroll
        for (int kb = 0; kb < NBK; ++kb)
#pragma unroll
            for (int vb = 0; vb < NB; ++vb) asm volatile("" : "+v"(S[kb][vb]));
        // K of chunk 0, the gates of chunks 0 and 1 and the gate products
        // of chunk 0 before the pipeline starts
        if (nchunks > 0) {
            for (int rg = w; rg < NBT; rg += NSW) issue_kq(kbase, L::oK, 0, rg);
            if (w == 0) {
                load_gb(0);
                if (nchunks > 1) load_gb(1);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (w == 0 && nchunks > 0) scan_gates(0);
        lds_barrier();
        // The state waves load K two chunks ahead and the gates three ahead,
        // at the start of phase a (they would otherwise wait at its end), and
        // wait for them before its barrier.
        auto issue_inputs = [&](int n) {
            if (n + 2 < nchunks)
                for (int rg = w; rg < NBT; rg += NSW) issue_kq(kbase, L::oK + ((n + 2) % 3) * L::KBUF, n + 2, rg);
            if (w == 0 && n + 3 < nchunks) load_gb(n + 3);
        };
        // (with two state waves, prep waves 5 and 4 issue these in the loop)
        issue_inputs(-1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();                           // A, T_ii of chunk 0
        lds_barrier();                           // first blocks of T of chunk 0, Q_0, V_0
        for (int n = 0; n < nchunks; ++n) {
            if constexpr (NSW == 2) asm volatile("" : "+v"(lane), "+v"(x), "+v"(qd));
            if constexpr (NSW == 4) issue_inputs(n);
            const unsigned lKt = f_lKt(), lA = f_lA();
            const unsigned kbn = L::oK + (n % 3) * L::KBUF;
            const float *gv = Gv(n);
            f32x4 Y[NB][NBT];
            X4 E[NBT][NB], Vf[NBT][NB];
            // ---------------- phase a ----------------
            {
                // Y^T = S Q^T and M = K S^T from the same 16-bit fragments of
                // the state, and this wave's Q K^T tiles from the same Q and K
                // fragments.  M: lane (x, qd) of tile (tb, vb) holds tokens
                // 16 tb + 4 qd .. + 3 of value column vcol(vb, x).
                f32x4 M[NBT][NB];
#pragma unroll
                for (int tb = 0; tb < NBT; ++tb)
#pragma unroll
                    for (int vb = 0; vb < NB; ++vb) Y[vb][tb] = M[tb][vb] = zero4();
                auto products = [&](auto W) {
                    constexpr auto TL = qk_state<NSW>(decltype(W)::value);
                    constexpr int nt = ntiles(TL);
                    f32x4 acc[nt > 0 ? nt : 1];
#pragma unroll
                    for (int i = 0; i < nt; ++i) acc[i] = zero4();
                    X8 nq[NBT], nk[NBT];
#pragma unroll
                    for (int tb = 0; tb < NBT; ++tb) {
                        nq[tb] = lds8<ET>(smem, L::oQ + lKt + 4096 * tb);
                        nk[tb] = lds8<ET>(smem, kbn + lKt + 4096 * tb);
                    }
#pragma unroll
                    for (int s = 0; s < NSK; ++s) {
                        X8 fs[NB];
#pragma unroll
                        for (int vb = 0; vb < NB; ++vb)
                            fs[vb] = cat8<ET>(cvt4<ET>(S[2 * s][vb]), cvt4<ET>(S[2 * s + 1][vb]));
                        X8 fq[NBT], fk[NBT];
#pragma unroll
                        for (int tb = 0; tb < NBT; ++tb) {
                            fq[tb] = nq[tb];
                            fk[tb] = nk[tb];
                        }
                        // the next key step's fragments are read during this
                        // step's products
                        if (s + 1 < NSK) {
                            const unsigned lo = lKt ^ (64 * (s + 1));
#pragma unroll
                            for (int tb = 0; tb < NBT; ++tb) {
                                nq[tb] = lds8<ET>(smem, L::oQ + lo + 4096 * tb);
                                nk[tb] = lds8<ET>(smem, kbn + lo + 4096 * tb);
                            }
                        }
#pragma unroll
                        for (int tb = 0; tb < NBT; ++tb)
#pragma unroll
                            for (int vb = 0; vb < NB; ++vb) {
                                Y[vb][tb] = mfma(fs[vb], fq[tb], Y[vb][tb]);
                                M[tb][vb] = mfma(fk[tb], fs[vb], M[tb][vb]);
                            }
#pragma unroll
                        for (int i = 0; i < nt; ++i)
                            acc[i] = mfma(fk[TL.t[i].jb], fq[TL.t[i].ib], acc[i]);
                        // one key step at a time: the 16-bit copy of the
                        // state is formed step by step, not held whole;
                        // vector ALU instructions alone may cross (mask
                        // 0x2), so that the next step's conversions and the
                        // right-hand side can issue under this step's
                        // matrix-core products
                        __builtin_amdgcn_sched_barrier(0x2);
                    }
#pragma unroll
                    for (int i = 0; i < nt; ++i) store_qkr(gv, n, TL.t[i].ib, TL.t[i].jb, acc[i]);
                };
                with_wave<NSW>(w, products);
                // the right-hand side E = V - G M in two 16-bit parts: V as
                // loaded (exact) and -G M rounded once; V read with the
                // permuted columns of the value tiles
                const unsigned vsl = L::oV + w * L::VSL + f_lVs();
#pragma unroll
                for (int tb = 0; tb < NBT; ++tb) {
                    const f32x4 g4 = *reinterpret_cast<const f32x4 *>(gv + kVG * C + 16 * tb + 4 * qd);
#pragma unroll
                    for (int vb = 0; vb < NB; ++vb) {
                        Vf[tb][vb] = ld_tr<ET>(smem, vsl + 8 * vb + 16 * L::VRB * tb);
                        E[tb][vb] = cvt4<ET>(g4 * M[tb][vb] * -1.f);
                    }
                }
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_barrier();
            // ---------------- phase b ----------------
            {
                // D = T diag(beta) V + T diag(beta) (-G M): [T_h | T_l] [V ; V]
                // and [T_h | T_l] [-G M ; -G M] per block
                const unsigned tub = L::oTU + (n & 1) * L::TBUF + f_lT();
                f32x4 D[NBT][NB];
#pragma unroll
                for (int tb = 0; tb < NBT; ++tb) {
#pragma unroll
                    for (int vb = 0; vb < NB; ++vb) D[tb][vb] = zero4();
#pragma unroll
                    for (int jb = 0; jb <= tb; ++jb) {
                        const unsigned to = tub + 2 * wy_tidx(tb, jb) * L::HBLK;
                        const X8 ft = cat8<ET>(ld_tr<ET>(smem, to), ld_tr<ET>(smem, to + L::HBLK));
#pragma unroll
                        for (int vb = 0; vb < NB; ++vb) {
                            D[tb][vb] = mfma(ft, cat8<ET>(Vf[jb][vb], Vf[jb][vb]), D[tb][vb]);
                            D[tb][vb] = mfma(ft, cat8<ET>(E[jb][vb], E[jb][vb]), D[tb][vb]);
                        }
                    }
                }
                // Y^T = G (S Q^T) / sqrt(Dk) + D^T QKR^T
#pragma unroll
                for (int tb = 0; tb < NBT; ++tb) {
                    const float gt = gv[kVG * C + 16 * tb + x] * scale;
#pragma unroll
                    for (int vb = 0; vb < NB; ++vb) Y[vb][tb] *= gt;
                }
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
                        const X8 fr = lds8<ET>(smem, L::oQKR + (lA ^ (64 * s)) + 2048 * tb);
#pragma unroll
                        for (int vb = 0; vb < NB; ++vb)
                            Y[vb][tb] = mfma(cat8<ET>(Df[2 * s][vb], Df[2 * s + 1][vb]), fr, Y[vb][tb]);
                    }
                }
                // y: lane (x, qd) holds token 16 tb + x, values vcol(vb, 4 qd + r),
                // 4 NB consecutive ones.
                // The stores go through a buffer resource that spans the
                // chunk's cn valid token rows: the hardware drops those past
                // the end of the sequence, with no branch around the stores.
                {
                    typedef int i32x4 __attribute__((ext_vector_type(4)));
                    const int t0 = n * C, cn = min(C, T - t0);
                    const unsigned rowb = (unsigned)(Hv * DV) * (unsigned)sizeof(ET);
                    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
                        (void *)(y + (((size_t)b * T + t0) * Hv + hv) * DV), (short)0, (int)(cn * rowb), 0x00020000);
                    typedef int i32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
                    for (int tb = 0; tb < NBT; ++tb) {
                        const int off = (int)((16 * tb + x) * rowb + vcol(0, 4 * qd) * sizeof(ET));
                        if constexpr (NB == 2)
                            __builtin_amdgcn_raw_buffer_store_b128(
                                __builtin_bit_cast(i32x4, cat8<ET>(cvt4<ET>(Y[0][tb]), cvt4<ET>(Y[1][tb]))), yr, off, 0, 0);
                        else
                            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, cvt4<ET>(Y[0][tb])), yr, off, 0, 0);
                    }
                }
                // S^T <- G_last S^T + K^T diag(Rl) D
                const unsigned lKu = f_lKu();
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
                        const unsigned ka = kbn + (lKu ^ (64 * (kb >> 1))) + 8 * (kb & 1) + 256 * 32 * s;
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
        // ================= prep waves =================
        const int p = w;
        lds_barrier();
        // Block (i, j) of T diag(beta) of chunk c, given in float32 (lane
        // (x, qd): rows 4 qd .. + 3, column x): scaled by beta of column x
        // and stored as a two-term 16-bit expansion, transposed by blocks.
        auto emit = [&](int c, int i, int j, f32x4 t) {
            const float bc = Gv(c)[kVb * C + 16 * j + x];
            const unsigned blk = L::oTU + (c & 1) * L::TBUF + 2 * wy_tidx(i, j) * L::HBLK +
                                 x * 32 + 8 * (qd ^ (2 * (x >> 3)));
            const f32x4 tu = t * bc;
            const X4 h = cvt4<ET>(tu);
            sts4<ET>(smem, blk, h);
            sts4<ET>(smem, blk + L::HBLK, cvt4<ET>(tu - to_f32x4<ET>(h)));
        };
        // Partial sums Z_2, Z_3 of column 0, carried from the first half of
        // the solve (prep wave 0) to its second half (prep wave 3, or 4 with
        // six prep waves) in 16-byte slots indexed by lane
        auto zst = [&](int i, f32x4 v) { *reinterpret_cast<f32x4 *>(smem + L::oZ + i * L::FBLK + 16 * lane) = v; };
        auto zld = [&](int i) { return *reinterpret_cast<const f32x4 *>(smem + L::oZ + i * L::FBLK + 16 * lane); };
        // iteration n: phase a finishes T of chunk n and builds A, T_ii of
        // chunk n+1; phase b starts T of chunk n+1 (n = -1 is the pipeline's
        // start).  The blocks below the diagonal, with -A stored:
        //   Z_i = sum_{j<=k<i} (-A_ik) T_kj,  T_ij = T_ii Z_i,
        // every product in float32 on the matrix cores.  First half (phase
        // b, prep wave p = column p): column 0 up to T_10 and the terms of
        // Z_2, Z_3 through T_10; columns 1 and 2 whole.  Second half (phase a
        // of the next iteration, prep wave 3 or 4): T_20, T_30.
        for (int n = -1; n < nchunks; ++n) {
            const int m = n + 1;
            const unsigned lF = f_lF();
            auto ff = [&](unsigned base) { return *reinterpret_cast<const f32x4 *>(smem + base + lF); };
            // ---------------- phase a ----------------
            if constexpr (NSW == 2) {
                // with two state waves, prep waves 5 and 6 load K two chunks
                // ahead and prep wave 6 the gates three ahead (the state
                // waves do with four)
                if ((p == 5 || p == 6) && n >= 0 && n + 2 < nchunks)
                    for (int rg = 2 * (p - 5); rg < 2 * (p - 5) + 2; ++rg)
                        issue_kq(kbase, L::oK + ((n + 2) % 3) * L::KBUF, n + 2, rg);
                if (p == 6 && n >= 0 && n + 3 < nchunks) load_gb(n + 3);
            }
            if (n >= 0 && p == (NSW == 4 ? 3 : 4)) {
                const unsigned ab = L::oA + (n & 1) * L::ABUF;
                const f32x4 t20 = mma_f32(ff(ab + L::bTd + 2 * L::FBLK), zld(0), zero4());
                const f32x4 z3 = mma_f32(ff(ab + wy_aidx(3, 2) * L::FBLK), t20, zld(1));
                emit(n, 2, 0, t20);
                emit(n, 3, 0, mma_f32(ff(ab + L::bTd + 3 * L::FBLK), z3, zero4()));
            }
            if (m < nchunks) {
                // K K^T tiles of chunk m -> A (float32): the diagonal tile to
                // Ad (for the inverse), the tiles below it to their blocks
                const unsigned kbm = L::oK + (m % 3) * L::KBUF;
                const unsigned ab = L::oA + (m & 1) * L::ABUF;
                const unsigned lKt = f_lKt();
                const float *gv = Gv(m);
                auto kk_tiles = [&](auto W) {
                    constexpr auto TL = kk_prep<NSW>(decltype(W)::value);
                    constexpr int nt = ntiles(TL);
                    if constexpr (nt > 0) {
                    f32x4 acc[nt];
#pragma unroll
                    for (int i = 0; i < nt; ++i) acc[i] = zero4();
#pragma unroll
                    for (int s = 0; s < NSK; ++s) {
                        const unsigned lo = lKt ^ (64 * s);
#pragma unroll
                        for (int i = 0; i < nt; ++i)
                            acc[i] = mfma(lds8<ET>(smem, kbm + lo + 4096 * TL.t[i].jb),
                                          lds8<ET>(smem, kbm + lo + 4096 * TL.t[i].ib), acc[i]);
                    }
#pragma unroll
                    for (int i = 0; i < nt; ++i) {
                        const int ib = TL.t[i].ib, jb = TL.t[i].jb;
                        const float bt = gv[kVb * C + 16 * ib + x];
                        if (ib == jb) {
                            const f32x4 R = diag_ratio(gv, ib);
                            // kept for the Q K^T tile (ib, ib) of this chunk
                            *reinterpret_cast<f32x4 *>(smem + L::oRd + (m & 1) * NBT * 1024 + ib * 1024 + 16 * lane) = R;
                            f32x4 a;
#pragma unroll
                            for (int r = 0; r < 4; ++r) a[r] = (4 * qd + r < x) ? bt * (R[r] * acc[i][r]) : 0.f;
                            *reinterpret_cast<f32x4 *>(smem + L::oAd + ((16 * ib + x) * L::LDD + 4 * qd) * 4) = a;
                        } else {
                            const f32x4 R = off_ratio(gv, ib, jb);
                            *reinterpret_cast<f32x4 *>(smem + ab + wy_aidx(ib, jb) * L::FBLK + lF) = R * acc[i] * (-bt);
                        }
                    }
                    }
                };
                with_wave<L::NP>(p, kk_tiles);
                // T_pp = (I + A_pp)^-1 by float32 forward substitution: four
                // lanes per column c, lane part pt holding rows pt, pt+4,
                // pt+8, pt+12.  Column sweep: once x_j is final (it sits in
                // part j%4), every later row subtracts A[i][j] x_j.  The rows
                // come from this wave's own writes above (LDS keeps a wave's
                // accesses in order).
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                if (p < NBT) {
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
                    // rows r = pt + 4 mm of column c, into the block by rows
                    // and the block by columns
                    float *td = reinterpret_cast<float *>(smem + ab + L::bTd + p * L::FBLK);
                    float *tdt = reinterpret_cast<float *>(smem + ab + L::bTdT + p * L::FBLK);
#pragma unroll
                    for (int mm = 0; mm < 4; ++mm) {
                        const int r = pt + 4 * mm;
                        td[r * 16 + 4 * ((c >> 2) ^ ((r >> 1) & 3)) + (c & 3)] = sv[mm];
                        tdt[c * 16 + 4 * (mm ^ ((c >> 1) & 3)) + pt] = sv[mm];
                    }
                }
            }
            if constexpr (NSW == 2) {
                // with two state waves, prep waves 7-9 compute the Q K^T
                // tiles of chunk n
                if (n >= 0 && p >= 7) {
                    const unsigned kbn = L::oK + (n % 3) * L::KBUF, lKt = f_lKt();
                    const float *gv = Gv(n);
                    auto qk_tiles = [&](auto W) {
                        constexpr auto TL = qk_prep<NSW>(decltype(W)::value);
                        constexpr int nt = ntiles(TL);
                        if constexpr (nt > 0) {
                        f32x4 acc[nt];
#pragma unroll
                        for (int i = 0; i < nt; ++i) acc[i] = zero4();
#pragma unroll
                        for (int s = 0; s < NSK; ++s) {
                            const unsigned lo = lKt ^ (64 * s);
#pragma unroll
                            for (int i = 0; i < nt; ++i)
                                acc[i] = mfma(lds8<ET>(smem, kbn + lo + 4096 * TL.t[i].jb),
                                              lds8<ET>(smem, L::oQ + lo + 4096 * TL.t[i].ib), acc[i]);
                        }
#pragma unroll
                        for (int i = 0; i < nt; ++i) store_qkr(gv, n, TL.t[i].ib, TL.t[i].jb, acc[i]);
                        }
                    };
                    with_wave<L::NP>(p, qk_tiles);
                }
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            lds_barrier();
            // ---------------- phase b ----------------
            if (m < nchunks) {
                // Q and V of chunk m (their buffers were last read in phase
                // a): with four prep waves, prep waves 3 and 2, whose blocks
                // of T need the least work; with ten, prep waves 7, 8 and 9
                if constexpr (NSW == 4) {
                    if (p == 3) {
#pragma unroll
                        for (int rg = 0; rg < 4; ++rg) issue_kq(qbase, L::oQ, m, rg);
                    } else if (p == 2) {
#pragma unroll
                        for (int sl = 0; sl < NSW; ++sl) issue_v(m, sl);
                    }
                } else {
                    if (p == 7 || p == 8) {
#pragma unroll
                        for (int i = 0; i < 2; ++i) issue_kq(qbase, L::oQ, m, 2 * (p - 7) + i);
                    } else if (p == 9) {
#pragma unroll
                        for (int sl = 0; sl < NSW; ++sl) issue_v(m, sl);
                    }
                }
                const unsigned ab = L::oA + (m & 1) * L::ABUF;
                if (p < NBT) {
                    const f32x4 tpp = ff(ab + L::bTdT + p * L::FBLK);   // T_pp, lane (x, qd): rows 4 qd .., column x
                    emit(m, p, p, tpp);
                }
                if (p == 0) {
                    const f32x4 tpp = ff(ab + L::bTdT);
                    const f32x4 z1 = mma_f32(ff(ab + wy_aidx(1, 0) * L::FBLK), tpp, zero4());
                    f32x4 z2 = mma_f32(ff(ab + wy_aidx(2, 0) * L::FBLK), tpp, zero4());
                    f32x4 z3 = mma_f32(ff(ab + wy_aidx(3, 0) * L::FBLK), tpp, zero4());
                    const f32x4 t10 = mma_f32(ff(ab + L::bTd + 1 * L::FBLK), z1, zero4());
                    z2 = mma_f32(ff(ab + wy_aidx(2, 1) * L::FBLK), t10, z2);
                    z3 = mma_f32(ff(ab + wy_aidx(3, 1) * L::FBLK), t10, z3);
                    zst(0, z2);
                    zst(1, z3);
                    emit(m, 1, 0, t10);
                } else if (p == 1) {
                    const f32x4 tpp = ff(ab + L::bTdT + 1 * L::FBLK);
                    const f32x4 z2 = mma_f32(ff(ab + wy_aidx(2, 1) * L::FBLK), tpp, zero4());
                    f32x4 z3 = mma_f32(ff(ab + wy_aidx(3, 1) * L::FBLK), tpp, zero4());
                    const f32x4 t21 = mma_f32(ff(ab + L::bTd + 2 * L::FBLK), z2, zero4());
                    z3 = mma_f32(ff(ab + wy_aidx(3, 2) * L::FBLK), t21, z3);
                    emit(m, 2, 1, t21);
                    emit(m, 3, 1, mma_f32(ff(ab + L::bTd + 3 * L::FBLK), z3, zero4()));
                } else if (p == 2) {
                    const f32x4 tpp = ff(ab + L::bTdT + 2 * L::FBLK);
                    const f32x4 z3 = mma_f32(ff(ab + wy_aidx(3, 2) * L::FBLK), tpp, zero4());
                    emit(m, 3, 2, mma_f32(ff(ab + L::bTd + 3 * L::FBLK), z3, zero4()));
                }
            }
            if (p == (NSW == 4 ? 3 : 6) && n + 2 < nchunks) scan_gates(n + 2);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_barrier();
        }
    }
}

}  // namespace gdn
