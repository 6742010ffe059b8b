// gdn_chunk_dispatch.h -- picks the chunk kernel instantiation for a shape.
#pragma once

#include "gdn_chunk_impl.h"
#include "gdn_chunk_wave.h"
#include "gdn_chunk_wy.h"
#include "gdn_internal.h"

#include <type_traits>

namespace gdn {

// Generic kernel on value slices of DVS columns: Dv / DVS workgroups per
// slot, each recomputing the slot's C x C work (gate products, K K^T, the
// solve) for its own slice of the state.
template <typename ET, int DK, int DV, int C, int DVS>
hipError_t launch_generic(const FwdArgs &a, hipStream_t st) {
    // 32 value columns per wave for a 128-column slice, else 16 (more waves,
    // fewer live registers per wave at small slices)
    constexpr int NB = DVS >= 128 ? 2 : 1;
    using L = ChunkCfg<ET, DK, DVS, C, NB>;
    const long nslots = (long)a.B * a.Hv;
    const int group = a.Hv / a.Hk;
    const int nsplit = DV / DVS;
    const long nblocks = nslots * nsplit;
    const int xcd_group = (nsplit == 1 && group > 1 && nblocks % (8L * group) == 0) ? group : 1;
    hipLaunchKernelGGL((chunk_fwd_kernel<ET, DK, DVS, C, NB>), dim3((unsigned)nblocks), dim3(L::NT), 0, st,
                       static_cast<const ET *>(a.q), static_cast<const ET *>(a.k),
                       static_cast<const ET *>(a.v), a.g, a.beta, a.state_in, a.state_out,
                       static_cast<ET *>(a.y), a.T, a.Hk, a.Hv, a.Dv, nsplit, xcd_group, a.scale,
                       a.flags);
    return hipGetLastError();
}

// Value slices per slot for the generic kernel, from timed sweeps over slot
// counts 8..384, T = 128 and 512, Dk = Dv in {64, 128}: while B Hv is small
// the extra workgroups fill idle CUs (up to 1.4x faster), once the grid
// fills the duplicated C x C work costs more than it gains.
inline int generic_split(int Dv, int C, bool f32, long nslots) {
    if (Dv == 128) {
        if (f32) return (C == 16 && nslots <= 128) ? 2 : 1;
        if (C == 32) return nslots <= 24 ? 4 : nslots <= 384 ? 2 : 1;
        if (C == 16) return nslots <= 16 ? 4 : nslots <= 128 ? 2 : 1;
        return 1;
    }
    if (Dv == 64 && !f32 && C == 16) return nslots <= 64 ? 2 : 1;
    return 1;
}

// Value slices per slot for the pipelined kernel: four while the grid
// stays within one workgroup per CU of the MI355X.
inline int wy_split(long nslots) { return nslots <= 64 ? 4 : 1; }

// The pipelined kernel's four-slice form (two state waves and ten prep
// waves per workgroup, at most 168 registers per wave) is compiled in a
// translation unit of its own, gdn_chunk_wy2_{bf16,f16}.hip, with the
// backend's instruction-level-parallelism scheduler: on the GQA ragged
// workload (B = 2, T = 1111, Hk = 16, Hv = 32, C = 64) it runs in 42.4
// against 45.1 us, bit-identical, while the same scheduler slows the
// one-slice form (long prefill 500.6 against 483.9 us) and the other chunk
// kernels.
hipError_t launch_wy2_bf16(const FwdArgs &a, hipStream_t st, unsigned nblocks, int xcd_group);
hipError_t launch_wy2_f16(const FwdArgs &a, hipStream_t st, unsigned nblocks, int xcd_group);

template <typename ET>
hipError_t launch_wy2_kernel(const FwdArgs &a, hipStream_t st, unsigned nblocks, int xcd_group) {
    hipLaunchKernelGGL((chunk_wy_kernel<ET, 2>), dim3(nblocks), dim3(768), 0, st,
                       static_cast<const ET *>(a.q), static_cast<const ET *>(a.k),
                       static_cast<const ET *>(a.v), a.g, a.beta, a.state_in, a.state_out,
                       static_cast<ET *>(a.y), a.T, a.Hk, a.Hv, xcd_group, a.scale, a.flags);
    return hipGetLastError();
}

// The C = 16 kernel with one wave per 16 value rows: a workgroup of four
// waves per 64 value rows of a slot.
template <typename ET>
hipError_t launch_wave(const FwdArgs &a, hipStream_t st) {
    const long nblocks = (long)a.B * a.Hv * (a.Dv / 64);
    hipLaunchKernelGGL((chunk_wave_kernel<ET>), dim3((unsigned)nblocks), dim3(256), 0, st,
                       static_cast<const ET *>(a.q), static_cast<const ET *>(a.k),
                       static_cast<const ET *>(a.v), a.g, a.beta, a.state_in, a.state_out,
                       static_cast<ET *>(a.y), a.T, a.Hk, a.Hv, a.Dv, a.scale, a.flags);
    return hipGetLastError();
}

// Whether the per-wave kernel serves a C = 16 call of 16-bit inputs with
// Dk = 128 and Dv a multiple of 64: one chunk (1..16 tokens).  Timed against
// the generic kernel at C = 16 over 64..2048 slots and T = 1..16 (GPU time of
// graph replays, the state read from HBM), it was faster everywhere: 5.5
// against 7.5 us at 64 slots, 50-52 against 60-63 us at 2048.
inline bool wave_for(int T) { return T >= 1 && T <= 16; }

template <typename ET, int DK, int DV, int C>
hipError_t launch_chunk_inst(const FwdArgs &a, hipStream_t st) {
    const long nslots = (long)a.B * a.Hv;
    const int group = a.Hv / a.Hk;
    if constexpr (sizeof(ET) == 2 && C == 16 && DK == 128 && DV % 64 == 0)
        if (wave_for(a.T)) return launch_wave<ET>(a, st);
    if constexpr (sizeof(ET) == 2 && DK == 128 && DV == 128 && C == 64) {
        // the pipelined kernel: one 8-wave workgroup per slot, or, while four
        // workgroups per slot still fit the 256 CUs in one round, four
        // 12-wave workgroups of 32 value rows each (two state waves, ten
        // prep waves)
        const int nsplit = wy_split(nslots);
        const long nblocks = nslots * nsplit;
        const int grp = group * nsplit;          // workgroups reading one q/k stream
        const int xcd_group = (grp > 1 && nblocks % (8L * grp) == 0) ? grp : 1;
        if (nsplit == 4) {
            if constexpr (std::is_same_v<ET, __bf16>) return launch_wy2_bf16(a, st, (unsigned)nblocks, xcd_group);
            else return launch_wy2_f16(a, st, (unsigned)nblocks, xcd_group);
        }
        hipLaunchKernelGGL((chunk_wy_kernel<ET, 4>), dim3((unsigned)nblocks), dim3(512), 0, st,
                           static_cast<const ET *>(a.q), static_cast<const ET *>(a.k),
                           static_cast<const ET *>(a.v), a.g, a.beta, a.state_in, a.state_out,
                           static_cast<ET *>(a.y), a.T, a.Hk, a.Hv, xcd_group, a.scale, a.flags);
        return hipGetLastError();
    } else {
        constexpr bool F32 = sizeof(ET) == 4;
        const int split = generic_split(DV, C, F32, nslots);
        if constexpr (DV == 128 && (C == 16 || (!F32 && C == 32))) {
            if constexpr (!F32)
                if (split == 4) return launch_generic<ET, DK, DV, C, 32>(a, st);
            if (split == 2) return launch_generic<ET, DK, DV, C, 64>(a, st);
        } else if constexpr (DV == 64 && !F32 && C == 16) {
            if (split == 2) return launch_generic<ET, DK, DV, C, 32>(a, st);
        }
        return launch_generic<ET, DK, DV, C, DV>(a, st);
    }
}

template <typename ET, int DK, int DV>
hipError_t launch_chunk_c(const FwdArgs &a, hipStream_t st) {
    int C = a.C;
    if (sizeof(ET) == 4 && C > kMaxChunkF32) C = kMaxChunkF32;
    switch (C) {
    case 16: return launch_chunk_inst<ET, DK, DV, 16>(a, st);
    case 32: return launch_chunk_inst<ET, DK, DV, 32>(a, st);
    case 64:
        if constexpr (sizeof(ET) != 4) return launch_chunk_inst<ET, DK, DV, 64>(a, st);
        [[fallthrough]];
    default: return hipErrorInvalidValue;
    }
}

template <typename ET, int DK>
hipError_t launch_chunk_dv(const FwdArgs &a, hipStream_t st) {
    switch (a.Dv) {
    case 32: return launch_chunk_c<ET, DK, 32>(a, st);
    case 64: return launch_chunk_c<ET, DK, 64>(a, st);
    case 128: return launch_chunk_c<ET, DK, 128>(a, st);
    default: return hipErrorInvalidValue;
    }
}

template <typename ET>
hipError_t launch_chunk_typed(const FwdArgs &a, hipStream_t st) {
    switch (a.Dk) {
    case 32: return launch_chunk_dv<ET, 32>(a, st);
    case 64: return launch_chunk_dv<ET, 64>(a, st);
    case 128: return launch_chunk_dv<ET, 128>(a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
