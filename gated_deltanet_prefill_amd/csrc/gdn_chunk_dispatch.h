// gdn_chunk_dispatch.h -- picks the chunk kernel instantiation for a shape.
#pragma once

#include "gdn_chunk_impl.h"
#include "gdn_chunk_pipe.h"
#include "gdn_internal.h"

namespace gdn {

template <typename ET, int DK, int DV, int C>
hipError_t launch_chunk_inst(const FwdArgs &a, hipStream_t st) {
    const long nslots = (long)a.B * a.Hv;
    const int group = a.Hv / a.Hk;
    if constexpr (sizeof(ET) == 2 && DK == 128 && DV == 128 && C == 64) {
        // the pipelined kernel: one 8-wave workgroup per slot
        const int xcd_group = (group > 1 && nslots % (8L * group) == 0) ? group : 1;
        hipLaunchKernelGGL((chunk_pipe_kernel<ET, DK, DV, C>), dim3((unsigned)nslots), dim3(512), 0, st,
                           static_cast<const ET *>(a.q), static_cast<const ET *>(a.k),
                           static_cast<const ET *>(a.v), a.g, a.beta, a.state_in, a.state_out,
                           static_cast<ET *>(a.y), a.T, a.Hk, a.Hv, xcd_group, a.scale, a.flags);
        return hipGetLastError();
    } else {
        // 32 value columns per wave for Dv = 128, else 16 (more waves, fewer
        // live registers per wave at small Dv)
        constexpr int NB = DV >= 128 ? 2 : 1;
        constexpr int DVS = DV;                      // one workgroup per slot
        using L = ChunkCfg<ET, DK, DVS, C, NB>;
        const int nsplit = DV / DVS;
        const long nblocks = nslots * nsplit;
        const int xcd_group = (nsplit == 1 && group > 1 && nblocks % (8L * group) == 0) ? group : 1;
        const dim3 grid((unsigned)nblocks), block(L::NT);
        hipLaunchKernelGGL((chunk_fwd_kernel<ET, DK, DVS, C, NB>), grid, block, 0, st,
                           static_cast<const ET *>(a.q), static_cast<const ET *>(a.k),
                           static_cast<const ET *>(a.v), a.g, a.beta, a.state_in, a.state_out,
                           static_cast<ET *>(a.y), a.T, a.Hk, a.Hv, a.Dv, nsplit, xcd_group, a.scale,
                           a.flags);
        return hipGetLastError();
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
