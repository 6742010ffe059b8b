// gdn_internal.h -- launchers shared between the kernel units and the C ABI.
#pragma once

#include <hip/hip_runtime_api.h>

namespace gdn {

// Bits of FwdArgs::flags (the GDN_HEADS_TILED and GDN_GATE_LOG values of
// the C ABI).
constexpr int kTiledHeads = 1;     // key head of value head hv is hv mod Hk
constexpr int kLogGate = 2;        // g holds log(decay)
constexpr int kVectorGate = 4;     // g is [B,T,Hv,Dk]: one decay per key dimension

struct FwdArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    const float *state_in;
    float *state_out;
    void *y;
    int B, T, Hk, Hv, Dk, Dv, C;
    float scale;
    int flags = 0;
};

// Each returns hipSuccess or the launch error; arguments are already valid.
hipError_t launch_chunk_f32(const FwdArgs &a, hipStream_t s);
hipError_t launch_chunk_bf16(const FwdArgs &a, hipStream_t s);
hipError_t launch_chunk_f16(const FwdArgs &a, hipStream_t s);
// the chunked kernel for a decay per key dimension (FwdArgs::flags & kVectorGate)
hipError_t launch_chunk_vg_f32(const FwdArgs &a, hipStream_t s);
hipError_t launch_chunk_vg_bf16(const FwdArgs &a, hipStream_t s);
hipError_t launch_chunk_vg_f16(const FwdArgs &a, hipStream_t s);
hipError_t launch_step(int dtype, const FwdArgs &a, hipStream_t s);
hipError_t launch_seq(int dtype, const FwdArgs &a, hipStream_t s);

// Largest chunk the float32 path can hold in LDS; bigger requests run with
// this chunk length (the result does not depend on the chunk length).
constexpr int kMaxChunkF32 = 32;

}  // namespace gdn
