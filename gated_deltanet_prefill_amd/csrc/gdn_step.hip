// gdn_step.hip -- one token of the gated delta rule (decode) for gfx950.
//
// The step reads every state row once and writes it once; it is bound by
// that traffic (the ferrox-core gdn_chunk.rs page, "Why": nothing about the
// loop is slow, the traffic is the cost).  Eight lanes own one state row
// (8 value rows per wave, 32 per workgroup); lane i of a row holds the
// 16-byte pieces i, i+8, ... of the row so that each load or store
// instruction of the 8 lanes covers 128 contiguous bytes.  Per row j:
//     a_j = S_j . k,   b_j = S_j . q          (one pass over the row)
//     d_j = beta (v_j - g a_j)
//     S'_j = g S_j + d_j k
//     y_j = (g b_j + d_j (k . q)) / sqrt(Dk)  (= S'_j . q / sqrt(Dk))
// The three dot products finish with a butterfly over the row's 8 lanes.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int kStepRowsPerBlock = 32;
constexpr int kStepLanesPerRow = 8;

template <typename ET, int DK>
__global__ __launch_bounds__(256)
void step_kernel(const ET *__restrict__ q, const ET *__restrict__ k,
                 const ET *__restrict__ v, const float *__restrict__ g,
                 const float *__restrict__ beta, const float *state_in,
                 float *state_out, ET *__restrict__ y,
                 int Hk, int Hv, int Dv, float scale)
{
    constexpr int LPR = kStepLanesPerRow;
    constexpr int NP = DK / (4 * LPR);            // 16-byte state pieces per lane
    const int tid = threadIdx.x;
    const int sub = tid & (LPR - 1);
    const int blocks_per_slot = Dv / kStepRowsPerBlock;
    const int slot = blockIdx.x / blocks_per_slot;
    const int j = (blockIdx.x - slot * blocks_per_slot) * kStepRowsPerBlock + tid / LPR;
    const int hv = slot % Hv, b = slot / Hv, hk = hv / (Hv / Hk);

    const ET *kp = k + ((size_t)b * Hk + hk) * DK;
    const ET *qp = q + ((size_t)b * Hk + hk) * DK;
    const size_t row = ((size_t)slot * Dv + j) * DK;

    f32x4 s[NP], kv[NP], qv[NP];
#pragma unroll
    for (int m = 0; m < NP; ++m) {
        const int e = 4 * (m * LPR + sub);
        kv[m] = to_f32x4<ET>(ld4<ET>(kp + e));
        qv[m] = to_f32x4<ET>(ld4<ET>(qp + e));
        s[m] = state_in ? *reinterpret_cast<const f32x4 *>(state_in + row + e) : zero4();
    }
    float a = 0.f, bq = 0.f, kq = 0.f;
#pragma unroll
    for (int m = 0; m < NP; ++m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a += s[m][i] * kv[m][i];
            bq += s[m][i] * qv[m][i];
            kq += kv[m][i] * qv[m][i];
        }
    }
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) {
        a += __shfl_xor(a, off);
        bq += __shfl_xor(bq, off);
        kq += __shfl_xor(kq, off);
    }
    const float gt = g[slot], bt = beta[slot];
    const float vj = to_f32(v[(size_t)slot * Dv + j]);
    const float d = bt * (vj - gt * a);
#pragma unroll
    for (int m = 0; m < NP; ++m) {
        const int e = 4 * (m * LPR + sub);
        *reinterpret_cast<f32x4 *>(state_out + row + e) = gt * s[m] + d * kv[m];
    }
    if (sub == 0) y[(size_t)slot * Dv + j] = from_f32<ET>((gt * bq + d * kq) * scale);
}

template <typename ET, int DK>
static hipError_t launch_step_inst(const FwdArgs &a, hipStream_t st) {
    const dim3 grid((unsigned)a.B * (unsigned)a.Hv * (unsigned)(a.Dv / kStepRowsPerBlock));
    const dim3 block(kStepRowsPerBlock * kStepLanesPerRow);
    hipLaunchKernelGGL((step_kernel<ET, DK>), grid, block, 0, st,
                       static_cast<const ET *>(a.q), static_cast<const ET *>(a.k),
                       static_cast<const ET *>(a.v), a.g, a.beta, a.state_in, a.state_out,
                       static_cast<ET *>(a.y), a.Hk, a.Hv, a.Dv, a.scale);
    return hipGetLastError();
}

template <typename ET>
static hipError_t launch_step_typed(const FwdArgs &a, hipStream_t st) {
    switch (a.Dk) {
    case 32: return launch_step_inst<ET, 32>(a, st);
    case 64: return launch_step_inst<ET, 64>(a, st);
    case 128: return launch_step_inst<ET, 128>(a, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_step(int dtype, const FwdArgs &a, hipStream_t st) {
    switch (dtype) {
    case 0: return launch_step_typed<float>(a, st);
    case 1: return launch_step_typed<__bf16>(a, st);
    case 2: return launch_step_typed<_Float16>(a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
