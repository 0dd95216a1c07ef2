// Reconstruct kernel: materialise W_eff = W_base + alpha * sign(Delta) in bf16.
//
// "BitDelta: Serving 14 Zen Models from One GPU Cluster", section "Serving
// Architecture", step 3 of the request flow (rebuild the effective weight)
// and the conceptual sketch (unpack the packed signs to {-1,+1}, scale by
// alpha per output row, add to the bf16 base).  The sum is formed in fp32
// and rounded once to bf16, nearest-even.
//
// Each thread handles one 8-column group per step: a 16-byte load of W_base,
// its sign byte, a 16-byte store of W_eff.  A workgroup covers 256 groups of
// one row; rows are split over ceil(groups / 256) workgroups.  Bandwidth-
// bound: 2 + 1/8 bytes read and 2 bytes written per weight.
#include "bd_device.h"
#include "bd_launch.h"

namespace bd {
namespace {

constexpr int kThreads = 256;

template <bool PER_MATRIX>
__global__ __launch_bounds__(kThreads) void reconstruct_rows(const uint16_t *__restrict__ w_base,
                                                             const uint8_t *__restrict__ signs,
                                                             const float *__restrict__ alpha,
                                                             int64_t C, int blocks_per_row,
                                                             uint16_t *__restrict__ w_eff)
{
    const int64_t r = blockIdx.x / blocks_per_row;
    const int64_t g = (int64_t)(blockIdx.x % blocks_per_row) * kThreads + threadIdx.x;
    const int64_t G = C >> 3;
    if (g >= G)
        return;
    const float a = PER_MATRIX ? alpha[0] : alpha[r];
    const uint4 w = reinterpret_cast<const uint4 *>(w_base + r * C)[g];
    const uint32_t byte = signs[r * G + g];
    reinterpret_cast<uint4 *>(w_eff + r * C)[g] = weff_group(w, byte, a);
}

}  // namespace

hipError_t launch_reconstruct(const uint16_t *w_base, const uint8_t *signs, const float *alpha,
                              bool per_matrix, int64_t d_out, int64_t d_in, uint16_t *w_eff,
                              hipStream_t s)
{
    const int64_t G = d_in >> 3;
    const int bpr = (int)((G + kThreads - 1) / kThreads);
    const dim3 grid((unsigned)(d_out * bpr)), block(kThreads);
    if (per_matrix)
        hipLaunchKernelGGL(reconstruct_rows<true>, grid, block, 0, s, w_base, signs, alpha, d_in, bpr, w_eff);
    else
        hipLaunchKernelGGL(reconstruct_rows<false>, grid, block, 0, s, w_base, signs, alpha, d_in, bpr, w_eff);
    return hipGetLastError();
}

}  // namespace bd
