// Definition of launch_mfma_op (see sgemm_launch.hpp): one workgroup per output tile
// (1-D grid, blockIdx.z = batch), and the kernel variant for the alignment (VEC) and
// for whether any tile crosses the matrix edge (EDGE).
#pragma once

#include "sgemm_launch.hpp"

namespace sgemm_impl {

template <int BM, int BN, int BK, int WGM, int WGN, int WGK, int PF, int GROUP_M, bool TA, bool TB>
hipError_t launch_mfma_op(const GemmArgs &p, int batch, bool vec, bool edge, hipStream_t s)
{
    const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    const dim3 grid(tiles, 1, batch), block(WGM * WGN * WGK * 64);
    if (vec && !edge)
        hipLaunchKernelGGL((sgemm_mfma<BM, BN, BK, WGM, WGN, WGK, PF, TA, TB, true, false>), grid, block, 0, s, p,
                           GROUP_M);
    else if (vec)
        hipLaunchKernelGGL((sgemm_mfma<BM, BN, BK, WGM, WGN, WGK, PF, TA, TB, true, true>), grid, block, 0, s, p,
                           GROUP_M);
    else
        hipLaunchKernelGGL((sgemm_mfma<BM, BN, BK, WGM, WGN, WGK, PF, TA, TB, false, true>), grid, block, 0, s, p,
                           GROUP_M);
    return hipGetLastError();
}

}  // namespace sgemm_impl
