// Definition of launch_mfma_op (see sgemm_launch.hpp): one workgroup per output tile
// (1-D grid, blockIdx.z = batch), and the kernel variant for the alignment (VEC) and
// for whether any tile crosses the matrix edge (EDGE). Unaligned operands (element-wise
// loads, several times the address registers) always take the register-staged kernel
// with one K-tile in flight, and with K-tiles of 16 * WGK for direct-copy configurations,
// so that variant fits the register file for every tile shape.
#pragma once

#include "sgemm_launch.hpp"

namespace sgemm_impl {

template <int BM, int BN, int BK, int WGM, int WGN, int WGK, int PF, bool DMA, int GROUP_M, bool TA, bool TB>
hipError_t launch_mfma_op(const GemmArgs &p, int batch, bool vec, bool edge, hipStream_t s)
{
    constexpr int BKU = DMA ? 16 * WGK : BK;            // K-tile of the unaligned variant
    const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    const dim3 grid(tiles, 1, batch), block(WGM * WGN * WGK * 64);
    if (vec && !edge)
        hipLaunchKernelGGL((sgemm_mfma<BM, BN, BK, WGM, WGN, WGK, PF, DMA, TA, TB, true, false>), grid, block, 0, s,
                           p, GROUP_M);
    else if (vec)
        hipLaunchKernelGGL((sgemm_mfma<BM, BN, BK, WGM, WGN, WGK, PF, DMA, TA, TB, true, true>), grid, block, 0, s,
                           p, GROUP_M);
    else
        hipLaunchKernelGGL((sgemm_mfma<BM, BN, BKU, WGM, WGN, WGK, 1, false, TA, TB, false, true>), grid, block, 0,
                           s, p, GROUP_M);
    return hipGetLastError();
}

template <int BM, int BN, int BK, int WGM, int WGN, int WGK, int PF, bool DMA, int GROUP_M, bool TA, bool TB>
hipError_t launch_mfma_sk_op(const GemmArgs &p, const StreamK &sk, int grid, bool vec, bool edge, hipStream_t s)
{
    const dim3 block(WGM * WGN * WGK * 64);
    if (vec && !edge)
        hipLaunchKernelGGL((sgemm_mfma_sk<BM, BN, BK, WGM, WGN, WGK, PF, DMA, TA, TB, true, false>), dim3(grid),
                           block, 0, s, p, sk);
    else if (vec)
        hipLaunchKernelGGL((sgemm_mfma_sk<BM, BN, BK, WGM, WGN, WGK, PF, DMA, TA, TB, true, true>), dim3(grid),
                           block, 0, s, p, sk);
    else    // unaligned operands: the data-parallel kernel of the same tile (see launch_mfma_op)
        hipLaunchKernelGGL((sgemm_mfma<BM, BN, BK, WGM, WGN, WGK, 1, false, TA, TB, false, true>),
                           dim3(sk.tiles_m * sk.tiles_n), block, 0, s, p, GROUP_M);
    return hipGetLastError();
}

}  // namespace sgemm_impl
