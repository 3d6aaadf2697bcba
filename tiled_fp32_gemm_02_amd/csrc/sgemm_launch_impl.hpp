// Definition of launch_mfma_op (see sgemm_launch.hpp): one workgroup per output tile
// (1-D grid, blockIdx.z = batch), and the kernel variant for the alignment (VEC) and
// for whether any tile crosses the matrix edge (EDGE).
//
// Unaligned operands (rows only 4-byte aligned): a direct-copy configuration keeps its
// 16-byte copies, from 4-byte aligned addresses, and copies the K-tile that holds the end
// of K in 4-byte words (TileDMA's U form), with its K-tiles in flight. A register-staged
// configuration keeps its own K-tile and loads in flight, with 16-byte loads of the chunks
// wholly inside a row and element-wise ones for the chunk that straddles its end. Calls
// the direct copies cannot take (dma_ok false: row strides too long for 32-bit copy
// offsets, or shorter than 4 floats) run the register-staged kernel with one K-tile in
// flight and K-tiles of two k groups per wave group (16 * WGK for 32x32 blocks, 32 * WGK
// for 16x16 ones), so that variant fits the register file for every tile shape. A
// register-staged stream-K configuration runs the data-parallel kernel of its tile on
// unaligned operands: stream-K itself was measured slower there on every odd-sized shape
// swept.
#pragma once

#include "sgemm_launch.hpp"

namespace sgemm_impl {

template <int BM, int BN, int BK, int WGM, int WGN, int WGK, int PF, bool DMA, int GROUP_M, int MB, bool TA,
          bool TB>
hipError_t launch_mfma_op(const GemmArgs &p, int batch, bool vec, bool edge, bool dma_ok, hipStream_t s)
{
    constexpr int NT = WGM * WGN * WGK * 64;
    constexpr int BKU = DMA ? 8 * (64 / MB) * WGK : BK;  // K-tile of the register-staged unaligned variant
    // The caller has checked that tiles x NT fits one launch; the sums are unsigned so that
    // M or N near 2^31 does not overflow.
    // With p.fringe > 0 the tiles stop at column N - fringe and kFringeRows rows of the last
    // columns go to each workgroup after them.
    const unsigned tiles = (((unsigned)p.M + BM - 1) / BM) * (((unsigned)(p.N - p.fringe) + BN - 1) / BN) +
                           (p.fringe > 0 ? ((unsigned)p.M + kFringeRows - 1) / kFringeRows : 0u);
    const dim3 grid(tiles, 1, batch), block(NT);
    if (DMA && !dma_ok)
        vec = false;                                    // only the register-staged variant takes long rows
    if (vec && !edge)
        hipLaunchKernelGGL((sgemm_mfma<BM, BN, BK, WGM, WGN, WGK, PF, DMA, TA, TB, true, false, MB>), grid, block, 0, s,
                           p, GROUP_M);
    else if (vec)
        hipLaunchKernelGGL((sgemm_mfma<BM, BN, BK, WGM, WGN, WGK, PF, DMA, TA, TB, true, true, MB>), grid, block, 0, s,
                           p, GROUP_M);
    else if constexpr (!DMA)    // register-staged configuration: its own K-tile and loads in flight
        hipLaunchKernelGGL((sgemm_mfma<BM, BN, BK, WGM, WGN, WGK, PF, false, TA, TB, false, true, MB>), grid, block, 0,
                           s, p, GROUP_M);
    else if (!dma_ok)
        hipLaunchKernelGGL((sgemm_mfma<BM, BN, BKU, WGM, WGN, WGK, 1, false, TA, TB, false, true, MB>), grid, block, 0,
                           s, p, GROUP_M);
    else    // direct copies on 4-byte aligned rows (the U form)
        hipLaunchKernelGGL((sgemm_mfma<BM, BN, BK, WGM, WGN, WGK, PF, true, TA, TB, false, true, MB>), grid, block, 0,
                           s, p, GROUP_M);
    return hipGetLastError();
}

template <int BM, int BN, int BK, int WGM, int WGN, int WGK, int PF, bool DMA, int GROUP_M, int MB, bool TA,
          bool TB>
hipError_t launch_mfma_sk_op(const GemmArgs &p, const StreamK &sk, int grid, bool vec, bool edge, bool dma_ok,
                             hipStream_t s)
{
    constexpr int NT = WGM * WGN * WGK * 64;
    const dim3 block(NT);
    // Calls the direct copies cannot take, and unaligned operands of a register-staged
    // configuration, run the register-staged data-parallel kernel of the tile.
    const bool staged = (DMA && !dma_ok) || (!vec && !DMA);
    if (staged)
        hipLaunchKernelGGL((sgemm_mfma<BM, BN, BK, WGM, WGN, WGK, PF, false, TA, TB, false, true, MB>),
                           dim3(sk.tiles_m * sk.tiles_n), block, 0, s, p, GROUP_M);
    else if (vec && !edge)
        hipLaunchKernelGGL((sgemm_mfma_sk<BM, BN, BK, WGM, WGN, WGK, PF, DMA, TA, TB, true, false, MB>), dim3(grid),
                           block, 0, s, p, sk);
    else if (vec)
        hipLaunchKernelGGL((sgemm_mfma_sk<BM, BN, BK, WGM, WGN, WGK, PF, DMA, TA, TB, true, true, MB>), dim3(grid),
                           block, 0, s, p, sk);
    else if constexpr (DMA)    // rows only 4-byte aligned: the U form of the direct copies
        hipLaunchKernelGGL((sgemm_mfma_sk<BM, BN, BK, WGM, WGN, WGK, PF, true, TA, TB, false, true, MB>), dim3(grid),
                           block, 0, s, p, sk);
    return hipGetLastError();
}

}  // namespace sgemm_impl
