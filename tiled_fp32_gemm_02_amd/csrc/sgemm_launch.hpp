// Host-side launcher of one MFMA kernel configuration for one operand form. Declared
// here, defined in sgemm_launch_impl.hpp and instantiated in sgemm_inst.hip, which is
// compiled once per operand form (TA, TB) so the four sets build in parallel.
#pragma once

#include <hip/hip_runtime.h>

#include "sgemm_kernels.hpp"

namespace sgemm_impl {

template <int BM, int BN, int BK, int WGM, int WGN, int WGK, int PF, bool DMA, int GROUP_M, int MB, bool TA,
          bool TB>
hipError_t launch_mfma_op(const GemmArgs &p, int batch, bool vec, bool edge, bool dma_ok, hipStream_t s);

// Stream-K launch of the same tile kernel: `grid` workgroups share the work described
// by sk (batch 1). Operands that the kernel cannot take (unaligned ones of a
// register-staged configuration, or row strides the direct copies cannot take) run the
// data-parallel kernel of the tile.
template <int BM, int BN, int BK, int WGM, int WGN, int WGK, int PF, bool DMA, int GROUP_M, int MB, bool TA,
          bool TB>
hipError_t launch_mfma_sk_op(const GemmArgs &p, const StreamK &sk, int grid, bool vec, bool edge, bool dma_ok,
                             hipStream_t s);

}  // namespace sgemm_impl
