// Instantiates the MFMA launchers of every configuration for one operand form, given
// on the compiler command line as SGEMM_TA and SGEMM_TB (0 or 1 each).
#include "sgemm_configs.inc"
#include "sgemm_launch_impl.hpp"

#if !defined(SGEMM_TA) || !defined(SGEMM_TB)
#error "compile with -DSGEMM_TA=<0|1> -DSGEMM_TB=<0|1>"
#endif

namespace sgemm_impl {

#define SGEMM_INSTANTIATE(name, BM, BN, BK, WGM, WGN, WGK, PF, DMA, GROUP_M, MB)                        \
    template hipError_t                                                                                 \
    launch_mfma_op<BM, BN, BK, WGM, WGN, WGK, PF, DMA, GROUP_M, MB, (SGEMM_TA != 0), (SGEMM_TB != 0)>(     \
        const GemmArgs &, int, bool, bool, bool, hipStream_t);
SGEMM_MFMA_CONFIGS(SGEMM_INSTANTIATE)
#undef SGEMM_INSTANTIATE

#define SGEMM_INSTANTIATE_SK(name, BM, BN, BK, WGM, WGN, WGK, PF, DMA, GROUP_M, MB)                     \
    template hipError_t                                                                                 \
    launch_mfma_sk_op<BM, BN, BK, WGM, WGN, WGK, PF, DMA, GROUP_M, MB, (SGEMM_TA != 0), (SGEMM_TB != 0)>(  \
        const GemmArgs &, const StreamK &, int, bool, bool, bool, hipStream_t);
SGEMM_SK_CONFIGS(SGEMM_INSTANTIATE_SK)
#undef SGEMM_INSTANTIATE_SK

}  // namespace sgemm_impl
