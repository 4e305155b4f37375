// Instantiations of the row-tiled GroupGEMM with a contraction-contiguous
// weight [N][Kd] (the dgrad GEMMs and the router's input gradient); the
// kernel template is in gemm_kernel.hpp.
#include "gemm_kernel.hpp"

namespace moe {

int launch_rows_kc(const GemmParams& p, int epi, hipStream_t s) {
    if (epi == EPI_SWIGLU_BWD) return launch<LAY_KC, EPI_SWIGLU_BWD, SCHED_ROWS>(p, s);
    return launch<LAY_KC, EPI_BF16, SCHED_ROWS>(p, s);
}

}  // namespace moe
