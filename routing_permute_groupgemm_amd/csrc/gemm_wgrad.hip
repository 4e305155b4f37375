// Entry point and instantiation of the weight-gradient GroupGEMM (the
// transposed GroupGEMM over each expert's rows); the kernel template is in
// gemm_kernel.hpp.
#include "gemm_kernel.hpp"

using moe_host::misaligned;

namespace moe {

int launch_wgrad(const GemmParams& p, hipStream_t s) { return launch<LAY_MN, EPI_F32, SCHED_WGRAD>(p, s); }

}  // namespace moe

extern "C" int moe_wgrad(const moe_bf16* a, int lda, const moe_bf16* b, int ldb, const int32_t* offsets,
                         int e_local, int M, int N, int cap_rows, float* dw, moe_stream stream) {
    using namespace moe;
    if (e_local < 0 || e_local > kMaxGroups || M < 0 || N < 0 || cap_rows < 0) return MOE_EINVAL;
    if (M % 64 || N % 64) return MOE_ESHAPE;
    if (lda < M || ldb < N || lda % 8 || ldb % 8) return MOE_EINVAL;
    if (!offsets) return MOE_EINVAL;
    if (e_local == 0 || M == 0 || N == 0) return MOE_OK;
    if (!dw || (cap_rows > 0 && (!a || !b))) return MOE_EINVAL;
    if (misaligned(a) || misaligned(b) || misaligned(offsets) || misaligned(dw)) return MOE_EALIGN;
    if ((int64_t)64 * lda * 2 >= (1ll << 31) || (int64_t)64 * ldb * 2 >= (1ll << 31)) return MOE_EINVAL;
    GemmParams p{};
    p.a = a;
    p.lda = lda;
    p.b = b;
    p.ldb = ldb;
    p.offsets = offsets;
    p.e_local = e_local;
    p.cap = cap_rows;
    p.M = M;
    p.N = N;
    p.cf = dw;
    return launch_wgrad(p, (hipStream_t)stream);
}

// ---- router projection -------------------------------------------------------
// Dense GEMMs on the same kernel: one group of all T rows (no offsets array).
// Few output tiles (E columns) would leave most of the chip idle, so the
// contraction is cut into chunks, each leaving an fp32 partial that a second
// pass adds in chunk order: the result is fixed for a given device, whatever
// the scheduling.
