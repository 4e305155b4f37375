// Entry point of the generic GroupGEMM (down projection and the dgrad GEMMs)
// and the instantiations with an N-contiguous weight [Kd][N]; the kernel
// template is in gemm_kernel.hpp.
#include "gemm_kernel.hpp"

using moe_host::misaligned;

namespace moe {

int launch_rows_mn(const GemmParams& p, int epi, hipStream_t s) {
    if (epi == EPI_SWIGLU_BWD) return launch<LAY_MN, EPI_SWIGLU_BWD, SCHED_ROWS>(p, s);
    return launch<LAY_MN, EPI_BF16, SCHED_ROWS>(p, s);
}

}  // namespace moe

extern "C" int moe_grouped_gemm(const moe_bf16* a, int lda, const moe_bf16* w0, const moe_bf16* w1, int trans_w,
                                const int32_t* offsets, int e_local, int Kd, int N, int cap_rows, int epilogue,
                                const moe_bf16* ab, moe_bf16* c, int ldc, moe_stream stream) {
    using namespace moe;
    if (e_local < 0 || e_local > kMaxGroups || Kd <= 0 || N < 0 || cap_rows < 0) return MOE_EINVAL;
    if (trans_w != 0 && trans_w != 1) return MOE_EINVAL;
    if (epilogue != MOE_EPI_NONE && epilogue != MOE_EPI_SWIGLU_BWD) return MOE_EINVAL;
    if (Kd % 64 || N % 64) return MOE_ESHAPE;
    if (w1 && !trans_w) return MOE_EINVAL;
    const int acols = w1 ? 2 * Kd : Kd;
    const int ccols = epilogue == MOE_EPI_SWIGLU_BWD ? 2 * N : N;
    if (lda < acols || ldc < ccols || lda % 8 || ldc % 8) return MOE_EINVAL;
    if (!offsets) return MOE_EINVAL;
    if (e_local == 0 || cap_rows == 0 || N == 0) return MOE_OK;
    if (!a || !w0 || !c || (epilogue == MOE_EPI_SWIGLU_BWD && !ab)) return MOE_EINVAL;
    if (misaligned(a) || misaligned(w0) || misaligned(w1) || misaligned(offsets) || misaligned(ab) ||
        misaligned(c))
        return MOE_EALIGN;
    // 32-bit load offsets below 2^31 (see moe_grouped_gemm_swiglu)
    if ((int64_t)256 * lda * 2 >= (1ll << 31) || (int64_t)256 * Kd * 2 >= (1ll << 31) ||
        (int64_t)Kd * N * 2 >= (1ll << 31))
        return MOE_EINVAL;
    GemmParams p{};
    p.a = a;
    p.lda = lda;
    p.w0 = w0;
    p.w1 = w1;
    p.w_stride = (int64_t)Kd * N;
    p.ldw = trans_w ? Kd : N;
    p.two_seg = w1 != nullptr;
    p.offsets = offsets;
    p.e_local = e_local;
    p.cap = cap_rows;
    p.N = N;
    p.Kd = Kd;
    p.c = c;
    p.ldc = ldc;
    p.ab = ab;
    hipStream_t s = (hipStream_t)stream;
    const int epi = epilogue == MOE_EPI_SWIGLU_BWD ? EPI_SWIGLU_BWD : EPI_BF16;
    return trans_w ? launch_rows_kc(p, epi, s) : launch_rows_mn(p, epi, s);
}
