// Entry point of the zero-copy gate/up GroupGEMM (A rows read from the tokens
// through src); the kernel template is in gemm_kernel.hpp.
#include "gemm_kernel.hpp"

using moe_host::misaligned;

extern "C" int moe_grouped_gemm_swiglu_gather(const moe_bf16* x, int T, const int32_t* src, int K,
                                              const moe_bf16* w_gate, const moe_bf16* w_up, const int32_t* offsets,
                                              int e_local, int H, int F, int cap_rows, moe_bf16* h,
                                              moe_bf16* ab_save, moe_stream stream) {
    using namespace moe;
    if (e_local < 0 || e_local > kMaxGroups || H <= 0 || F < 0 || cap_rows < 0 || T < 0 || K < 1 || K > 16)
        return MOE_EINVAL;
    if (H % 64 || F % 64) return MOE_ESHAPE;
    // every A load offset (row * H * 2 + column bytes) must stay below the
    // out-of-range offset that masks rows past an expert's end
    if ((int64_t)T * H * 2 > (int64_t)kOOB_GATHER || (int64_t)H * F * 2 >= (1ll << 31)) return MOE_EINVAL;
    if ((int64_t)cap_rows > (int64_t)T * K) return MOE_EINVAL;
    if (!offsets) return MOE_EINVAL;
    if (e_local == 0 || cap_rows == 0 || F == 0) return MOE_OK;
    if (!x || !src || !w_gate || !w_up || !h) return MOE_EINVAL;
    if (misaligned(x) || misaligned(src) || misaligned(w_gate) || misaligned(w_up) || misaligned(offsets) ||
        misaligned(h) || misaligned(ab_save))
        return MOE_EALIGN;
    GemmParams p{};
    p.a = x;
    p.lda = H;
    p.src = src;
    p.topk = K;
    p.topk_rcp = 0xffffffffu / (uint32_t)K;
    p.a_rows = T;
    p.w0 = w_gate;
    p.w1 = w_up;
    p.w_stride = (int64_t)H * F;
    p.ldw = F;
    p.offsets = offsets;
    p.e_local = e_local;
    p.cap = cap_rows;
    p.N = F;
    p.Kd = H;
    p.c = h;
    p.ldc = F;
    p.c2 = ab_save;
    return launch<LAY_MN, EPI_SWIGLU, SCHED_ROWS, true>(p, (hipStream_t)stream);
}
