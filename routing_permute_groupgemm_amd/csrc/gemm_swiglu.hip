// Entry point of the gate/up GroupGEMM with fused SwiGLU on the permuted rows;
// the kernel template is in gemm_kernel.hpp.
#include "gemm_kernel.hpp"

using moe_host::misaligned;

extern "C" int moe_grouped_gemm_swiglu(const moe_bf16* x_perm, const moe_bf16* w_gate, const moe_bf16* w_up,
                                       const int32_t* offsets, int e_local, int H, int F, int cap_rows,
                                       moe_bf16* h, moe_bf16* ab_save, moe_stream stream) {
    using namespace moe;
    if (e_local < 0 || e_local > kMaxGroups || H < 0 || F < 0 || cap_rows < 0) return MOE_EINVAL;
    if (H % 64 || F % 64) return MOE_ESHAPE;
    if (!offsets) return MOE_EINVAL;
    if (e_local == 0 || cap_rows == 0 || F == 0) return MOE_OK;
    if (!x_perm || !w_gate || !w_up || !h) return MOE_EINVAL;
    if (misaligned(x_perm) || misaligned(w_gate) || misaligned(w_up) || misaligned(offsets) || misaligned(h) ||
        misaligned(ab_save))
        return MOE_EALIGN;
    // load offsets are 32-bit and those at or past 2^31 mean "out of range":
    // 256 rows of A, and one expert's whole weight matrix, stay below that
    if ((int64_t)256 * H * 2 >= (1ll << 31) || (int64_t)H * F * 2 >= (1ll << 31)) return MOE_EINVAL;
    GemmParams p{};
    p.a = x_perm;
    p.lda = H;
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
    if (H == 0) return MOE_EINVAL;
    return launch<LAY_MN, EPI_SWIGLU, SCHED_ROWS>(p, (hipStream_t)stream);
}
