// Entry points and instantiation of the weight-gradient GroupGEMM (the
// transposed GroupGEMM over each expert's rows); the kernel template is in
// gemm_kernel.hpp.
//
// moe_wgrad sums each expert's rows in one fixed order per output element.
// moe_wgrad_split is the non-bitwise variant the UniEP paper measures against
// it (evaluation, "Performance Cost of Bitwise Reproducibility", Table 7):
// each expert's rows are cut into `splits` fixed chunks, the chunks run as
// separate groups of the same kernel, each leaving an fp32 partial, and a
// second pass adds the partials in chunk order.  The result is identical from
// run to run but is not the one-pass order of moe_wgrad.
#include "gemm_kernel.hpp"

using moe_host::misaligned;

namespace moe {

int launch_wgrad(const GemmParams& p, hipStream_t s) { return launch<LAY_MN, EPI_F32, SCHED_WGRAD>(p, s); }
static int launch_wgrad_gather(const GemmParams& p, hipStream_t s) {
    return launch<LAY_MN, EPI_F32, SCHED_WGRAD, true>(p, s);
}

// Offsets of the split groups: group j*S + c holds chunk c of expert j, rows
// [off[j] + min(c*len, n), off[j] + min((c+1)*len, n)) with n the expert's
// rows and len = ceil(n / S) rounded up to whole 32-row k-steps, so every
// chunk but the last of an expert starts and ends on a k-step.  The groups
// stay in row order: this is a refinement of the experts' row partition.
__global__ __launch_bounds__(256) void split_offsets_kernel(const int32_t* __restrict__ off, int EL, int S,
                                                            int32_t* __restrict__ off2) {
    for (int j = blockIdx.x * 256 + threadIdx.x; j < EL; j += gridDim.x * 256) {
        const int lo = off[j], n = off[j + 1] - lo;
        const int len = ((n + S - 1) / S + 31) / 32 * 32;
        for (int c = 0; c < S; ++c) off2[j * S + c] = lo + min(c * len, n);
        if (j == EL - 1) off2[EL * S] = off[EL];
    }
}

// dw[j][i] = part[j*S][i] + part[j*S + 1][i] + ... (chunk order), i < MN
__global__ __launch_bounds__(256) void sum_split_kernel(const f32x4* __restrict__ part, int EL, int S, int64_t mn4,
                                                        f32x4* __restrict__ out) {
    const int64_t n4 = (int64_t)EL * mn4;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < n4; q += (int64_t)gridDim.x * 256) {
        const int64_t j = q / mn4, i = q - j * mn4;
        const f32x4* pj = part + j * S * mn4 + i;
        f32x4 acc = __builtin_nontemporal_load(pj);
        for (int c = 1; c < S; ++c) acc += __builtin_nontemporal_load(pj + c * mn4);
        out[q] = acc;
    }
}

static size_t round256(size_t b) { return (b + 255) / 256 * 256; }

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
    p.n_split = N;
    return launch_wgrad(p, (hipStream_t)stream);
}

extern "C" int moe_wgrad_gate_up(const moe_bf16* x_perm, int H, const moe_bf16* dab, int F, const int32_t* offsets,
                                 int e_local, int cap_rows, float* dw_gate, float* dw_up, moe_stream stream) {
    using namespace moe;
    if (e_local < 0 || e_local > kMaxGroups || H < 0 || F < 0 || cap_rows < 0) return MOE_EINVAL;
    if (H % 64 || F % 64) return MOE_ESHAPE;
    if (!offsets) return MOE_EINVAL;
    if (e_local == 0 || H == 0 || F == 0) return MOE_OK;
    if (!dw_gate || !dw_up || (cap_rows > 0 && (!x_perm || !dab))) return MOE_EINVAL;
    if (misaligned(x_perm) || misaligned(dab) || misaligned(offsets) || misaligned(dw_gate) || misaligned(dw_up))
        return MOE_EALIGN;
    if ((int64_t)64 * H * 2 >= (1ll << 31) || (int64_t)64 * 2 * F * 2 >= (1ll << 31)) return MOE_EINVAL;
    // one transposed GroupGEMM over [da | db]: output columns n < F are dW_gate, the rest dW_up
    GemmParams p{};
    p.a = x_perm;
    p.lda = H;
    p.b = dab;
    p.ldb = 2 * F;
    p.offsets = offsets;
    p.e_local = e_local;
    p.cap = cap_rows;
    p.M = H;
    p.N = 2 * F;
    p.cf = dw_gate;
    p.cf2 = dw_up;
    p.n_split = F;
    return launch_wgrad(p, (hipStream_t)stream);
}

extern "C" int moe_wgrad_gate_up_gather(const moe_bf16* x, int T, const int32_t* src, int K, int H,
                                        const moe_bf16* dab, int F, const int32_t* offsets, int e_local,
                                        int cap_rows, float* dw_gate, float* dw_up, moe_stream stream) {
    using namespace moe;
    if (e_local < 0 || e_local > kMaxGroups || H < 0 || F < 0 || cap_rows < 0 || T < 0 || K < 1 || K > 16)
        return MOE_EINVAL;
    if (H % 64 || F % 64) return MOE_ESHAPE;
    // every A load offset (token * H * 2 + column bytes) must stay below the
    // out-of-range offset that masks rows past an expert's end
    if ((int64_t)T * H * 2 > (int64_t)kOOB_GATHER || (int64_t)64 * 2 * F * 2 >= (1ll << 31)) return MOE_EINVAL;
    if ((int64_t)cap_rows > (int64_t)T * K) return MOE_EINVAL;
    if (!offsets) return MOE_EINVAL;
    if (e_local == 0 || H == 0 || F == 0) return MOE_OK;
    if (!dw_gate || !dw_up || (cap_rows > 0 && (!x || !src || !dab))) return MOE_EINVAL;
    if (misaligned(x) || misaligned(src) || misaligned(dab) || misaligned(offsets) || misaligned(dw_gate) ||
        misaligned(dw_up))
        return MOE_EALIGN;
    GemmParams p{};
    p.a = x;
    p.lda = H;
    p.a_rows = T;
    p.src = src;
    p.topk = K;
    p.topk_rcp = 0xffffffffu / (uint32_t)K;
    p.b = dab;
    p.ldb = 2 * F;
    p.offsets = offsets;
    p.e_local = e_local;
    p.cap = cap_rows;
    p.M = H;
    p.N = 2 * F;
    p.cf = dw_gate;
    p.cf2 = dw_up;
    p.n_split = F;
    return launch_wgrad_gather(p, (hipStream_t)stream);
}

extern "C" size_t moe_wgrad_split_workspace_size(int e_local, int M, int N, int splits) {
    using namespace moe;
    if (e_local < 0 || M < 0 || N < 0 || splits < 1 || (int64_t)e_local * splits > kMaxGroups) return 0;
    if (splits == 1) return 0;
    return round256((size_t)(e_local * splits + 1) * 4) + (size_t)e_local * splits * M * N * 4;
}

extern "C" int moe_wgrad_split(const moe_bf16* a, int lda, const moe_bf16* b, int ldb, const int32_t* offsets,
                               int e_local, int M, int N, int cap_rows, int splits, float* dw, void* ws,
                               size_t ws_bytes, moe_stream stream) {
    using namespace moe;
    if (splits < 1 || e_local < 0 || (int64_t)e_local * splits > kMaxGroups) return MOE_EINVAL;
    if (splits == 1) return moe_wgrad(a, lda, b, ldb, offsets, e_local, M, N, cap_rows, dw, stream);
    // the same checks as moe_wgrad, then the workspace
    if (M < 0 || N < 0 || cap_rows < 0) return MOE_EINVAL;
    if (M % 64 || N % 64) return MOE_ESHAPE;
    if (lda < M || ldb < N || lda % 8 || ldb % 8) return MOE_EINVAL;
    if (!offsets) return MOE_EINVAL;
    if (e_local == 0 || M == 0 || N == 0) return MOE_OK;
    if (!dw || (cap_rows > 0 && (!a || !b))) return MOE_EINVAL;
    if (misaligned(a) || misaligned(b) || misaligned(offsets) || misaligned(dw) || misaligned(ws)) return MOE_EALIGN;
    if ((int64_t)64 * lda * 2 >= (1ll << 31) || (int64_t)64 * ldb * 2 >= (1ll << 31)) return MOE_EINVAL;
    const size_t need = moe_wgrad_split_workspace_size(e_local, M, N, splits);
    if (!ws || ws_bytes < need) return MOE_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    int32_t* off2 = (int32_t*)ws;
    float* part = (float*)((char*)ws + round256((size_t)(e_local * splits + 1) * 4));
    split_offsets_kernel<<<(e_local + 255) / 256, 256, 0, s>>>(offsets, e_local, splits, off2);
    int rc = moe_host::launch_status();
    if (rc != MOE_OK) return rc;
    GemmParams p{};
    p.a = a;
    p.lda = lda;
    p.b = b;
    p.ldb = ldb;
    p.offsets = off2;
    p.e_local = e_local * splits;
    p.cap = cap_rows;
    p.M = M;
    p.N = N;
    p.cf = part;
    p.n_split = N;
    rc = launch_wgrad(p, s);
    if (rc != MOE_OK) return rc;
    const int64_t mn4 = (int64_t)M * N / 4;
    const int64_t blocks = std::min<int64_t>((e_local * mn4 + 255) / 256, (int64_t)moe_host::num_cus() * 8);
    sum_split_kernel<<<(int)blocks, 256, 0, s>>>((const f32x4*)part, e_local, splits, mn4, (f32x4*)dw);
    return moe_host::launch_status();
}
