// Router projection and its backward on the GroupGEMM kernel (dense mode:
// one group of all T rows); the kernel template is in gemm_kernel.hpp.
#include "gemm_kernel.hpp"

using moe_host::misaligned;

namespace moe {

// Chunks of a contraction of kt_total steps so that `tiles` output tiles
// become at most one workgroup per compute unit (a second, partial round of
// workgroups would double the time), each chunk at least 8 steps.
static void split_steps(int64_t tiles, int64_t kt_total, int* n_chunks, int* steps) {
    kt_total = std::max<int64_t>(kt_total, 1);  // no tokens: one (empty) chunk
    const int64_t cus = moe_host::num_cus();
    int64_t s = std::min<int64_t>(cus / std::max<int64_t>(tiles, 1), std::max<int64_t>(kt_total / 8, 1));
    s = std::max<int64_t>(s, 1);
    const int64_t st = (kt_total + s - 1) / s;
    *steps = (int)st;
    *n_chunks = (int)((kt_total + st - 1) / st);
}

struct RouterPlan {
    bool fwd_small;               // forward on 128x128 tiles (too few 256x256 tiles to fill the GPU)
    int fwd_chunks, fwd_steps;    // forward: contraction over H in chunks of fwd_steps * 32
    int bwd_chunks, bwd_rows;     // weight gradient: token rows in chunks of bwd_rows
    size_t fwd_bytes, bwd_bytes;  // workspace
};

static size_t round256(size_t b) { return (b + 255) / 256 * 256; }

static RouterPlan router_plan(int T, int H, int E) {
    RouterPlan r{};
    // Few rows: 128x128 tiles, whose smaller fp32 partials cost less to write
    // and add than the 256x256 tiles' (the partials, not the MFMAs, bound a
    // forward cut into many chunks).
    const int64_t big_tiles = (int64_t)((T + 255) / 256) * ((E + 255) / 256);
    r.fwd_small = big_tiles < moe_host::num_cus();
    const int tm = r.fwd_small ? 128 : 256;
    split_steps((int64_t)((T + tm - 1) / tm) * ((E + tm - 1) / tm), H / 32, &r.fwd_chunks, &r.fwd_steps);
    int steps;
    split_steps((int64_t)((H + 255) / 256) * ((E + 255) / 256), (T + 31) / 32, &r.bwd_chunks, &steps);
    r.bwd_rows = steps * 32;
    r.bwd_chunks = std::max(1, (T + r.bwd_rows - 1) / r.bwd_rows);
    r.fwd_bytes = r.fwd_chunks > 1 ? (size_t)r.fwd_chunks * T * E * 4 : 0;
    r.bwd_bytes = round256((size_t)T * E * 2) + (r.bwd_chunks > 1 ? (size_t)r.bwd_chunks * H * E * 4 : 0);
    return r;
}

static int router_check(int T, int H, int E) {
    if (T < 0 || H <= 0 || E <= 0 || E > 4096) return MOE_EINVAL;
    if (H % 64 || E % 64) return MOE_ESHAPE;
    // every buffer descriptor spans at most 256 rows of x or all of W_r
    if ((int64_t)T * E >= (1ll << 31) || (int64_t)T * H >= (1ll << 40) || (int64_t)256 * H * 2 >= (1ll << 31) ||
        (int64_t)H * E * 2 >= (1ll << 31))
        return MOE_EINVAL;
    return MOE_OK;
}

}  // namespace moe

extern "C" size_t moe_router_workspace_size(int T, int H, int E) {
    using namespace moe;
    if (router_check(T, H, E) != MOE_OK) return 0;
    const RouterPlan r = router_plan(T, H, E);
    return std::max(r.fwd_bytes, r.bwd_bytes) + 256;
}

extern "C" int moe_router_logits(const moe_bf16* x, int T, int H, const moe_bf16* w_r, int E, const float* bias,
                                 float* logits, void* ws, size_t ws_bytes, moe_stream stream) {
    using namespace moe;
    const int st = router_check(T, H, E);
    if (st != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    if (!x || !w_r || !logits) return MOE_EINVAL;
    if (misaligned(x) || misaligned(w_r) || misaligned(bias) || misaligned(logits) || misaligned(ws))
        return MOE_EALIGN;
    const RouterPlan r = router_plan(T, H, E);
    if (r.fwd_bytes && (!ws || ws_bytes < r.fwd_bytes)) return MOE_EWORKSPACE;
    const bool split = r.fwd_chunks > 1;
    GemmParams p{};
    p.a = x;
    p.lda = H;
    p.w0 = w_r;
    p.ldw = E;
    p.dense_rows = T;
    p.row_chunk = T;
    p.e_local = 1;
    p.cap = T;
    p.N = E;
    p.Kd = H;
    p.cf = split ? (float*)ws : logits;
    p.ldc = E;
    p.ksplit = r.fwd_chunks;
    p.kchunk = r.fwd_steps * 32;
    p.part_stride = (int64_t)T * E;
    p.bias = split ? nullptr : bias;
    hipStream_t s = (hipStream_t)stream;
    int rc = r.fwd_small ? launch_cfg<128, 128, 32, 2, 2, LAY_MN, EPI_F32, SCHED_ROWS, kLdsBudget>(p, s)
                         : launch<LAY_MN, EPI_F32, SCHED_ROWS>(p, s);
    if (rc != MOE_OK || !split) return rc;
    return moe_host::sum_partials((const float*)ws, r.fwd_chunks, (int64_t)T * E, (int64_t)T * E, bias, E, logits, s);
}

extern "C" int moe_router_backward(const moe_bf16* x, int T, int H, const moe_bf16* w_r, int E, const float* dlogits,
                                   moe_bf16* dx, float* dw_r, void* ws, size_t ws_bytes, moe_stream stream) {
    using namespace moe;
    const int st = router_check(T, H, E);
    if (st != MOE_OK) return st;
    if (!w_r || !dw_r || (T > 0 && (!x || !dlogits || !dx))) return MOE_EINVAL;
    if (misaligned(x) || misaligned(w_r) || misaligned(dlogits) || misaligned(dx) || misaligned(dw_r) ||
        misaligned(ws))
        return MOE_EALIGN;
    const RouterPlan r = router_plan(T, H, E);
    if (!ws || ws_bytes < r.bwd_bytes) return MOE_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    uint16_t* dl16 = (uint16_t*)ws;
    float* part = (float*)((char*)ws + round256((size_t)T * E * 2));
    int rc = moe_host::cast_f32_bf16(dlogits, (int64_t)T * E, dl16, s);
    if (rc != MOE_OK) return rc;
    // dx = bf16(dlogits) . W_r^T: W_r [H][E] is the [N][Kd] weight, contraction contiguous
    GemmParams p{};
    p.a = dl16;
    p.lda = E;
    p.w0 = w_r;
    p.ldw = E;
    p.dense_rows = T;
    p.row_chunk = T;
    p.e_local = 1;
    p.cap = T;
    p.N = H;
    p.Kd = E;
    p.c = dx;
    p.ldc = H;
    if (T > 0) {
        rc = launch_rows_kc(p, EPI_BF16, s);
        if (rc != MOE_OK) return rc;
    }
    // dW_r = x^T . bf16(dlogits): the token rows in chunks, one fp32 partial each
    const bool split = r.bwd_chunks > 1;
    GemmParams q{};
    q.a = x;
    q.lda = H;
    q.b = dl16;
    q.ldb = E;
    q.dense_rows = T;
    q.row_chunk = r.bwd_rows;
    q.e_local = r.bwd_chunks;
    q.cap = T;
    q.M = H;
    q.N = E;
    q.cf = split ? part : dw_r;
    q.n_split = E;
    rc = launch_wgrad(q, s);
    if (rc != MOE_OK || !split) return rc;
    return moe_host::sum_partials(part, r.bwd_chunks, (int64_t)H * E, (int64_t)H * E, nullptr, E, dw_r, s);
}
