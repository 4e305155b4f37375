/*
 * moe.h -- C ABI of the one-GPU MoE layer hot path for AMD Instinct MI355X
 * (gfx950).  Plain pointers and sizes only.
 *
 * What is computed follows the UniEP paper (arXiv 2604.19241): the "MoE
 * workflow" paragraph (routing probabilities and top-k, a stable expert-grouped
 * permutation, GroupGEMM -> SwiGLU -> GroupGEMM, gate-weighted combine, and a
 * backward whose weight gradient is a transposed GroupGEMM), the "Deterministic
 * Token Mapping" section (destination row = exclusive prefix of per-expert
 * counts + the token's stable index inside its expert, no atomics deciding
 * order), the "Top-k accumulation constraint" paragraph (a token's K
 * contributions are summed together in one fixed order) and the MoonEP page
 * (the dispatch gradient sums each token's K copies).
 *
 * Notation: T tokens, H hidden, F expert intermediate, E router experts,
 * K top-k, e_local local experts [e_begin, e_begin+e_local), R routed local
 * rows (= offsets[e_local], lives on the device), cap_rows the row capacity
 * of every permuted buffer.  All matrices are row-major, last index
 * contiguous.  bf16 values are raw 16-bit patterns; fp32 -> bf16 rounding is
 * round-to-nearest-even.
 *
 * Conventions common to every entry point:
 *  - All data pointers are DEVICE pointers, owned by the caller, and must be
 *    16-byte aligned.  The library allocates nothing and keeps no state
 *    between calls (the one exception is moe_permute_noalloc's device
 *    array); calls on different streams with disjoint buffers may run
 *    concurrently.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    negative moe_status is returned and nothing runs on error.  Launch
 *    failures are reported as MOE_EHIP.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *    returns without waiting.  No call ever reads device memory from the
 *    host, so R and per-expert row counts never leave the device.
 *  - Results are bitwise identical from run to run: no floating-point
 *    atomics, every sum has a fixed order.
 *  - Rows of the permuted buffers at or beyond R are unspecified.
 *  - Limits: H and F multiples of 64; 1 <= K <= 16, K <= E <= 512;
 *    e_local <= 512; T*K < 2^31; cap_rows <= T*K; one expert's weight
 *    matrix below 2 GiB (H*F*2 < 2^31) and 256 rows of any GEMM operand
 *    below 2 GiB, since load offsets are 32-bit (MOE_EINVAL).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t moe_bf16;  /* raw bf16 bit pattern */
typedef void* moe_stream;   /* hipStream_t */

enum moe_status {
    MOE_OK = 0,
    MOE_EINVAL = -1,      /* NULL pointer, or a size/count out of range */
    MOE_ESHAPE = -2,      /* H or F not a multiple of 64, K > E, ... */
    MOE_EALIGN = -3,      /* a pointer not 16-byte aligned */
    MOE_EWORKSPACE = -4,  /* workspace NULL or smaller than required */
    MOE_EHIP = -5         /* the HIP runtime reported a launch error */
};

enum moe_epilogue {
    MOE_EPI_NONE = 0,       /* c = bf16(acc) */
    MOE_EPI_SWIGLU_BWD = 1  /* acc is dh[rows,F]; writes c = [bf16(da) | bf16(db)] of width 2F */
};

/* Human-readable text of a moe_status value (static storage). */
const char* moe_strerror(int status);

/* Version of this ABI (incremented on any signature change). */
int moe_abi_version(void);

/*
 * Routing (UniEP "MoE workflow": the router yields a probability
 * distribution over experts per token, and each token goes to its top-k).
 *   logits   fp32 [T,E]  router scores x.W_r (+bias), in.
 *   topk_idx int32 [T,K] out: the K experts with the largest scores, ordered
 *            by (score descending, expert id ascending); -0 == +0.
 *   gates    fp32 [T,K] out: softmax probabilities of the chosen experts
 *            renormalised over the K choices (they sum to 1).
 */
int moe_route(const float* logits, int T, int E, int K,
              int32_t* topk_idx, float* gates, moe_stream stream);

/*
 * Router backward (second half): the gradient of the routing scores through
 * the renormalised top-K gates of moe_route.  The gates are the softmax of the
 * chosen scores alone (the full softmax normaliser cancels in the
 * renormalisation) and the top-K choice is piecewise constant, so for the
 * chosen expert e = topk_idx[t,k]:
 *   dlogits[t,e] = gates[t,k] * (dgates[t,k] - sum_j gates[t,j]*dgates[t,j])
 * (sum over j ascending, fp32) and dlogits[t,e] = 0 for the other experts.
 * A token's K experts must be distinct (those of moe_route are).
 * Linear in dgates, so per-GPU partial gate gradients give per-GPU partial
 * score gradients that sum to the full one.
 *   topk_idx int32 [T,K], gates fp32 [T,K] (from moe_route);
 *   dgates fp32 [T,K] (from moe_gather_gate_grad);  dlogits fp32 [T,E] out.
 */
int moe_route_backward(const int32_t* topk_idx, const float* gates, const float* dgates,
                       int T, int E, int K, float* dlogits, moe_stream stream);

/* Bytes of workspace moe_permute needs for these sizes. */
size_t moe_permute_workspace_size(int T, int K, int e_local);

/*
 * Stable expert-grouped permutation (UniEP "MoE workflow": tokens are
 * grouped by expert in a deterministic order, a stable sort preserving the
 * source sequence; "Deterministic Token Mapping": destination = exclusive
 * prefix of counts + stable local index).
 *   topk_idx int32 [T,K] in.  Pairs with e_begin <= idx < e_begin+e_local
 *            are local; others are skipped.
 *   x        bf16 [T,H] in.
 *   counts   int32 [e_local]   out: local pairs per expert.
 *   offsets  int32 [e_local+1] out: offsets[0]=0, offsets[j+1]=offsets[j]+counts[j].
 *   pos      int32 [T,K] out: destination row of pair (t,k), or -1.
 *   src      int32 [cap_rows] out: src[pos[t,k]] = t*K+k.
 *   x_perm   bf16 [cap_rows,H] out: x_perm[pos[t,k]] = x[t] (bit copy).
 *            x_perm NULL: the index-only permutation, no row copy and x
 *            not read (for moe_grouped_gemm_swiglu_gather).
 *   status   int32 [1] out: 0, or 1 if R > cap_rows (rows >= cap_rows are
 *            dropped: their pos is -1 and nothing is written for them;
 *            counts/offsets still hold the true totals).
 *   ws       device workspace of ws_bytes >= moe_permute_workspace_size().
 * Rows are ordered by expert, then by token: bit-exact and independent of
 * thread scheduling.
 */
int moe_permute(const int32_t* topk_idx, int T, int K, int e_begin, int e_local,
                const moe_bf16* x, int H, int cap_rows,
                int32_t* counts, int32_t* offsets, int32_t* pos, int32_t* src,
                moe_bf16* x_perm, int32_t* status, void* ws, size_t ws_bytes,
                moe_stream stream);

/*
 * moe_permute for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same permutation with the same results, but the per-(expert, block) count
 * matrix that moe_permute keeps in the caller's ws lives in a device array of
 * this library instead, MOE_PERMUTE_SCRATCH_BYTES per GPU, held until the
 * process ends.  Nothing is allocated: no hipMalloc, hipFree or allocating
 * library call.  The array's device address is looked up once per device
 * (hipGetSymbolAddress) on the first call with that device current.
 *   Arguments as moe_permute, without ws / ws_bytes.
 *   Errors: as moe_permute; MOE_EWORKSPACE when
 *   moe_permute_workspace_size(T, K, e_local) > MOE_PERMUTE_SCRATCH_BYTES
 *   (T = 131072 fits with e_local up to 256, T = 2^20 with e_local up to
 *   32); MOE_EHIP if the address lookup fails.
 * Every call on one GPU uses that GPU's one array, so calls that overlap on
 * one GPU (different streams, or host threads without ordering) race and
 * must not be made.  Each call writes every entry it later reads, so no
 * clearing is needed between calls.
 */
#define MOE_PERMUTE_SCRATCH_BYTES ((size_t)1 << 20)
int moe_permute_noalloc(const int32_t* topk_idx, int T, int K, int e_begin, int e_local,
                        const moe_bf16* x, int H, int cap_rows,
                        int32_t* counts, int32_t* offsets, int32_t* pos, int32_t* src,
                        moe_bf16* x_perm, int32_t* status, moe_stream stream);

/*
 * Gate-scaled gather of the output gradient into expert-grouped order
 * (UniEP "MoE workflow", backward: gradients with respect to the output are
 * dispatched to the experts).
 *   d_out   bf16 [T,H] in;  pos int32 [T,K] in (from moe_permute);
 *   gates   fp32 [T,K] in, or NULL for weight 1.
 *   dy_perm bf16 [cap_rows,H] out: dy_perm[pos[t,k]] = bf16(gate[t,k]*d_out[t]).
 */
int moe_gather(const moe_bf16* d_out, const int32_t* pos, const float* gates,
               int T, int K, int H, moe_bf16* dy_perm, moe_stream stream);

/*
 * moe_gather plus the gradient of the gates (router backward, first half).
 * UniEP "MoE workflow": the combine weights each expert output by its gating
 * score, so the gradient of a gate is the dot product of the token's output
 * gradient with the expert output it weighted.  For k < K, r = pos[t,k]:
 *   dy_perm[r]  = bf16(gates[t,k] * d_out[t])       (as moe_gather)
 *   dgates[t,k] = sum_c d_out[t,c] * y[r,c]          (fp32, fixed order)
 * and dgates[t,k] = 0 when pos[t,k] < 0: that expert is on another GPU, and
 * the full gradient of a gate is the sum of the per-GPU values.
 *   d_out bf16 [T,H];  pos int32 [T,K];  gates fp32 [T,K] (required);
 *   y bf16 [cap_rows,H], the forward's down-projection output;
 *   dy_perm bf16 [cap_rows,H] out;  dgates fp32 [T,K] out.
 */
int moe_gather_gate_grad(const moe_bf16* d_out, const int32_t* pos, const float* gates,
                         const moe_bf16* y, int T, int K, int H, moe_bf16* dy_perm,
                         float* dgates, moe_stream stream);

/*
 * Padding-free gate/up GroupGEMM with fused SwiGLU (UniEP "MoE workflow":
 * a GroupGEMM projects the tokens, then SwiGLU; "Scoreboard-based
 * Synchronization": padding-free GroupGEMM over irregular per-expert tiles).
 * For every row r of local expert j (offsets[j] <= r < offsets[j+1], rows at
 * or beyond cap_rows ignored):
 *   a = x_perm[r] . w_gate[j],  b = x_perm[r] . w_up[j]   (fp32 accumulate)
 *   h[r] = bf16(silu(a) * b),   silu(a) = a / (1 + exp(-a))
 *   ab_save[r] = [bf16(a) | bf16(b)]   (optional, for the backward)
 *   x_perm  bf16 [cap_rows,H];  w_gate, w_up bf16 [e_local,H,F];
 *   offsets int32 [e_local+1] (device);  h bf16 [cap_rows,F];
 *   ab_save bf16 [cap_rows,2F] or NULL.
 */
int moe_grouped_gemm_swiglu(const moe_bf16* x_perm, const moe_bf16* w_gate,
                            const moe_bf16* w_up, const int32_t* offsets,
                            int e_local, int H, int F, int cap_rows,
                            moe_bf16* h, moe_bf16* ab_save, moe_stream stream);

/*
 * moe_grouped_gemm_swiglu without the permuted copy of the tokens (MoonEP
 * page, "How Redundant Expert Planning Achieves Perfect Balance": zero-copy
 * dispatch puts tokens at their expert-grouped positions with no copy through
 * an intermediate buffer; on one GPU the GEMM reads each token where it
 * already is).  Row r of the expert-grouped
 * order is read from x[src[r] / K], so the index-only moe_permute (x_perm
 * NULL) replaces the row copy.  h and ab_save are bit-identical to
 * moe_grouped_gemm_swiglu on the x_perm that moe_permute would have written.
 *   x    bf16 [T,H], the tokens;  src int32 [cap_rows] from moe_permute
 *        (src[r] = t*K + k);  K the top-k of src's encoding;
 *   other arguments as moe_grouped_gemm_swiglu.
 * Errors: x must be at most 0xF0000000 bytes (T*H*2 <= 3.75 GiB; T up to
 * 280870 at H = 7168), H*F*2 below 2^31, and cap_rows <= T*K (MOE_EINVAL).
 * A src value outside [0, T*K) reads a zero row (no access outside x).
 * The weight gradient needs x_perm, so a forward that is followed by the
 * backward keeps the row copy.
 */
int moe_grouped_gemm_swiglu_gather(const moe_bf16* x, int T, const int32_t* src, int K,
                                   const moe_bf16* w_gate, const moe_bf16* w_up,
                                   const int32_t* offsets, int e_local, int H, int F,
                                   int cap_rows, moe_bf16* h, moe_bf16* ab_save,
                                   moe_stream stream);

/*
 * Generic padding-free GroupGEMM over expert row groups (UniEP "MoE
 * workflow": the second GroupGEMM projects back to H; backward: the dgrad
 * GEMMs mirror the forward).
 * For rows r of expert j:
 *   trans_w = 0: w0[j] is [Kd,N] and acc = a[r,0:Kd] . w0[j]
 *   trans_w = 1: w0[j] is [N,Kd] and acc = a[r,0:Kd] . w0[j]^T
 *   w1 != NULL (trans_w = 1 only): a has 2*Kd columns and
 *        acc = a[r,0:Kd] . w0[j]^T + a[r,Kd:2Kd] . w1[j]^T   (one accumulator)
 *   epilogue MOE_EPI_NONE:       c[r,0:N] = bf16(acc)
 *   epilogue MOE_EPI_SWIGLU_BWD: acc is dh; with a_, b_ = ab[r,0:N], ab[r,N:2N]
 *        and s = sigmoid(a_): c[r,0:N] = bf16(dh*b_*s*(1+a_*(1-s))),
 *        c[r,N:2N] = bf16(dh*a_*s).
 *   lda, ldc: row strides in elements (multiples of 8).
 * Forward down projection: (h, F, w_down, NULL, 0, ..., Kd=F, N=H) -> y.
 * Backward: (dy_perm, H, w_down, NULL, 1, ..., Kd=H, N=F, SWIGLU_BWD, ab) -> dab;
 *           (dab, 2F, w_gate, w_up, 1, ..., Kd=F, N=H) -> dx_perm.
 */
int moe_grouped_gemm(const moe_bf16* a, int lda, const moe_bf16* w0, const moe_bf16* w1,
                     int trans_w, const int32_t* offsets, int e_local, int Kd, int N,
                     int cap_rows, int epilogue, const moe_bf16* ab,
                     moe_bf16* c, int ldc, moe_stream stream);

/*
 * Gate-weighted combine back to token order (UniEP "MoE workflow": results
 * are weighted by their gating scores and aggregated per token; "Top-k
 * accumulation constraint": a token's K contributions are summed only all
 * together, in one fixed order).
 *   out[t] = bf16( sum over k ascending with pos[t,k] >= 0 of gate[t,k]*y[pos[t,k]] )
 * in fp32 from +0; a token with no local pair gets +0.  gates == NULL means
 * weight 1: the backward's combine-gradient dX[t] = sum_k dx_perm[pos[t,k]]
 * (MoonEP: the dispatch gradient sums each token's K copies).
 *   y bf16 [cap_rows,H];  pos int32 [T,K] as moe_permute writes it (-1, or
 *   a row of y: the rows are not bounds-checked);  gates fp32 [T,K] or
 *   NULL;  out bf16 [T,H].
 */
int moe_combine(const moe_bf16* y, const int32_t* pos, const float* gates,
                int T, int K, int H, moe_bf16* out, moe_stream stream);

/*
 * Transposed GroupGEMM for weight gradients (UniEP "MoE workflow",
 * backward: the weight gradient needs a transposed GroupGEMM that reduces
 * over the token dimension; splitting that reduction changes the summation
 * tree, so it runs in one fixed order).
 *   dw[j] = a_j^T . b_j  (fp32 [e_local,M,N]), a_j = rows offsets[j]..offsets[j+1]-1
 *   of a (bf16 [.,M], row stride lda), b_j likewise of b (bf16 [.,N], ldb).
 * Each output element is one fp32 sum over the group's rows in a fixed
 * blocked order (no split over rows, no atomics); an empty group writes 0.
 *   dW_gate: (x_perm, H, dab, 2F, M=H, N=F);  dW_up: b = dab + F;
 *   dW_down: (h, F, dy_perm, H, M=F, N=H).   M, N multiples of 64.
 */
int moe_wgrad(const moe_bf16* a, int lda, const moe_bf16* b, int ldb,
              const int32_t* offsets, int e_local, int M, int N, int cap_rows,
              float* dw, moe_stream stream);

/*
 * dW_gate and dW_up in one transposed GroupGEMM (UniEP "MoE workflow",
 * backward: the weight gradients reduce over the token dimension): both
 * contract the same rows of x_perm, against the two halves of dab, so one pass
 * over [da | db] reads x_perm once instead of twice.  For expert j:
 *   dw_gate[j] = x_perm_j^T . dab_j[:, 0:F],  dw_up[j] = x_perm_j^T . dab_j[:, F:2F]
 * bitwise equal to moe_wgrad(x_perm, H, dab, 2F, ..., M=H, N=F) and to the
 * same call on dab + F (the same fixed order per output element).
 *   x_perm bf16 [cap_rows,H];  dab bf16 [cap_rows,2F];  offsets as moe_wgrad;
 *   dw_gate, dw_up fp32 [e_local,H,F] out.  H, F multiples of 64.
 */
int moe_wgrad_gate_up(const moe_bf16* x_perm, int H, const moe_bf16* dab, int F,
                      const int32_t* offsets, int e_local, int cap_rows,
                      float* dw_gate, float* dw_up, moe_stream stream);

/*
 * moe_wgrad_gate_up without the permuted copy of the tokens, the backward
 * half of zero-copy dispatch (MoonEP page, "How Redundant Expert Planning
 * Achieves Perfect Balance": tokens are used where they are, with no copy
 * through an intermediate buffer).  Row r of the expert-grouped order is
 * read from x[src[r] / K], so a training step needs no x_perm: the forward
 * runs moe_grouped_gemm_swiglu_gather on the index-only moe_permute.
 * dw_gate and dw_up are bit-identical to moe_wgrad_gate_up on the x_perm
 * that moe_permute would have written (the same fixed order per element).
 *   x    bf16 [T,H], the tokens;  src int32 [cap_rows] from moe_permute
 *        (src[r] = t*K + k);  K the top-k of src's encoding;
 *   dab, F, offsets, e_local, cap_rows, dw_gate, dw_up as moe_wgrad_gate_up.
 * Errors: as moe_grouped_gemm_swiglu_gather for x, T, src, K (x at most
 * 0xF0000000 bytes, cap_rows <= T*K: MOE_EINVAL); H, F multiples of 64
 * (MOE_ESHAPE).  A src value outside [0, T*K) reads a zero row.
 */
int moe_wgrad_gate_up_gather(const moe_bf16* x, int T, const int32_t* src, int K, int H,
                             const moe_bf16* dab, int F, const int32_t* offsets, int e_local,
                             int cap_rows, float* dw_gate, float* dw_up, moe_stream stream);

/*
 * The non-bitwise variant of moe_wgrad (UniEP evaluation, "Performance Cost
 * of Bitwise Reproducibility" and Table 7: splitting the weight gradient's
 * reduction over tokens gives more parallel work but changes the summation
 * tree).  Each expert's rows are cut into `splits` fixed chunks (every chunk
 * but the last a whole number of 32-row steps); each chunk is summed as in
 * moe_wgrad into an fp32 partial in ws, and the partials are added in chunk
 * order:
 *   dw[j] = sum over chunks c ascending of (a_jc^T . b_jc)
 * Identical bits from run to run, within the fp32 rounding of moe_wgrad, but
 * not the same bits.  splits == 1 is moe_wgrad itself (ws unused).
 *   Arguments as moe_wgrad, plus splits (1 <= splits, e_local*splits <= 512)
 *   and ws: device workspace of at least
 *   moe_wgrad_split_workspace_size(e_local, M, N, splits) bytes
 *   (e_local*splits fp32 [M,N] partials and the chunk offsets).
 * Errors as moe_wgrad; MOE_EWORKSPACE if ws is NULL or too small.
 */
size_t moe_wgrad_split_workspace_size(int e_local, int M, int N, int splits);
int moe_wgrad_split(const moe_bf16* a, int lda, const moe_bf16* b, int ldb,
                    const int32_t* offsets, int e_local, int M, int N, int cap_rows,
                    int splits, float* dw, void* ws, size_t ws_bytes, moe_stream stream);

/*
 * Router projection (UniEP "MoE workflow": the router network produces each
 * token's scores over the experts, from which routing takes the top-k):
 *   logits[t,e] = sum_i x[t,i] * w_r[i,e]  (+ bias[e])      fp32 accumulate
 *   x bf16 [T,H];  w_r bf16 [H,E];  bias fp32 [E] or NULL;  logits fp32 [T,E].
 * When the tiles are too few to fill the GPU the contraction over H is cut
 * into chunks whose fp32 partials are added in chunk order (then the bias):
 * repeated calls on one device give identical bits.  H and E must be
 * multiples of 64 (MOE_ESHAPE), E <= 4096.  ws: device workspace of at least
 * moe_router_workspace_size(T, H, E) bytes (may be NULL when that is 0 for
 * the forward; the backward always needs it).
 * The routing step consumes logits; whether they come from here or from the
 * caller, moe_route selects exactly on the fp32 values it is given.
 */
size_t moe_router_workspace_size(int T, int H, int E);
int moe_router_logits(const moe_bf16* x, int T, int H, const moe_bf16* w_r, int E,
                      const float* bias, float* logits, void* ws, size_t ws_bytes,
                      moe_stream stream);

/*
 * Backward of the router projection, from the score gradient dlogits fp32
 * [T,E] (moe_route_backward's output), rounded to bf16 like the other
 * activation gradients of the path:
 *   dx[t,i]   = bf16( sum_e bf16(dlogits[t,e]) * w_r[i,e] )   bf16 [T,H]
 *   dw_r[i,e] = sum_t x[t,i] * bf16(dlogits[t,e])             fp32 [H,E]
 * dx is the router's share of the input gradient only (the caller adds the
 * experts' dX).  dw_r sums the tokens in fixed chunks added in chunk order
 * (the non-bitwise-serial variant of the weight gradient: run-to-run
 * identical, not the serial order).  Shapes and ws as moe_router_logits.
 */
int moe_router_backward(const moe_bf16* x, int T, int H, const moe_bf16* w_r, int E,
                        const float* dlogits, moe_bf16* dx, float* dw_r, void* ws,
                        size_t ws_bytes, moe_stream stream);

/*
 * Measurement aid, not a step of the layer: the bf16 MFMA rate this GPU
 * sustains.  Each of the blocks x 4 waves keeps its own 8 fragments of
 * operands in registers and runs iters rounds of a 4 x 4 block of
 * independent 32x32x16 bf16 MFMAs (16 * 32768 flop per round and wave),
 * then writes one float per lane: the sum of its accumulator elements.
 *   operands  bf16 [blocks*4][8][64][8]: for wave w, fragments 0..3 are its
 *             A operands, 4..7 its B operands; lane l of fragment f holds the
 *             8 values at [w][f][l][0..7].
 *   out       fp32 [blocks*4*64].
 * For each wave the sum of out over its 64 lanes equals
 *   iters * sum_{m,n<4} sum_{h<2, j<8} (sum_{l in half h} A_m[l][j]) * (sum_{l in half h} B_n[l][j])
 * (lanes 0..31 and 32..63 carry the two halves of the 16-deep contraction).
 * blocks in 1..2^20, iters >= 0 (MOE_EINVAL), both pointers 16-byte aligned
 * (MOE_EALIGN).  The caller owns both buffers; nothing is allocated.
 */
int moe_probe_mfma(const moe_bf16* operands, int blocks, int iters, float* out, moe_stream stream);

/*
 * The same measurement aid on the other bf16 MFMA shape,
 * v_mfma_f32_16x16x32_bf16: each wave runs iters rounds of an 8 x 8 block of
 * independent 16x16x32 MFMAs (the same 16 * 32768 flop per round and wave).
 *   operands  bf16 [blocks*4][16][64][8]: fragments 0..7 of wave w are its A
 *             operands, 8..15 its B operands; lane l of a fragment holds row
 *             (or column) l%16 and contraction index 8*(l/16) + 0..7.
 *   out       fp32 [blocks*4*64].
 * For each wave the sum of out over its 64 lanes equals
 *   iters * sum_{m,n<8} sum_{g<4, j<8} (sum_{l in group g} A_m[l][j]) * (sum_{l in group g} B_n[l][j])
 * (lanes 16g .. 16g+15 form group g).  Limits and errors as moe_probe_mfma.
 */
int moe_probe_mfma16(const moe_bf16* operands, int blocks, int iters, float* out, moe_stream stream);

/*
 * Measurement aid, not a step of the layer: the rate of a plain streaming
 * copy, the practical ceiling of a kernel that reads and writes as many bytes
 * as it moves.  Copies bytes from src to dst (device buffers, no overlap)
 * with 16-byte coalesced loads and stores.
 *   nontemporal  bit 0: non-temporal loads; bit 1: non-temporal stores.
 *   blocks       workgroups of 256 lanes, each copying 16 KiB per pass over
 *                the buffer; 0 picks 8 per compute unit.
 * bytes >= 0 and a multiple of 16, nontemporal in 0..3, blocks in 0..2^20
 * (MOE_EINVAL; a null pointer with bytes > 0 too); both pointers 16-byte
 * aligned (MOE_EALIGN).  bytes = 0 launches nothing.  The caller owns both
 * buffers; nothing is allocated.
 */
int moe_probe_copy(const void* src, void* dst, int64_t bytes, int nontemporal, int blocks, moe_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
