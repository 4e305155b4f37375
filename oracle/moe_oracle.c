/*
 * moe_oracle.c -- plain, slow, obviously-correct CPU oracle of the one-GPU
 * MoE layer hot path.  TEST INFRASTRUCTURE ONLY: it exists so the tests, the
 * smoke check and the benchmark's CPU-baseline leg can check the HIP path.
 * Nothing in the product path may call it, and it shares no code, header,
 * table or helper with the HIP kernels.
 *
 * Source of what is computed: the UniEP paper (arXiv 2604.19241), section
 * "MoE workflow" (forward: routing probabilities, top-k, stable expert-grouped
 * permutation, GroupGEMM -> SwiGLU -> GroupGEMM, gate-weighted combine;
 * backward: dgrad and the transposed GroupGEMM for weight gradients), the
 * "Deterministic Token Mapping" section (destination = exclusive prefix of
 * per-expert counts + stable local index), the "Top-k accumulation
 * constraint" paragraph (a token's K contributions are summed together, in
 * one fixed order) and the MoonEP page ("dispatch gradient" = combine of the
 * K copies).  Readings where the pages are silent are stated per function.
 *
 * Precision: inputs are bf16 bit patterns; every product is taken in fp32
 * (exact for bf16 x bf16) and every sum is an fp32 running sum in the stated
 * order, starting from +0.  Build with -ffp-contract=off and no fast-math so
 * that the compiler keeps each multiply and add separate and in order.
 * Stored intermediates are rounded to bf16 nearest-even.
 *
 * Loops are parallelised with OpenMP only over independent outputs (tokens,
 * rows, experts); the order inside every single sum is the sequential one.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* threads an OpenMP parallel region of the oracle uses */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- bf16 <-> fp32 --------------------------------------------------- */

static float bf(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint16_t rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return 0x7fc0; /* NaN */
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* exported so the tests can pin the rounding helper itself */
uint16_t oracle_f32_to_bf16(float f) { return rne(f); }

/* ---- O1: routing ------------------------------------------------------
 * Router probabilities are the softmax of the fp32 scores; the K experts
 * with the largest scores are chosen, ordered by (score descending, expert
 * id ascending) -- IEEE comparison, so -0 == +0 and equal scores go to the
 * lower id.  Selection on scores equals selection on probabilities in exact
 * arithmetic (softmax is monotonic) and cannot be perturbed by rounding.
 * Gates are the chosen probabilities renormalised over the K choices.
 */
void oracle_route(const float* logits, int T, int E, int K, int32_t* topk_idx, float* gates) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const float* s = logits + (int64_t)t * E;
        unsigned char taken[1024];
        memset(taken, 0, (size_t)E);
        for (int k = 0; k < K; ++k) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || s[e] > s[best]) best = e; /* ties keep the lower id */
            }
            taken[best] = 1;
            topk_idx[(int64_t)t * K + k] = best;
        }
        float m = s[0];
        for (int e = 1; e < E; ++e)
            if (s[e] > m) m = s[e];
        float z = 0.0f;
        for (int e = 0; e < E; ++e) z += expf(s[e] - m);
        float p[64];
        for (int k = 0; k < K; ++k) p[k] = expf(s[topk_idx[(int64_t)t * K + k]] - m) / z;
        float sum = 0.0f;
        for (int k = 0; k < K; ++k) sum += p[k];
        for (int k = 0; k < K; ++k) gates[(int64_t)t * K + k] = p[k] / sum;
    }
}

/* ---- O2: permutation --------------------------------------------------
 * Local pairs are (t,k) with e_begin <= idx[t,k] < e_begin+e_local.
 * counts[j] = number of local pairs choosing expert e_begin+j;
 * offsets = exclusive prefix sum of counts (offsets[0]=0, e_local+1 entries).
 * Rows are ordered by local expert, then by token index (a stable sort of the
 * pairs by expert; a token picks an expert at most once, so this is unique).
 * pos[t,k] = destination row (-1 if not local); src[row] = t*K+k;
 * x_perm[row] = x[t] (bit copy).  A row at or beyond cap_rows is dropped:
 * its pos is -1, nothing is written for it, and *status gets bit 0.
 */
void oracle_permute(const int32_t* topk_idx, int T, int K, int e_begin, int e_local,
                    const uint16_t* x, int H, int64_t cap_rows,
                    int32_t* counts, int32_t* offsets, int32_t* pos, int32_t* src,
                    uint16_t* x_perm, int32_t* status) {
    for (int j = 0; j < e_local; ++j) counts[j] = 0;
    for (int64_t p = 0; p < (int64_t)T * K; ++p) {
        int j = topk_idx[p] - e_begin;
        if (j >= 0 && j < e_local) counts[j]++;
    }
    offsets[0] = 0;
    for (int j = 0; j < e_local; ++j) offsets[j + 1] = offsets[j] + counts[j];
    int32_t fill[1024];
    for (int j = 0; j < e_local; ++j) fill[j] = 0;
    int32_t st = 0;
    for (int t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            int64_t p = (int64_t)t * K + k;
            int j = topk_idx[p] - e_begin;
            if (j < 0 || j >= e_local) {
                pos[p] = -1;
                continue;
            }
            int64_t r = (int64_t)offsets[j] + fill[j]++;
            if (r >= cap_rows) {
                pos[p] = -1;
                st |= 1;
                continue;
            }
            pos[p] = (int32_t)r;
            src[r] = (int32_t)p;
            if (x && x_perm) memcpy(x_perm + r * H, x + (int64_t)t * H, (size_t)H * 2);
        }
    }
    if (status) *status = st;
}

/* Rows of group j are [offsets[j], offsets[j+1]) clipped to cap_rows. */
static int group_of_row(const int32_t* offsets, int e_local, int64_t r) {
    for (int j = 0; j < e_local; ++j)
        if (r >= offsets[j] && r < offsets[j + 1]) return j;
    return -1;
}

static int64_t rows_total(const int32_t* offsets, int e_local, int64_t cap_rows) {
    int64_t R = offsets[e_local];
    return R < cap_rows ? R : cap_rows;
}

/* ---- O3: gate/up GroupGEMM with SwiGLU --------------------------------
 * For row r of group j: a[c] = sum_{i<H} x_perm[r,i]*Wg[j,i,c] and
 * b[c] = sum_{i<H} x_perm[r,i]*Wu[j,i,c] (i ascending);
 * h[r,c] = bf16(silu(a)*b) with silu(a) = a/(1+exp(-a)) applied to the gate
 * half; ab_save[r] = [bf16(a) | bf16(b)] (columns [0,F) and [F,2F)).
 * rows: optional list of n_rows row indices to compute (NULL: all rows).
 */
void oracle_expert_up(const uint16_t* x_perm, const uint16_t* w_gate, const uint16_t* w_up,
                      const int32_t* offsets, int e_local, int H, int F, int64_t cap_rows,
                      const int64_t* rows, int64_t n_rows, uint16_t* h, uint16_t* ab_save) {
    int64_t R = rows_total(offsets, e_local, cap_rows);
    int64_t n = rows ? n_rows : R;
#pragma omp parallel
    {
        float* a = (float*)__builtin_alloca(sizeof(float) * (size_t)F);
        float* b = (float*)__builtin_alloca(sizeof(float) * (size_t)F);
#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < n; ++q) {
            int64_t r = rows ? rows[q] : q;
            if (r < 0 || r >= R) continue;
            int j = group_of_row(offsets, e_local, r);
            const uint16_t* xr = x_perm + r * H;
            const uint16_t* wg = w_gate + (int64_t)j * H * F;
            const uint16_t* wu = w_up + (int64_t)j * H * F;
            for (int c = 0; c < F; ++c) { a[c] = 0.0f; b[c] = 0.0f; }
            for (int i = 0; i < H; ++i) {
                float xv = bf(xr[i]);
                const uint16_t* g = wg + (int64_t)i * F;
                const uint16_t* u = wu + (int64_t)i * F;
                for (int c = 0; c < F; ++c) {
                    a[c] += xv * bf(g[c]);
                    b[c] += xv * bf(u[c]);
                }
            }
            for (int c = 0; c < F; ++c) {
                float silu = a[c] / (1.0f + expf(-a[c]));
                h[r * F + c] = rne(silu * b[c]);
                if (ab_save) {
                    ab_save[r * 2 * F + c] = rne(a[c]);
                    ab_save[r * 2 * F + F + c] = rne(b[c]);
                }
            }
        }
    }
}

/* ---- O4: down GroupGEMM --------------------------------------------
 * y[r,c] = bf16( sum_{i<F} h[r,i]*Wd[j,i,c] ), i ascending.
 */
void oracle_expert_down(const uint16_t* h, const uint16_t* w_down, const int32_t* offsets,
                        int e_local, int F, int H, int64_t cap_rows,
                        const int64_t* rows, int64_t n_rows, uint16_t* y) {
    int64_t R = rows_total(offsets, e_local, cap_rows);
    int64_t n = rows ? n_rows : R;
#pragma omp parallel
    {
        float* acc = (float*)__builtin_alloca(sizeof(float) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
        for (int64_t q = 0; q < n; ++q) {
            int64_t r = rows ? rows[q] : q;
            if (r < 0 || r >= R) continue;
            int j = group_of_row(offsets, e_local, r);
            const uint16_t* hr = h + r * F;
            const uint16_t* wd = w_down + (int64_t)j * F * H;
            for (int c = 0; c < H; ++c) acc[c] = 0.0f;
            for (int i = 0; i < F; ++i) {
                float hv = bf(hr[i]);
                const uint16_t* w = wd + (int64_t)i * H;
                for (int c = 0; c < H; ++c) acc[c] += hv * bf(w[c]);
            }
            for (int c = 0; c < H; ++c) y[r * H + c] = rne(acc[c]);
        }
    }
}

/* ---- O5: combine ------------------------------------------------------
 * out[t,c] = bf16( sum over k ascending with pos[t,k] >= 0 of
 *                  gate[t,k] * y[pos[t,k], c] ), accumulator from +0,
 * multiply then add.  gates == NULL means weight 1 (the backward's
 * combine-gradient: the K dispatched gradient copies summed per token).
 * A token with no local pair gets +0.
 */
void oracle_combine(const uint16_t* y, const int32_t* pos, const float* gates,
                    int T, int K, int H, const int64_t* tokens, int64_t n_tokens, uint16_t* out) {
    int64_t n = tokens ? n_tokens : T;
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < n; ++q) {
        int64_t t = tokens ? tokens[q] : q;
        for (int c = 0; c < H; ++c) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                int32_t r = pos[t * K + k];
                if (r < 0) continue;
                float v = bf(y[(int64_t)r * H + c]);
                if (gates) v = gates[t * K + k] * v;
                acc += v;
            }
            out[t * H + c] = rne(acc);
        }
    }
}

/* ---- B1: gate-scaled gather of the output gradient --------------------
 * dy_perm[r] = bf16( gate[t,k] * dOut[t] ) where src[r] = t*K+k.
 */
void oracle_bwd_gather(const uint16_t* d_out, const int32_t* src, const int32_t* offsets,
                       const float* gates, int K, int H, int e_local, int64_t cap_rows,
                       uint16_t* dy_perm) {
    int64_t R = rows_total(offsets, e_local, cap_rows);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        int64_t p = src[r];
        int64_t t = p / K;
        for (int c = 0; c < H; ++c) {
            float v = bf(d_out[t * H + c]);
            dy_perm[r * H + c] = gates ? rne(gates[p] * v) : d_out[t * H + c];
        }
    }
}

/* ---- B2: down-projection dgrad and SwiGLU backward ---------------------
 * dh[r,i] = sum_{c<H} dy_perm[r,c]*Wd[j,i,c] (c ascending).  With a, b the
 * saved pre-activations and s = 1/(1+exp(-a)):
 *   da = dh*b*s*(1 + a*(1-s))   (d silu(a)/da = s*(1+a*(1-s)))
 *   db = dh*silu(a) = dh*a*s
 * dab[r] = [bf16(da) | bf16(db)].
 */
void oracle_bwd_down(const uint16_t* dy_perm, const uint16_t* w_down, const uint16_t* ab_save,
                     const int32_t* offsets, int e_local, int F, int H, int64_t cap_rows,
                     const int64_t* rows, int64_t n_rows, uint16_t* dab) {
    int64_t R = rows_total(offsets, e_local, cap_rows);
    int64_t n = rows ? n_rows : R;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < n; ++q) {
        int64_t r = rows ? rows[q] : q;
        if (r < 0 || r >= R) continue;
        int j = group_of_row(offsets, e_local, r);
        const uint16_t* g = dy_perm + r * H;
        const uint16_t* wd = w_down + (int64_t)j * F * H;
        for (int i = 0; i < F; ++i) {
            const uint16_t* w = wd + (int64_t)i * H;
            float dh = 0.0f;
            for (int c = 0; c < H; ++c) dh += bf(g[c]) * bf(w[c]);
            float a = bf(ab_save[r * 2 * F + i]);
            float b = bf(ab_save[r * 2 * F + F + i]);
            float s = 1.0f / (1.0f + expf(-a));
            float da = dh * b * s * (1.0f + a * (1.0f - s));
            float db = dh * a * s;
            dab[r * 2 * F + i] = rne(da);
            dab[r * 2 * F + F + i] = rne(db);
        }
    }
}

/* ---- B3: gate/up dgrad -------------------------------------------------
 * dx_perm[r,i] = bf16( sum_{c<F} da[r,c]*Wg[j,i,c] + sum_{c<F} db[r,c]*Wu[j,i,c] )
 * in one fp32 accumulator: the gate segment first (c ascending), then the
 * up segment (c ascending).
 */
void oracle_bwd_up(const uint16_t* dab, const uint16_t* w_gate, const uint16_t* w_up,
                   const int32_t* offsets, int e_local, int H, int F, int64_t cap_rows,
                   const int64_t* rows, int64_t n_rows, uint16_t* dx_perm) {
    int64_t R = rows_total(offsets, e_local, cap_rows);
    int64_t n = rows ? n_rows : R;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < n; ++q) {
        int64_t r = rows ? rows[q] : q;
        if (r < 0 || r >= R) continue;
        int j = group_of_row(offsets, e_local, r);
        const uint16_t* da = dab + r * 2 * F;
        const uint16_t* db = da + F;
        for (int i = 0; i < H; ++i) {
            const uint16_t* g = w_gate + ((int64_t)j * H + i) * F;
            const uint16_t* u = w_up + ((int64_t)j * H + i) * F;
            float acc = 0.0f;
            for (int c = 0; c < F; ++c) acc += bf(da[c]) * bf(g[c]);
            for (int c = 0; c < F; ++c) acc += bf(db[c]) * bf(u[c]);
            dx_perm[r * H + i] = rne(acc);
        }
    }
}

/* ---- B5: transposed GroupGEMM (weight gradient) ------------------------
 * dW[j,m,n] = sum over rows r of group j, r ascending, of A[r,m]*B[r,n]
 * (fp32 result; an empty group gives +0).  A has row stride lda, B ldb.
 *   dW_gate: A = x_perm (M=H), B = da;  dW_up: B = db;
 *   dW_down: A = h (M=F), B = dy_perm (N=H).
 * groups: optional list of groups to compute (NULL: all); cols: optional
 * list of n indices (NULL: all N).  Untouched outputs are left as they were.
 */
void oracle_wgrad(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                  const int32_t* offsets, int e_local, int M, int N, int64_t cap_rows,
                  const int32_t* groups, int n_groups, const int32_t* cols, int n_cols, float* dw) {
    int ng = groups ? n_groups : e_local;
    int nc = cols ? n_cols : N;
    for (int gi = 0; gi < ng; ++gi) {
        int j = groups ? groups[gi] : gi;
        int64_t r0 = offsets[j] < cap_rows ? offsets[j] : cap_rows;
        int64_t r1 = offsets[j + 1] < cap_rows ? offsets[j + 1] : cap_rows;
#pragma omp parallel
        {
            float* acc = (float*)__builtin_alloca(sizeof(float) * (size_t)nc);
#pragma omp for schedule(static)
            for (int m = 0; m < M; ++m) {
                for (int ci = 0; ci < nc; ++ci) acc[ci] = 0.0f;
                for (int64_t r = r0; r < r1; ++r) {
                    float av = bf(A[r * lda + m]);
                    const uint16_t* b = B + r * ldb;
                    if (cols)
                        for (int ci = 0; ci < nc; ++ci) acc[ci] += av * bf(b[cols[ci]]);
                    else
                        for (int ci = 0; ci < nc; ++ci) acc[ci] += av * bf(b[ci]);
                }
                for (int ci = 0; ci < nc; ++ci) {
                    int c = cols ? cols[ci] : ci;
                    dw[((int64_t)j * M + m) * N + c] = acc[ci];
                }
            }
        }
    }
}

/* ---- R1: gate gradient --------------------------------------------------
 * The combine is out[t] = sum_k gate[t,k] * y[pos[t,k]], so the gradient of
 * a gate is the dot product of the output gradient with the expert output it
 * weighted: dgates[t,k] = sum_{c<H} dOut[t,c] * y[pos[t,k],c] (c ascending,
 * fp32 running sum from +0).  A non-local pair gets 0: its expert and y row
 * are on another GPU, and the gate's full gradient is the sum of the per-GPU
 * parts, exactly one of which is non-zero.
 */
void oracle_gate_grad(const uint16_t* d_out, const uint16_t* y, const int32_t* pos, int T, int K, int H,
                      float* dgates) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            int32_t r = pos[(int64_t)t * K + k];
            float acc = 0.0f;
            if (r >= 0)
                for (int c = 0; c < H; ++c) acc += bf(d_out[(int64_t)t * H + c]) * bf(y[(int64_t)r * H + c]);
            dgates[(int64_t)t * K + k] = acc;
        }
    }
}

/* ---- R2: router backward --------------------------------------------------
 * The gates are the chosen experts' softmax probabilities renormalised over
 * the K choices, which equals the softmax of the chosen scores alone (the
 * full normaliser cancels); the choice itself is piecewise constant in the
 * scores and contributes nothing.  So, with g = gates[t,:], dg = dgates[t,:]:
 *   sum = sum_j g_j * dg_j                      (j ascending, fp32)
 *   dlogits[t, idx[t,k]] = g_k * (dg_k - sum)
 * and dlogits[t,e] = 0 for every expert e not chosen.  The map is linear in
 * dg, so per-GPU partial gate gradients give per-GPU partial dlogits.
 */
void oracle_route_backward(const int32_t* topk_idx, const float* gates, const float* dgates, int T, int E,
                           int K, float* dlogits) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const float* g = gates + (int64_t)t * K;
        const float* dg = dgates + (int64_t)t * K;
        float sum = 0.0f;
        for (int j = 0; j < K; ++j) sum += g[j] * dg[j];
        float* row = dlogits + (int64_t)t * E;
        for (int e = 0; e < E; ++e) row[e] = 0.0f;
        for (int k = 0; k < K; ++k) row[topk_idx[(int64_t)t * K + k]] = g[k] * (dg[k] - sum);
    }
}

/* ---- R3: router projection ----------------------------------------------
 * UniEP "MoE workflow": the router network scores every token against every
 * expert.  The scores are the token times the router weight, plus the
 * per-expert bias of the synthetic routing recipe:
 *   logits[t,e] = fp32( sum_i x[t,i] * W_r[i,e] ) + bias[e]
 * with the sum in fp64, i ascending (the definition the scores handed to the
 * routing step are made by; the fp64 sum is exact enough that its rounding
 * to fp32 is the correctly rounded dot product but for ties), then one fp32
 * add of the bias.  Only `rows` (if given) are filled.
 */
void oracle_router_logits(const uint16_t* x, const uint16_t* w_r, const float* bias, int T, int H, int E,
                          const int64_t* rows, int n_rows, float* logits) {
    int n = rows ? n_rows : T;
#pragma omp parallel for schedule(static)
    for (int ri = 0; ri < n; ++ri) {
        int64_t t = rows ? rows[ri] : ri;
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int i = 0; i < H; ++i) acc += (double)bf(x[t * H + i]) * (double)bf(w_r[(int64_t)i * E + e]);
            float v = (float)acc;
            if (bias) v = v + bias[e];
            logits[t * E + e] = v;
        }
    }
}

/* ---- R4: router projection backward --------------------------------------
 * The gradient of logits = x . W_r with respect to x, from the score
 * gradient rounded to bf16 (as every stored activation gradient of the path):
 *   dx[t,i] = bf16( sum_e dl[t,e] * W_r[i,e] ),   e ascending, fp32
 * (the weight gradient, sum_t x[t,i] * dl[t,e], is oracle_wgrad over the one
 * group of all T rows).  oracle_round_bf16 gives dl = bf16(dlogits).
 */
void oracle_round_bf16(const float* in, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = rne(in[i]);
}

void oracle_router_dx(const uint16_t* dl, const uint16_t* w_r, int T, int H, int E, const int64_t* rows,
                      int n_rows, uint16_t* dx) {
    int n = rows ? n_rows : T;
#pragma omp parallel for schedule(static)
    for (int ri = 0; ri < n; ++ri) {
        int64_t t = rows ? rows[ri] : ri;
        for (int i = 0; i < H; ++i) {
            float acc = 0.0f;
            for (int e = 0; e < E; ++e) acc += bf(dl[t * E + e]) * bf(w_r[(int64_t)i * E + e]);
            dx[t * H + i] = rne(acc);
        }
    }
}
