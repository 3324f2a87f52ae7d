/*
 * CPU oracle for scaled dot-product attention and the multi-head layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link,
 * load or call this file; only the tests, the smoke check and the bench's
 * CPU-baseline leg use it. It shares no code with the HIP library.
 *
 * Everything is computed in float64 on inputs already widened to float64,
 * with plain loops and no blocking, fusion or reordering, so that each step
 * can be checked against the pages by eye:
 *
 *   Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k) + M) V
 *
 * as the four stages of "04. Self-Attention: Transformer 的核心计算"
 * section 四 (scores, scaling, row softmax, weighted sum), with the mask
 * added before the softmax as in its section 七 (causal) and the padding
 * mask of "attention-mechanism" (page 2), section 掩码. The softmax is the
 * stable form that subtracts the row maximum before exponentiating (page 2,
 * section 最小实现) -- deliberately NOT the online recurrence, so that the
 * GPU's online softmax is checked against an independent formulation.
 *
 * Readings of points the pages leave open (each is also listed in the design
 * notes of the repository):
 *  - scale is an explicit argument; the pages fix it at 1/sqrt(d_k) with d_k
 *    the per-head width ("attention-mechanism", 工程权衡与边界).
 *  - a masked position is excluded exactly: its weight is 0.0 (the pages'
 *    e^{-inf} = 0), never exp(-1e9 - m).
 *  - the padding mask removes KEY positions j >= valid_len[b] for every
 *    query row; padded query rows are computed normally.
 *  - causal hides keys j > i (diagonal visible); it is defined here for any
 *    N_q, N_k with that same index rule.
 *  - causal and padding together (the decoder's masked self-attention over a
 *    padded batch) hide a key when either rule hides it: visible iff j <= i
 *    and j < valid_len.
 *  - grouped K/V heads (page 5, section MHA -> MQA -> GQA -> MLA: every h/g
 *    query heads share one K/V head): query head h reads K/V head
 *    h / (H / H_kv), i.e. consecutive query heads form a group. H_kv = H is
 *    the plain multi-head case, H_kv = 1 the single shared K/V head.
 *  - the optional per-row log-sum-exp is ln sum_j exp(s_j) over the visible
 *    scaled scores s_j (-inf for a row without a visible key): the log of
 *    the softmax denominator, so that weight_j = exp(s_j - lse).
 *  - a row with no visible key has no softmax; its output is 0 (convention,
 *    not fixed by the pages: parity unpinned for that case).
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC attn_oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_MASK_NONE = 0, ORACLE_MASK_CAUSAL = 1, ORACLE_MASK_PADDING = 2, ORACLE_MASK_CAUSAL_PADDING = 3 };

/* Is key j visible to query i?  (page 1 section 七; page 2 section 掩码) */
static int visible(int mask_kind, int64_t i, int64_t j, int64_t valid_len)
{
    if (mask_kind == ORACLE_MASK_CAUSAL) return j <= i;
    if (mask_kind == ORACLE_MASK_PADDING) return j < valid_len;
    if (mask_kind == ORACLE_MASK_CAUSAL_PADDING) return j <= i && j < valid_len;
    return 1;
}

static int uses_valid_lens(int mask_kind)
{
    return mask_kind == ORACLE_MASK_PADDING || mask_kind == ORACLE_MASK_CAUSAL_PADDING;
}

/*
 * One query row i of one (batch, head):
 *   q    : [d]        the query row
 *   Kbh  : [Nk, d]    keys of this (batch, head)
 *   Vbh  : [Nk, dv]   values of this (batch, head)
 *   s    : [Nk]       caller's scratch for the row of scaled scores
 *   o    : [dv]       output row
 *   a    : [Nk]       optional attention-weight row (may be NULL)
 *   lse  : [1]        optional log-sum-exp of the row's visible scaled scores (may be NULL)
 */
static void attention_row(const double *q, const double *Kbh, const double *Vbh, int64_t Nk, int64_t d,
                          int64_t dv, int mask_kind, int64_t i, int64_t valid_len, double scale, double *s,
                          double *o, double *a, double *lse)
{
    /* stage 1 + 2: s_j = (q . k_j) * scale for every visible key */
    int any = 0;
    for (int64_t j = 0; j < Nk; ++j) {
        if (!visible(mask_kind, i, j, valid_len)) continue;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += q[c] * Kbh[j * d + c];
        s[j] = dot * scale;
        any = 1;
    }

    for (int64_t c = 0; c < dv; ++c) o[c] = 0.0;
    if (!any) { /* no visible key: output 0, weights 0, log of an empty sum */
        if (a) for (int64_t j = 0; j < Nk; ++j) a[j] = 0.0;
        if (lse) *lse = -INFINITY;
        return;
    }

    /* stage 3: stable softmax over the visible keys */
    double m = -INFINITY;
    for (int64_t j = 0; j < Nk; ++j)
        if (visible(mask_kind, i, j, valid_len) && s[j] > m) m = s[j];
    double z = 0.0;
    for (int64_t j = 0; j < Nk; ++j) {
        if (visible(mask_kind, i, j, valid_len)) {
            s[j] = exp(s[j] - m);
            z += s[j];
        } else {
            s[j] = 0.0; /* e^{-inf} = 0 exactly */
        }
    }
    /* ln sum_j exp(s_j) = m + ln sum_j exp(s_j - m) */
    if (lse) *lse = m + log(z);
    for (int64_t j = 0; j < Nk; ++j) s[j] = s[j] / z;

    /* stage 4: weighted sum of the value rows */
    for (int64_t j = 0; j < Nk; ++j) {
        if (s[j] == 0.0) continue;
        for (int64_t c = 0; c < dv; ++c) o[c] += s[j] * Vbh[j * dv + c];
    }
    if (a) for (int64_t j = 0; j < Nk; ++j) a[j] = s[j];
}

static int set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Threads an oracle call uses (OpenMP's current maximum). */
int oracle_max_threads(void) { return set_threads(0); }

/* Offset of the K (or V) head that query head bh = b*H + h reads: head
 * h / (H / Hkv) of batch b, heads of n elements each. */
static int64_t kv_head_offset(int64_t bh, int64_t H, int64_t Hkv, int64_t n)
{
    int64_t b = bh / H, h = bh % H;
    return (b * Hkv + h / (H / Hkv)) * n;
}

static int bad_args(int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, int64_t dv,
                    int mask_kind, const int32_t *valid_lens)
{
    if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || d <= 0 || dv <= 0) return 1;
    if (Hkv <= 0 || (H > 0 && H % Hkv != 0)) return 1;
    if (mask_kind < 0 || mask_kind > ORACLE_MASK_CAUSAL_PADDING) return 1;
    return uses_valid_lens(mask_kind) && !valid_lens;
}

/*
 * Full attention. Q [B,H,Nq,d], K [B,Hkv,Nk,d], V [B,Hkv,Nk,dv] row-major
 * float64; O [B,H,Nq,dv]; A optional [B,H,Nq,Nk]; LSE optional [B,H,Nq].
 * valid_lens [B] is read only for the masks that use it. Returns the number
 * of threads used, or -1 on bad arguments.
 */
int oracle_attn(const double *Q, const double *K, const double *V, int64_t B, int64_t H, int64_t Hkv, int64_t Nq,
                int64_t Nk, int64_t d, int64_t dv, int mask_kind, const int32_t *valid_lens, double scale, double *O,
                double *A, double *LSE, int nthreads)
{
    if (bad_args(B, H, Hkv, Nq, Nk, d, dv, mask_kind, valid_lens)) return -1;
    int used = set_threads(nthreads);
    int64_t rows = B * H * Nq;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < rows; ++r) {
            int64_t i = r % Nq;
            int64_t bh = r / Nq;
            int64_t b = bh / H;
            int64_t L = uses_valid_lens(mask_kind) ? valid_lens[b] : Nk;
            attention_row(Q + r * d, K + kv_head_offset(bh, H, Hkv, Nk * d), V + kv_head_offset(bh, H, Hkv, Nk * dv),
                          Nk, d, dv, mask_kind, i, L, scale, s, O + r * dv, A ? A + r * Nk : NULL,
                          LSE ? LSE + r : NULL);
        }
        free(s);
    }
    return used;
}

/*
 * A subset of rows of the same attention: rows[] holds flat indices
 * r = (b*H + h)*Nq + i; O_rows is [nrows, dv], LSE_rows optional [nrows].
 * Rows are independent, so each one is exact, not an approximation of the
 * full computation.
 */
int oracle_attn_rows(const double *Q, const double *K, const double *V, int64_t B, int64_t H, int64_t Hkv,
                     int64_t Nq, int64_t Nk, int64_t d, int64_t dv, int mask_kind, const int32_t *valid_lens,
                     double scale, const int64_t *rows, int64_t nrows, double *O_rows, double *LSE_rows, int nthreads)
{
    if (bad_args(B, H, Hkv, Nq, Nk, d, dv, mask_kind, valid_lens)) return -1;
    int used = set_threads(nthreads);
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
#pragma omp for schedule(dynamic, 1) reduction(| : bad)
        for (int64_t t = 0; t < nrows; ++t) {
            int64_t r = rows[t];
            if (r < 0 || r >= B * H * Nq) { bad = 1; continue; }
            int64_t i = r % Nq;
            int64_t bh = r / Nq;
            int64_t b = bh / H;
            int64_t L = uses_valid_lens(mask_kind) ? valid_lens[b] : Nk;
            attention_row(Q + r * d, K + kv_head_offset(bh, H, Hkv, Nk * d), V + kv_head_offset(bh, H, Hkv, Nk * dv),
                          Nk, d, dv, mask_kind, i, L, scale, s, O_rows + t * dv, NULL,
                          LSE_rows ? LSE_rows + t : NULL);
        }
        free(s);
    }
    return bad ? -1 : used;
}

/*
 * Gradients of the attention above with respect to Q, K and V, given the
 * gradient dO of the output (same shapes as Q, K, V, O; float64). The pages
 * give no backward algorithm (they motivate gradients through the scaling:
 * "04. Self-Attention", section 四 stage 2); this is the chain rule applied
 * to the four forward stages in reverse, per (batch, query head, row i):
 *   a_j  = the row's softmax weights (stage 3; 0 at masked j)
 *   dV_j += a_j dO_i                       (stage 4: o_i = sum_j a_j v_j)
 *   da_j  = dO_i . v_j
 *   ds_j  = a_j (da_j - sum_k a_k da_k)    (stage 3: the softmax Jacobian)
 *   dQ_i  = scale sum_j ds_j k_j           (stages 1-2: s_j = scale q_i . k_j)
 *   dK_j += scale ds_j q_i
 * With grouped K/V heads the contributions of every query head of a group
 * add up in its K/V head. A row without a visible key contributes nothing.
 * Parallel over (batch, K/V head): the rows that add into one K/V head run
 * in one thread, in a fixed order.
 */
int oracle_attn_bwd(const double *Q, const double *K, const double *V, const double *dO, int64_t B, int64_t H,
                    int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, int64_t dv, int mask_kind,
                    const int32_t *valid_lens, double scale, double *dQ, double *dK, double *dV, int nthreads)
{
    if (bad_args(B, H, Hkv, Nq, Nk, d, dv, mask_kind, valid_lens)) return -1;
    int used = set_threads(nthreads);
    const int64_t group = H > 0 ? H / Hkv : 1;
    for (int64_t x = 0; x < B * Hkv * Nk * d; ++x) dK[x] = 0.0;
    for (int64_t x = 0; x < B * Hkv * Nk * dv; ++x) dV[x] = 0.0;
#pragma omp parallel
    {
        double *a = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        double *s = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        double *o = (double *)malloc(sizeof(double) * (size_t)(dv > 0 ? dv : 1));
        double *da = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t bk = 0; bk < B * Hkv; ++bk) {
            const int64_t b = bk / Hkv, hk = bk % Hkv;
            const double *Kbh = K + bk * Nk * d, *Vbh = V + bk * Nk * dv;
            double *dKbh = dK + bk * Nk * d, *dVbh = dV + bk * Nk * dv;
            const int64_t L = uses_valid_lens(mask_kind) ? valid_lens[b] : Nk;
            for (int64_t h = hk * group; h < (hk + 1) * group; ++h) {
                const int64_t bh = b * H + h;
                for (int64_t i = 0; i < Nq; ++i) {
                    const int64_t r = bh * Nq + i;
                    const double *q = Q + r * d, *g = dO + r * dv;
                    double *dq = dQ + r * d;
                    for (int64_t c = 0; c < d; ++c) dq[c] = 0.0;
                    attention_row(q, Kbh, Vbh, Nk, d, dv, mask_kind, i, L, scale, s, o, a, NULL);
                    double dot = 0.0; /* sum_k a_k da_k */
                    for (int64_t j = 0; j < Nk; ++j) {
                        da[j] = 0.0;
                        if (a[j] == 0.0) continue;
                        for (int64_t c = 0; c < dv; ++c) da[j] += g[c] * Vbh[j * dv + c];
                        dot += a[j] * da[j];
                    }
                    for (int64_t j = 0; j < Nk; ++j) {
                        if (a[j] == 0.0) continue;
                        for (int64_t c = 0; c < dv; ++c) dVbh[j * dv + c] += a[j] * g[c];
                        const double ds = a[j] * (da[j] - dot);
                        for (int64_t c = 0; c < d; ++c) {
                            dq[c] += scale * ds * Kbh[j * d + c];
                            dKbh[j * d + c] += scale * ds * q[c];
                        }
                    }
                }
            }
        }
        free(a);
        free(s);
        free(o);
        free(da);
    }
    return used;
}

/*
 * C[M,N] = A[M,Kd] B[Kd,N], row-major. Each output element is summed over
 * the inner index in ascending order; the loop nest walks B by rows only so
 * that the plain triple loop stays cache friendly.
 */
static void matmul_f64(const double *A, const double *Bm, double *C, int64_t M, int64_t Kd, int64_t N)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double *c = C + m * N;
        for (int64_t n = 0; n < N; ++n) c[n] = 0.0;
        for (int64_t k = 0; k < Kd; ++k) {
            const double a = A[m * Kd + k];
            const double *b = Bm + k * N;
            for (int64_t n = 0; n < N; ++n) c[n] += a * b[n];
        }
    }
}

/*
 * Multi-head attention layer without bias ("Self-Attention 机制", page 5,
 * sections 五步计算 and 维度全程跟踪; page 1 section 八):
 *   P = X W_qkv with W_qkv = [W_Q | W_K | W_V]  (d_model x 3 d_model)
 *   head i uses columns [i*d_k, (i+1)*d_k) of the Q, K and V blocks,
 *   d_k = d_model / h, scale 1/sqrt(d_k), no mask
 *   C[:, i*d_k:(i+1)*d_k] = head_i ;  Y = C W_o
 * X [B,N,d_model], Y [B,N,d_model]; no intermediate rounding.
 */
int oracle_mha(const double *X, const double *Wqkv, const double *Wo, int64_t B, int64_t N, int64_t d_model,
               int64_t h, double *Y, int nthreads)
{
    if (B < 0 || N < 0 || d_model <= 0 || h <= 0 || d_model % h) return -1;
    int used = set_threads(nthreads);
    const int64_t dk = d_model / h, M = B * N, W3 = 3 * d_model;
    double *P = (double *)malloc(sizeof(double) * (size_t)(M * W3 > 0 ? M * W3 : 1));
    double *C = (double *)malloc(sizeof(double) * (size_t)(M * d_model > 0 ? M * d_model : 1));
    double *Qh = (double *)malloc(sizeof(double) * (size_t)(M * d_model > 0 ? M * d_model : 1));
    double *Kh = (double *)malloc(sizeof(double) * (size_t)(M * d_model > 0 ? M * d_model : 1));
    double *Vh = (double *)malloc(sizeof(double) * (size_t)(M * d_model > 0 ? M * d_model : 1));
    if (!P || !C || !Qh || !Kh || !Vh) { free(P); free(C); free(Qh); free(Kh); free(Vh); return -1; }

    /* step 1: one projection GEMM with the concatenated weight */
    matmul_f64(X, Wqkv, P, M, d_model, W3);

    /* split: [B,N,h,dk] -> [B,h,N,dk] for each of Q, K, V */
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < N; ++t)
            for (int64_t hh = 0; hh < h; ++hh)
                for (int64_t c = 0; c < dk; ++c) {
                    int64_t src = (b * N + t) * W3 + hh * dk + c;
                    int64_t dst = ((b * h + hh) * N + t) * dk + c;
                    Qh[dst] = P[src];
                    Kh[dst] = P[src + d_model];
                    Vh[dst] = P[src + 2 * d_model];
                }

    /* per-head attention, no mask, scale 1/sqrt(d_k) */
    double *Oh = P; /* P is no longer needed; reuse its first B*h*N*dk doubles */
    oracle_attn(Qh, Kh, Vh, B, h, h, N, N, dk, dk, ORACLE_MASK_NONE, NULL, 1.0 / sqrt((double)dk), Oh, NULL, NULL,
                nthreads);

    /* concat: [B,h,N,dk] -> [B,N,h*dk] */
    for (int64_t b = 0; b < B; ++b)
        for (int64_t hh = 0; hh < h; ++hh)
            for (int64_t t = 0; t < N; ++t)
                for (int64_t c = 0; c < dk; ++c)
                    C[(b * N + t) * d_model + hh * dk + c] = Oh[((b * h + hh) * N + t) * dk + c];

    /* output projection */
    matmul_f64(C, Wo, Y, M, d_model, d_model);

    free(P); free(C); free(Qh); free(Kh); free(Vh);
    return used;
}

/*
 * Multi-head cross-attention layer without bias: the queries come from one
 * sequence and the keys and values from another ("多模态大模型学习笔记（十四）"
 * section 4: in the decoder's cross-attention Q is the decoder's and K, V
 * the encoder's; "Transformer 详解" section 编码器、解码器与因果掩码), with
 * the same weights and head split as oracle_mha:
 *   Q = Xq W_Q,  [K | V] = Xkv [W_K | W_V],  W_qkv = [W_Q | W_K | W_V]
 *   head i: columns [i*d_k, (i+1)*d_k) of Q, K and V, scale 1/sqrt(d_k)
 *   mask: none, or padding of the key sequence (keys j >= valid_lens[b])
 *   C[:, i*d_k:(i+1)*d_k] = head_i ;  Y = C W_o
 * Xq [B,Nq,d_model], Xkv [B,Nkv,d_model], Y [B,Nq,d_model]; no intermediate
 * rounding.
 */
int oracle_mha_cross(const double *Xq, const double *Xkv, const double *Wqkv, const double *Wo, int64_t B,
                     int64_t Nq, int64_t Nkv, int64_t d_model, int64_t h, int mask_kind, const int32_t *valid_lens,
                     double *Y, int nthreads)
{
    if (B < 0 || Nq < 0 || Nkv < 0 || d_model <= 0 || h <= 0 || d_model % h) return -1;
    if (mask_kind != ORACLE_MASK_NONE && mask_kind != ORACLE_MASK_PADDING) return -1;
    if (mask_kind == ORACLE_MASK_PADDING && !valid_lens && B > 0) return -1;
    int used = set_threads(nthreads);
    const int64_t dk = d_model / h, Mq = B * Nq, Mk = B * Nkv, W3 = 3 * d_model;
    const size_t nq = (size_t)(Mq * d_model > 0 ? Mq * d_model : 1), nk = (size_t)(Mk * d_model > 0 ? Mk * d_model : 1);
    double *Wq = (double *)malloc(sizeof(double) * (size_t)(d_model * d_model));
    double *Wkv = (double *)malloc(sizeof(double) * (size_t)(d_model * 2 * d_model));
    double *Pq = (double *)malloc(sizeof(double) * nq), *Pkv = (double *)malloc(sizeof(double) * 2 * nk);
    double *Qh = (double *)malloc(sizeof(double) * nq), *Oh = (double *)malloc(sizeof(double) * nq);
    double *C = (double *)malloc(sizeof(double) * nq);
    double *Kh = (double *)malloc(sizeof(double) * nk), *Vh = (double *)malloc(sizeof(double) * nk);
    if (!Wq || !Wkv || !Pq || !Pkv || !Qh || !Oh || !C || !Kh || !Vh) {
        free(Wq); free(Wkv); free(Pq); free(Pkv); free(Qh); free(Oh); free(C); free(Kh); free(Vh);
        return -1;
    }
    /* the weight's column blocks: W_Q, and W_K | W_V side by side */
    for (int64_t r = 0; r < d_model; ++r) {
        for (int64_t c = 0; c < d_model; ++c) Wq[r * d_model + c] = Wqkv[r * W3 + c];
        for (int64_t c = 0; c < 2 * d_model; ++c) Wkv[r * 2 * d_model + c] = Wqkv[r * W3 + d_model + c];
    }
    matmul_f64(Xq, Wq, Pq, Mq, d_model, d_model);
    matmul_f64(Xkv, Wkv, Pkv, Mk, d_model, 2 * d_model);

    /* split into heads: [B,N,h,dk] -> [B,h,N,dk] */
    for (int64_t b = 0; b < B; ++b)
        for (int64_t hh = 0; hh < h; ++hh)
            for (int64_t c = 0; c < dk; ++c) {
                for (int64_t t = 0; t < Nq; ++t)
                    Qh[((b * h + hh) * Nq + t) * dk + c] = Pq[(b * Nq + t) * d_model + hh * dk + c];
                for (int64_t t = 0; t < Nkv; ++t) {
                    Kh[((b * h + hh) * Nkv + t) * dk + c] = Pkv[(b * Nkv + t) * 2 * d_model + hh * dk + c];
                    Vh[((b * h + hh) * Nkv + t) * dk + c] = Pkv[(b * Nkv + t) * 2 * d_model + d_model + hh * dk + c];
                }
            }

    oracle_attn(Qh, Kh, Vh, B, h, h, Nq, Nkv, dk, dk, mask_kind, valid_lens, 1.0 / sqrt((double)dk), Oh, NULL, NULL,
                nthreads);

    /* concat: [B,h,Nq,dk] -> [B,Nq,h*dk] */
    for (int64_t b = 0; b < B; ++b)
        for (int64_t hh = 0; hh < h; ++hh)
            for (int64_t t = 0; t < Nq; ++t)
                for (int64_t c = 0; c < dk; ++c)
                    C[(b * Nq + t) * d_model + hh * dk + c] = Oh[((b * h + hh) * Nq + t) * dk + c];
    matmul_f64(C, Wo, Y, Mq, d_model, d_model);

    free(Wq); free(Wkv); free(Pq); free(Pkv); free(Qh); free(Oh); free(C); free(Kh); free(Vh);
    return used;
}
