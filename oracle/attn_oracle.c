/*
 * attn_oracle.c -- plain, slow, fp64 CPU oracle for tiled online-softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, calls or
 * includes this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark load it (through oracle/__init__.py).  It shares no code,
 * header, table or constant with the HIP kernels.
 *
 * What it computes (sources are the four web pages on tiled attention):
 *   - "Sequence length doubles, inference time quadruples" (answer.freetools.me),
 *     section "The mathematical nature of attention", displayed equation:
 *         Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k)) V
 *   - "Flash Attention and Paged Attention" (ipipp.com), section 1: the forward
 *     pass is three steps -- S = Q K^T, P = row-softmax(S), O = P V -- and
 *     section 2: the method only keeps O and the softmax normalisation
 *     statistics (here: LSE = log-sum-exp of each masked, scaled score row).
 *   - same page, section 2, PyTorch call: is_causal=True (query i may attend
 *     keys j <= i).  When the query rows are the last Nq of Nk positions (a
 *     decode step or an appended chunk) the causal limit is aligned to the
 *     bottom-right: query i sits at absolute position Nk - Nq + i.
 *   - same page, section 3, PagedKVCache: the physical pool is
 *     [num_blocks, 2, num_heads, block_size, head_dim], K at index 0, V at 1;
 *     and "Chunked attention ... 70x slower" (cf-1.com), section 2.1: logical
 *     block = token / block_size, physical block = block_table[logical block],
 *     offset = token % block_size.
 *   - same ipipp.com page, section 2, the block-wise forward with running
 *     max m and running sum l: oracle_tiled_online() follows that algorithm
 *     step by step in fp64 (plus the mask); it exists only to pin the online
 *     algebra against the two-pass definition.
 *   - same ipipp.com page, section 2: the forward keeps the softmax statistics
 *     so that the backward can recompute S and P.  oracle_attention_bwd()
 *     gives the gradients dQ, dK, dV of the definition (chain rule through
 *     the three steps of section 1; formulas at that function).
 *
 * Every result is the plain definition, materialised: the full masked score
 * matrix S (-inf outside the allowed set), a two-pass softmax P, then P V.
 * Inputs are upcast exactly (bf16 -> fp64 and fp32 -> fp64 are exact).
 *
 * Preconditions (the definition is undefined otherwise): every query row has
 * at least one allowed key.  A row with none yields NaN, as the definition does.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BF16 0
#define ORACLE_F32 1
#define ORACLE_F64 2

#define ORACLE_OK 0
#define ORACLE_ERR_ARG -1
#define ORACLE_ERR_TABLE -2
#define ORACLE_ERR_ALLOC -3

/* ---- element access: exact upcast of one stored element to fp64 ---------- */
static double elem(const void* base, int dtype, int64_t idx)
{
    if (dtype == ORACLE_BF16) {
        /* bf16 is the top half of an IEEE binary32: shift into place. */
        uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
    return ((const double*)base)[idx];
}

static int elem_size(int dtype)
{
    return dtype == ORACLE_BF16 ? 2 : (dtype == ORACLE_F32 ? 4 : 8);
}

/* Number of keys query row i may attend.
 * mask_mode 0: none (all nk keys).
 * mask_mode 1: causal, bottom-right aligned: key j allowed iff j <= nk - nq + i.
 *              For nq == nk this is the square is_causal rule j <= i. */
static int64_t allowed_keys(int mask_mode, int64_t i, int64_t nq, int64_t nk)
{
    if (mask_mode == 0) return nk;
    int64_t lim = nk - nq + i + 1;
    if (lim < 0) lim = 0;
    if (lim > nk) lim = nk;
    return lim;
}

/*
 * The definition for a block of query rows against one key/value set.
 *   S[i][j] = scale * sum_c Q[i][c] K[j][c]          (j allowed) else -inf
 *   P[i][j] = exp(S[i][j] - m_i) / sum_j' exp(S[i][j'] - m_i),  m_i = max_j S[i][j]
 *   O[i][c] = sum_j P[i][j] V[j][c]
 *   LSE[i]  = m_i + ln sum_j exp(S[i][j] - m_i)
 * Q: [nq][d], K, V: [nk][d], all fp64, row-major.  S and P are materialised
 * as full nq x nk matrices in the caller-provided scratch.
 */
static void attention_dense(const double* Q, const double* K, const double* V,
                            int64_t nq, int64_t nk, int d, double scale,
                            const int64_t* n_allowed, double* S, double* P,
                            double* O, double* LSE)
{
    /* step 1: S = scale * Q K^T, masked */
    for (int64_t i = 0; i < nq; ++i)
        for (int64_t j = 0; j < nk; ++j) {
            if (j < n_allowed[i]) {
                double acc = 0.0;
                for (int c = 0; c < d; ++c) acc += Q[i * d + c] * K[j * d + c];
                S[i * nk + j] = scale * acc;
            } else {
                S[i * nk + j] = -INFINITY;
            }
        }
    /* step 2: P = row-softmax(S), two passes (max, then exp-sum) */
    for (int64_t i = 0; i < nq; ++i) {
        double m = -INFINITY;
        for (int64_t j = 0; j < nk; ++j)
            if (S[i * nk + j] > m) m = S[i * nk + j];
        double l = 0.0;
        for (int64_t j = 0; j < nk; ++j) l += exp(S[i * nk + j] - m);
        for (int64_t j = 0; j < nk; ++j) P[i * nk + j] = exp(S[i * nk + j] - m) / l;
        if (LSE) LSE[i] = m + log(l);
    }
    /* step 3: O = P V */
    for (int64_t i = 0; i < nq; ++i)
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int64_t j = 0; j < nk; ++j) acc += P[i * nk + j] * V[j * d + c];
            O[i * d + c] = acc;
        }
}

/* Copy one [rows][d] head slice out of a [B,H,rows,d] tensor into fp64. */
static void load_head(const void* x, int dtype, int64_t bh, int64_t rows, int d, double* out)
{
    int64_t base = bh * rows * d;
    for (int64_t r = 0; r < rows * d; ++r) out[r] = elem(x, dtype, base + r);
}

/* K/V head of query head h when Hkv K/V heads serve H query heads: groups of
 * H / Hkv consecutive query heads share one K/V head ("Sequence length
 * doubles, inference time quadruples", further optimisations: grouped-query
 * attention; Hkv == H is ordinary multi-head attention, Hkv == 1 is MQA). */
static int kv_head(int h, int H, int Hkv) { return h / (H / Hkv); }

/*
 * Contiguous attention over [B,H,Nq,d] queries and [B,Hkv,Nk,d] keys/values
 * (H a multiple of Hkv).  o: fp64 [B,H,Nq,d]; lse: fp64 [B,H,Nq] (may be NULL).
 */
int oracle_attention(const void* q, const void* k, const void* v, int dtype,
                     int B, int H, int Hkv, int Nq, int Nk, int d, double scale, int mask_mode,
                     double* o, double* lse)
{
    if (!q || !k || !v || !o || B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return ORACLE_ERR_ARG;
    if (Hkv < 1 || H % Hkv != 0) return ORACLE_ERR_ARG;
    if (dtype < ORACLE_BF16 || dtype > ORACLE_F64 || mask_mode < 0 || mask_mode > 1) return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        double* Q = malloc(sizeof(double) * Nq * d);
        double* K = malloc(sizeof(double) * Nk * d);
        double* V = malloc(sizeof(double) * Nk * d);
        double* S = malloc(sizeof(double) * (int64_t)Nq * Nk);
        double* P = malloc(sizeof(double) * (int64_t)Nq * Nk);
        int64_t* lim = malloc(sizeof(int64_t) * Nq);
        if (!Q || !K || !V || !S || !P || !lim) {
#pragma omp atomic write
            err = ORACLE_ERR_ALLOC;
        } else {
            int64_t bkv = (bh / H) * Hkv + kv_head((int)(bh % H), H, Hkv);
            load_head(q, dtype, bh, Nq, d, Q);
            load_head(k, dtype, bkv, Nk, d, K);
            load_head(v, dtype, bkv, Nk, d, V);
            for (int64_t i = 0; i < Nq; ++i) lim[i] = allowed_keys(mask_mode, i, Nq, Nk);
            attention_dense(Q, K, V, Nq, Nk, d, scale, lim, S, P, o + bh * Nq * d,
                            lse ? lse + bh * Nq : NULL);
        }
        free(Q); free(K); free(V); free(S); free(P); free(lim);
    }
    return err;
}

/*
 * Selected rows only (for workloads too large to evaluate in full): sample s
 * is query row rows[s] of head (bidx[s], hidx[s]).  o: fp64 [n][d], lse: [n].
 * Each sample materialises its full masked score row against all Nk keys.
 */
int oracle_attention_rows(const void* q, const void* k, const void* v, int dtype,
                          int B, int H, int Hkv, int Nq, int Nk, int d, double scale, int mask_mode,
                          int n, const int* bidx, const int* hidx, const int* rows,
                          double* o, double* lse)
{
    if (!q || !k || !v || !o || !bidx || !hidx || !rows || n < 0) return ORACLE_ERR_ARG;
    if (Hkv < 1 || H % Hkv != 0) return ORACLE_ERR_ARG;
    for (int s = 0; s < n; ++s)
        if (bidx[s] < 0 || bidx[s] >= B || hidx[s] < 0 || hidx[s] >= H || rows[s] < 0 || rows[s] >= Nq)
            return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int s = 0; s < n; ++s) {
        int64_t bh = (int64_t)bidx[s] * H + hidx[s];
        double* Q = malloc(sizeof(double) * d);
        double* K = malloc(sizeof(double) * (int64_t)Nk * d);
        double* V = malloc(sizeof(double) * (int64_t)Nk * d);
        double* S = malloc(sizeof(double) * Nk);
        double* P = malloc(sizeof(double) * Nk);
        if (!Q || !K || !V || !S || !P) {
#pragma omp atomic write
            err = ORACLE_ERR_ALLOC;
        } else {
            int64_t bkv = (int64_t)bidx[s] * Hkv + kv_head(hidx[s], H, Hkv);
            for (int c = 0; c < d; ++c) Q[c] = elem(q, dtype, (bh * Nq + rows[s]) * d + c);
            load_head(k, dtype, bkv, Nk, d, K);
            load_head(v, dtype, bkv, Nk, d, V);
            int64_t lim = allowed_keys(mask_mode, rows[s], Nq, Nk);
            attention_dense(Q, K, V, 1, Nk, d, scale, &lim, S, P, o + (int64_t)s * d,
                            lse ? lse + s : NULL);
        }
        free(Q); free(K); free(V); free(S); free(P);
    }
    return err;
}

/* ---- backward ------------------------------------------------------------ */
/*
 * Gradients of the forward above with respect to Q, K and V, given the
 * gradient dO of the output.  "Flash Attention and Paged Attention", section
 * 2, keeps the softmax normalisation statistics from the forward so that the
 * backward can recompute S and P instead of storing them; the pages give no
 * formulas for the pass itself, so this is the chain rule through the three
 * forward steps of section 1, for one head:
 *   O = P V                  ->  dV = P^T dO,  dP = dO V^T
 *   P = row-softmax(S)       ->  dS[i][j] = P[i][j] (dP[i][j] - D_i),
 *                                D_i = sum_j P[i][j] dP[i][j]
 *   S = scale Q K^T          ->  dQ = scale dS K,  dK = scale dS^T Q
 * Masked keys have P = 0 and contribute nothing.  With Hkv < H a K/V head's
 * dK and dV are the sums over the query heads of its group.  P is recomputed
 * here by the plain two-pass softmax of the definition, not from saved
 * statistics.
 */

/* One query row: its masked score row against all nk keys, the softmax p,
 * and ds[j] = p[j] (dp[j] - D) with dp[j] = do_i . V[j], D = sum_j p[j] dp[j].
 * o: d doubles of scratch (the row's output, unused here). */
static void grad_row(const double* qi, const double* doi, const double* K, const double* V, int64_t nk, int d,
                     double scale, int64_t lim, double* p, double* ds, double* o)
{
    attention_dense(qi, K, V, 1, nk, d, scale, &lim, ds /* scores; overwritten below */, p, o, NULL);
    double D = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += doi[c] * V[j * d + c];
        ds[j] = acc;
        D += p[j] * acc;
    }
    for (int64_t j = 0; j < nk; ++j) ds[j] = p[j] * (ds[j] - D);
}

/*
 * Contiguous backward over [B,H,Nq,d] queries and output gradients dout and
 * [B,Hkv,Nk,d] keys/values.  dq: fp64 [B,H,Nq,d]; dk, dv: fp64 [B,Hkv,Nk,d].
 */
int oracle_attention_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype,
                         int B, int H, int Hkv, int Nq, int Nk, int d, double scale, int mask_mode,
                         double* dq, double* dk, double* dv)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return ORACLE_ERR_ARG;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1 || Hkv < 1 || H % Hkv != 0) return ORACLE_ERR_ARG;
    if (dtype < ORACLE_BF16 || dtype > ORACLE_F64 || mask_mode < 0 || mask_mode > 1) return ORACLE_ERR_ARG;
    const int G = H / Hkv;
    int err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bk = 0; bk < (int64_t)B * Hkv; ++bk) {
        double* Q = malloc(sizeof(double) * (int64_t)Nq * d);
        double* dO = malloc(sizeof(double) * (int64_t)Nq * d);
        double* K = malloc(sizeof(double) * (int64_t)Nk * d);
        double* V = malloc(sizeof(double) * (int64_t)Nk * d);
        double* p = malloc(sizeof(double) * Nk);
        double* ds = malloc(sizeof(double) * Nk);
        double* o = malloc(sizeof(double) * d);
        if (!Q || !dO || !K || !V || !p || !ds || !o) {
#pragma omp atomic write
            err = ORACLE_ERR_ALLOC;
        } else {
            double* dK = dk + bk * Nk * d;
            double* dV = dv + bk * Nk * d;
            for (int64_t x = 0; x < (int64_t)Nk * d; ++x) dK[x] = dV[x] = 0.0;
            load_head(k, dtype, bk, Nk, d, K);
            load_head(v, dtype, bk, Nk, d, V);
            const int64_t b = bk / Hkv, hk = bk % Hkv;
            for (int gh = 0; gh < G; ++gh) {
                const int64_t bh = b * H + hk * G + gh;
                load_head(q, dtype, bh, Nq, d, Q);
                load_head(dout, dtype, bh, Nq, d, dO);
                for (int64_t i = 0; i < Nq; ++i) {
                    const double* qi = Q + i * d;
                    const double* doi = dO + i * d;
                    grad_row(qi, doi, K, V, Nk, d, scale, allowed_keys(mask_mode, i, Nq, Nk), p, ds, o);
                    double* dQ = dq + (bh * Nq + i) * d;
                    for (int c = 0; c < d; ++c) {
                        double acc = 0.0;
                        for (int64_t j = 0; j < Nk; ++j) acc += ds[j] * K[j * d + c];
                        dQ[c] = scale * acc;
                    }
                    for (int64_t j = 0; j < Nk; ++j)
                        for (int c = 0; c < d; ++c) {
                            dK[j * d + c] += scale * ds[j] * qi[c];
                            dV[j * d + c] += p[j] * doi[c];
                        }
                }
            }
        }
        free(Q); free(dO); free(K); free(V); free(p); free(ds); free(o);
    }
    return err;
}

/*
 * Selected rows of the backward, for workloads too large to evaluate whole.
 *   dQ sample s: query row qrow[s] of head (qb[s], qh[s])        -> dq_rows [nq][d]
 *   dK/dV sample s: key row krow[s] of K/V head (kb[s], khk[s])  -> dk_rows, dv_rows [nk][d]
 * A key sample visits every query row of every query head of the group that
 * may attend that key and materialises its full score row (its softmax needs
 * all of it).  Query rows are split over threads in fixed contiguous ranges
 * whose partial sums are added in thread order.
 */
int oracle_attention_bwd_rows(const void* q, const void* k, const void* v, const void* dout, int dtype,
                              int B, int H, int Hkv, int Nq, int Nk, int d, double scale, int mask_mode,
                              int nq_s, const int* qb, const int* qh, const int* qrow, double* dq_rows,
                              int nk_s, const int* kb, const int* khk, const int* krow, double* dk_rows,
                              double* dv_rows)
{
    if (!q || !k || !v || !dout || nq_s < 0 || nk_s < 0) return ORACLE_ERR_ARG;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1 || Hkv < 1 || H % Hkv != 0) return ORACLE_ERR_ARG;
    if (dtype < ORACLE_BF16 || dtype > ORACLE_F64 || mask_mode < 0 || mask_mode > 1) return ORACLE_ERR_ARG;
    if (nq_s > 0 && (!qb || !qh || !qrow || !dq_rows)) return ORACLE_ERR_ARG;
    if (nk_s > 0 && (!kb || !khk || !krow || !dk_rows || !dv_rows)) return ORACLE_ERR_ARG;
    for (int s = 0; s < nq_s; ++s)
        if (qb[s] < 0 || qb[s] >= B || qh[s] < 0 || qh[s] >= H || qrow[s] < 0 || qrow[s] >= Nq) return ORACLE_ERR_ARG;
    for (int s = 0; s < nk_s; ++s)
        if (kb[s] < 0 || kb[s] >= B || khk[s] < 0 || khk[s] >= Hkv || krow[s] < 0 || krow[s] >= Nk)
            return ORACLE_ERR_ARG;
    const int G = H / Hkv;
    int err = ORACLE_OK;

#pragma omp parallel for schedule(dynamic, 1)
    for (int s = 0; s < nq_s; ++s) {
        double* Q = malloc(sizeof(double) * d);
        double* dO = malloc(sizeof(double) * d);
        double* K = malloc(sizeof(double) * (int64_t)Nk * d);
        double* V = malloc(sizeof(double) * (int64_t)Nk * d);
        double* p = malloc(sizeof(double) * Nk);
        double* ds = malloc(sizeof(double) * Nk);
        double* o = malloc(sizeof(double) * d);
        if (!Q || !dO || !K || !V || !p || !ds || !o) {
#pragma omp atomic write
            err = ORACLE_ERR_ALLOC;
        } else {
            const int64_t bh = (int64_t)qb[s] * H + qh[s];
            const int64_t bkv = (int64_t)qb[s] * Hkv + kv_head(qh[s], H, Hkv);
            for (int c = 0; c < d; ++c) {
                Q[c] = elem(q, dtype, (bh * Nq + qrow[s]) * d + c);
                dO[c] = elem(dout, dtype, (bh * Nq + qrow[s]) * d + c);
            }
            load_head(k, dtype, bkv, Nk, d, K);
            load_head(v, dtype, bkv, Nk, d, V);
            grad_row(Q, dO, K, V, Nk, d, scale, allowed_keys(mask_mode, qrow[s], Nq, Nk), p, ds, o);
            for (int c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j < Nk; ++j) acc += ds[j] * K[j * d + c];
                dq_rows[(int64_t)s * d + c] = scale * acc;
            }
        }
        free(Q); free(dO); free(K); free(V); free(p); free(ds); free(o);
    }
    if (err) return err;

    int nthr = 1;
#ifdef _OPENMP
    nthr = omp_get_max_threads();
#endif
    double* part = calloc((size_t)nthr * 2 * d, sizeof(double));
    double* K = malloc(sizeof(double) * (int64_t)Nk * d);
    double* V = malloc(sizeof(double) * (int64_t)Nk * d);
    if (!part || !K || !V) err = ORACLE_ERR_ALLOC;
    for (int s = 0; s < nk_s && !err; ++s) {
        const int64_t bkv = (int64_t)kb[s] * Hkv + khk[s];
        const int64_t j = krow[s];
        load_head(k, dtype, bkv, Nk, d, K);
        load_head(v, dtype, bkv, Nk, d, V);
        for (int64_t x = 0; x < (int64_t)nthr * 2 * d; ++x) part[x] = 0.0;
#pragma omp parallel num_threads(nthr)
        {
            int t = 0, nt = 1;
#ifdef _OPENMP
            t = omp_get_thread_num();
            nt = omp_get_num_threads();
#endif
            double* acc_k = part + (int64_t)t * 2 * d;
            double* acc_v = acc_k + d;
            double* qi = malloc(sizeof(double) * d);
            double* doi = malloc(sizeof(double) * d);
            double* p = malloc(sizeof(double) * Nk);
            double* ds = malloc(sizeof(double) * Nk);
            double* o = malloc(sizeof(double) * d);
            if (!qi || !doi || !p || !ds || !o) {
#pragma omp atomic write
                err = ORACLE_ERR_ALLOC;
            } else {
                const int64_t rows = (int64_t)G * Nq;
                const int64_t lo = rows * t / nt, hi = rows * (t + 1) / nt;
                for (int64_t x = lo; x < hi; ++x) {
                    const int64_t gh = x / Nq, i = x % Nq;
                    const int64_t lim = allowed_keys(mask_mode, i, Nq, Nk);
                    if (j >= lim) continue;                  /* row i does not attend key j */
                    const int64_t bh = (int64_t)kb[s] * H + (int64_t)khk[s] * G + gh;
                    for (int c = 0; c < d; ++c) {
                        qi[c] = elem(q, dtype, (bh * Nq + i) * d + c);
                        doi[c] = elem(dout, dtype, (bh * Nq + i) * d + c);
                    }
                    grad_row(qi, doi, K, V, Nk, d, scale, lim, p, ds, o);
                    for (int c = 0; c < d; ++c) {
                        acc_k[c] += scale * ds[j] * qi[c];
                        acc_v[c] += p[j] * doi[c];
                    }
                }
            }
            free(qi); free(doi); free(p); free(ds); free(o);
        }
        for (int c = 0; c < d; ++c) {
            double sk = 0.0, sv = 0.0;
            for (int t = 0; t < nthr; ++t) {
                sk += part[(int64_t)t * 2 * d + c];
                sv += part[(int64_t)t * 2 * d + d + c];
            }
            dk_rows[(int64_t)s * d + c] = sk;
            dv_rows[(int64_t)s * d + c] = sv;
        }
    }
    free(part); free(K); free(V);
    return err;
}

/* ---- paged KV cache ------------------------------------------------------ */

/* Element index of (physical block pb, kv in {0:K, 1:V}, head h, in-block
 * offset off, channel c) in the [num_blocks, 2, H, block_size, d] pool. */
static int64_t pool_index(int64_t pb, int kv, int h, int off, int c, int H, int bs, int d)
{
    return (((pb * 2 + kv) * H + h) * bs + off) * (int64_t)d + c;
}

/* Per-token gather of request r, head h: token t lives in logical block
 * t / bs, at offset t % bs of physical block block_table[r][t / bs].
 * Returns ORACLE_ERR_TABLE if an entry needed is outside [0, num_blocks). */
static int gather_head(const void* pool, int dtype, const int* table, int maxb, int num_blocks,
                       int r, int h, int64_t ctx, int H, int bs, int d, double* K, double* V)
{
    for (int64_t t = 0; t < ctx; ++t) {
        int64_t lb = t / bs;
        int off = (int)(t % bs);
        if (lb >= maxb) return ORACLE_ERR_TABLE;
        int64_t pb = table[(int64_t)r * maxb + lb];
        if (pb < 0 || pb >= num_blocks) return ORACLE_ERR_TABLE;
        for (int c = 0; c < d; ++c) {
            K[t * d + c] = elem(pool, dtype, pool_index(pb, 0, h, off, c, H, bs, d));
            V[t * d + c] = elem(pool, dtype, pool_index(pb, 1, h, off, c, H, bs, d));
        }
    }
    return ORACLE_OK;
}

static int64_t prefix_q(const int* q_lens, int r)
{
    int64_t s = 0;
    for (int i = 0; i < r; ++i) s += q_lens[i];
    return s;
}

static int check_paged_args(const int* ctx_lens, const int* q_lens, int num_seqs, int H, int d,
                            int bs, int maxb)
{
    if (num_seqs < 1 || H < 1 || d < 1 || bs < 1 || maxb < 1) return ORACLE_ERR_ARG;
    for (int r = 0; r < num_seqs; ++r)
        if (q_lens[r] < 1 || ctx_lens[r] < q_lens[r]) return ORACLE_ERR_ARG;
    return ORACLE_OK;
}

/*
 * Paged attention, all rows.  q: packed [sum(q_lens), H, d] (request r's rows
 * start at sum_{s<r} q_lens[s]); pool: [num_blocks, 2, Hkv, bs, d] (query
 * head h reads K/V head kv_head(h, H, Hkv));
 * block_table: int32 [num_seqs][maxb]; ctx_lens includes the q_lens new tokens.
 * Query row i of request r attends keys j <= ctx_r - q_r + i.
 * o: fp64 [sum(q_lens), H, d]; lse: fp64 [sum(q_lens), H] (may be NULL).
 */
int oracle_paged_attention(const void* q, int q_dtype, const void* pool, int pool_dtype,
                           const int* block_table, const int* ctx_lens, const int* q_lens,
                           int num_seqs, int H, int Hkv, int d, int bs, int maxb, int num_blocks,
                           double scale, double* o, double* lse)
{
    if (!q || !pool || !block_table || !ctx_lens || !q_lens || !o) return ORACLE_ERR_ARG;
    if (Hkv < 1 || H % Hkv != 0) return ORACLE_ERR_ARG;
    int rc = check_paged_args(ctx_lens, q_lens, num_seqs, H, d, bs, maxb);
    if (rc) return rc;
    int err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t rh = 0; rh < (int64_t)num_seqs * H; ++rh) {
        int r = (int)(rh / H), h = (int)(rh % H);
        int64_t ctx = ctx_lens[r], nq = q_lens[r], row0 = prefix_q(q_lens, r);
        double* Q = malloc(sizeof(double) * nq * d);
        double* K = malloc(sizeof(double) * ctx * d);
        double* V = malloc(sizeof(double) * ctx * d);
        double* S = malloc(sizeof(double) * nq * ctx);
        double* P = malloc(sizeof(double) * nq * ctx);
        double* O = malloc(sizeof(double) * nq * d);
        double* L = malloc(sizeof(double) * nq);
        int64_t* lim = malloc(sizeof(int64_t) * nq);
        int my = ORACLE_OK;
        if (!Q || !K || !V || !S || !P || !O || !L || !lim) my = ORACLE_ERR_ALLOC;
        if (my == ORACLE_OK)
            my = gather_head(pool, pool_dtype, block_table, maxb, num_blocks, r, kv_head(h, H, Hkv), ctx, Hkv,
                             bs, d, K, V);
        if (my == ORACLE_OK) {
            for (int64_t i = 0; i < nq; ++i) {
                for (int c = 0; c < d; ++c) Q[i * d + c] = elem(q, q_dtype, ((row0 + i) * H + h) * d + c);
                lim[i] = allowed_keys(1, i, nq, ctx);
            }
            attention_dense(Q, K, V, nq, ctx, d, scale, lim, S, P, O, L);
            for (int64_t i = 0; i < nq; ++i) {
                for (int c = 0; c < d; ++c) o[((row0 + i) * H + h) * d + c] = O[i * d + c];
                if (lse) lse[(row0 + i) * H + h] = L[i];
            }
        }
        if (my != ORACLE_OK) {
#pragma omp atomic write
            err = my;
        }
        free(Q); free(K); free(V); free(S); free(P); free(O); free(L); free(lim);
    }
    return err;
}

/* Paged attention for sampled (request, head, row-in-request) triples.
 * o: fp64 [n][d]; lse: [n]. */
int oracle_paged_attention_rows(const void* q, int q_dtype, const void* pool, int pool_dtype,
                                const int* block_table, const int* ctx_lens, const int* q_lens,
                                int num_seqs, int H, int Hkv, int d, int bs, int maxb, int num_blocks,
                                double scale, int n, const int* ridx, const int* hidx,
                                const int* iidx, double* o, double* lse)
{
    if (!q || !pool || !block_table || !ctx_lens || !q_lens || !o || !ridx || !hidx || !iidx || n < 0)
        return ORACLE_ERR_ARG;
    if (Hkv < 1 || H % Hkv != 0) return ORACLE_ERR_ARG;
    int rc = check_paged_args(ctx_lens, q_lens, num_seqs, H, d, bs, maxb);
    if (rc) return rc;
    for (int s = 0; s < n; ++s)
        if (ridx[s] < 0 || ridx[s] >= num_seqs || hidx[s] < 0 || hidx[s] >= H ||
            iidx[s] < 0 || iidx[s] >= q_lens[ridx[s]])
            return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int s = 0; s < n; ++s) {
        int r = ridx[s], h = hidx[s];
        int64_t ctx = ctx_lens[r], nq = q_lens[r], i = iidx[s];
        int64_t row = prefix_q(q_lens, r) + i;
        double* Q = malloc(sizeof(double) * d);
        double* K = malloc(sizeof(double) * ctx * d);
        double* V = malloc(sizeof(double) * ctx * d);
        double* S = malloc(sizeof(double) * ctx);
        double* P = malloc(sizeof(double) * ctx);
        int my = ORACLE_OK;
        if (!Q || !K || !V || !S || !P) my = ORACLE_ERR_ALLOC;
        if (my == ORACLE_OK)
            my = gather_head(pool, pool_dtype, block_table, maxb, num_blocks, r, kv_head(h, H, Hkv), ctx, Hkv,
                             bs, d, K, V);
        if (my == ORACLE_OK) {
            for (int c = 0; c < d; ++c) Q[c] = elem(q, q_dtype, (row * H + h) * d + c);
            int64_t lim = allowed_keys(1, i, nq, ctx);
            attention_dense(Q, K, V, 1, ctx, d, scale, &lim, S, P, o + (int64_t)s * d,
                            lse ? lse + s : NULL);
        }
        if (my != ORACLE_OK) {
#pragma omp atomic write
            err = my;
        }
        free(Q); free(K); free(V); free(S); free(P);
    }
    return err;
}

/*
 * Bit-exact gather: copies the stored bytes of K and V of every request,
 * tokens [0, ctx_r), into packed token-major [sum(ctx_lens), H, d] outputs
 * (request r's tokens start at sum_{s<r} ctx_lens[s]).  No arithmetic.
 */
int oracle_paged_gather(const void* pool, int dtype, const int* block_table, const int* ctx_lens,
                        int num_seqs, int H, int d, int bs, int maxb, int num_blocks,
                        void* k_out, void* v_out)
{
    if (!pool || !block_table || !ctx_lens || !k_out || !v_out || num_seqs < 1 || H < 1 || d < 1 ||
        bs < 1 || maxb < 1)
        return ORACLE_ERR_ARG;
    int es = elem_size(dtype);
    int64_t tok0 = 0;
    for (int r = 0; r < num_seqs; ++r) {
        for (int64_t t = 0; t < ctx_lens[r]; ++t) {
            int64_t lb = t / bs;
            int off = (int)(t % bs);
            if (lb >= maxb) return ORACLE_ERR_TABLE;
            int64_t pb = block_table[(int64_t)r * maxb + lb];
            if (pb < 0 || pb >= num_blocks) return ORACLE_ERR_TABLE;
            for (int h = 0; h < H; ++h) {
                int64_t dst = ((tok0 + t) * H + h) * (int64_t)d;
                memcpy((char*)k_out + dst * es, (const char*)pool + pool_index(pb, 0, h, off, 0, H, bs, d) * es,
                       (size_t)d * es);
                memcpy((char*)v_out + dst * es, (const char*)pool + pool_index(pb, 1, h, off, 0, H, bs, d) * es,
                       (size_t)d * es);
            }
        }
        tok0 += ctx_lens[r];
    }
    return ORACLE_OK;
}

/*
 * The block-wise forward with online softmax (ipipp.com page, section 2),
 * one head, in fp64, with the same mask as above.  Keys are visited in blocks
 * of block_size; per row it keeps the running max m (start -inf), running sum
 * l (start 0) and an unnormalised output; each block rescales the old l and O
 * by exp(m_old - m_new) and adds exp(S - m_new) and exp(S - m_new) V; O is
 * divided by l once at the end.  Used only to check that this algorithm and
 * the two-pass definition agree.
 */
int oracle_tiled_online(const void* q, const void* k, const void* v, int dtype, int Nq, int Nk, int d,
                        double scale, int mask_mode, int block_size, double* o, double* lse)
{
    if (!q || !k || !v || !o || Nq < 1 || Nk < 1 || d < 1 || block_size < 1) return ORACLE_ERR_ARG;
    double* m = malloc(sizeof(double) * Nq);
    double* l = malloc(sizeof(double) * Nq);
    double* S = malloc(sizeof(double) * (int64_t)Nq * block_size);
    if (!m || !l || !S) { free(m); free(l); free(S); return ORACLE_ERR_ALLOC; }
    for (int64_t i = 0; i < Nq; ++i) {
        m[i] = -INFINITY;
        l[i] = 0.0;
        for (int c = 0; c < d; ++c) o[i * d + c] = 0.0;
    }
    for (int64_t start = 0; start < Nk; start += block_size) {
        int64_t end = start + block_size < Nk ? start + block_size : Nk;
        int64_t nb = end - start;
        for (int64_t i = 0; i < Nq; ++i) {
            int64_t lim = allowed_keys(mask_mode, i, Nq, Nk);
            double bmax = -INFINITY;
            for (int64_t j = 0; j < nb; ++j) {
                double s = -INFINITY;
                if (start + j < lim) {
                    double acc = 0.0;
                    for (int c = 0; c < d; ++c) acc += elem(q, dtype, i * d + c) * elem(k, dtype, (start + j) * d + c);
                    s = acc * scale;
                }
                S[i * block_size + j] = s;
                if (s > bmax) bmax = s;
            }
            double m_new = m[i] > bmax ? m[i] : bmax;
            double alpha = exp(m[i] - m_new);
            double psum = 0.0;
            for (int c = 0; c < d; ++c) o[i * d + c] *= alpha;
            for (int64_t j = 0; j < nb; ++j) {
                double p = exp(S[i * block_size + j] - m_new);
                psum += p;
                for (int c = 0; c < d; ++c) o[i * d + c] += p * elem(v, dtype, (start + j) * d + c);
            }
            l[i] = alpha * l[i] + psum;
            m[i] = m_new;
        }
    }
    for (int64_t i = 0; i < Nq; ++i) {
        for (int c = 0; c < d; ++c) o[i * d + c] /= l[i];
        if (lse) lse[i] = m[i] + log(l[i]);
    }
    free(m); free(l); free(S);
    return ORACLE_OK;
}

/*
 * Merge of partial results over a partition of one row's keys: part s holds
 * its normalised output O_s and its log-sum-exp lse_s.  With M = max_s lse_s,
 * LSE = M + ln sum_s exp(lse_s - M) and O = sum_s exp(lse_s - LSE) O_s.  This
 * is the same rescaling algebra as the online update above, applied once.
 */
int oracle_lse_merge(int nparts, int d, const double* o_parts, const double* lse_parts,
                     double* o, double* lse)
{
    if (nparts < 1 || d < 1 || !o_parts || !lse_parts || !o) return ORACLE_ERR_ARG;
    double M = -INFINITY;
    for (int s = 0; s < nparts; ++s)
        if (lse_parts[s] > M) M = lse_parts[s];
    double sum = 0.0;
    for (int s = 0; s < nparts; ++s) sum += exp(lse_parts[s] - M);
    double L = M + log(sum);
    for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int s = 0; s < nparts; ++s) acc += exp(lse_parts[s] - L) * o_parts[(int64_t)s * d + c];
        o[c] = acc;
    }
    if (lse) *lse = L;
    return ORACLE_OK;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
