/*
 * CPU fp64 oracle for the scaled-dot-product attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU-baseline
 * leg may load this library.  It shares no code, header, table or helper with the HIP
 * path, and the product path never calls it.
 *
 * Every function is the plain definition, written out in double precision:
 *   - scores s_ij = scale * sum_d q_id k_jd over the allowed keys j of row i,
 *   - m_i = max_j s_ij, l_i = sum_j exp(s_ij - m_i),
 *   - out_i = sum_j exp(s_ij - m_i) v_j / l_i,
 * a two-pass softmax with no tiling and no online rescaling.
 *
 * Sources (web pages, cited by title and section):
 *   - formula and the 1/sqrt(d) scale: Paddle "sparse_attention" API page, formula section;
 *     the blog "高效 AI 模型开发：PyTorch torch.nn.attention 报错排查与高效替代方法",
 *     manual_attention section (scores, softmax over the last dim, times V).
 *   - packed TND batches, cumulative END offsets, GQA ratio, band/causal masks:
 *     "aclnnFlashAttentionVarLenScore", 功能说明 (function) and 约束说明 (constraints).
 *   - the merge of two partial (out, max, sum) triples:
 *     "npu_ring_attention_update对外接口", equivalent small-operator logic section.
 *   - CSR rows (row pointer `offset`, `columns`): Paddle "sparse_attention", parameters
 *     and code example sections.
 *
 * Readings where the pages are silent (each listed with its reason in the design notes):
 *   - mask: keep(i, j) <=> -pre <= j - i <= next on sequence-local positions, top-left
 *     aligned; causal = (pre = +inf, next = 0); "none" keeps every key.
 *   - a row with no allowed key gives out = 0, max = -inf, sum = 0.
 *   - GQA: query head h reads kv head h / (Nq / Nkv).
 *   - softmax_max is in natural-log units of the SCALED logits; softmax_sum is taken at
 *     the final max.
 *
 * Parity pins live in tests/test_oracle_pins.py (CPU only).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_MASK_NONE = 0, OR_MASK_CAUSAL = 1, OR_MASK_BAND = 2 };

/* Is key j visible from query i (both sequence-local)? */
static int allowed(int mask, int64_t i, int64_t j, int64_t pre, int64_t next)
{
    if (mask == OR_MASK_NONE) return 1;
    if (mask == OR_MASK_CAUSAL) return j <= i;
    /* band: -pre <= j - i <= next, evaluated without overflow */
    __int128 d = (__int128)j - (__int128)i;
    return d >= -(__int128)pre && d <= (__int128)next;
}

/*
 * One query row against a key/value sequence.
 *   q: D values;  k_row(j) = k + j*kstride (D values);  v_row(j) = v + j*vstride (Dv values);
 *   keys j in [0, Skv) filtered by keep_row[j] when keep_row is given, else by
 *   allowed(mask, i, j, ...).
 *   s: scratch of Skv doubles.  out: Dv values.  probs (optional): Skv outputs, 0 for
 *   masked keys.
 */
static int visible(const unsigned char* keep_row, int mask, int64_t i, int64_t j, int64_t pre,
                   int64_t next)
{
    return keep_row ? keep_row[j] != 0 : allowed(mask, i, j, pre, next);
}

static void attend_row(const double* q, const double* k, int64_t kstride,
                       const double* v, int64_t vstride, int64_t Skv, int64_t D, int64_t Dv,
                       double scale, int mask, int64_t i, int64_t pre, int64_t next,
                       const unsigned char* keep_row,
                       double* out, double* m_out, double* l_out, double* s, double* probs)
{
    /* pass 1: scores and their max */
    double m = -INFINITY;
    int64_t n_allowed = 0;
    for (int64_t j = 0; j < Skv; ++j) {
        if (!visible(keep_row, mask, i, j, pre, next)) continue;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += q[d] * k[j * kstride + d];
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
        ++n_allowed;
    }
    for (int64_t d = 0; d < Dv; ++d) out[d] = 0.0;
    if (probs)
        for (int64_t j = 0; j < Skv; ++j) probs[j] = 0.0;
    if (n_allowed == 0) {
        *m_out = -INFINITY;
        *l_out = 0.0;
        return;
    }
    /* pass 2: exponentials, their sum, and the weighted sum of values */
    double l = 0.0;
    for (int64_t j = 0; j < Skv; ++j) {
        if (!visible(keep_row, mask, i, j, pre, next)) continue;
        double e = exp(s[j] - m);
        l += e;
        for (int64_t d = 0; d < Dv; ++d) out[d] += e * v[j * vstride + d];
    }
    for (int64_t d = 0; d < Dv; ++d) out[d] /= l;
    if (probs)
        for (int64_t j = 0; j < Skv; ++j)
            if (visible(keep_row, mask, i, j, pre, next)) probs[j] = exp(s[j] - m) / l;
    *m_out = m;
    *l_out = l;
}

static int pick_threads(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

static int mask_ok(int mask) { return mask == OR_MASK_NONE || mask == OR_MASK_CAUSAL || mask == OR_MASK_BAND; }

/*
 * Dense attention.  q [B][Nq][Sq][D], k/v [B][Nkv][Skv][D], out [B][Nq][Sq][D],
 * smax/ssum [B][Nq][Sq], probs (optional) [B][Nq][Sq][Skv]; all contiguous fp64.
 * Returns 0, or -1 on an invalid argument.
 */
int oracle_attn(const double* q, const double* k, const double* v, double* out,
                double* smax, double* ssum, double* probs,
                int64_t B, int64_t Nq, int64_t Nkv, int64_t Sq, int64_t Skv, int64_t D,
                double scale, int mask, int64_t pre, int64_t next, int nthreads)
{
    if (B < 0 || Nq <= 0 || Nkv <= 0 || Sq < 0 || Skv < 0 || D <= 0) return -1;
    if (Nq % Nkv != 0 || !mask_ok(mask)) return -1;
    const int64_t G = Nq / Nkv;
    const int64_t rows = B * Nq * Sq;
    int nt = pick_threads(nthreads);
#pragma omp parallel num_threads(nt)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < rows; ++r) {
            int64_t i = r % Sq, h = (r / Sq) % Nq, b = r / (Sq * Nq);
            int64_t g = h / G;
            const double* qr = q + ((b * Nq + h) * Sq + i) * D;
            const double* kb = k + (b * Nkv + g) * Skv * D;
            const double* vb = v + (b * Nkv + g) * Skv * D;
            double* o = out + ((b * Nq + h) * Sq + i) * D;
            double* pr = probs ? probs + ((b * Nq + h) * Sq + i) * Skv : NULL;
            attend_row(qr, kb, D, vb, D, Skv, D, D, scale, mask, i, pre, next, NULL,
                       o, smax + r, ssum + r, s, pr);
        }
        free(s);
    }
    return 0;
}

/*
 * Packed variable-length attention (TND).  q [Tq][Nq][D], k/v [Tkv][Nkv][D],
 * out [Tq][Nq][D], smax/ssum [Nq][Tq].  cu_q/cu_kv: B END offsets (no leading 0),
 * so sequence b spans rows [cu[b-1], cu[b]) with cu[-1] = 0.  Positions inside the
 * mask are local to the sequence.
 */
int oracle_attn_varlen(const double* q, const double* k, const double* v, double* out,
                       double* smax, double* ssum,
                       const int64_t* cu_q, const int64_t* cu_kv, int64_t B,
                       int64_t Tq, int64_t Tkv, int64_t Nq, int64_t Nkv, int64_t D,
                       double scale, int mask, int64_t pre, int64_t next, int nthreads)
{
    if (B <= 0 || Nq <= 0 || Nkv <= 0 || D <= 0 || Nq % Nkv != 0 || !mask_ok(mask)) return -1;
    int64_t prev_q = 0, prev_kv = 0, max_kv = 1;
    for (int64_t b = 0; b < B; ++b) {
        if (cu_q[b] < prev_q || cu_kv[b] < prev_kv) return -1;
        if (cu_kv[b] - prev_kv > max_kv) max_kv = cu_kv[b] - prev_kv;
        prev_q = cu_q[b];
        prev_kv = cu_kv[b];
    }
    if (prev_q != Tq || prev_kv != Tkv) return -1;
    const int64_t G = Nq / Nkv;
    int nt = pick_threads(nthreads);
#pragma omp parallel num_threads(nt)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)max_kv);
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < Tq * Nq; ++r) {
            int64_t t = r / Nq, h = r % Nq, g = h / G;
            int64_t b = 0;
            while (cu_q[b] <= t) ++b; /* sequence holding row t */
            int64_t q0 = b ? cu_q[b - 1] : 0, kv0 = b ? cu_kv[b - 1] : 0;
            int64_t Skv = cu_kv[b] - kv0;
            const double* kb = k + (kv0 * Nkv + g) * D;
            const double* vb = v + (kv0 * Nkv + g) * D;
            attend_row(q + (t * Nq + h) * D, kb, Nkv * D, vb, Nkv * D, Skv, D, D, scale, mask,
                       t - q0, pre, next, NULL, out + (t * Nq + h) * D, smax + h * Tq + t,
                       ssum + h * Tq + t, s, NULL);
        }
        free(s);
    }
    return 0;
}

/*
 * Dense attention with an explicit visibility matrix and a value head dim of its own.
 *   q [B][Nq][Sq][D], k [B][Nkv][Skv][D], v [B][Nkv][Skv][Dv], out [B][Nq][Sq][Dv],
 *   smax/ssum [B][Nq][Sq]; keep [B][Sq][Skv] bytes (nonzero: key j visible from query i),
 *   shared by the heads of a batch entry.  Each row is the plain definition over its
 *   visible keys; a row with none gives out = 0, max = -inf, sum = 0.
 */
int oracle_attn_keep(const double* q, const double* k, const double* v, double* out,
                     double* smax, double* ssum, const unsigned char* keep,
                     int64_t B, int64_t Nq, int64_t Nkv, int64_t Sq, int64_t Skv, int64_t D,
                     int64_t Dv, double scale, int nthreads)
{
    if (B < 0 || Nq <= 0 || Nkv <= 0 || Sq < 0 || Skv < 0 || D <= 0 || Dv <= 0) return -1;
    if (Nq % Nkv != 0 || !keep) return -1;
    const int64_t G = Nq / Nkv;
    const int64_t rows = B * Nq * Sq;
    int nt = pick_threads(nthreads);
#pragma omp parallel num_threads(nt)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < rows; ++r) {
            int64_t i = r % Sq, h = (r / Sq) % Nq, b = r / (Sq * Nq);
            int64_t g = h / G;
            attend_row(q + ((b * Nq + h) * Sq + i) * D, k + (b * Nkv + g) * Skv * D, D,
                       v + (b * Nkv + g) * Skv * Dv, Dv, Skv, D, Dv, scale, OR_MASK_NONE, i, 0, 0,
                       keep + (b * Sq + i) * Skv, out + ((b * Nq + h) * Sq + i) * Dv, smax + r,
                       ssum + r, s, NULL);
        }
        free(s);
    }
    return 0;
}

/*
 * Merge of two partial results of the same queries over disjoint key sets (the update of
 * "npu_ring_attention_update对外接口"), written from the log-sum-exp identity rather than
 * in that page's step order: a partial (o_i, m_i, l_i) stands for keys whose softmax
 * weights sum to Z_i = l_i e^{m_i}, i.e. log|Z_i| = m_i + ln|l_i| (the sign of l_i is kept,
 * so that the page's example with arbitrary, even negative, sums is covered).  The union of
 * the keys has Z = Z_1 + Z_2, taken as a signed log-add-exp; each partial output enters
 * with weight Z_i / Z; the union's max is max(m_1, m_2) and its sum l = Z e^{-max}.
 *   o1, o2, out [B][N][S][D]; m1, l1, m2, l2, mo, lo [B][N][S]; contiguous fp64.
 * Reading for an all-empty pair (both max = -inf, where the plain formula divides 0/0):
 * out = 0, max = -inf, sum = 0.  A pair whose sums are both 0 has no weight at all and
 * gives out = 0, sum = 0 with the larger max.
 */
int oracle_merge(const double* o1, const double* m1, const double* l1,
                 const double* o2, const double* m2, const double* l2,
                 double* out, double* mo, double* lo,
                 int64_t B, int64_t N, int64_t S, int64_t D, int nthreads)
{
    if (B < 0 || N <= 0 || S < 0 || D <= 0) return -1;
    const int64_t rows = B * N * S;
    int nt = pick_threads(nthreads);
#pragma omp parallel for num_threads(nt) schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double m = m1[r] > m2[r] ? m1[r] : m2[r];
        /* log|Z_i| and sign of Z_i; an empty partial (sum 0) has log|Z_i| = -inf */
        const double a1 = l1[r] == 0.0 ? -INFINITY : m1[r] + log(fabs(l1[r]));
        const double a2 = l2[r] == 0.0 ? -INFINITY : m2[r] + log(fabs(l2[r]));
        const double g1 = l1[r] < 0.0 ? -1.0 : 1.0, g2 = l2[r] < 0.0 ? -1.0 : 1.0;
        const double amax = a1 > a2 ? a1 : a2;
        if (m == -INFINITY || amax == -INFINITY) {
            mo[r] = m;
            lo[r] = 0.0;
            for (int64_t d = 0; d < D; ++d) out[r * D + d] = 0.0;
            continue;
        }
        /* Z = Z_1 + Z_2 = e^{amax} (g1 e^{a1 - amax} + g2 e^{a2 - amax}) */
        const double rel = g1 * exp(a1 - amax) + g2 * exp(a2 - amax);
        const double gz = rel < 0.0 ? -1.0 : 1.0;
        const double az = amax + log(fabs(rel));             /* log|Z| */
        const double w1 = g1 * gz * exp(a1 - az);              /* Z_1 / Z */
        const double w2 = g2 * gz * exp(a2 - az);              /* Z_2 / Z */
        for (int64_t d = 0; d < D; ++d) out[r * D + d] = o1[r * D + d] * w1 + o2[r * D + d] * w2;
        mo[r] = m;
        lo[r] = gz * exp(az - m);
    }
    return 0;
}

/*
 * CSR-sparse attention.  q/k/v/out [B][N][S][D] fp64; offset [B][N][S+1] int32 row
 * pointer; columns [B][N][nnz] int32.  Row i of slice (b, n) attends to the entries
 * columns[b][n][offset[b][n][i] .. offset[b][n][i+1]) of the same slice; every stored
 * entry counts once (a repeated column counts as often as it is stored); an empty row
 * gives 0.  smax/ssum (optional) [B][N][S] as for dense attention.
 */
int oracle_sparse(const double* q, const double* k, const double* v, double* out,
                  double* smax, double* ssum, const int32_t* offset, const int32_t* columns,
                  int64_t nnz, int64_t B, int64_t N, int64_t S, int64_t D, double scale,
                  int nthreads)
{
    if (B < 0 || N <= 0 || S < 0 || D <= 0 || nnz < 0) return -1;
    const int64_t rows = B * N * S;
    for (int64_t bn = 0; bn < B * N; ++bn) {
        const int32_t* off = offset + bn * (S + 1);
        if (off[0] < 0 || off[S] > nnz) return -1;
        for (int64_t i = 0; i < S; ++i)
            if (off[i + 1] < off[i]) return -1;
        for (int64_t e = 0; e < off[S]; ++e)
            if (columns[bn * nnz + e] < 0 || columns[bn * nnz + e] >= S) return -1;
    }
    int nt = pick_threads(nthreads);
#pragma omp parallel num_threads(nt)
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(nnz > 0 ? nnz : 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < rows; ++r) {
            int64_t i = r % S, bn = r / S;
            const int32_t* off = offset + bn * (S + 1);
            const int32_t* col = columns + bn * nnz;
            const double* qr = q + r * D;
            const double* kb = k + bn * S * D;
            const double* vb = v + bn * S * D;
            double* o = out + r * D;
            int64_t e0 = off[i], e1 = off[i + 1];
            double m = -INFINITY;
            for (int64_t e = e0; e < e1; ++e) {
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d) dot += qr[d] * kb[(int64_t)col[e] * D + d];
                s[e - e0] = scale * dot;
                if (s[e - e0] > m) m = s[e - e0];
            }
            for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
            double l = 0.0;
            for (int64_t e = e0; e < e1; ++e) {
                double w = exp(s[e - e0] - m);
                l += w;
                for (int64_t d = 0; d < D; ++d) o[d] += w * vb[(int64_t)col[e] * D + d];
            }
            if (e1 > e0)
                for (int64_t d = 0; d < D; ++d) o[d] /= l;
            if (smax) smax[r] = e1 > e0 ? m : -INFINITY;
            if (ssum) ssum[r] = l;
        }
        free(s);
    }
    return 0;
}
