/*
 * attn_oracle.c -- plain fp64 CPU oracle for one Ulysses rank's attention and
 * its post-attention All-to-All layout.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header or constant with the HIP path.
 *
 * What it computes (X-Stage paper, arXiv 2607.23264):
 *   - Fig. 5 of the pith.science review page (Ulysses sequence-parallel
 *     attention): after the pre-attention All-to-All a rank holds the full
 *     sequence for H/P heads; attention runs there; the post-attention
 *     All-to-All puts the output back into the sequence partition.
 *   - Abstract (arXiv abstract page): the fused design lets the owner of an
 *     output tile store it straight into that post-All-to-All placement.
 *   - The attention itself is the ordinary non-causal softmax attention that
 *     FlashAttention (refs. of the review page) computes exactly, up to
 *     rounding; so this oracle is that definition written out, row by row,
 *     with no tiling and no online rescaling.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - scale = 1/sqrt(d) is passed in by the caller; no mask, no dropout.
 *   - rank r owns the contiguous head block g = r*Hl + h_l (Hl = H/P).
 *   - destination rank p owns the contiguous sequence chunk
 *     [p*S/P, (p+1)*S/P); dest layout is [B][P][S/P][H][d].
 *   - tensors hold bf16 bit patterns (uint16); they are widened exactly.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC attn_oracle.c -o liboracle.so -lm
 * (no -ffast-math: evaluation order is the one written here).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Exact widening of a bf16 bit pattern: a bf16 is the top half of an IEEE
 * binary32, so shifting it up 16 bits gives the same value as a float. */
static double widen(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

void oracle_widen(const uint16_t *in, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = widen(in[i]);
}

/* Element offset of (b, s, h, k) in a [B][S][Hl][d] tensor. */
static int64_t bshd(int64_t b, int64_t s, int64_t h, int64_t k,
                    int64_t S, int64_t Hl, int64_t d)
{
    return ((b * S + s) * Hl + h) * d + k;
}

/*
 * Softmax weights of one query row (b, h, s), written to w[0..S).
 *   x_j = scale * sum_k Q[b,s,h,k] * K[b,j,h,k]
 *   w_j = exp(x_j - max_j x_j) / sum_j exp(x_j - max_j x_j)
 * Subtracting the max changes nothing mathematically; it only keeps exp()
 * finite.  Returns the normaliser l (sum of the unnormalised weights), which
 * is always >= 1 because the max term contributes exp(0) = 1.
 */
double oracle_softmax_row(const uint16_t *Q, const uint16_t *K,
                          int64_t S, int64_t Hl, int64_t d, double scale,
                          int64_t b, int64_t h, int64_t s, double *w)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < S; ++j) {
        double acc = 0.0;
        for (int64_t k = 0; k < d; ++k)
            acc += widen(Q[bshd(b, s, h, k, S, Hl, d)]) *
                   widen(K[bshd(b, j, h, k, S, Hl, d)]);
        w[j] = acc * scale;
        if (w[j] > m) m = w[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < S; ++j) {
        w[j] = exp(w[j] - m);
        l += w[j];
    }
    for (int64_t j = 0; j < S; ++j) w[j] /= l;
    return l;
}

/*
 * Attention output for a list of query rows.
 *   rows: nrows triples (b, h, s); out: nrows * d doubles,
 *   out[n][k] = sum_j w_j * V[b,j,h,k]  with w from oracle_softmax_row.
 * nthreads <= 0 uses the OpenMP default.  Returns 0, or -1 on a bad row or
 * allocation failure (out is then unspecified).
 */
int oracle_attn_rows(const uint16_t *Q, const uint16_t *K, const uint16_t *V,
                     int64_t B, int64_t S, int64_t Hl, int64_t d, double scale,
                     const int64_t *rows, int64_t nrows, double *out,
                     int nthreads)
{
    for (int64_t n = 0; n < nrows; ++n) {
        int64_t b = rows[3 * n], h = rows[3 * n + 1], s = rows[3 * n + 2];
        if (b < 0 || b >= B || h < 0 || h >= Hl || s < 0 || s >= S) return -1;
    }
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        double *w = (double *)malloc((size_t)(S > 0 ? S : 1) * sizeof(double));
        if (!w) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t n = 0; n < nrows; ++n) {
            if (!w) continue;
            int64_t b = rows[3 * n], h = rows[3 * n + 1], s = rows[3 * n + 2];
            oracle_softmax_row(Q, K, S, Hl, d, scale, b, h, s, w);
            double *o = out + n * d;
            for (int64_t k = 0; k < d; ++k) {
                double acc = 0.0;
                for (int64_t j = 0; j < S; ++j)
                    acc += w[j] * widen(V[bshd(b, j, h, k, S, Hl, d)]);
                o[k] = acc;
            }
        }
        free(w);
    }
    return failed ? -1 : 0;
}

/* Number of threads an OpenMP region would use here (for reporting). */
int oracle_max_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/*
 * Post-attention All-to-All placement (Fig. 5, steps d-e).
 * Query row s of local head h_l on rank r goes to destination rank
 * p = s / (S/P), at local row i = s mod (S/P), global head g = r*Hl + h_l,
 * inside the destination buffer laid out [B][P][S/P][H][d].
 * Returns the element offset of that row's first element, or -1 if any
 * argument is out of range.
 */
int64_t oracle_dest_offset(int64_t b, int64_t s, int64_t h_l,
                           int64_t B, int64_t S, int64_t H, int64_t d,
                           int64_t P, int64_t rank)
{
    if (P <= 0 || H % P != 0 || S % P != 0) return -1;
    int64_t Hl = H / P, chunk = S / P;
    if (b < 0 || b >= B || s < 0 || s >= S || h_l < 0 || h_l >= Hl ||
        rank < 0 || rank >= P)
        return -1;
    int64_t p = s / chunk;
    int64_t i = s % chunk;
    int64_t g = rank * Hl + h_l;
    return (((b * P + p) * chunk + i) * H + g) * d;
}

/* Vector form: rows are (b, h_l, s) triples; out[n] = dest offset or -1. */
void oracle_dest_offsets(const int64_t *rows, int64_t nrows,
                         int64_t B, int64_t S, int64_t H, int64_t d,
                         int64_t P, int64_t rank, int64_t *out)
{
    for (int64_t n = 0; n < nrows; ++n)
        out[n] = oracle_dest_offset(rows[3 * n], rows[3 * n + 2],
                                    rows[3 * n + 1], B, S, H, d, P, rank);
}

/*
 * The pre-attention All-to-All for one rank (Fig. 5, steps a-c: sequence
 * partitions become head partitions) as a plain copy.  Before it, source rank
 * p holds rows [p*S/P, (p+1)*S/P) of all H heads; laid out as P adjacent
 * regions this is the same [B][P][S/P][H][d] buffer as the destination of the
 * post-attention exchange, so row (b, s, h_l) of this rank's X_local
 * [B][S][Hl][d] is read from oracle_dest_offset(b, s, h_l, ...).  Returns 0 or -1.
 */
int oracle_gather(const uint16_t *X, int64_t B, int64_t S, int64_t H, int64_t d,
                  int64_t P, int64_t rank, uint16_t *X_local)
{
    if (P <= 0 || H % P != 0 || S % P != 0 || rank < 0 || rank >= P) return -1;
    int64_t Hl = H / P;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t s = 0; s < S; ++s)
            for (int64_t h = 0; h < Hl; ++h) {
                int64_t off = oracle_dest_offset(b, s, h, B, S, H, d, P, rank);
                memcpy(X_local + bshd(b, s, h, 0, S, Hl, d), X + off,
                       (size_t)d * sizeof(uint16_t));
            }
    return 0;
}

/*
 * The serial All-to-All as a plain copy: every row (b, s, h_l) of the local
 * output O_local [B][S][Hl][d] is copied bit-for-bit to its destination slot.
 * Slots of other ranks' heads are not touched.  Returns 0 or -1.
 */
int oracle_permute(const uint16_t *O_local, int64_t B, int64_t S, int64_t H,
                   int64_t d, int64_t P, int64_t rank, uint16_t *dest)
{
    if (P <= 0 || H % P != 0 || S % P != 0 || rank < 0 || rank >= P) return -1;
    int64_t Hl = H / P;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t s = 0; s < S; ++s)
            for (int64_t h = 0; h < Hl; ++h) {
                int64_t off = oracle_dest_offset(b, s, h, B, S, H, d, P, rank);
                memcpy(dest + off, O_local + bshd(b, s, h, 0, S, Hl, d),
                       (size_t)d * sizeof(uint16_t));
            }
    return 0;
}
