/*
 * sketch_oracle.c -- plain, slow, obviously-correct CPU oracle for the
 * UltraSketchLLM sketch encoder and the sketch-decoded matrix product.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this code.  It shares nothing with
 * the HIP path (no headers, no helpers, no tables); the two are compared on
 * the same seeded inputs.
 *
 * Source of the method: "UltraSketchLLM: Sub-1-Bit LLM Compression via
 * Sketch and Hardware-Friendly Operators" (gist.science explainer, Spanish
 * page "Resumen Técnico" and its Dutch twin "Technische Samenvatting"):
 *   - Metodología §1 "Diseño de Sketch AbsMaxMin": the sketch state keeps,
 *     per bucket, the weight of minimum absolute value among the weights the
 *     hash drops into it; reconstruction is the original value or one of
 *     smaller magnitude (the underestimation bound).
 *   - Metodología §4 "Mapeo de Operadores de Matriz": compression is a
 *     MIN-reduction over absolute values through a projection matrix P;
 *     decompression is the plain product W_hat = S * P^T.
 *   - Resultados › Ablación: the matrix form equals the sequential form.
 * Readings where the pages are silent (hash function, key arithmetic,
 * tie-break, empty buckets, rounding, rejection rules) are the ones listed
 * in the design notes; each is restated at the function that uses it.
 *
 * Everything here is a direct loop over the definition: no blocking, no
 * fusion, no reordering.  Blocks (and output rows) are independent by
 * definition, so an OpenMP loop over them changes no result.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_OK = 0, OR_EINVAL = -1, OR_ERANGE = -2 };
enum { OR_F32 = 0, OR_BF16 = 1, OR_F16 = 2 };
enum { OR_ABSMIN = 0, OR_ABSMAX = 1 };

/* ------------------------------------------------------------------ */
/* Number formats (IEEE 754 binary16, and bfloat16 = top half of a    */
/* binary32).  Written from the format definitions, value by value.   */
/* ------------------------------------------------------------------ */

/* binary16 bit pattern -> exact double value. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0x1F)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -24);              /* subnormal: m * 2^-24 */
    else
        v = ldexp((double)(1024 + m), e - 25);  /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* binary32 -> binary16, round to nearest, ties to even; subnormals kept,
 * sign of zero kept, overflow to infinity.  Value-based: find the spacing q
 * of binary16 numbers around |f|, round |f|/q to an integer with the
 * current (nearest-even) rounding mode, then encode the rounded value. */
uint16_t oracle_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    if (isnan(f))
        return sign | 0x7E00;
    double a = fabs((double)f);
    if (a == 0.0)
        return sign;
    if (isinf(f))
        return sign | 0x7C00;
    int e2;
    frexp(a, &e2);                  /* a = m * 2^e2, m in [0.5, 1) */
    int E = e2 - 1;                 /* floor(log2 a) */
    if (E < -14)
        E = -14;                    /* below the normal range the spacing is 2^-24 */
    double q = ldexp(1.0, E - 10);  /* 10 fraction bits */
    double n = nearbyint(a / q);    /* a/q is exact: q is a power of two */
    double r = n * q;               /* rounded magnitude, exact */
    if (r >= 65536.0)
        return sign | 0x7C00;       /* beyond the largest finite binary16 */
    if (r < ldexp(1.0, -14))
        return sign | (uint16_t)(r / ldexp(1.0, -24));   /* subnormal (or 2^-14 exactly handled below) */
    int er;
    double mr = frexp(r, &er);      /* r = mr * 2^er, mr in [0.5,1) */
    int Er = er - 1;
    uint16_t frac = (uint16_t)((mr * 2.0 - 1.0) * 1024.0);
    return sign | (uint16_t)((Er + 15) << 10) | frac;
}

/* Array form of oracle_f32_to_f16, element by element. */
void oracle_f32_to_f16_n(const float* f, int64_t n, uint16_t* h)
{
    for (int64_t e = 0; e < n; ++e)
        h[e] = oracle_f32_to_f16(f[e]);
}

/* bfloat16 bit pattern -> float: the 16 bits are the top half of a binary32. */
static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Element e of an input array of the given dtype, widened exactly to float. */
static float load_as_f32(const void* base, int dtype, int64_t e)
{
    if (dtype == OR_F32)
        return ((const float*)base)[e];
    if (dtype == OR_BF16)
        return bf16_to_f32(((const uint16_t*)base)[e]);
    return (float)oracle_f16_to_f64(((const uint16_t*)base)[e]);
}

/* ------------------------------------------------------------------ */
/* Budget and layout.                                                 */
/* The method's operating point is 0.5 bits per weight ("Resultados", */
/* compression efficiency); a bucket is one binary16 value, so a      */
/* block of R rows x N columns holds Bg = R*N*bpw/16 buckets.         */
/* ------------------------------------------------------------------ */
int oracle_layout(int64_t M, int64_t N, int32_t R, double bpw, int64_t* nb, int64_t* Bg)
{
    if (M < 0 || N <= 0 || R <= 0 || !(bpw > 0.0) || !isfinite(bpw))
        return OR_EINVAL;
    if (M % R != 0)
        return OR_EINVAL;
    double bg = (double)R * (double)N * bpw / 16.0;
    double bgi = floor(bg);
    if (bg != bgi || bgi < 1.0 || bgi > 4294967295.0)
        return OR_EINVAL;
    if ((double)R * (double)N > 4294967295.0)   /* local index l must fit 32 bits */
        return OR_EINVAL;
    *nb = M / R;
    *Bg = (int64_t)bgi;
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Hash: the projection matrix P is one-hot, row l has its single 1   */
/* at column k(l).  l = r*N + j is the position inside a row block,   */
/* row-major; the map does not depend on the block.                   */
/*   k(l) = (u64(hash32((u32)(l * 0x9E3779B1) ^ seed)) * Bg) >> 32    */
/* hash32 is read as MurmurHash3's 32-bit finalizer (fmix32).         */
/* ------------------------------------------------------------------ */
uint32_t oracle_hash32(uint32_t h)
{
    h ^= h >> 16;
    h *= 0x85EBCA6Bu;
    h ^= h >> 13;
    h *= 0xC2B2AE35u;
    h ^= h >> 16;
    return h;
}

uint32_t oracle_bucket(uint32_t l, uint32_t seed, uint32_t Bg)
{
    uint32_t u = (uint32_t)(l * 0x9E3779B1u) ^ seed;
    uint64_t h = oracle_hash32(u);
    return (uint32_t)((h * (uint64_t)Bg) >> 32);
}

/* Fill k[l] for every local position l in [0, R*N). */
void oracle_bucket_map(int64_t R, int64_t N, uint32_t seed, uint32_t Bg, uint32_t* k)
{
    for (int64_t l = 0; l < R * N; ++l)
        k[l] = oracle_bucket((uint32_t)l, seed, Bg);
}

/* ------------------------------------------------------------------ */
/* Encode (compression).                                              */
/*                                                                    */
/* AbsMaxMin sketch, "Metodología §1": each bucket keeps the weight   */
/* with the minimum absolute value among those hashed into it.        */
/* Importance ("Metodología §2", E[a^2]) scales the comparison per    */
/* input column: key = |w| * imp[j], one binary32 multiply.  With     */
/* imp == 1 this is the pages' |w| rule.  rule ABSMAX keeps the       */
/* largest key instead (the explainer's plain-language "keep the      */
/* biggest / most important" reading).                                */
/* Scan order: blocks independently, l ascending; a bucket's holder   */
/* is replaced only on a strict improvement, so among equal keys the  */
/* smallest l wins.  Bucket value = binary16 RNE of the winning       */
/* weight; a bucket nobody hashes into holds +0.                      */
/* Rejections: any weight that is NaN/Inf or whose magnitude rounds   */
/* to binary16 infinity (|w| >= 65520) -> OR_ERANGE; any importance   */
/* that is NaN, infinite or negative -> OR_EINVAL.  On error S is     */
/* left untouched.                                                    */
/* ------------------------------------------------------------------ */
int oracle_encode(int64_t M, int64_t N, int32_t R, double bpw, uint32_t seed, int rule,
                  int w_dtype, const void* W, const float* imp, uint16_t* S, int nthreads)
{
    int64_t nb, Bg;
    if (oracle_layout(M, N, R, bpw, &nb, &Bg) != OR_OK)
        return OR_EINVAL;
    if (rule != OR_ABSMIN && rule != OR_ABSMAX)
        return OR_EINVAL;
    if (w_dtype != OR_F32 && w_dtype != OR_BF16 && w_dtype != OR_F16)
        return OR_EINVAL;

    if (imp)
        for (int64_t j = 0; j < N; ++j)
            if (!isfinite(imp[j]) || imp[j] < 0.0f)
                return OR_EINVAL;

    for (int64_t e = 0; e < M * N; ++e) {
        float w = load_as_f32(W, w_dtype, e);
        if (!isfinite(w) || fabsf(w) >= 65520.0f)
            return OR_ERANGE;
    }

    int64_t L = (int64_t)R * N;
    uint32_t* k = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)L);
    if (!k)
        return OR_EINVAL;
    oracle_bucket_map(R, N, seed, (uint32_t)Bg, k);

#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        int64_t* best_l = (int64_t*)malloc(sizeof(int64_t) * (size_t)Bg);
        float* best_key = (float*)malloc(sizeof(float) * (size_t)Bg);
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t b = 0; b < nb; ++b) {
            for (int64_t q = 0; q < Bg; ++q)
                best_l[q] = -1;
            for (int64_t l = 0; l < L; ++l) {
                int64_t r = l / N, j = l % N;
                float w = load_as_f32(W, w_dtype, (b * R + r) * N + j);
                float key = fabsf(w) * (imp ? imp[j] : 1.0f);
                uint32_t q = k[l];
                int better;
                if (best_l[q] < 0)
                    better = 1;
                else if (rule == OR_ABSMIN)
                    better = key < best_key[q];
                else
                    better = key > best_key[q];
                if (better) {
                    best_l[q] = l;
                    best_key[q] = key;
                }
            }
            for (int64_t q = 0; q < Bg; ++q) {
                uint16_t v = 0;
                if (best_l[q] >= 0) {
                    int64_t l = best_l[q];
                    v = oracle_f32_to_f16(load_as_f32(W, w_dtype, (b * R + l / N) * N + l % N));
                }
                S[b * Bg + q] = v;
            }
        }
        free(best_l);
        free(best_key);
    }
    free(k);
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Decode (decompression), "Metodología §4": W_hat = S * P^T, i.e.    */
/* W_hat[i][j] = S[i / R][k((i % R) * N + j)], exactly as a double.   */
/* ------------------------------------------------------------------ */
int oracle_decode(int64_t M, int64_t N, int32_t R, double bpw, uint32_t seed,
                  const uint16_t* S, double* What)
{
    int64_t nb, Bg;
    if (oracle_layout(M, N, R, bpw, &nb, &Bg) != OR_OK)
        return OR_EINVAL;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            uint32_t q = oracle_bucket((uint32_t)((i % R) * N + j), seed, (uint32_t)Bg);
            What[i * N + j] = oracle_f16_to_f64(S[(i / R) * Bg + q]);
        }
    return OR_OK;
}

/* One output of the product, from its definition:
 * Y[t][i] = sum_j X[t][j] * W_hat[i][j], in double, j ascending. */
static double product_one(int64_t N, int32_t R, int64_t Bg, uint32_t seed, const uint16_t* S,
                          const void* X, int x_dtype, int64_t t, int64_t i)
{
    double acc = 0.0;
    for (int64_t j = 0; j < N; ++j) {
        uint32_t q = oracle_bucket((uint32_t)((i % R) * N + j), seed, (uint32_t)Bg);
        double w = oracle_f16_to_f64(S[(i / R) * Bg + q]);
        double x = (double)load_as_f32(X, x_dtype, t * N + j);
        acc += x * w;
    }
    return acc;
}

/* Full product Y[batch][M] = X[batch][N] * W_hat^T, double. */
int oracle_matmul(int64_t M, int64_t N, int32_t R, double bpw, uint32_t seed, const uint16_t* S,
                  const void* X, int x_dtype, int64_t batch, double* Y, int nthreads)
{
    int64_t nb, Bg;
    if (oracle_layout(M, N, R, bpw, &nb, &Bg) != OR_OK)
        return OR_EINVAL;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t i = 0; i < M; ++i)
        for (int64_t t = 0; t < batch; ++t)
            Y[t * M + i] = product_one(N, R, Bg, seed, S, X, x_dtype, t, i);
    return OR_OK;
}

/* Selected outputs only: y[s] = Y[t_idx[s]][i_idx[s]]. */
int oracle_matmul_sampled(int64_t M, int64_t N, int32_t R, double bpw, uint32_t seed,
                          const uint16_t* S, const void* X, int x_dtype, int64_t batch,
                          int64_t n, const int64_t* t_idx, const int64_t* i_idx, double* y,
                          int nthreads)
{
    int64_t nb, Bg;
    if (oracle_layout(M, N, R, bpw, &nb, &Bg) != OR_OK)
        return OR_EINVAL;
    for (int64_t s = 0; s < n; ++s)
        if (t_idx[s] < 0 || t_idx[s] >= batch || i_idx[s] < 0 || i_idx[s] >= M)
            return OR_EINVAL;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16)
#endif
    for (int64_t s = 0; s < n; ++s)
        y[s] = product_one(N, R, Bg, seed, S, X, x_dtype, t_idx[s], i_idx[s]);
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Multi-row AbsMaxMin sketch, "Metodología §1" (multi-row design):   */
/* several independent hash functions, each with its own sketch row,  */
/* so that similar weights are more likely to share a bucket in some  */
/* row; decompression takes the Max over the rows.  Readings:         */
/*   - row rho (0 <= rho < rows) hashes with seed + rho (one hash     */
/*     family, rows seeds);                                           */
/*   - the block's Bg buckets (the same bit budget) are split into    */
/*     rows contiguous segments of Bgr = Bg / rows; row rho's bucket  */
/*     of position l is rho * Bgr + k_rho(l), k_rho taken over Bgr    */
/*     buckets with seed + rho;                                       */
/*   - each row keeps, per bucket, the same winner as the single-row  */
/*     sketch over its own segment (AbsMin, or AbsMax for the plain-  */
/*     language rule);                                                */
/*   - decompression: among the rows' buckets of a position, the one */
/*     of largest magnitude (AbsMin rule; of smallest magnitude for   */
/*     AbsMax), the first row among equal magnitudes.                 */
/* rows == 1 is the single-row sketch.                                */
/* ------------------------------------------------------------------ */
static int rows_layout(int64_t M, int64_t N, int32_t R, double bpw, int32_t rows, int64_t* nb, int64_t* Bg)
{
    if (rows < 1 || oracle_layout(M, N, R, bpw, nb, Bg) != OR_OK || *Bg % rows != 0)
        return OR_EINVAL;
    return OR_OK;
}

/* Bucket of position l in row rho, as an index into the block's Bg. */
static uint32_t row_bucket(uint32_t l, uint32_t seed, int32_t rho, uint32_t Bgr)
{
    return (uint32_t)rho * Bgr + oracle_bucket(l, seed + (uint32_t)rho, Bgr);
}

int oracle_encode_rows(int64_t M, int64_t N, int32_t R, double bpw, uint32_t seed, int rule, int32_t rows,
                       int w_dtype, const void* W, const float* imp, uint16_t* S, int nthreads)
{
    int64_t nb, Bg;
    if (rows_layout(M, N, R, bpw, rows, &nb, &Bg) != OR_OK)
        return OR_EINVAL;
    if (rule != OR_ABSMIN && rule != OR_ABSMAX)
        return OR_EINVAL;
    if (w_dtype != OR_F32 && w_dtype != OR_BF16 && w_dtype != OR_F16)
        return OR_EINVAL;
    if (imp)
        for (int64_t j = 0; j < N; ++j)
            if (!isfinite(imp[j]) || imp[j] < 0.0f)
                return OR_EINVAL;
    for (int64_t e = 0; e < M * N; ++e) {
        float w = load_as_f32(W, w_dtype, e);
        if (!isfinite(w) || fabsf(w) >= 65520.0f)
            return OR_ERANGE;
    }
    const uint32_t Bgr = (uint32_t)(Bg / rows);
    const int64_t L = (int64_t)R * N;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        int64_t* best_l = (int64_t*)malloc(sizeof(int64_t) * (size_t)Bg);
        float* best_key = (float*)malloc(sizeof(float) * (size_t)Bg);
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t b = 0; b < nb; ++b) {
            for (int64_t q = 0; q < Bg; ++q)
                best_l[q] = -1;
            /* each row scans the block in l order into its own segment */
            for (int32_t rho = 0; rho < rows; ++rho)
                for (int64_t l = 0; l < L; ++l) {
                    int64_t r = l / N, j = l % N;
                    float w = load_as_f32(W, w_dtype, (b * R + r) * N + j);
                    float key = fabsf(w) * (imp ? imp[j] : 1.0f);
                    uint32_t q = row_bucket((uint32_t)l, seed, rho, Bgr);
                    int better;
                    if (best_l[q] < 0)
                        better = 1;
                    else if (rule == OR_ABSMIN)
                        better = key < best_key[q];
                    else
                        better = key > best_key[q];
                    if (better) {
                        best_l[q] = l;
                        best_key[q] = key;
                    }
                }
            for (int64_t q = 0; q < Bg; ++q) {
                uint16_t v = 0;
                if (best_l[q] >= 0) {
                    int64_t l = best_l[q];
                    v = oracle_f32_to_f16(load_as_f32(W, w_dtype, (b * R + l / N) * N + l % N));
                }
                S[b * Bg + q] = v;
            }
        }
        free(best_l);
        free(best_key);
    }
    return OR_OK;
}

/* W_hat[i][j] of a multi-row sketch, exactly as a double. */
static double decode_rows_one(int64_t N, int32_t R, int64_t Bg, uint32_t seed, int rule, int32_t rows,
                              const uint16_t* S, int64_t i, int64_t j)
{
    const uint32_t Bgr = (uint32_t)(Bg / rows);
    const uint32_t l = (uint32_t)((i % R) * N + j);
    double best = oracle_f16_to_f64(S[(i / R) * Bg + row_bucket(l, seed, 0, Bgr)]);
    for (int32_t rho = 1; rho < rows; ++rho) {
        double v = oracle_f16_to_f64(S[(i / R) * Bg + row_bucket(l, seed, rho, Bgr)]);
        int better = rule == OR_ABSMIN ? fabs(v) > fabs(best) : fabs(v) < fabs(best);
        if (better)
            best = v;
    }
    return best;
}

int oracle_decode_rows(int64_t M, int64_t N, int32_t R, double bpw, uint32_t seed, int rule, int32_t rows,
                       const uint16_t* S, double* What)
{
    int64_t nb, Bg;
    if (rows_layout(M, N, R, bpw, rows, &nb, &Bg) != OR_OK || (rule != OR_ABSMIN && rule != OR_ABSMAX))
        return OR_EINVAL;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            What[i * N + j] = decode_rows_one(N, R, Bg, seed, rule, rows, S, i, j);
    return OR_OK;
}

/* Y[t][i] = sum_j X[t][j] * W_hat[i][j] for a multi-row sketch, double, j ascending. */
static double product_rows_one(int64_t N, int32_t R, int64_t Bg, uint32_t seed, int rule, int32_t rows,
                               const uint16_t* S, const void* X, int x_dtype, int64_t t, int64_t i)
{
    double acc = 0.0;
    for (int64_t j = 0; j < N; ++j)
        acc += (double)load_as_f32(X, x_dtype, t * N + j) * decode_rows_one(N, R, Bg, seed, rule, rows, S, i, j);
    return acc;
}

int oracle_matmul_rows(int64_t M, int64_t N, int32_t R, double bpw, uint32_t seed, int rule, int32_t rows,
                       const uint16_t* S, const void* X, int x_dtype, int64_t batch, double* Y, int nthreads)
{
    int64_t nb, Bg;
    if (rows_layout(M, N, R, bpw, rows, &nb, &Bg) != OR_OK || (rule != OR_ABSMIN && rule != OR_ABSMAX))
        return OR_EINVAL;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t i = 0; i < M; ++i)
        for (int64_t t = 0; t < batch; ++t)
            Y[t * M + i] = product_rows_one(N, R, Bg, seed, rule, rows, S, X, x_dtype, t, i);
    return OR_OK;
}

int oracle_matmul_sampled_rows(int64_t M, int64_t N, int32_t R, double bpw, uint32_t seed, int rule,
                               int32_t rows, const uint16_t* S, const void* X, int x_dtype, int64_t batch,
                               int64_t n, const int64_t* t_idx, const int64_t* i_idx, double* y, int nthreads)
{
    int64_t nb, Bg;
    if (rows_layout(M, N, R, bpw, rows, &nb, &Bg) != OR_OK || (rule != OR_ABSMIN && rule != OR_ABSMAX))
        return OR_EINVAL;
    for (int64_t s = 0; s < n; ++s)
        if (t_idx[s] < 0 || t_idx[s] >= batch || i_idx[s] < 0 || i_idx[s] >= M)
            return OR_EINVAL;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16)
#endif
    for (int64_t s = 0; s < n; ++s)
        y[s] = product_rows_one(N, R, Bg, seed, rule, rows, S, X, x_dtype, t_idx[s], i_idx[s]);
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* Importance-aware space allocation, "Metodología §2": rows or       */
/* layers of higher importance get more sketch space (more buckets),  */
/* the metric being the expected squared activation E[a^2].           */
/* Readings (the pages give no formulas):                             */
/*   - the unit is the row block; its importance is                   */
/*       s_b = sum over its rows i of E[y_i^2],                       */
/*       E[y_i^2] = sum_j W[i][j]^2 * E[x_j^2]                        */
/*     (independent zero-mean inputs), i.e. E[a^2] of the outputs     */
/*     computed from E[a^2] of the inputs;                            */
/*   - the bit budget is kept: the block bucket counts Bg_b add up to */
/*     the uniform sketch's nb * Bg; every block gets a floor of lo   */
/*     buckets and the rest, E = total - nb * lo, is shared in        */
/*     proportion to s_b by largest remainder (Hamilton): quota       */
/*     q_b = (E * s_b) / sum(s) in double, floor(q_b) each, the       */
/*     leftover units to the largest fractional parts, ties to the    */
/*     lower block (all s zero: equal shares);                        */
/*   - block b hashes with the same function reduced to its own count */
/*       k_b(l) = (u64(hash32((u32)(l * 0x9E3779B1) ^ seed)) * Bg_b) >> 32 */
/*     and its table is the Bg_b buckets at offset sum_{c<b} Bg_c;    */
/*   - everything else (key, tie-break, empty buckets, rounding,      */
/*     rejections) is the single-row sketch's.                        */
/* ------------------------------------------------------------------ */

/* s[b] for every row block b of an M x N weight (double, r then j ascending). */
int oracle_block_importance(int64_t M, int64_t N, int32_t R, int w_dtype, const void* W, const float* a2,
                            double* s)
{
    if (R < 1 || N < 1 || M < 0 || M % R != 0)
        return OR_EINVAL;
    if (w_dtype != OR_F32 && w_dtype != OR_BF16 && w_dtype != OR_F16)
        return OR_EINVAL;
    for (int64_t j = 0; j < N; ++j)
        if (!isfinite(a2[j]) || a2[j] < 0.0f)
            return OR_EINVAL;
    for (int64_t b = 0; b < M / R; ++b) {
        double acc = 0.0;
        for (int64_t r = 0; r < R; ++r)
            for (int64_t j = 0; j < N; ++j) {
                double w = (double)load_as_f32(W, w_dtype, (b * R + r) * N + j);
                acc += w * w * (double)a2[j];
            }
        s[b] = acc;
    }
    return OR_OK;
}

/* Bucket counts bg[nb] from the importances s[nb] (see above). */
int oracle_alloc_plan(int64_t nb, int64_t total, int64_t lo, const double* s, int64_t* bg)
{
    if (nb < 1 || lo < 1 || total < nb * lo)
        return OR_EINVAL;
    double sum = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
        if (!isfinite(s[b]) || s[b] < 0.0)
            return OR_EINVAL;
        sum += s[b];
    }
    if (!isfinite(sum))
        return OR_EINVAL;
    const int64_t E = total - nb * lo;
    double* rem = (double*)malloc(sizeof(double) * (size_t)nb);
    char* used = (char*)calloc((size_t)nb, 1);
    if (!rem || !used) {
        free(rem);
        free(used);
        return OR_EINVAL;
    }
    int64_t left = E;
    for (int64_t b = 0; b < nb; ++b) {
        double q = sum > 0.0 ? ((double)E * s[b]) / sum : (double)E / (double)nb;
        double f = floor(q);
        bg[b] = (int64_t)f;
        rem[b] = q - f;
        left -= bg[b];
    }
    /* leftover units: largest remainder first, ties to the lower block */
    while (left > 0) {
        int64_t pick = -1;
        for (int64_t b = 0; b < nb; ++b)
            if (!used[b] && (pick < 0 || rem[b] > rem[pick]))
                pick = b;
        used[pick] = 1;
        bg[pick] += 1;
        --left;
    }
    /* rounding of the quotas can overshoot by a unit: smallest remainder
     * gives one back first, ties to the higher block */
    while (left < 0) {
        int64_t pick = -1;
        for (int64_t b = nb - 1; b >= 0; --b)
            if (!used[b] && bg[b] > 0 && (pick < 0 || rem[b] < rem[pick]))
                pick = b;
        used[pick] = 1;
        bg[pick] -= 1;
        ++left;
    }
    for (int64_t b = 0; b < nb; ++b)
        bg[b] += lo;
    free(rem);
    free(used);
    return OR_OK;
}

static int alloc_check(int64_t M, int64_t N, int32_t R, const int64_t* bg)
{
    if (R < 1 || N < 1 || M < 0 || M % R != 0 || (int64_t)R * N > 4294967296LL)
        return OR_EINVAL;
    for (int64_t b = 0; b < M / R; ++b)
        if (bg[b] < 1 || bg[b] > 4294967295LL)
            return OR_EINVAL;
    return OR_OK;
}

int oracle_encode_alloc(int64_t M, int64_t N, int32_t R, uint32_t seed, int rule, int w_dtype, const void* W,
                        const float* imp, const int64_t* bg, uint16_t* S, int nthreads)
{
    if (alloc_check(M, N, R, bg) != OR_OK || (rule != OR_ABSMIN && rule != OR_ABSMAX))
        return OR_EINVAL;
    if (w_dtype != OR_F32 && w_dtype != OR_BF16 && w_dtype != OR_F16)
        return OR_EINVAL;
    if (imp)
        for (int64_t j = 0; j < N; ++j)
            if (!isfinite(imp[j]) || imp[j] < 0.0f)
                return OR_EINVAL;
    for (int64_t e = 0; e < M * N; ++e) {
        float w = load_as_f32(W, w_dtype, e);
        if (!isfinite(w) || fabsf(w) >= 65520.0f)
            return OR_ERANGE;
    }
    const int64_t nb = M / R, L = (int64_t)R * N;
    int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nb + 1));
    if (!off)
        return OR_EINVAL;
    off[0] = 0;
    for (int64_t b = 0; b < nb; ++b)
        off[b + 1] = off[b] + bg[b];
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 4)
#endif
    for (int64_t b = 0; b < nb; ++b) {
        const int64_t Bg = bg[b];
        int64_t* best_l = (int64_t*)malloc(sizeof(int64_t) * (size_t)Bg);
        float* best_key = (float*)malloc(sizeof(float) * (size_t)Bg);
        for (int64_t q = 0; q < Bg; ++q)
            best_l[q] = -1;
        for (int64_t l = 0; l < L; ++l) {
            int64_t r = l / N, j = l % N;
            float w = load_as_f32(W, w_dtype, (b * R + r) * N + j);
            float key = fabsf(w) * (imp ? imp[j] : 1.0f);
            uint32_t q = oracle_bucket((uint32_t)l, seed, (uint32_t)Bg);
            int better;
            if (best_l[q] < 0)
                better = 1;
            else if (rule == OR_ABSMIN)
                better = key < best_key[q];
            else
                better = key > best_key[q];
            if (better) {
                best_l[q] = l;
                best_key[q] = key;
            }
        }
        for (int64_t q = 0; q < Bg; ++q) {
            uint16_t v = 0;
            if (best_l[q] >= 0) {
                int64_t l = best_l[q];
                v = oracle_f32_to_f16(load_as_f32(W, w_dtype, (b * R + l / N) * N + l % N));
            }
            S[off[b] + q] = v;
        }
        free(best_l);
        free(best_key);
    }
    free(off);
    return OR_OK;
}

/* W_hat[i][j] of an allocated sketch: S[off_b + k_b(l)], b = i / R. */
static double decode_alloc_one(int64_t N, int32_t R, uint32_t seed, const int64_t* bg, const int64_t* off,
                               const uint16_t* S, int64_t i, int64_t j)
{
    const int64_t b = i / R;
    const uint32_t q = oracle_bucket((uint32_t)((i % R) * N + j), seed, (uint32_t)bg[b]);
    return oracle_f16_to_f64(S[off[b] + q]);
}

static int64_t* alloc_offsets(int64_t nb, const int64_t* bg)
{
    int64_t* off = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nb + 1));
    if (!off)
        return NULL;
    off[0] = 0;
    for (int64_t b = 0; b < nb; ++b)
        off[b + 1] = off[b] + bg[b];
    return off;
}

int oracle_decode_alloc(int64_t M, int64_t N, int32_t R, uint32_t seed, const int64_t* bg, const uint16_t* S,
                        double* What)
{
    if (alloc_check(M, N, R, bg) != OR_OK)
        return OR_EINVAL;
    int64_t* off = alloc_offsets(M / R, bg);
    if (!off)
        return OR_EINVAL;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            What[i * N + j] = decode_alloc_one(N, R, seed, bg, off, S, i, j);
    free(off);
    return OR_OK;
}

static double product_alloc_one(int64_t N, int32_t R, uint32_t seed, const int64_t* bg, const int64_t* off,
                                const uint16_t* S, const void* X, int x_dtype, int64_t t, int64_t i)
{
    double acc = 0.0;
    for (int64_t j = 0; j < N; ++j)
        acc += (double)load_as_f32(X, x_dtype, t * N + j) * decode_alloc_one(N, R, seed, bg, off, S, i, j);
    return acc;
}

int oracle_matmul_alloc(int64_t M, int64_t N, int32_t R, uint32_t seed, const int64_t* bg, const uint16_t* S,
                        const void* X, int x_dtype, int64_t batch, double* Y, int nthreads)
{
    if (alloc_check(M, N, R, bg) != OR_OK)
        return OR_EINVAL;
    int64_t* off = alloc_offsets(M / R, bg);
    if (!off)
        return OR_EINVAL;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t i = 0; i < M; ++i)
        for (int64_t t = 0; t < batch; ++t)
            Y[t * M + i] = product_alloc_one(N, R, seed, bg, off, S, X, x_dtype, t, i);
    free(off);
    return OR_OK;
}

int oracle_matmul_sampled_alloc(int64_t M, int64_t N, int32_t R, uint32_t seed, const int64_t* bg,
                                const uint16_t* S, const void* X, int x_dtype, int64_t batch, int64_t n,
                                const int64_t* t_idx, const int64_t* i_idx, double* y, int nthreads)
{
    if (alloc_check(M, N, R, bg) != OR_OK)
        return OR_EINVAL;
    for (int64_t s = 0; s < n; ++s)
        if (t_idx[s] < 0 || t_idx[s] >= batch || i_idx[s] < 0 || i_idx[s] >= M)
            return OR_EINVAL;
    int64_t* off = alloc_offsets(M / R, bg);
    if (!off)
        return OR_EINVAL;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16)
#endif
    for (int64_t s = 0; s < n; ++s)
        y[s] = product_alloc_one(N, R, seed, bg, off, S, X, x_dtype, t_idx[s], i_idx[s]);
    free(off);
    return OR_OK;
}

/* ------------------------------------------------------------------ */
/* 4-bit buckets, "Resultados" (0.5 bits per weight combined with     */
/* 4-bit quantization).  Readings (the pages give no formulas):       */
/*   - a bucket holds a signed 4-bit code q in [-7, 7]; at bpw bits   */
/*     per weight a block has Bg4 = R*N*bpw/4 buckets (8 weights per  */
/*     bucket at 0.5 bpw), Bg4 even (two codes per byte);             */
/*   - the winner of a bucket is chosen exactly as in the binary16    */
/*     sketch with Bg4 buckets (AbsMin/AbsMax on |w| * imp[j], ties   */
/*     to the smallest l), before any quantization;                   */
/*   - one binary16 scale per block: s = f16_rne(amax / 7.0f), amax   */
/*     the largest |w| among the block's winners (float32);           */
/*   - q = clamp(rint(w / s), -7, 7) with w the winner's float32      */
/*     value, the division correctly rounded and rint ties-to-even;   */
/*     s == 0 (all winners zero, or amax / 7 below binary16's range)  */
/*     gives q = 0; an empty bucket holds 0;                          */
/*   - W_hat[i][j] = q * s (exact in double);                         */
/*   - storage: block b's codes at bytes [b*Bg4/2, (b+1)*Bg4/2),      */
/*     bucket k in the low nibble of byte k/2 when k is even, the     */
/*     high nibble when odd, two's complement; the scales are a       */
/*     separate binary16 array [nb].                                  */
/* ------------------------------------------------------------------ */
int oracle_layout_q4(int64_t M, int64_t N, int32_t R, double bpw, int64_t* nb, int64_t* Bg4)
{
    if (M < 0 || N <= 0 || R <= 0 || !(bpw > 0.0) || !isfinite(bpw) || M % R != 0)
        return OR_EINVAL;
    double bg = (double)R * (double)N * bpw / 4.0;
    double bgi = floor(bg);
    if (bg != bgi || bgi < 2.0 || bgi > 4294967294.0 || fmod(bgi, 2.0) != 0.0)
        return OR_EINVAL;
    if ((double)R * (double)N > 4294967295.0)
        return OR_EINVAL;
    *nb = M / R;
    *Bg4 = (int64_t)bgi;
    return OR_OK;
}

static int q4_get(const uint8_t* T, int64_t b, int64_t Bg4, int64_t k)
{
    uint8_t byte = T[b * (Bg4 / 2) + k / 2];
    int v = (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
    return v >= 8 ? v - 16 : v;
}

int oracle_encode_q4(int64_t M, int64_t N, int32_t R, double bpw, uint32_t seed, int rule, int w_dtype,
                     const void* W, const float* imp, uint8_t* T, uint16_t* scales, int nthreads)
{
    int64_t nb, Bg4;
    if (oracle_layout_q4(M, N, R, bpw, &nb, &Bg4) != OR_OK || (rule != OR_ABSMIN && rule != OR_ABSMAX))
        return OR_EINVAL;
    if (w_dtype != OR_F32 && w_dtype != OR_BF16 && w_dtype != OR_F16)
        return OR_EINVAL;
    if (imp)
        for (int64_t j = 0; j < N; ++j)
            if (!isfinite(imp[j]) || imp[j] < 0.0f)
                return OR_EINVAL;
    for (int64_t e = 0; e < M * N; ++e) {
        float w = load_as_f32(W, w_dtype, e);
        if (!isfinite(w) || fabsf(w) >= 65520.0f)
            return OR_ERANGE;
    }
    const int64_t L = (int64_t)R * N;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        int64_t* best_l = (int64_t*)malloc(sizeof(int64_t) * (size_t)Bg4);
        float* best_key = (float*)malloc(sizeof(float) * (size_t)Bg4);
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t b = 0; b < nb; ++b) {
            for (int64_t q = 0; q < Bg4; ++q)
                best_l[q] = -1;
            for (int64_t l = 0; l < L; ++l) {
                int64_t r = l / N, j = l % N;
                float w = load_as_f32(W, w_dtype, (b * R + r) * N + j);
                float key = fabsf(w) * (imp ? imp[j] : 1.0f);
                uint32_t q = oracle_bucket((uint32_t)l, seed, (uint32_t)Bg4);
                int better;
                if (best_l[q] < 0)
                    better = 1;
                else if (rule == OR_ABSMIN)
                    better = key < best_key[q];
                else
                    better = key > best_key[q];
                if (better) {
                    best_l[q] = l;
                    best_key[q] = key;
                }
            }
            /* block scale from the winners */
            float amax = 0.0f;
            for (int64_t q = 0; q < Bg4; ++q)
                if (best_l[q] >= 0) {
                    int64_t l = best_l[q];
                    float w = fabsf(load_as_f32(W, w_dtype, (b * R + l / N) * N + l % N));
                    if (w > amax)
                        amax = w;
                }
            uint16_t s16 = oracle_f32_to_f16(amax / 7.0f);
            float s = (float)oracle_f16_to_f64(s16);
            scales[b] = s16;
            uint8_t* Tb = T + b * (Bg4 / 2);
            for (int64_t k = 0; k < Bg4 / 2; ++k)
                Tb[k] = 0;
            for (int64_t q = 0; q < Bg4; ++q) {
                int code = 0;
                if (best_l[q] >= 0 && s > 0.0f) {
                    int64_t l = best_l[q];
                    float w = load_as_f32(W, w_dtype, (b * R + l / N) * N + l % N);
                    float v = rintf(w / s);
                    if (v > 7.0f)
                        v = 7.0f;
                    if (v < -7.0f)
                        v = -7.0f;
                    code = (int)v;
                }
                uint8_t nib = (uint8_t)(code & 0x0F);
                Tb[q / 2] |= (q % 2 == 0) ? nib : (uint8_t)(nib << 4);
            }
        }
        free(best_l);
        free(best_key);
    }
    return OR_OK;
}

static double decode_q4_one(int64_t N, int32_t R, int64_t Bg4, uint32_t seed, const uint8_t* T,
                            const uint16_t* scales, int64_t i, int64_t j)
{
    const int64_t b = i / R;
    const uint32_t k = oracle_bucket((uint32_t)((i % R) * N + j), seed, (uint32_t)Bg4);
    return (double)q4_get(T, b, Bg4, k) * oracle_f16_to_f64(scales[b]);
}

int oracle_decode_q4(int64_t M, int64_t N, int32_t R, double bpw, uint32_t seed, const uint8_t* T,
                     const uint16_t* scales, double* What)
{
    int64_t nb, Bg4;
    if (oracle_layout_q4(M, N, R, bpw, &nb, &Bg4) != OR_OK)
        return OR_EINVAL;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            What[i * N + j] = decode_q4_one(N, R, Bg4, seed, T, scales, i, j);
    return OR_OK;
}

static double product_q4_one(int64_t N, int32_t R, int64_t Bg4, uint32_t seed, const uint8_t* T,
                             const uint16_t* scales, const void* X, int x_dtype, int64_t t, int64_t i)
{
    double acc = 0.0;
    for (int64_t j = 0; j < N; ++j)
        acc += (double)load_as_f32(X, x_dtype, t * N + j) * decode_q4_one(N, R, Bg4, seed, T, scales, i, j);
    return acc;
}

int oracle_matmul_q4(int64_t M, int64_t N, int32_t R, double bpw, uint32_t seed, const uint8_t* T,
                     const uint16_t* scales, const void* X, int x_dtype, int64_t batch, double* Y, int nthreads)
{
    int64_t nb, Bg4;
    if (oracle_layout_q4(M, N, R, bpw, &nb, &Bg4) != OR_OK)
        return OR_EINVAL;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (int64_t i = 0; i < M; ++i)
        for (int64_t t = 0; t < batch; ++t)
            Y[t * M + i] = product_q4_one(N, R, Bg4, seed, T, scales, X, x_dtype, t, i);
    return OR_OK;
}

int oracle_matmul_sampled_q4(int64_t M, int64_t N, int32_t R, double bpw, uint32_t seed, const uint8_t* T,
                             const uint16_t* scales, const void* X, int x_dtype, int64_t batch, int64_t n,
                             const int64_t* t_idx, const int64_t* i_idx, double* y, int nthreads)
{
    int64_t nb, Bg4;
    if (oracle_layout_q4(M, N, R, bpw, &nb, &Bg4) != OR_OK)
        return OR_EINVAL;
    for (int64_t s = 0; s < n; ++s)
        if (t_idx[s] < 0 || t_idx[s] >= batch || i_idx[s] < 0 || i_idx[s] >= M)
            return OR_EINVAL;
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16)
#endif
    for (int64_t s = 0; s < n; ++s)
        y[s] = product_q4_one(N, R, Bg4, seed, T, scales, X, x_dtype, t_idx[s], i_idx[s]);
    return OR_OK;
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
