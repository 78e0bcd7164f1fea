/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the replayed SSM decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the reference the GPU library is checked
 * against.  Only the test suite, the package's smoke check and the CPU-baseline
 * leg of the benchmark may load it.  It shares no code, header, table or helper
 * with the GPU library under hybrid_decode_replay_amd/.
 *
 * Pages cited (the only description of the method available):
 *   [DE] "ReplaySSM beschleunigt das Decoding von Hybridmodellen durch Caching
 *        der Eingaben statt des Zustands" (bytechap.com, German)
 *   [ES] "ReplaySSM acelera la decodificacion de modelos hibridos mediante el
 *        almacenamiento en cache de entradas en lugar del estado" (Spanish
 *        translation of [DE])
 *   [TR] "NVIDIA ve Dao AI Lab, hibrit model cozumlemesini hizlandirmak icin
 *        ReplaySSM'i sundu" (sitech.ge, Turkish)
 *
 * What the oracle computes.  The pages state that the replayed path produces
 * the same outputs as ordinary token-by-token decoding, apart from floating-
 * point rounding ([TR] section "ReplaySSM nasil calisir?").  Ordinary decoding
 * is the step the pages describe as: load the previous state, decay it, add
 * the update, read out the output, store the state ([DE] "Wie es
 * funktioniert", [ES] "Como funciona").  The oracle is therefore exactly that
 * step, in fp64, one token at a time.  The per-token formulas themselves are
 * not printed on the pages; the pages name the two layer families (Mamba-2 and
 * Gated DeltaNet, [DE] "Wichtige Details") and the formulas below are their
 * standard published decode recurrences:
 *   Mamba-2 (Dao & Gu, "Transformers are SSMs", 2024), per head h, group g:
 *       a      = exp(dt * A_h)
 *       S      = a * S + dt * x B^T          (S is P x N)
 *       y      = S C + D_h * x
 *   Gated DeltaNet (Yang, Kautz & Hatamizadeh, "Gated Delta Networks", 2024):
 *       S      = alpha * S (I - beta k k^T) + beta v k^T   (S is d_v x d_k)
 *       o      = scale * S q
 *
 * The quantizers implement the OCP Microscaling (MX) v1.0 element formats
 * FP8 E4M3 and FP4 E2M1 with the E8M0 shared scale, by nearest-value search
 * over the decoded code table (ties to the even code).
 *
 * Parity unpinned: nothing here.  Every function is pinned by the CPU tests
 * (brute-force unrolled sums, closed forms, special cases, library casts).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_ABI 1

int oracle_abi(void) { return ORACLE_ABI; }

/* ------------------------------------------------------------------------ */
/* Mamba-2: one decode token for every (b, h) whose sequence is active.      */
/* Layouts (row-major):                                                      */
/*   S  [B][H][P][N]   state, updated in place                               */
/*   x  [B][H][P]      Bm, Cm [B][G][N]      dt [B][H]                       */
/*   A, D [H]          y [B][H][P] output (written only for active b)        */
/*   active [B]        nonzero = this sequence takes the token (NULL = all)  */
/* ------------------------------------------------------------------------ */
void oracle_mamba2_token(int B, int H, int G, int P, int N,
                         double *S, const double *x, const double *Bm,
                         const double *Cm, const double *dt,
                         const double *A, const double *D,
                         double *y, const unsigned char *active)
{
    const int heads_per_group = H / G;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
            if (active && !active[b]) continue;
            const int g = h / heads_per_group;
            double *s = S + ((size_t)b * H + h) * (size_t)P * N;
            const double *xv = x + ((size_t)b * H + h) * P;
            const double *bv = Bm + ((size_t)b * G + g) * N;
            const double *cv = Cm + ((size_t)b * G + g) * N;
            const double d = dt[(size_t)b * H + h];
            const double a = exp(d * A[h]);              /* decay */
            for (int p = 0; p < P; ++p) {
                double acc = 0.0;
                for (int n = 0; n < N; ++n) {
                    /* decay, then the outer-product update dt * x B^T */
                    s[(size_t)p * N + n] = a * s[(size_t)p * N + n] + d * xv[p] * bv[n];
                    acc += s[(size_t)p * N + n] * cv[n]; /* read-out S C */
                }
                y[((size_t)b * H + h) * P + p] = acc + D[h] * xv[p];
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Gated DeltaNet: one decode token for every active (b, h).                 */
/*   S  [B][H][DV][DK]  state, updated in place                              */
/*   q, k [B][G][DK]    v [B][H][DV]    alpha, beta [B][H]                   */
/*   o  [B][H][DV]      output (active b only)                               */
/* The update S <- alpha S (I - beta k k^T) + beta v k^T is evaluated as     */
/*   u = S k ;  S[i][j] <- alpha (S[i][j] - beta u[i] k[j]) + beta v[i] k[j] */
/* which is the same expression with the product (I - beta k k^T) expanded.  */
/* ------------------------------------------------------------------------ */
void oracle_gdn_token(int B, int H, int G, int DK, int DV,
                      double *S, const double *q, const double *k,
                      const double *v, const double *alpha, const double *beta,
                      double scale, double *o, const unsigned char *active)
{
    const int heads_per_group = H / G;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
            if (active && !active[b]) continue;
            const int g = h / heads_per_group;
            double *s = S + ((size_t)b * H + h) * (size_t)DV * DK;
            const double *qv = q + ((size_t)b * G + g) * DK;
            const double *kv = k + ((size_t)b * G + g) * DK;
            const double *vv = v + ((size_t)b * H + h) * DV;
            const double al = alpha[(size_t)b * H + h];
            const double be = beta[(size_t)b * H + h];
            for (int i = 0; i < DV; ++i) {
                double u = 0.0;                          /* (S k)[i] */
                for (int j = 0; j < DK; ++j) u += s[(size_t)i * DK + j] * kv[j];
                double acc = 0.0;
                for (int j = 0; j < DK; ++j) {
                    double nv = al * (s[(size_t)i * DK + j] - be * u * kv[j]) + be * vv[i] * kv[j];
                    s[(size_t)i * DK + j] = nv;
                    acc += nv * qv[j];                   /* read-out S q */
                }
                o[((size_t)b * H + h) * DV + i] = scale * acc;
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* OCP MX v1.0 element formats.                                              */
/* ------------------------------------------------------------------------ */

/* FP8 E4M3 ("fn" variant: no infinities, S.1111.111 is NaN).  Exponent bias */
/* 7, 3 mantissa bits, subnormals when the exponent field is 0.             */
double oracle_e4m3_decode(int code)
{
    code &= 0xFF;
    const int sign = code >> 7, e = (code >> 3) & 0xF, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m / 8.0, 1 - 7)
                          : ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* Nearest E4M3 code to v; exact ties go to the code with an even mantissa  */
/* (round-half-to-even).  Finite magnitudes beyond the largest finite value  */
/* (448) saturate to it; +-inf saturate too; NaN maps to 0x7F.              */
int oracle_e4m3_encode(double v)
{
    if (isnan(v)) return 0x7F;
    const int sign = signbit(v) ? 0x80 : 0;
    const double a = fabs(v);
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {                  /* all finite magnitudes */
        const double err = fabs(oracle_e4m3_decode(c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return sign | best;
}

/* FP4 E2M1: bias 1, 1 mantissa bit, no inf/NaN.  Magnitudes 0, 0.5, 1,     */
/* 1.5, 2, 3, 4, 6.                                                          */
double oracle_e2m1_decode(int code)
{
    code &= 0xF;
    const int sign = code >> 3, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -mag : mag;
}

int oracle_e2m1_encode(double v)
{
    const int sign = signbit(v) ? 8 : 0;
    const double a = fabs(v);
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c <= 7; ++c) {
        const double err = fabs(oracle_e2m1_decode(c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return sign | best;        /* beyond 6 the nearest value is 6: saturates */
}

/* E8M0 scale: value 2^(code - 127); code 255 is NaN and never produced.    */
double oracle_e8m0_decode(int code)
{
    code &= 0xFF;
    if (code == 255) return NAN;
    return ldexp(1.0, code - 127);
}

/* MX block quantization of n values (n = 32 in use) to E2M1 with one E8M0  */
/* scale.  Shared exponent X = floor(log2(amax)) - 2, where 2 is the largest */
/* E2M1 exponent; X is clamped to [-127, 127]; an all-zero block uses -127. */
/* Elements are v / 2^X rounded to E2M1 (saturating at 6).  codes[] receives */
/* one 4-bit code per element (not packed); returns the E8M0 scale code.    */
int oracle_mxfp4_quantize_block(const double *v, int n, unsigned char *codes)
{
    double amax = 0.0;
    for (int i = 0; i < n; ++i) {
        const double a = fabs(v[i]);
        if (a > amax) amax = a;
    }
    int X;
    if (amax == 0.0) {
        X = -127;
    } else {
        int e2;
        frexp(amax, &e2);          /* amax = f * 2^e2 with f in [0.5, 1) */
        X = (e2 - 1) - 2;          /* floor(log2(amax)) - emax(E2M1)     */
        if (X < -127) X = -127;
        if (X > 127) X = 127;
    }
    for (int i = 0; i < n; ++i) codes[i] = (unsigned char)oracle_e2m1_encode(ldexp(v[i], -X));
    return X + 127;
}

/* The same block quantization with the non-clipping scale rule: X is the   */
/* smallest integer in [-127, 127] with amax <= 6 * 2^X (6 is E2M1's largest */
/* magnitude), so no element saturates; 127 if there is none.  Found by a    */
/* plain upward search; an all-zero block gets -127.                         */
int oracle_mxfp4_quantize_block_ceil(const double *v, int n, unsigned char *codes)
{
    double amax = 0.0;
    for (int i = 0; i < n; ++i) {
        const double a = fabs(v[i]);
        if (a > amax) amax = a;
    }
    int X = -127;
    while (X < 127 && !(amax <= ldexp(6.0, X))) ++X;
    for (int i = 0; i < n; ++i) codes[i] = (unsigned char)oracle_e2m1_encode(ldexp(v[i], -X));
    return X + 127;
}

/* Bulk helpers over arrays (plain loops over the scalar definitions).      */
void oracle_e4m3_encode_array(const double *v, long n, unsigned char *out)
{
#pragma omp parallel for schedule(static)
    for (long i = 0; i < n; ++i) out[i] = (unsigned char)oracle_e4m3_encode(v[i]);
}

void oracle_e4m3_decode_array(const unsigned char *c, long n, double *out)
{
    for (long i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(c[i]);
}

/* v is [nblocks][32]; codes [nblocks][32] (one code per byte); scales      */
/* [nblocks].                                                               */
void oracle_mxfp4_quantize_array(const double *v, long nblocks,
                                 unsigned char *codes, unsigned char *scales)
{
#pragma omp parallel for schedule(static)
    for (long b = 0; b < nblocks; ++b)
        scales[b] = (unsigned char)oracle_mxfp4_quantize_block(v + b * 32, 32, codes + b * 32);
}

void oracle_mxfp4_quantize_array_ceil(const double *v, long nblocks,
                                      unsigned char *codes, unsigned char *scales)
{
#pragma omp parallel for schedule(static)
    for (long b = 0; b < nblocks; ++b)
        scales[b] = (unsigned char)oracle_mxfp4_quantize_block_ceil(v + b * 32, 32, codes + b * 32);
}

void oracle_mxfp4_dequantize_array(const unsigned char *codes, const unsigned char *scales,
                                   long nblocks, double *out)
{
    for (long b = 0; b < nblocks; ++b) {
        const double s = oracle_e8m0_decode(scales[b]);
        for (int i = 0; i < 32; ++i) out[b * 32 + i] = oracle_e2m1_decode(codes[b * 32 + i]) * s;
    }
}

/* Threads the OpenMP loops above use (for reporting the CPU baseline). */
#ifdef _OPENMP
#include <omp.h>
int oracle_threads(void) { return omp_get_max_threads(); }
/* Threads for the loops above from now on (n >= 1); used to time the oracle on
 * one core beside all of them. */
void oracle_set_threads(int n) { omp_set_num_threads(n < 1 ? 1 : n); }
#else
int oracle_threads(void) { return 1; }
void oracle_set_threads(int n) { (void)n; }
#endif
