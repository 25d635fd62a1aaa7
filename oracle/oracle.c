/*
 * Reference oracle for the ring-decomposed all-gather + GEMM and GEMM + reduce-scatter.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  It shares no code, header or constant with the HIP library and
 * includes none of its files.
 *
 * What it computes is the plain definition of the operations on the pages:
 *
 *   - TransformerEngine issue #1583 ("curious about atomic_gemm_overlap_ag"), the C++ listing:
 *     the GEMM dimensions are m = rows of the weight (TN layout), n = rows of the gathered buffer,
 *     n_chunk = n / tp; the gathered buffer holds every rank's chunk contiguously in rank order.
 *     The result is D = G * A^T with G [n, k] and A [m, k], both K-contiguous ("TN").
 *   - nvFuser PR #5742 ("Reference implementation for Linear+Allreduce with overlapping"),
 *     walkthrough: a chunked linear must equal the unchunked linear, and each chunk's partial
 *     products are summed over ranks.
 *   - TransformerEngine PR #2443, sequence diagram: GEMM + reduce-scatter = the local GEMM followed
 *     by a reduction of each output chunk over ranks.
 *
 * Precision: inputs are widened exactly to fp32; every product and every sum is a separate fp32
 * IEEE operation (built with -ffp-contract=off, so no FMA), k in increasing order.  The fp32
 * accumulation is the precision the workloads fix ("fp32 accumulate").
 */
#include <stdint.h>
#include <string.h>
#include <math.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of threads the OpenMP loops below will use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* bf16 -> fp32: a bf16 value is the upper 16 bits of the fp32 value with the same bits, so the
 * widening is exact (IEEE 754 binary32 layout; bfloat16 = truncated binary32). */
void oracle_bf16_to_f32(const uint16_t* src, float* dst, long n) {
    for (long i = 0; i < n; ++i) {
        uint32_t bits = ((uint32_t)src[i]) << 16;
        float f;
        memcpy(&f, &bits, 4);
        dst[i] = f;
    }
}

/* fp32 -> bf16, round to nearest, ties to even.  NaN stays NaN (quiet bit set); +-inf stays inf;
 * values above the largest bf16 round to inf as IEEE rounding prescribes. */
void oracle_f32_to_bf16_rne(const float* src, uint16_t* dst, long n) {
    for (long i = 0; i < n; ++i) {
        uint32_t bits;
        memcpy(&bits, &src[i], 4);
        if ((bits & 0x7f800000u) == 0x7f800000u && (bits & 0x007fffffu) != 0u) {
            dst[i] = (uint16_t)((bits >> 16) | 0x0040u);   /* NaN: keep sign, force quiet */
            continue;
        }
        uint32_t upper = bits >> 16;
        uint32_t lower = bits & 0xffffu;
        /* round half to even on the 16 dropped bits */
        if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
        dst[i] = (uint16_t)upper;
    }
}

/* OCP 8-bit floating point, E4M3 ("FN" variant: no infinities): 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6; the codes S.1111.111 are
 * NaN; every other code is finite, the largest being 448. */
void oracle_e4m3fn_to_f32(const uint8_t* src, float* dst, long n) {
    for (long i = 0; i < n; ++i) {
        uint8_t c = src[i];
        int sign = (c >> 7) & 1;
        int e = (c >> 3) & 0xf;
        int m = c & 0x7;
        float v;
        if (e == 0xf && m == 0x7) {
            v = NAN;
        } else if (e == 0) {
            v = ldexpf((float)m / 8.0f, -6);
        } else {
            v = ldexpf(1.0f + (float)m / 8.0f, e - 7);
        }
        dst[i] = sign ? -v : v;
    }
}

/* fp32 -> OCP E4M3 (no-infinity variant) codes: saturate to +-448 (the largest finite value,
 * code 0x7e), then round to the nearest representable value with ties to even mantissa.  From
 * the format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; normals (1 + m/8) 2^(e-7)
 * for e = 1..15 (e = 15, m = 7 is NaN), subnormals (m/8) 2^-6.  NaN keeps its sign: 0x7f / 0xff.
 * The arithmetic is in double, where every step below is exact; nearbyint rounds ties to even in
 * the default rounding mode. */
void oracle_f32_to_e4m3fn_sat(const float* src, uint8_t* dst, long n) {
    for (long i = 0; i < n; ++i) {
        const float v = src[i];
        const uint8_t sign = signbit(v) ? 0x80 : 0x00;
        if (isnan(v)) {
            dst[i] = sign | 0x7f;
            continue;
        }
        const double a = fabs((double)v);
        if (a >= 448.0) {
            dst[i] = sign | 0x7e;
            continue;
        }
        if (a < ldexp(1.0, -6)) {
            /* subnormal range: multiples of 2^-9; a count of 8 is the smallest normal, code 8 */
            dst[i] = sign | (uint8_t)nearbyint(a / ldexp(1.0, -9));
            continue;
        }
        int e2;
        (void)frexp(a, &e2);               /* a = f * 2^e2, f in [0.5, 1) */
        int E = e2 - 1;                    /* a = (1 + r) * 2^E, r in [0, 1) */
        double q = nearbyint((a / ldexp(1.0, E) - 1.0) * 8.0);
        if (q == 8.0) {
            q = 0.0;
            E += 1;
        }
        int code = ((E + 7) << 3) | (int)q;
        if (code > 0x7e) code = 0x7e;
        dst[i] = sign | (uint8_t)code;
    }
}

/* out[n][m] = sum_k G[n][k] * A[m][k] for n in [0, N), m in [0, M).
 * G is [N, K] with row stride ldg, A is [M, K] with row stride lda, out is [N, M] with row stride
 * ldo (all in elements, row-major).  Plain triple loop, k ascending, separate multiply and add. */
void oracle_gemm_tn_f32(const float* G, long ldg, const float* A, long lda, float* out, long ldo,
                        long N, long M, long K) {
#pragma omp parallel for schedule(dynamic, 1)
    for (long n = 0; n < N; ++n) {
        const float* g = G + n * ldg;
        for (long m = 0; m < M; ++m) {
            const float* a = A + m * lda;
            float acc = 0.0f;
            for (long k = 0; k < K; ++k) {
                float p = g[k] * a[k];
                acc = acc + p;
            }
            out[n * ldo + m] = acc;
        }
    }
}

/* The same sum for a chosen list of rows of G only: out[i][m] = sum_k G[rows[i]][k] * A[m][k].
 * Used where the full product is too large to compute on the host in a test. */
void oracle_gemm_tn_rows_f32(const float* G, long ldg, const float* A, long lda,
                             const long* rows, long nrows, float* out, long ldo, long M, long K) {
#pragma omp parallel for schedule(dynamic, 1)
    for (long i = 0; i < nrows; ++i) {
        const float* g = G + rows[i] * ldg;
        for (long m = 0; m < M; ++m) {
            const float* a = A + m * lda;
            float acc = 0.0f;
            for (long k = 0; k < K; ++k) {
                float p = g[k] * a[k];
                acc = acc + p;
            }
            out[i * ldo + m] = acc;
        }
    }
}
