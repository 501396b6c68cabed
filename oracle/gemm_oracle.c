/*
 * Reference (oracle) GEMM: D_ref = alpha * A*B + beta * C in fp64, plain
 * i-j-k loops. TEST INFRASTRUCTURE: only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg load this library; the product never does.
 *
 * What it follows: the GEMM definition D = alpha*A*B + beta*C with A of shape
 * MxK and B of shape KxN ("CUTLASS, in depth", "The problem CUTLASS solves"),
 * checked the way "CUTLASS and CuTe layouts" checks its GEMM ("Two programs:
 * the algebra, then the GEMM"): the CPU reads the very same 16-bit values the
 * GPU read (already widened exactly to double by the caller) and sums in
 * double, so the only difference it can measure is accumulation order.
 *
 * Every operand is addressed as a rank-2 Shape:Stride layout in elements:
 * A(i,k) = A[i*sa0 + k*sa1], B(k,j) = B[k*sb0 + j*sb1], C(i,j) = C[i*sc0 +
 * j*sc1]. The sum over k is strictly sequential, k = 0 .. K-1, with no
 * reassociation (built without fast-math). T accumulates |a_ik * b_kj| in
 * the same order; it scales the error bound.
 */
#include <stdint.h>
#include <math.h>

static void one_point(const double* A, int64_t sa0, int64_t sa1,
                      const double* B, int64_t sb0, int64_t sb1,
                      int64_t K, int64_t i, int64_t j,
                      double* s_out, double* t_out) {
    double s = 0.0, t = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = A[i * sa0 + k * sa1] * B[k * sb0 + j * sb1];
        s += p;
        t += fabs(p);
    }
    *s_out = s;
    *t_out = t;
}

/* S and T for an explicit list of output coordinates (pairs i,j). */
void oracle_gemm_points(const double* A, int64_t sa0, int64_t sa1,
                        const double* B, int64_t sb0, int64_t sb1,
                        int64_t K, const int64_t* ij, int64_t npts,
                        double* S, double* T) {
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t p = 0; p < npts; ++p)
        one_point(A, sa0, sa1, B, sb0, sb1, K, ij[2 * p], ij[2 * p + 1], &S[p], &T[p]);
}

/* S and T for whole rows: rows[r] for r < nrows, every column j < N.
 * Outputs are row-major nrows x N. */
void oracle_gemm_rows(const double* A, int64_t sa0, int64_t sa1,
                      const double* B, int64_t sb0, int64_t sb1,
                      int64_t N, int64_t K, const int64_t* rows, int64_t nrows,
                      double* S, double* T) {
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r)
        for (int64_t j = 0; j < N; ++j)
            one_point(A, sa0, sa1, B, sb0, sb1, K, rows[r], j, &S[r * N + j], &T[r * N + j]);
}

/* D_ref = alpha * S + beta * c for the same points (c read through C's
 * layout; beta == 0 never reads C). */
void oracle_epilogue_points(const double* S, const double* C, int64_t sc0, int64_t sc1,
                            const int64_t* ij, int64_t npts, double alpha, double beta,
                            double* Dref, double* Cabs) {
    for (int64_t p = 0; p < npts; ++p) {
        double c = 0.0;
        if (beta != 0.0) c = C[ij[2 * p] * sc0 + ij[2 * p + 1] * sc1];
        Dref[p] = alpha * S[p] + beta * c;
        Cabs[p] = fabs(beta * c);
    }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
