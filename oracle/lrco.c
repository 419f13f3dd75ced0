/*
 * lrco.c -- fp64 CPU oracle kernels.  TEST INFRASTRUCTURE ONLY: nothing in the GPU
 * library links, includes or calls this file, and this file uses nothing from it.
 *
 * Swift-SVD page ("Swift-SVD: Theoretical Optimality Meets Practical Efficiency in
 * Low-Rank LLM Compression"), section 2-ga: the right singular vectors and squared
 * singular values of Y = XW come from one symmetric eigendecomposition of Y^T Y.
 * The oracle solves that eigenproblem with a textbook method that is unrelated to the
 * GPU's: the cyclic two-sided Jacobi method (Golub & Van Loan, "Matrix Computations",
 * the symmetric Schur 2x2 step plus cyclic sweeps, with the round-robin parallel
 * ordering of disjoint pairs).
 *
 * The LASER page ("LASER: Loss-Aware Singular-value Decomposition and Rank
 * Allocation", method 1, "Transformation") whitens W with Cholesky factors of the
 * activation and gradient covariances; lrco_cholesky is the textbook column-by-column
 * (Cholesky-Crout) factorisation used by the oracle for that variant.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC lrco.c -o liblrco.so -lm
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Round-robin ("circle") pairing of m players, m even, round r in [0, m-1):
 * pair 0 = (r, m-1); pair i > 0 = ((r+i) mod (m-1), (r-i) mod (m-1)).
 * Over the m-1 rounds every unordered pair appears exactly once. */
static void rr_pairs(int m, int r, int *P, int *Q) {
    P[0] = r;
    Q[0] = m - 1;
    for (int i = 1; i < m / 2; ++i) {
        P[i] = (r + i) % (m - 1);
        Q[i] = (r - i + (m - 1)) % (m - 1);
    }
}

typedef struct {
    double val;
    int idx;
} lrco_pair_t;

static int cmp_desc_stable(const void *a, const void *b) {
    const lrco_pair_t *x = (const lrco_pair_t *)a, *y = (const lrco_pair_t *)b;
    if (x->val > y->val) return -1;
    if (x->val < y->val) return 1;
    return (x->idx > y->idx) - (x->idx < y->idx);
}

/*
 * Eigendecomposition of a symmetric n x n matrix A (row-major, both triangles
 * present; destroyed).  On return lam[0..n) holds the eigenvalues in descending order
 * (stable by original diagonal position) and V (n x n row-major) holds the matching
 * eigenvectors as columns, each scaled so that its entry of largest magnitude is
 * positive (first such index on ties).
 *
 * A pair (p, q) is rotated when a_pq != 0 and |a_pq| > 2^-52 sqrt(|a_pp a_qq|)
 * (the relative criterion of Demmel and Veselic).  The angle: theta = (a_qq - a_pp) /
 * (2 a_pq), t = sign(theta) / (|theta| + sqrt(theta^2 + 1)) with sign(0) = +1,
 * c = 1/sqrt(t^2 + 1), s = t c; then A <- J^T A J, V <- V J with J = [[c, s], [-s, c]]
 * on rows/columns (p, q), and a_pq = a_qp = 0.  Iteration stops after a sweep without
 * a rotation.
 *
 * Returns 0 on convergence, 1 if max_sweeps sweeps did not converge, -1 on bad input.
 */
int lrco_jacobi_eigh(int n, double *A, double *lam, double *V, int max_sweeps, int *sweeps_done) {
    if (n <= 0 || !A || !lam || !V) return -1;
    for (int64_t i = 0; i < (int64_t)n * n; ++i) V[i] = 0.0;
    for (int i = 0; i < n; ++i) V[(int64_t)i * n + i] = 1.0;
    if (sweeps_done) *sweeps_done = 0;
    int status = 1;
    if (n == 1) {
        status = 0;
    } else {
        const int m = n + (n & 1);
        const int np = m / 2;
        int *P = (int *)malloc(sizeof(int) * np), *Q = (int *)malloc(sizeof(int) * np);
        int *ap = (int *)malloc(sizeof(int) * np), *aq = (int *)malloc(sizeof(int) * np);
        double *cc = (double *)malloc(sizeof(double) * np), *ss = (double *)malloc(sizeof(double) * np);
        for (int sweep = 0; sweep < max_sweeps; ++sweep) {
            int64_t rotations = 0;
            for (int r = 0; r < m - 1; ++r) {
                rr_pairs(m, r, P, Q);
                int na = 0;
                for (int i = 0; i < np; ++i) {
                    int p = P[i] < Q[i] ? P[i] : Q[i];
                    int q = P[i] < Q[i] ? Q[i] : P[i];
                    if (q >= n) continue; /* dummy player when n is odd */
                    double apq = A[(int64_t)p * n + q];
                    double app = A[(int64_t)p * n + p];
                    double aqq = A[(int64_t)q * n + q];
                    if (apq == 0.0 || !(fabs(apq) > DBL_EPSILON * sqrt(fabs(app) * fabs(aqq)))) continue;
                    double theta = (aqq - app) / (2.0 * apq);
                    double sg = theta >= 0.0 ? 1.0 : -1.0;
                    double t;
                    if (fabs(theta) > 1e150)
                        t = 0.5 / theta; /* theta^2 would overflow; 1/(2 theta) to working precision */
                    else
                        t = sg / (fabs(theta) + sqrt(theta * theta + 1.0));
                    double c = 1.0 / sqrt(t * t + 1.0);
                    ap[na] = p;
                    aq[na] = q;
                    cc[na] = c;
                    ss[na] = t * c;
                    ++na;
                }
                if (na == 0) continue;
                rotations += na;
                /* rows: A <- J^T A */
#pragma omp parallel for schedule(static)
                for (int i = 0; i < na; ++i) {
                    double *rp = A + (int64_t)ap[i] * n, *rq = A + (int64_t)aq[i] * n;
                    const double c = cc[i], s = ss[i];
                    for (int j = 0; j < n; ++j) {
                        double x = rp[j], y = rq[j];
                        rp[j] = c * x - s * y;
                        rq[j] = s * x + c * y;
                    }
                }
                /* columns: A <- A J, V <- V J */
#pragma omp parallel for schedule(static)
                for (int row = 0; row < n; ++row) {
                    double *ra = A + (int64_t)row * n, *rv = V + (int64_t)row * n;
                    for (int i = 0; i < na; ++i) {
                        const int p = ap[i], q = aq[i];
                        const double c = cc[i], s = ss[i];
                        double x = ra[p], y = ra[q];
                        ra[p] = c * x - s * y;
                        ra[q] = s * x + c * y;
                        x = rv[p];
                        y = rv[q];
                        rv[p] = c * x - s * y;
                        rv[q] = s * x + c * y;
                    }
                }
                for (int i = 0; i < na; ++i) {
                    A[(int64_t)ap[i] * n + aq[i]] = 0.0;
                    A[(int64_t)aq[i] * n + ap[i]] = 0.0;
                }
            }
            if (sweeps_done) *sweeps_done = sweep + 1;
            if (rotations == 0) {
                status = 0;
                break;
            }
        }
        free(P);
        free(Q);
        free(ap);
        free(aq);
        free(cc);
        free(ss);
    }
    /* sort descending (stable) and permute the columns of V */
    lrco_pair_t *pr = (lrco_pair_t *)malloc(sizeof(lrco_pair_t) * n);
    for (int i = 0; i < n; ++i) {
        pr[i].val = A[(int64_t)i * n + i];
        pr[i].idx = i;
    }
    qsort(pr, n, sizeof(lrco_pair_t), cmp_desc_stable);
    double *tmp = (double *)malloc(sizeof(double) * n);
    for (int row = 0; row < n; ++row) {
        double *rv = V + (int64_t)row * n;
        for (int j = 0; j < n; ++j) tmp[j] = rv[pr[j].idx];
        memcpy(rv, tmp, sizeof(double) * n);
    }
    for (int j = 0; j < n; ++j) lam[j] = pr[j].val;
    /* sign: largest |v| entry of each column positive, first index on ties */
    for (int j = 0; j < n; ++j) {
        int best = 0;
        double bv = -1.0;
        for (int i = 0; i < n; ++i) {
            double a = fabs(V[(int64_t)i * n + j]);
            if (a > bv) {
                bv = a;
                best = i;
            }
        }
        if (V[(int64_t)best * n + j] < 0.0)
            for (int i = 0; i < n; ++i) V[(int64_t)i * n + j] = -V[(int64_t)i * n + j];
    }
    free(pr);
    free(tmp);
    return status;
}

/*
 * In-place lower Cholesky factor of a symmetric positive definite n x n matrix
 * (row-major; the lower triangle is read, the strict upper triangle is zeroed on
 * return).  Column by column: L_jj = sqrt(A_jj - sum_{k<j} L_jk^2), then
 * L_ij = (A_ij - sum_{k<j} L_ik L_jk) / L_jj for i > j.
 * Returns 0, or j+1 when pivot j is not positive (or not finite).
 */
int lrco_cholesky(int n, double *A) {
    if (n <= 0 || !A) return -1;
    for (int j = 0; j < n; ++j) {
        double *rj = A + (int64_t)j * n;
        double d = rj[j];
        for (int k = 0; k < j; ++k) d -= rj[k] * rj[k];
        if (!(d > 0.0) || !isfinite(d)) return j + 1;
        const double ljj = sqrt(d);
        rj[j] = ljj;
#pragma omp parallel for schedule(static)
        for (int i = j + 1; i < n; ++i) {
            double *ri = A + (int64_t)i * n;
            double x = ri[j];
            for (int k = 0; k < j; ++k) x -= ri[k] * rj[k];
            ri[j] = x / ljj;
        }
    }
    for (int i = 0; i < n; ++i)
        for (int j = i + 1; j < n; ++j) A[(int64_t)i * n + j] = 0.0;
    return 0;
}
