/*
 * Sign-bias diagnostic of 2-bit codebooks - TEST INFRASTRUCTURE (the oracle), plain C.
 *
 * The pages (README, bullet "2-bit expert planes - the sign-bias finding"; vLLM-Moet article,
 * section "Sign symmetry, not error size, is what collapses naive 2-bit experts") compare 2-bit
 * codebooks on each expert tensor by two numbers: the relative RMS error of the quantized tensor
 * and its mean bias, and report that the L2-optimal codebook is sign-asymmetric and biased while
 * the sign-symmetric {-4,-1,1,4} reaches the same relative RMS with a far smaller bias.
 *
 * Definition (readings where the pages are silent):
 *  - a codebook is 4 values q0 < q1 < q2 < q3; a tensor [R][C] is cut into blocks of 32 along C,
 *    each with its own power-of-two scale 2^e, e in [-127, 127] (the planes' UE8M0 block-32 scale);
 *  - element x takes the code whose value q_c 2^e is nearest; exactly halfway between two codes
 *    it takes the one of smaller magnitude, and between equal magnitudes (x = 0) the one on the
 *    side of x's sign bit (the zero rule of the 2-bit re-quantizer);
 *  - the exponent minimises the block's squared error over the ten exponents from 7 below to 2
 *    above e_c, the smallest exponent with max(|q0|, |q3|) 2^e_c >= max|x| (e_c = -127 for an
 *    all-zero block), equal errors going to the lower exponent;
 *  - the squared error is accumulated in float64 in element order, each term (x - v)^2 rounded
 *    as a product of two float64 values, then added (no fused operations): float64 is the pages'
 *    precision for load-time quantization ("float64-exact"), and the order makes the decision
 *    reproducible;
 *  - per tensor: sse = sum of block errors, err = sum of (v - x), rel_rms = sqrt(sse / sum x^2),
 *    bias = err / sqrt(N sum x^2) (mean error over rms of x); best symmetric / asymmetric
 *    codebook = least sse among those with q0 = -q3 and q1 = -q2 / among the others, ties to the
 *    lower index.
 * Built with -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>

static int exp_top(double amax, double qmax)
{
    if (amax == 0.0) return -127;
    int e = ilogb(amax) - ilogb(qmax);
    if (ldexp(qmax, e) < amax) e += 1;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* index of the code taken by x at scale 2^e */
static int nearest_code(double x, const double q[4], int e)
{
    int c = 0;
    for (int k = 0; k < 3; ++k) {
        double mid = ldexp(0.5 * (q[k] + q[k + 1]), e);
        int up;
        if (x > mid) up = 1;
        else if (x < mid) up = 0;
        else if (fabs(q[k + 1]) != fabs(q[k])) up = fabs(q[k + 1]) < fabs(q[k]);
        else up = !signbit(x);
        if (up) c = k + 1;
    }
    return c;
}

static double block_sse(const float* x, const double q[4], int e)
{
    double acc = 0.0;
    for (int i = 0; i < 32; ++i) {
        double v = ldexp(q[nearest_code((double)x[i], q, e)], e);
        double d = (double)x[i] - v;
        double t = d * d;
        acc = acc + t;
    }
    return acc;
}

/* chosen exponent of one block; *sse and *err receive its squared error and sum of (v - x) */
int oracle_block_choice(const float* x, const float* qf, double* sse, double* err)
{
    double q[4] = {qf[0], qf[1], qf[2], qf[3]};
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) if (fabs((double)x[i]) > amax) amax = fabs((double)x[i]);
    double qmax = fabs(q[0]) > fabs(q[3]) ? fabs(q[0]) : fabs(q[3]);
    int ec = exp_top(amax, qmax);
    int best_e = 0;
    double best = INFINITY;
    for (int e = ec - 7; e <= ec + 2; ++e) {
        if (e < -127 || e > 127) continue;
        double s = block_sse(x, q, e);
        if (s < best) { best = s; best_e = e; }
    }
    double acc = 0.0;
    for (int i = 0; i < 32; ++i) {
        double v = ldexp(q[nearest_code((double)x[i], q, best_e)], best_e);
        acc = acc + (v - (double)x[i]);
    }
    *sse = best;
    *err = acc;
    return best_e;
}

/*
 * x [n][R][C] fp32, cb [M][4]; stats [n][M][4] = {sse, err, rel_rms, bias},
 * moments [n][2] = {sum x^2, sum x}, best [n][2] = {best symmetric, best asymmetric} (-1: none).
 */
void oracle_codebook_sweep(int n, int R, int C, const float* x, int M, const float* cb,
                           double* stats, double* moments, int* best, int nthreads)
{
    const long N = (long)R * C, nb = N / 32;
#pragma omp parallel for collapse(2) schedule(dynamic) num_threads(nthreads)
    for (int t = 0; t < n; ++t)
        for (int m = 0; m < M; ++m) {
            const float* xt = x + (long)t * N;
            double sse = 0.0, err = 0.0;
            for (long b = 0; b < nb; ++b) {
                double s, e;
                oracle_block_choice(xt + 32 * b, cb + 4 * m, &s, &e);
                sse += s;
                err += e;
            }
            double* o = stats + ((long)t * M + m) * 4;
            o[0] = sse;
            o[1] = err;
        }
    for (int t = 0; t < n; ++t) {
        const float* xt = x + (long)t * N;
        double s2 = 0.0, s1 = 0.0;
        for (long i = 0; i < N; ++i) {
            s2 += (double)xt[i] * (double)xt[i];
            s1 += (double)xt[i];
        }
        moments[2 * t] = s2;
        moments[2 * t + 1] = s1;
        int bs = -1, ba = -1;
        for (int m = 0; m < M; ++m) {
            double* o = stats + ((long)t * M + m) * 4;
            o[2] = s2 > 0.0 ? sqrt(o[0] / s2) : 0.0;
            o[3] = s2 > 0.0 ? o[1] / sqrt((double)N * s2) : 0.0;
            const float* q = cb + 4 * m;
            int sym = q[0] == -q[3] && q[1] == -q[2];
            int* slot = sym ? &bs : &ba;
            if (*slot < 0 || o[0] < stats[((long)t * M + *slot) * 4]) *slot = m;
        }
        best[2 * t] = bs;
        best[2 * t + 1] = ba;
    }
}
