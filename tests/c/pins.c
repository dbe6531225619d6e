/*
 * pins.c -- exhaustive CPU pins for the oracle's primitives.
 *
 *   pins exp   : EXP over every fp32 input vs binary64 exp(); prints max ulp
 *   pins log   : LOG over every positive fp32 input vs binary64 log()
 *   pins prod  : every pair of finite bf16 values: the fp32 product equals
 *                the exact (binary64) product unless it over- or underflows
 *   pins rne   : bf16 rounding of every fp32 pattern vs an independent
 *                nearest-even rule computed in binary64
 *
 * The claim behind "prod": a bf16 significand has 8 bits, a product of two
 * has at most 16, so it fits the 24-bit fp32 significand (the rounding-
 * alignment article, "the problem": bf16 keeps 7 stored mantissa bits).
 *
 * An optional fourth argument visits every step-th pattern only (a sampled
 * run, as under the sanitizer build); the default 1 is exhaustive.
 *
 * Output: one line "key=value ..." parsed by the test suite.
 */
#define _GNU_SOURCE
#include <dlfcn.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef float (*f1)(float);
typedef uint16_t (*rnef)(float);
static f1 fn_exp, fn_log;
static rnef fn_rne;

static float fb(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* ulp of the binary32 grid at |ref| (subnormal spacing below 2^-126). */
static double ulp32(double ref) {
    double a = fabs(ref);
    if (a < ldexp(1.0, -126)) return ldexp(1.0, -149);
    int e;
    frexp(a, &e);                 /* a = m * 2^e, m in [0.5, 1) */
    return ldexp(1.0, e - 24);
}

static uint64_t step = 1;

typedef struct {
    int mode, tid, nth;
    double max_err;
    uint32_t worst;
    uint64_t bad;
} job;

static void *work(void *p) {
    job *j = (job *)p;
    uint64_t lo = (uint64_t)j->tid * (1ull << 32) / j->nth;
    uint64_t hi = (uint64_t)(j->tid + 1) * (1ull << 32) / j->nth;
    for (uint64_t u = lo; u < hi; u += step) {
        uint32_t bits = (uint32_t)u;
        float x = fb(bits);
        if (j->mode == 0 || j->mode == 1) {
            if (isnan(x)) continue;
            double ref;
            float y;
            if (j->mode == 0) {
                ref = exp((double)x);
                y = fn_exp(x);
                if (ref > 3.4028235677973366e38) { /* beyond FLT_MAX: must be inf or FLT_MAX */
                    if (!(isinf(y) || y == 3.40282347e38f)) { j->bad++; }
                    continue;
                }
            } else {
                if (x <= 0.0f || isinf(x)) continue;
                ref = log((double)x);
                y = fn_log(x);
            }
            if (isinf(y) || isnan(y)) { j->bad++; j->worst = bits; continue; }
            double err = fabs((double)y - ref) / ulp32(ref);
            if (err > j->max_err) { j->max_err = err; j->worst = bits; }
        } else if (j->mode == 2) {
            uint32_t a16 = bits >> 16, b16 = bits & 0xffffu;
            float a = fb(a16 << 16), b = fb(b16 << 16);
            if (!isfinite(a) || !isfinite(b)) continue;
            double exact = (double)a * (double)b;   /* exact in binary64 */
            double ae = fabs(exact);
            if (ae != 0.0 && (ae < ldexp(1.0, -126) || ae > 3.4028234663852886e38)) continue;
            float prod = a * b;
            if ((double)prod != exact) { j->bad++; j->worst = bits; }
        } else {
            if (isnan(x)) {
                uint16_t h = fn_rne(x);
                if ((h & 0x7fc0u) != 0x7fc0u) { j->bad++; j->worst = bits; }
                continue;
            }
            /* nearest bf16 by binary64 arithmetic: neighbours lo <= x <= hi */
            uint32_t tr = bits & 0xffff0000u;
            double xd = (double)x;
            double lo_v = (double)fb(tr);
            uint32_t up = tr + 0x10000u;                 /* next pattern away from zero */
            double hi_v = ((up & 0x7f800000u) == 0x7f800000u)
                              ? copysign(ldexp(1.0, 128), xd) : (double)fb(up);
            double dlo = fabs(xd - lo_v), dhi = fabs(hi_v - xd);
            uint32_t expect;
            if (dlo < dhi) expect = tr;
            else if (dhi < dlo) expect = up;
            else expect = ((tr >> 16) & 1u) ? up : tr;  /* tie: even */
            uint16_t h = fn_rne(x);
            if ((uint32_t)h << 16 != expect) { j->bad++; j->worst = bits; }
        }
    }
    return NULL;
}

int main(int argc, char **argv) {
    if (argc < 3) { fprintf(stderr, "usage: pins <liboracle.so> exp|log|prod|rne [threads [step]]\n"); return 2; }
    void *h = dlopen(argv[1], RTLD_NOW);
    if (!h) { fprintf(stderr, "dlopen: %s\n", dlerror()); return 2; }
    fn_exp = (f1)dlsym(h, "or_expf");
    fn_log = (f1)dlsym(h, "or_logf");
    fn_rne = (rnef)dlsym(h, "or_f32_to_bf16");
    int mode = !strcmp(argv[2], "exp") ? 0 : !strcmp(argv[2], "log") ? 1
             : !strcmp(argv[2], "prod") ? 2 : 3;
    int nth = argc > 3 ? atoi(argv[3]) : 8;
    if (nth < 1) nth = 1;
    if (nth > 64) nth = 64;
    if (argc > 4) step = strtoull(argv[4], NULL, 10);
    if (step < 1) step = 1;
    fn_exp(0.0f);   /* initialise the oracle's constants before threading */
    pthread_t th[64];
    job jobs[64];
    for (int t = 0; t < nth; t++) {
        memset(&jobs[t], 0, sizeof(job));
        jobs[t].mode = mode; jobs[t].tid = t; jobs[t].nth = nth;
        pthread_create(&th[t], NULL, work, &jobs[t]);
    }
    double mx = 0.0; uint32_t worst = 0; uint64_t bad = 0;
    for (int t = 0; t < nth; t++) {
        pthread_join(th[t], NULL);
        if (jobs[t].max_err > mx) { mx = jobs[t].max_err; worst = jobs[t].worst; }
        if (jobs[t].bad && !bad) worst = jobs[t].worst;
        bad += jobs[t].bad;
    }
    printf("max_ulp=%.6f worst=0x%08x bad=%llu\n", mx, worst, (unsigned long long)bad);
    return 0;
}
