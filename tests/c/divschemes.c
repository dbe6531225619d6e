/*
 * divschemes.c -- CPU check of the division scheme the SwiGLU kernels use in
 * place of the IEEE fp32 division.  It rests on Markstein's theorem
 * (binary floating point, round to nearest, no underflow): if y is within
 * half an ulp of 1/b and q within one ulp of a/b, the remainder
 * r = a - q b is exact in one FMA and RN(q + r y) = RN(a / b).
 *
 *   divschemes <liboracle.so> silu [threads]
 *       SwiGLU's gate: silu(g) = g / d, d = 1 + EXP(-g).  For every bf16 g
 *       with g >= -87 and |g| >= 2^-20, and for each reciprocal y0 within
 *       3 ulp of RN(1/d) (what v_rcp_f32 may return), one Newton step
 *       y1 = y0 + y0 (1 - d y0), then q0 = g y1 and the correction must give
 *       the IEEE quotient.
 *
 * The oracle library supplies EXP (the check needs the exact d the kernels
 * see).  Output: "checked=N bad=M worst=..." parsed by the tests.
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
static f1 fn_exp;

static float fb(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bf(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* the SiLU scheme: y0 any approximate reciprocal of d */
static float div_silu(float g, float d, float y0) {
    float e0 = fmaf(-d, y0, 1.0f);
    float y1 = fmaf(e0, y0, y0);
    float q0 = g * y1;
    float rm = fmaf(-d, q0, g);
    return fmaf(rm, y1, q0);
}

typedef struct {
    int tid, nth;
    uint64_t checked, bad;
    uint32_t worst_a, worst_b;
} job;

static void note_bad(job *j, float a, float b) {
    if (!j->bad) { j->worst_a = bf(a); j->worst_b = bf(b); }
    j->bad++;
}

static void *work(void *p) {
    job *j = (job *)p;
    for (uint32_t h = (uint32_t)j->tid; h < 65536u; h += (uint32_t)j->nth) {   /* bf16 gates */
        float g = fb(h << 16);
        if (!(g >= -87.0f) || !(fabsf(g) >= 0x1p-20f) || isinf(g)) continue;
        float d = 1.0f + fn_exp(-g);
        float want = g / d;
        float y = 1.0f / d;
        for (int k = -3; k <= 3; k++) {
            float y0 = fb((uint32_t)((int32_t)bf(y) + k));
            j->checked++;
            if (bf(div_silu(g, d, y0)) != bf(want)) note_bad(j, g, d);
        }
    }
    return NULL;
}

int main(int argc, char **argv) {
    if (argc < 3) { fprintf(stderr, "usage: divschemes <liboracle.so> silu [threads]\n"); return 2; }
    void *h = dlopen(argv[1], RTLD_NOW);
    if (!h) { fprintf(stderr, "dlopen: %s\n", dlerror()); return 2; }
    fn_exp = (f1)dlsym(h, "or_expf");
    if (!fn_exp) { fprintf(stderr, "or_expf missing\n"); return 2; }
    if (strcmp(argv[2], "silu")) { fprintf(stderr, "unknown mode %s\n", argv[2]); return 2; }
    int nth = argc > 3 ? atoi(argv[3]) : 8;
    if (nth < 1) nth = 1;
    if (nth > 64) nth = 64;
    fn_exp(0.0f);   /* initialise the oracle's constants before threading */
    pthread_t th[64];
    job jobs[64];
    for (int t = 0; t < nth; t++) {
        memset(&jobs[t], 0, sizeof(job));
        jobs[t].tid = t; jobs[t].nth = nth;
        pthread_create(&th[t], NULL, work, &jobs[t]);
    }
    uint64_t checked = 0, bad = 0;
    uint32_t wa = 0, wb = 0;
    for (int t = 0; t < nth; t++) {
        pthread_join(th[t], NULL);
        if (jobs[t].bad && !bad) { wa = jobs[t].worst_a; wb = jobs[t].worst_b; }
        checked += jobs[t].checked;
        bad += jobs[t].bad;
    }
    printf("checked=%llu bad=%llu worst=0x%08x/0x%08x\n", (unsigned long long)checked,
           (unsigned long long)bad, wa, wb);
    return 0;
}
