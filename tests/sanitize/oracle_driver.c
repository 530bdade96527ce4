/* Drives every entry point of the C oracle on small inputs (all dtypes, with
 * and without optional arguments) and on rejected arguments, for a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_host_sanitizer.py).
 * Exit status 0 means every call returned what it should; the sanitizers
 * abort the process on their own findings. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int ckda_oracle_fwd(const void*, const void*, const void*, const void*, const void*, int, const void*, int, double*,
                    double*, int, int, int, int, int, int);
int ckda_oracle_decode(const void*, const void*, const void*, const void*, const void*, int, double*, double*, int,
                       int, int, int, int);
int ckda_oracle_num_threads(void);
int ckda_oracle_prologue(const void*, const void*, const void*, const void*, int, int, long long, int, double*,
                         double*, double*, double*);
int ckda_oracle_prologue_bwd(const void*, const void*, const void*, const void*, int, int, long long, int,
                             const double*, const double*, const double*, const double*, double*, double*, double*,
                             double*);
int ckda_oracle_deltaproduct2(const void*, const void*, const void*, const void*, const void*, int, const void*, int,
                              double*, double*, int, int, int, int, int, int);
int ckda_oracle_deltaproduct2_decode(const void*, const void*, const void*, const void*, const void*, int, double*,
                                     double*, int, int, int, int);
int ckda_oracle_bwd(const void*, const void*, const void*, const void*, const void*, int, const void*, int,
                    const void*, const void*, int, double*, double*, double*, double*, double*, double*, int, int, int,
                    int, int, int);

enum { F32 = 0, BF16 = 1, F64 = 2 };
static int failures = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static uint32_t rng = 12345u;
static double uni(void) { /* xorshift32 in [-1, 1) */
  rng ^= rng << 13;
  rng ^= rng >> 17;
  rng ^= rng << 5;
  return (double)rng / 2147483648.0 - 1.0;
}

/* n values as the given dtype; the caller frees */
static void* make(size_t n, int dtype, double scale, double shift) {
  size_t es = dtype == F64 ? 8 : dtype == F32 ? 4 : 2;
  unsigned char* p = (unsigned char*)malloc(n * es);
  for (size_t i = 0; i < n; ++i) {
    const double x = shift + scale * uni();
    if (dtype == F64) {
      ((double*)p)[i] = x;
    } else {
      float f = (float)x;
      if (dtype == F32) {
        ((float*)p)[i] = f;
      } else {
        uint32_t b;
        memcpy(&b, &f, 4);
        ((uint16_t*)p)[i] = (uint16_t)(b >> 16);
      }
    }
  }
  return p;
}

int main(void) {
  const int B = 1, H = 2, T = 37, dk = 8, dv = 4;
  const size_t nq = (size_t)B * H * T * dk, nv = (size_t)B * H * T * dv, nb = (size_t)B * H * T;
  const size_t ns = (size_t)B * H * dk * dv;
  EXPECT(ckda_oracle_num_threads() >= 1);
  for (int dtype = 0; dtype < 3; ++dtype) {
    void *q = make(nq, dtype, 1, 0), *k = make(nq, dtype, 0.3, 0), *v = make(nv, dtype, 1, 0);
    void *a = make(nq, dtype, 1, 0), *b = make(nb, dtype, 1, 1), *h0 = make(ns, F32, 0.1, 0);
    double *o = malloc(nv * 8), *hT = malloc(ns * 8);
    for (int nt = 0; nt < 2; ++nt) {
      EXPECT(ckda_oracle_fwd(q, k, v, a, b, dtype, h0, F32, o, hT, B, H, T, dk, dv, nt) == 0);
      EXPECT(ckda_oracle_fwd(q, k, v, a, b, dtype, NULL, F32, o, hT, B, H, T, dk, dv, nt) == 0);
      EXPECT(ckda_oracle_fwd(q, k, v, a, b, dtype, h0, F32, NULL, hT, B, H, T, dk, dv, nt) == 0);
    }
    EXPECT(ckda_oracle_fwd(q, k, v, a, b, dtype, h0, F32, o, hT, B, H, 0, dk, dv, 0) == 0);
    EXPECT(ckda_oracle_fwd(NULL, k, v, a, b, dtype, h0, F32, o, hT, B, H, T, dk, dv, 0) != 0);
    EXPECT(ckda_oracle_fwd(q, k, v, a, b, dtype, h0, F32, o, hT, -1, H, T, dk, dv, 0) != 0);
    EXPECT(ckda_oracle_fwd(q, k, v, a, b, 7, h0, F32, o, hT, B, H, T, dk, dv, 0) != 0);
    /* decode on the states just computed, T of them as N sequences */
    double *S = malloc(ns * 8), *od = malloc((size_t)B * H * dv * 8);
    memcpy(S, hT, ns * 8);
    EXPECT(ckda_oracle_decode(q, k, v, a, b, dtype, S, od, B, H, dk, dv, 0) == 0);
    EXPECT(ckda_oracle_decode(q, k, v, a, b, dtype, NULL, od, B, H, dk, dv, 0) != 0);
    /* prologue and its backward, every flag combination */
    double *pa = malloc(nq * 8), *pb = malloc(nb * 8), *pk = malloc(nq * 8), *pq = malloc(nq * 8);
    double *ga = malloc(nq * 8), *gb = malloc(nb * 8), *gk = malloc(nq * 8), *gq = malloc(nq * 8);
    for (int flags = 0; flags < 8; ++flags) {
      EXPECT(ckda_oracle_prologue(a, b, k, q, dtype, flags, (long long)nb, dk, pa, pb, pk, pq) == 0);
      EXPECT(ckda_oracle_prologue_bwd(a, b, k, q, dtype, flags, (long long)nb, dk, pa, pb, pk, pq, ga, gb, gk, gq) ==
             0);
    }
    EXPECT(ckda_oracle_prologue(a, b, k, q, dtype, 8, (long long)nb, dk, pa, pb, pk, pq) != 0);
    /* backward */
    /* do and dhT share one fp32 or fp64 dtype */
    const int gdt = dtype == F64 ? F64 : F32;
    void* dout = make(nv, gdt, 1, 0);
    void* dhT = make(ns, gdt, 1, 0);
    double *dq = malloc(nq * 8), *dkk = malloc(nq * 8), *dvv = malloc(nv * 8), *dal = malloc(nq * 8);
    double *dbe = malloc(nb * 8), *dh0 = malloc(ns * 8);
    EXPECT(ckda_oracle_bwd(q, k, v, a, b, dtype, h0, F32, dout, dhT, gdt, dq, dkk, dvv, dal, dbe, dh0, B, H, T, dk,
                           dv, 0) == 0);
    EXPECT(ckda_oracle_bwd(q, k, v, a, b, dtype, NULL, F32, dout, NULL, gdt, dq, dkk, dvv, dal, dbe, dh0, B, H, T,
                           dk, dv, 1) == 0);
    EXPECT(ckda_oracle_bwd(q, k, v, a, b, dtype, h0, F32, dout, dhT, gdt, NULL, dkk, dvv, dal, dbe, dh0, B, H, T,
                           dk, dv, 0) != 0);
    /* DeltaProduct_2: 2 sub-steps per token */
    void *k2 = make(2 * nq, dtype, 0.3, 0), *v2 = make(2 * nv, dtype, 1, 0), *b2 = make(2 * nb, dtype, 1, 1);
    void* a1 = make(nb, dtype, 1, 0);
    EXPECT(ckda_oracle_deltaproduct2(q, k2, v2, a1, b2, dtype, h0, F32, o, hT, B, H, T, dk, dv, 0) == 0);
    EXPECT(ckda_oracle_deltaproduct2(q, k2, v2, NULL, b2, dtype, NULL, F32, o, hT, B, H, T, dk, dv, 1) == 0);
    EXPECT(ckda_oracle_deltaproduct2_decode(q, k2, v2, a1, b2, dtype, S, od, B, H, dk, dv) == 0);
    EXPECT(ckda_oracle_deltaproduct2_decode(q, k2, v2, NULL, b2, dtype, S, od, B, H, dk, dv) == 0);
    for (size_t i = 0; i < ns; ++i) EXPECT(isfinite(S[i]));
    free(q); free(k); free(v); free(a); free(b); free(h0); free(o); free(hT); free(S); free(od);
    free(pa); free(pb); free(pk); free(pq); free(ga); free(gb); free(gk); free(gq);
    free(dout); free(dhT); free(dq); free(dkk); free(dvv); free(dal); free(dbe); free(dh0);
    free(k2); free(v2); free(b2); free(a1);
  }
  printf("oracle driver: %d failures\n", failures);
  return failures ? 1 : 0;
}
