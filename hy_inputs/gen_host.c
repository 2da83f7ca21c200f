/*
 * Host build of the seeded input generator (see gen_core.h). Threaded with
 * pthreads; element i of a tensor depends only on (seed, stream, i), so the
 * result does not depend on the thread count or on the sub-range requested.
 * Compiled with gcc -O2 -ffp-contract=off.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include "gen_core.h"

enum { KIND_GAUSS = 0, KIND_UNIFORM = 1, KIND_U32 = 2 };

typedef struct {
  int kind;
  uint64_t seed;
  uint32_t stream;
  uint64_t start, begin, end; /* global index range [begin, end) of this worker */
  double a, b;
  void* out;
} job_t;

static void* worker(void* p) {
  job_t* j = (job_t*)p;
  for (uint64_t i = j->begin; i < j->end; ++i) {
    uint64_t o = i - j->start;
    if (j->kind == KIND_GAUSS)
      ((uint16_t*)j->out)[o] = gen_gauss_bf16_elem(j->seed, j->stream, i, j->a);
    else if (j->kind == KIND_UNIFORM)
      ((uint16_t*)j->out)[o] = gen_uniform_bf16_elem(j->seed, j->stream, i, j->a, j->b);
    else
      ((uint32_t*)j->out)[o] = gen_u32_elem(j->seed, j->stream, i);
  }
  return NULL;
}

static int run(int kind, uint64_t seed, uint32_t stream, uint64_t start, uint64_t count,
               double a, double b, void* out, int nthreads) {
  if (count == 0) return 0;
  if (!out) return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((uint64_t)nthreads > count) nthreads = (int)count;
  pthread_t th[256];
  job_t jobs[256];
  uint64_t per = (count + (uint64_t)nthreads - 1) / (uint64_t)nthreads;
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    uint64_t b0 = start + (uint64_t)t * per;
    uint64_t b1 = b0 + per;
    if (b1 > start + count) b1 = start + count;
    if (b0 >= b1) break;
    jobs[t].kind = kind; jobs[t].seed = seed; jobs[t].stream = stream;
    jobs[t].start = start; jobs[t].begin = b0; jobs[t].end = b1;
    jobs[t].a = a; jobs[t].b = b; jobs[t].out = out;
    if (t == 0) continue; /* run the first slice on the calling thread */
    if (pthread_create(&th[t], NULL, worker, &jobs[t]) != 0) {
      worker(&jobs[t]); /* fall back to running it inline */
      th[t] = 0;
    }
    started = t + 1;
  }
  worker(&jobs[0]);
  for (int t = 1; t < started; ++t)
    if (th[t]) pthread_join(th[t], NULL);
  return 0;
}

/* Elements [start, start+count) of a bf16 Gaussian tensor N(0, std^2). */
int hy_gen_gauss_bf16(uint64_t seed, uint32_t stream, uint64_t start, uint64_t count,
                      double std, uint16_t* out, int nthreads) {
  return run(KIND_GAUSS, seed, stream, start, count, std, 0.0, out, nthreads);
}

/* Elements [start, start+count) of a bf16 tensor uniform on [lo, lo+width). */
int hy_gen_uniform_bf16(uint64_t seed, uint32_t stream, uint64_t start, uint64_t count,
                        double lo, double width, uint16_t* out, int nthreads) {
  return run(KIND_UNIFORM, seed, stream, start, count, lo, width, out, nthreads);
}

/* Words [start, start+count) of a tensor of uniform random 32-bit words. */
int hy_gen_u32(uint64_t seed, uint32_t stream, uint64_t start, uint64_t count,
               uint32_t* out, int nthreads) {
  return run(KIND_U32, seed, stream, start, count, 0.0, 0.0, out, nthreads);
}

/* One raw Philox4x32-10 block, for known-answer tests. */
void hy_gen_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  gen_u32x4 r = gen_philox4x32_10(ctr[0], ctr[1], ctr[2], ctr[3], key[0], key[1]);
  for (int i = 0; i < 4; ++i) out[i] = r.v[i];
}

/* The elementary functions, exported so tests can bound their error. */
double hy_gen_ln(double u) { return gen_ln(u); }
double hy_gen_sqrt(double x) { return gen_sqrt(x); }
void hy_gen_cossin_turn(double a, double* c, double* s) { gen_cossin_turn(a, c, s); }
