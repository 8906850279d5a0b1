/*
 * fvgen.c -- seeded synthetic Q/K/V for video-DiT attention layers.
 *
 * Test and benchmark harness only.  It holds none of the attention method's
 * arithmetic: it draws inputs.  The GPU library and the CPU oracle both consume
 * the bytes it writes; neither links it.
 *
 * Recipe (one head h of one tensor X in {Q,K,V}):
 *   - M Fourier modes per head.  Mode m has an integer wave vector
 *     (kt,ky,kx) drawn uniformly from {0,1,2}^3 without the zero vector, a
 *     phase phi_m ~ U[0,2pi), and per channel c an amplitude a[m][c] ~ N(0,1).
 *   - f_c(t,y,x) = sum_m a[m][c] * cos(2pi(kt*t/T + ky*y/H + kx*x/W) + phi_m),
 *     standardised per channel to zero mean and unit variance over the grid.
 *   - The field f is shared by Q, K and V of the head; each tensor draws its
 *     own noise eps ~ N(0,1):   X = s_X * (0.7 f + 0.3 eps)
 *     with s_Q = tau_h (the head's logit temperature) and s_K = s_V = 1.
 *   - The value is formed in double, rounded to fp32, then to bf16 (RNE).
 *
 * Randomness is counter based: every draw is a SplitMix64-style finaliser of a
 * key built from (seed, config tag, stream, indices), so the bytes do not
 * depend on the number of threads.  Normals come from Box-Muller.
 *
 * Layout of the output: BSHD with B = 1, i.e. out[(l*heads + h)*D + c] with
 * token l = (t*H + y)*W + x.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define FVGEN_TWO_PI 6.283185307179586476925286766559

static inline uint64_t fvgen_fmix(uint64_t z) {
  z += 0x9e3779b97f4a7c15ULL;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

/* 64-bit hash of (seed, tag, stream, a, b). */
uint64_t fvgen_hash(uint64_t seed, uint64_t tag, uint64_t stream, uint64_t a, uint64_t b) {
  uint64_t z = fvgen_fmix(seed);
  z = fvgen_fmix(z ^ tag);
  z = fvgen_fmix(z ^ (stream * 0x100000001b3ULL));
  z = fvgen_fmix(z ^ a);
  z = fvgen_fmix(z ^ (b + 0x632be59bd9b4e019ULL));
  return z;
}

/* Uniform in [0,1) from the top 53 bits. */
double fvgen_uniform(uint64_t seed, uint64_t tag, uint64_t stream, uint64_t a, uint64_t b) {
  return (double)(fvgen_hash(seed, tag, stream, a, b) >> 11) * (1.0 / 9007199254740992.0);
}

/* Standard normal: Box-Muller over two hashed uniforms; u1 in (0,1]. */
static double fvgen_normal(uint64_t seed, uint64_t tag, uint64_t stream, uint64_t idx) {
  uint64_t pair = idx >> 1;
  double u1 = ((double)(fvgen_hash(seed, tag, stream, pair, 0) >> 11) + 1.0) * (1.0 / 9007199254740992.0);
  double u2 = (double)(fvgen_hash(seed, tag, stream, pair, 1) >> 11) * (1.0 / 9007199254740992.0);
  double r = sqrt(-2.0 * log(u1));
  return (idx & 1) ? r * sin(FVGEN_TWO_PI * u2) : r * cos(FVGEN_TWO_PI * u2);
}

double fvgen_normal_at(uint64_t seed, uint64_t tag, uint64_t stream, uint64_t idx) {
  return fvgen_normal(seed, tag, stream, idx);
}

/* fp32 -> bf16 bits, round to nearest even (NaN kept quiet). */
static inline uint16_t fvgen_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

enum { STREAM_MODE = 1, STREAM_PHASE = 2, STREAM_AMP = 3, STREAM_NOISE = 16 };

typedef struct {
  int T, H, W, heads, D, modes, which;
  int h;                 /* head being generated */
  uint64_t seed, tag;
  double scale;          /* tau for Q, 1 for K and V */
  const double* cosv;    /* [modes][L] */
  const double* amp;     /* [modes][D] */
  const double* mean;    /* [D] */
  const double* inv_std; /* [D] */
  uint16_t* out;
  int64_t l0, l1;
} fvgen_job;

static void* fvgen_worker(void* arg) {
  fvgen_job* j = (fvgen_job*)arg;
  const int64_t L = (int64_t)j->T * j->H * j->W;
  for (int64_t l = j->l0; l < j->l1; ++l) {
    uint16_t* row = j->out + (l * j->heads + j->h) * (int64_t)j->D;
    for (int c = 0; c < j->D; ++c) {
      double f = 0.0;
      for (int m = 0; m < j->modes; ++m) f += j->amp[(int64_t)m * j->D + c] * j->cosv[(int64_t)m * L + l];
      f = (f - j->mean[c]) * j->inv_std[c];
      uint64_t nidx = ((uint64_t)j->h * (uint64_t)L + (uint64_t)l) * (uint64_t)j->D + (uint64_t)c;
      double eps = fvgen_normal(j->seed, j->tag, STREAM_NOISE + (uint64_t)j->which, nidx);
      double v = j->scale * (0.7 * f + 0.3 * eps);
      row[c] = fvgen_f32_to_bf16((float)v);
    }
  }
  return NULL;
}

/* Generate one tensor (which: 0=Q, 1=K, 2=V) for all heads.
 * tau[heads] scales Q only.  Returns 0 on success, -1 on bad arguments or
 * allocation failure. */
int fvgen_qkv(uint64_t seed, uint64_t tag, int T, int H, int W, int heads, int D, int modes,
              const double* tau, int which, uint16_t* out, int nthreads) {
  if (T <= 0 || H <= 0 || W <= 0 || heads <= 0 || D <= 0 || modes <= 0 || which < 0 || which > 2 || !out || !tau)
    return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  const int64_t L = (int64_t)T * H * W;
  double* cosv = (double*)malloc(sizeof(double) * (size_t)modes * (size_t)L);
  double* amp = (double*)malloc(sizeof(double) * (size_t)modes * (size_t)D);
  double* mean = (double*)malloc(sizeof(double) * (size_t)D);
  double* inv_std = (double*)malloc(sizeof(double) * (size_t)D);
  double* mu = (double*)malloc(sizeof(double) * (size_t)modes);
  double* gram = (double*)malloc(sizeof(double) * (size_t)modes * (size_t)modes);
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  fvgen_job* jobs = (fvgen_job*)malloc(sizeof(fvgen_job) * (size_t)nthreads);
  if (!cosv || !amp || !mean || !inv_std || !mu || !gram || !th || !jobs) {
    free(cosv); free(amp); free(mean); free(inv_std); free(mu); free(gram); free(th); free(jobs);
    return -1;
  }
  for (int h = 0; h < heads; ++h) {
    /* modes of this head: shared by Q, K and V (streams do not depend on `which`) */
    for (int m = 0; m < modes; ++m) {
      uint64_t u = fvgen_hash(seed, tag, STREAM_MODE, (uint64_t)h, (uint64_t)m) % 26u; /* 26 nonzero vectors */
      int code = (int)u + 1;                                                             /* 1..26 in base 3 */
      int kt = code / 9, ky = (code / 3) % 3, kx = code % 3;
      double phi = FVGEN_TWO_PI * fvgen_uniform(seed, tag, STREAM_PHASE, (uint64_t)h, (uint64_t)m);
      for (int c = 0; c < D; ++c)
        amp[(int64_t)m * D + c] =
            fvgen_normal(seed, tag, STREAM_AMP, ((uint64_t)h * (uint64_t)modes + (uint64_t)m) * (uint64_t)D + (uint64_t)c);
      for (int t = 0; t < T; ++t)
        for (int y = 0; y < H; ++y)
          for (int x = 0; x < W; ++x) {
            double arg = FVGEN_TWO_PI * ((double)kt * t / T + (double)ky * y / H + (double)kx * x / W) + phi;
            cosv[(int64_t)m * L + ((int64_t)t * H + y) * W + x] = cos(arg);
          }
    }
    /* per-channel mean and variance of f from the mode means and Gram matrix
     * (sequential sums: independent of the thread count) */
    for (int m = 0; m < modes; ++m) {
      double s = 0.0;
      for (int64_t l = 0; l < L; ++l) s += cosv[(int64_t)m * L + l];
      mu[m] = s / (double)L;
      for (int n = 0; n <= m; ++n) {
        double g = 0.0;
        for (int64_t l = 0; l < L; ++l) g += cosv[(int64_t)m * L + l] * cosv[(int64_t)n * L + l];
        gram[m * modes + n] = gram[n * modes + m] = g / (double)L;
      }
    }
    for (int c = 0; c < D; ++c) {
      double e1 = 0.0, e2 = 0.0;
      for (int m = 0; m < modes; ++m) {
        e1 += amp[(int64_t)m * D + c] * mu[m];
        for (int n = 0; n < modes; ++n) e2 += amp[(int64_t)m * D + c] * amp[(int64_t)n * D + c] * gram[m * modes + n];
      }
      double var = e2 - e1 * e1;
      mean[c] = e1;
      inv_std[c] = var > 1e-300 ? 1.0 / sqrt(var) : 0.0;
    }
    int nt = nthreads;
    if ((int64_t)nt > L) nt = (int)L;
    for (int i = 0; i < nt; ++i) {
      fvgen_job* j = &jobs[i];
      j->T = T; j->H = H; j->W = W; j->heads = heads; j->D = D; j->modes = modes; j->which = which;
      j->h = h; j->seed = seed; j->tag = tag;
      j->scale = (which == 0) ? tau[h] : 1.0;
      j->cosv = cosv; j->amp = amp; j->mean = mean; j->inv_std = inv_std; j->out = out;
      j->l0 = L * i / nt;
      j->l1 = L * (i + 1) / nt;
    }
    for (int i = 1; i < nt; ++i) pthread_create(&th[i], NULL, fvgen_worker, &jobs[i]);
    fvgen_worker(&jobs[0]);
    for (int i = 1; i < nt; ++i) pthread_join(th[i], NULL);
  }
  free(cosv); free(amp); free(mean); free(inv_std); free(mu); free(gram); free(th); free(jobs);
  return 0;
}
