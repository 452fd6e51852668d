/* Drives every entry point of the C oracle over small seeded inputs, for a build with the
 * address and undefined-behaviour sanitizers (tests/test_host_sanitizers.py). The oracle source
 * is included whole so the driver sees its codec struct. Exit status 0 = no finding. */
#include "../../oracle/kvq_oracle.c"

#include <stdio.h>

static uint64_t lcg_state = 0x9E3779B97F4A7C15ull;
static double uniform01(void) {
  lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(lcg_state >> 11) * (1.0 / 9007199254740992.0);
}
static double normal(void) {  /* Box-Muller */
  double u = uniform01(), v = uniform01();
  if (u < 1e-300) u = 1e-300;
  return sqrt(-2.0 * log(u)) * cos(2.0 * M_PI * v);
}

static void run(int D, int bits, int r, int rule, double T, int64_t n) {
  const int m = r > 0 ? r : D, L = 1 << bits, rb = kvq_ref_record_bytes(m, bits);
  double c64[16];
  float c32[16];
  if (kvq_ref_lloyd_max_gaussian(bits, c64, c32) < 0) exit(2);
  uint16_t* x = malloc(sizeof(uint16_t) * n * D);
  for (int64_t i = 0; i < n * D; ++i) x[i] = float_to_bf16_rne((float)(normal() * (i % 7 == 0 ? 8.0 : 1.0)));
  uint16_t* basis = NULL;
  float* mean = NULL;
  if (r > 0) {
    basis = malloc(sizeof(uint16_t) * D * r);
    mean = malloc(sizeof(float) * D);
    for (int i = 0; i < D * r; ++i) basis[i] = float_to_bf16_rne((float)(normal() / sqrt((double)D)));
    for (int i = 0; i < D; ++i) mean[i] = (float)(0.1 * normal());
  }
  ref_codec cd = {D, bits, r, rule, 1234567ull + (uint64_t)D, T, c32, basis, mean, NULL};
  uint8_t* rec = malloc((size_t)rb * n);
  uint8_t* codes = malloc((size_t)m * n);
  uint8_t* flags = malloc((size_t)m * n);
  double* z = malloc(sizeof(double) * m * n);
  double* norms = malloc(sizeof(double) * n);
  const int64_t cap = n * m / 8;
  uint32_t* off = T > 0 ? malloc(sizeof(uint32_t) * (n + 1)) : NULL;
  uint16_t* idx = T > 0 ? malloc(sizeof(uint16_t) * cap) : NULL;
  uint16_t* val = T > 0 ? malloc(sizeof(uint16_t) * cap) : NULL;
  const int64_t total = kvq_ref_encode(&cd, n, x, D, rec, codes, flags, z, norms, off, idx, val, cap);
  if (total < 0) exit(3);
  double* y = malloc(sizeof(double) * n * D);
  kvq_ref_decode(&cd, n, rec, off, idx, val, cap, y);
  double* s = malloc(sizeof(double) * n);
  kvq_ref_score(&cd, n, x, rec, s);
  uint8_t code1[512];
  float nrm;
  kvq_ref_unpack_codes(m, bits, rec, code1, &nrm);
  float fit[16];
  memcpy(fit, c32, sizeof(float) * L);
  kvq_ref_lloyd_fit(z, n * m, L, 3, fit);
  if (!(kvq_ref_table_mse(z, n * m, L, fit) >= 0.0)) exit(4);
  free(x); free(basis); free(mean); free(rec); free(codes); free(flags); free(z); free(norms);
  free(off); free(idx); free(val); free(y); free(s);
}

int main(void) {
  static const int dims[] = {64, 128, 256, 512};
  for (int di = 0; di < 4; ++di)
    for (int b = 1; b <= 4; ++b) {
      run(dims[di], b, 0, 0, 0.0, 37);
      run(dims[di], b, 0, 0, 2.0, 29);
    }
  for (int rule = 1; rule <= 3; ++rule) run(128, 3, 0, rule, 0.0, 21);
  run(128, 3, 32, 0, 0.0, 19);
  run(128, 2, 64, 0, 0.0, 19);
  run(64, 4, 64, 0, 0.0, 11);
  double* a = malloc(sizeof(double) * 3 * 512);
  for (int i = 0; i < 3 * 512; ++i) a[i] = normal();
  kvq_ref_fwht_rows(a, 3, 512);
  int8_t sg[512];
  kvq_ref_signs(42, 512, sg);
  float t[15], c[16];
  double c64[16];
  kvq_ref_lloyd_max_gaussian(4, c64, c);
  kvq_ref_thresholds(c, 16, t);
  free(a);
  printf("oracle driver ok\n");
  return 0;
}
