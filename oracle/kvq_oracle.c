/*
 * kvq_oracle.c — plain, slow, single-threaded CPU reference of the KV-cache vector codec.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library. It shares no code, header, table or constant generator with the
 * GPU library; the two meet only in the byte format of a record.
 *
 * Arithmetic is f64 throughout; f32 / bf16 appear only where the record format stores a value
 * (centroids, thresholds, norm, outlier values). Each function cites the passage it follows:
 *   [PR15 M4A]  kakeyaturbo PR #15 "v1.3 PPL on vLLM ...", commit "M4 Phase A" (stages 2..5:
 *               project, rotate H.D.x, scale, Lloyd-Max quantise, pack; nearest centroid)
 *   [PR15 M4B]  same page, commit "M4 Phase B" (Sylvester Hadamard, scale by 1/||r||)
 *   [PR15 M5]   same page, commit "M5" (decode: LUT, outlier scatter before the inverse
 *               rotation, y = z^ * norm, x = H y * sign / wht_len, unproject)
 *   [PR15 OL]   same page, commit adding calibrated Lloyd-Max + outlier compensation
 *               (|scaled residual| > T become sparse overrides at decode)
 *   [LARQL TQ]  larql PR #196, turbo-quant commit (one N(0,1) Lloyd-Max table per bit width)
 *   [ARC98 WL]  arc PR #98 "TurboQuant KV storage for DeepSeek-V4", section "What landed"
 *               (record = packed codes + one f32 norm, 260 B at head_dim 512 / 4 bits)
 *
 * Parity pins for every function live in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------ */
/* Storage conversions (the only places f32 / bf16 enter).                                     */

static double bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* f32 -> bf16, round to nearest, ties to even (finite inputs). */
static uint16_t float_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------------------------ */
/* Gaussian Lloyd-Max table [PR15 M4A "centroids_gaussian(bits)"; LARQL TQ].                   */
/* Lloyd's two conditions for a density p: each boundary is the midpoint of its neighbouring  */
/* centroids, each centroid the conditional mean of its cell. For N(0,1) the conditional mean */
/* of (a, b) is (phi(a) - phi(b)) / (Phi(b) - Phi(a)).                                          */

static double std_normal_pdf(double x) {
  if (isinf(x)) return 0.0;
  return exp(-0.5 * x * x) / sqrt(2.0 * M_PI);
}

/* P(a < Z < b) for Z ~ N(0,1), evaluated on the side of zero where it does not cancel. */
static double std_normal_mass(double a, double b) {
  if (a >= 0.0) return 0.5 * erfc(a / sqrt(2.0)) - 0.5 * erfc(b / sqrt(2.0));
  if (b <= 0.0) return 0.5 * erfc(-b / sqrt(2.0)) - 0.5 * erfc(-a / sqrt(2.0));
  return 1.0 - 0.5 * erfc(b / sqrt(2.0)) - 0.5 * erfc(-a / sqrt(2.0));
}

/* Iterates Lloyd's conditions on N(0,1) with L = 2^bits cells until no centroid moves by
 * 1e-14, then makes the table exactly antisymmetric. Writes the f64 centroids and their f32
 * (round-to-nearest) values. Returns the iteration count, or -1 on bad input / no convergence. */
int kvq_ref_lloyd_max_gaussian(int bits, double* c64, float* c32) {
  if (bits < 1 || bits > 8) return -1;
  const int L = 1 << bits;
  double c[256], t[256];
  for (int k = 0; k < L; ++k) c[k] = -3.0 + 6.0 * (k + 0.5) / L; /* any ascending start */
  int it;
  for (it = 1; it <= 200000; ++it) {
    for (int k = 0; k + 1 < L; ++k) t[k] = 0.5 * (c[k] + c[k + 1]);
    double moved = 0.0;
    for (int k = 0; k < L; ++k) {
      double a = (k == 0) ? -INFINITY : t[k - 1];
      double b = (k == L - 1) ? INFINITY : t[k];
      double mass = std_normal_mass(a, b);
      double cm = (std_normal_pdf(a) - std_normal_pdf(b)) / mass;
      double d = fabs(cm - c[k]);
      if (d > moved) moved = d;
      c[k] = cm;
    }
    if (moved < 1e-14) break;
  }
  if (it > 200000) return -1;
  for (int k = 0; k < L / 2; ++k) {
    double s = 0.5 * (c[L - 1 - k] - c[k]);
    c[k] = -s;
    c[L - 1 - k] = s;
  }
  for (int k = 0; k < L; ++k) {
    if (c64) c64[k] = c[k];
    if (c32) c32[k] = (float)c[k];
  }
  return it;
}

/* Decision thresholds: t_k = f32 of the midpoint of the f32 centroids c_k, c_{k+1}
 * (the nearest-centroid boundaries of the stored table) [PR15 M4A]. */
void kvq_ref_thresholds(const float* c, int L, float* t) {
  for (int k = 0; k + 1 < L; ++k) t[k] = (float)(0.5 * ((double)c[k] + (double)c[k + 1]));
}

/* ------------------------------------------------------------------------------------------ */
/* Sign diagonal. The pages draw it from a seeded RNG ("wht_sign_pattern(seed, n)" [PR15 M4A]); */
/* the generator here is SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): the state advances by  */
/* the golden-ratio increment and each output is the state run through the published mixing   */
/* function; the sign is the top bit of output i.                                             */

static uint64_t splitmix64_output(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Exposed for the pins: the first n raw generator outputs from `seed`. */
void kvq_ref_splitmix64(uint64_t seed, int n, uint64_t* out) {
  uint64_t state = seed;
  for (int i = 0; i < n; ++i) {
    state += 0x9E3779B97F4A7C15ull;
    out[i] = splitmix64_output(state);
  }
}

void kvq_ref_signs(uint64_t seed, int m, int8_t* s) {
  uint64_t state = seed;
  for (int i = 0; i < m; ++i) {
    state += 0x9E3779B97F4A7C15ull;
    s[i] = (splitmix64_output(state) >> 63) ? (int8_t)-1 : (int8_t)1;
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Walsh-Hadamard transform, natural (Sylvester) order, unnormalised: a <- H_m a with          */
/* H[i][j] = (-1)^popcount(i & j) [PR15 M4B "128x128 Sylvester Hadamard"].                      */

static void fwht(double* a, int m) {
  for (int h = 1; h < m; h <<= 1)
    for (int i = 0; i < m; i += 2 * h)
      for (int j = i; j < i + h; ++j) {
        double x = a[j], y = a[j + h];
        a[j] = x + y;
        a[j + h] = x - y;
      }
}

/* Exposed for the pins: in-place FWHT of n rows of length m (f64). */
void kvq_ref_fwht_rows(double* a, int64_t n, int m) {
  for (int64_t r = 0; r < n; ++r) fwht(a + r * m, m);
}

/* ------------------------------------------------------------------------------------------ */
/* Record format [ARC98 WL: codes then one f32 norm]. The bit layout is this codec's own:      */
/* plane position pi(i) = (i mod 8)*(m/8) + i/8; word[g*b + p] bit j = bit p of the code at    */
/* plane position 32g + j; then f32 norm.                                                      */

int kvq_ref_record_bytes(int m, int bits) { return m * bits / 8 + 4; }

int kvq_ref_plane_position(int i, int m) { return (i % 8) * (m / 8) + i / 8; }

static void pack_record(const uint8_t* code, int m, int bits, float norm, uint8_t* rec) {
  const int nwords = (m / 32) * bits;
  uint32_t w[64];
  memset(w, 0, sizeof(w));
  for (int i = 0; i < m; ++i) {
    int pos = kvq_ref_plane_position(i, m);
    for (int p = 0; p < bits; ++p)
      if ((code[i] >> p) & 1u) w[(pos / 32) * bits + p] |= 1u << (pos % 32);
  }
  for (int k = 0; k < nwords; ++k) {
    rec[4 * k + 0] = (uint8_t)(w[k] & 0xFF);
    rec[4 * k + 1] = (uint8_t)((w[k] >> 8) & 0xFF);
    rec[4 * k + 2] = (uint8_t)((w[k] >> 16) & 0xFF);
    rec[4 * k + 3] = (uint8_t)((w[k] >> 24) & 0xFF);
  }
  uint32_t nb;
  memcpy(&nb, &norm, 4);
  for (int q = 0; q < 4; ++q) rec[4 * nwords + q] = (uint8_t)((nb >> (8 * q)) & 0xFF);
}

/* Inverse of pack_record: codes[m] and the stored f32 norm. */
void kvq_ref_unpack_codes(int m, int bits, const uint8_t* rec, uint8_t* code, float* norm) {
  const int nwords = (m / 32) * bits;
  for (int i = 0; i < m; ++i) {
    int pos = kvq_ref_plane_position(i, m);
    uint8_t c = 0;
    for (int p = 0; p < bits; ++p) {
      int k = (pos / 32) * bits + p;
      uint32_t word = (uint32_t)rec[4 * k] | ((uint32_t)rec[4 * k + 1] << 8) |
                      ((uint32_t)rec[4 * k + 2] << 16) | ((uint32_t)rec[4 * k + 3] << 24);
      if ((word >> (pos % 32)) & 1u) c |= (uint8_t)(1u << p);
    }
    code[i] = c;
  }
  if (norm) {
    uint32_t nb = (uint32_t)rec[4 * nwords] | ((uint32_t)rec[4 * nwords + 1] << 8) |
                  ((uint32_t)rec[4 * nwords + 2] << 16) | ((uint32_t)rec[4 * nwords + 3] << 24);
    memcpy(norm, &nb, 4);
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Codec parameters as the oracle sees them.                                                   */

typedef struct {
  int32_t D;               /* head_dim                                                        */
  int32_t bits;            /* b                                                               */
  int32_t r;               /* 0 = no projection; else PCA rank                                */
  int32_t scale_rule;      /* stored scale: 0 = ||v||, 1 = matched norm, 2 = inner-product     */
                           /* preserving, 3 = least-squares optimal                           */
  uint64_t seed;           /* sign seed                                                       */
  double T;                /* outlier threshold, 0 = off                                      */
  const float* centroids;  /* f32[2^b] ascending                                              */
  const uint16_t* basis;   /* bf16 [D][r] (PCA only)                                          */
  const float* mean;       /* f32 [D] or NULL (PCA only)                                      */
  const uint16_t* unbasis; /* bf16 [D][r] decode basis C, or NULL = basis (PCA only). Q-       */
                           /* preconditioning with Sigma_q = L L^T [kakeyaturbo PR #15: the    */
                           /* artefacts commit (K_tilde = K @ L), the full-recipe commit (K is */
                           /* whitened before the codec and unwhitened after it) and "M6 Phase */
                           /* B.2a" (whiten by the Cholesky factor before encode, multiply by  */
                           /* its inverse after decode)] gives the pair basis = L B_w,          */
                           /* unbasis = L^-T B_w, mean = L^-T mu_w for a whitened-domain fit   */
                           /* (B_w, mu_w); B_w = I when nothing is projected away.             */
} ref_codec;

#define FLAG_NEAR_BOUNDARY 1u
#define FLAG_NEAR_T 2u
#define NEAR 1e-5

/* Encode n vectors (x: bf16 rows, leading dimension ld) [PR15 M4A, PR15 M4B, PR15 OL, ARC98 WL].
 * Outputs (each may be NULL): records (n * record bytes), codes[n][m], flags[n][m]
 * (bit0: |z - t_k| < 1e-5 for some k; bit1: ||z| - T| < 1e-5), z[n][m] (f64 scaled rotated
 * coordinates), norms[n] (f64). Outliers (T > 0): CSR offsets[n+1], entries written while the
 * running count is below ol_cap; an entry is the coordinate index (held as u16: the record format
 * stores it in one byte while m <= 256 and in two above [PR15 OL: u16 index]) and the bf16 value
 * of z. Returns the total outlier count. */
int64_t kvq_ref_encode(const ref_codec* cd, int64_t n, const uint16_t* x, int64_t ld,
                       uint8_t* records, uint8_t* codes, uint8_t* flags, double* zout,
                       double* norms, uint32_t* ol_off, uint16_t* ol_idx, uint16_t* ol_val,
                       int64_t ol_cap) {
  const int D = cd->D, b = cd->bits, L = 1 << b;
  const int m = cd->r > 0 ? cd->r : D;
  const int rb = kvq_ref_record_bytes(m, b);
  float t[255];
  kvq_ref_thresholds(cd->centroids, L, t);
  int8_t s[512];
  kvq_ref_signs(cd->seed, m, s);
  double v[512], u[512];
  uint8_t code[512];
  int64_t total = 0;
  if (ol_off) ol_off[0] = 0;
  for (int64_t row = 0; row < n; ++row) {
    const uint16_t* xr = x + row * ld;
    /* project (PCA) or take the row as is [PR15 M4A: (X - mu) @ basis^T] */
    if (cd->r > 0) {
      for (int j = 0; j < m; ++j) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d) {
          double xm = bf16_to_double(xr[d]) - (cd->mean ? (double)cd->mean[d] : 0.0);
          acc += bf16_to_double(cd->basis[(int64_t)d * m + j]) * xm;
        }
        v[j] = acc;
      }
    } else {
      for (int d = 0; d < D; ++d) v[d] = bf16_to_double(xr[d]);
    }
    /* norm of the coded vector */
    double ss = 0.0;
    for (int i = 0; i < m; ++i) ss += v[i] * v[i];
    const double nrm = sqrt(ss);
    if (norms) norms[row] = nrm;
    /* rotate: u = H (s .* v) [PR15 M4A "rotate = H.D.x"] */
    for (int i = 0; i < m; ++i) u[i] = (double)s[i] * v[i];
    fwht(u, m);
    /* scale to unit-variance units, quantise to the nearest centroid (ties to the lower cell) */
    for (int i = 0; i < m; ++i) {
      double z = nrm > 0.0 ? u[i] / nrm : 0.0;
      int cnt = 0;
      double dmin = INFINITY;
      for (int k = 0; k + 1 < L; ++k) {
        if (z > (double)t[k]) ++cnt;
        double d = fabs(z - (double)t[k]);
        if (d < dmin) dmin = d;
      }
      code[i] = (uint8_t)cnt;
      uint8_t fl = (dmin < NEAR) ? FLAG_NEAR_BOUNDARY : 0u;
      if (cd->T > 0.0 && fabs(fabs(z) - cd->T) < NEAR) fl |= FLAG_NEAR_T;
      if (flags) flags[row * m + i] = fl;
      if (codes) codes[row * m + i] = code[i];
      if (zout) zout[row * m + i] = z;
      /* outlier side list, ascending coordinate within the vector [PR15 OL] */
      if (cd->T > 0.0 && fabs(z) > cd->T) {
        if (total < ol_cap) {
          if (ol_idx) ol_idx[total] = (uint16_t)i;
          if (ol_val) ol_val[total] = float_to_bf16_rne((float)z);
        }
        ++total;
      }
    }
    if (ol_off) ol_off[row + 1] = (uint32_t)total;
    /* stored scale. Decode gives x^ = (scale/m) s .* H z^, so ||x^||^2 = scale^2 ||z^||^2 / m and
     * <x^, v> = (scale/m) ||v|| <z, z^>. The rules [turboquant_plus log: EDEN and matched-norm
     * scales]: 1 matched norm, ||x^|| = ||v||; 2 inner-product preserving (EDEN's S), <x^, v> =
     * ||v||^2; 3 least-squares optimal (the per-vector MSE minimum), <v - x^, x^> = 0. */
    double scale = nrm;
    if (cd->scale_rule != 0 && nrm > 0.0) {
      double zz = 0.0, zh2 = 0.0;
      for (int i = 0; i < m; ++i) {
        const double zh = (double)cd->centroids[code[i]];
        zz += (u[i] / nrm) * zh;
        zh2 += zh * zh;
      }
      /* a rule whose denominator is not positive keeps the plain norm */
      if (cd->scale_rule == 1 && zh2 > 0.0) scale = nrm * sqrt((double)m / zh2);
      else if (cd->scale_rule == 2 && zz > 0.0) scale = nrm * (double)m / zz;
      else if (cd->scale_rule == 3 && zh2 > 0.0) scale = nrm * zz / zh2;
    }
    if (records) pack_record(code, m, b, (float)scale, records + row * rb);
  }
  return total;
}

/* Decode n records into y[n][D] (f64) [PR15 M5]: z^_i = centroid[code_i], outlier entries
 * override their coordinate, v^ = norm * s .* (H z^) / m, then x^ = mu + B v^ (PCA). */
void kvq_ref_decode(const ref_codec* cd, int64_t n, const uint8_t* records,
                    const uint32_t* ol_off, const uint16_t* ol_idx, const uint16_t* ol_val,
                    int64_t ol_cap, double* y) {
  const int D = cd->D, b = cd->bits;
  const int m = cd->r > 0 ? cd->r : D;
  const int rb = kvq_ref_record_bytes(m, b);
  int8_t s[512];
  kvq_ref_signs(cd->seed, m, s);
  uint8_t code[512];
  double w[512];
  for (int64_t row = 0; row < n; ++row) {
    float nrm32;
    kvq_ref_unpack_codes(m, b, records + row * rb, code, &nrm32);
    for (int i = 0; i < m; ++i) w[i] = (double)cd->centroids[code[i]];
    if (ol_off) {
      for (int64_t e = ol_off[row]; e < (int64_t)ol_off[row + 1] && e < ol_cap; ++e)
        w[ol_idx[e]] = bf16_to_double(ol_val[e]);
    }
    fwht(w, m);
    double* yr = y + row * D;
    if (cd->r > 0) {
      /* x^ = mu + C v^, C the decode basis (the projection basis itself unless a separate one
         is given) */
      const uint16_t* C = cd->unbasis ? cd->unbasis : cd->basis;
      double vh[512];
      for (int i = 0; i < m; ++i) vh[i] = (double)nrm32 * (double)s[i] * w[i] / m;
      for (int d = 0; d < D; ++d) {
        double acc = cd->mean ? (double)cd->mean[d] : 0.0;
        for (int j = 0; j < m; ++j) acc += bf16_to_double(C[(int64_t)d * m + j]) * vh[j];
        yr[d] = acc;
      }
    } else {
      for (int i = 0; i < m; ++i) yr[i] = (double)nrm32 * (double)s[i] * w[i] / m;
    }
  }
}

/* Score of n (query, record) pairs by the plain definition: q . decode(record), f64.
 * q: bf16 [n][D]; records: n records back to back. No outliers (the packed score reads codes
 * and norms only). [arc PR #94 kernel commit: attention over packed K] */
void kvq_ref_score(const ref_codec* cd, int64_t n, const uint16_t* q, const uint8_t* records,
                   double* out) {
  const int D = cd->D;
  const int m = cd->r > 0 ? cd->r : D;
  const int rb = kvq_ref_record_bytes(m, cd->bits);
  double y[512];
  for (int64_t k = 0; k < n; ++k) {
    kvq_ref_decode(cd, 1, records + k * rb, NULL, NULL, NULL, 0, y);
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += bf16_to_double(q[k * D + d]) * y[d];
    out[k] = acc;
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Lloyd-Max table refitted to a sample [kakeyaturbo PR #15, calibration-artefacts commit: the  */
/* table refitted to the codec's own post-rotation coordinates, MSE below the Gaussian table's; */
/* LARQL TQ: the same two optimality conditions with the sample's distribution in place of      */
/* N(0,1)]. One iteration: the f32 thresholds of the current f32 table (midpoints of adjacent   */
/* centroids, as the quantiser uses them), each sample z in the cell #{k : z > t_k}, each       */
/* centroid replaced by the f64 mean of its cell, rounded to f32 (the stored table). An empty   */
/* cell keeps its centroid. `iters` iterations in place on c32 (ascending, L entries).          */
void kvq_ref_lloyd_fit(const double* z, int64_t n, int L, int iters, float* c32) {
  float t[255];
  double sum[256];
  int64_t cnt[256];
  for (int it = 0; it < iters; ++it) {
    kvq_ref_thresholds(c32, L, t);
    for (int k = 0; k < L; ++k) {
      sum[k] = 0.0;
      cnt[k] = 0;
    }
    for (int64_t i = 0; i < n; ++i) {
      int code = 0;
      for (int k = 0; k + 1 < L; ++k)
        if (z[i] > (double)t[k]) ++code;
      sum[code] += z[i];
      ++cnt[code];
    }
    for (int k = 0; k < L; ++k)
      if (cnt[k] > 0) c32[k] = (float)(sum[k] / (double)cnt[k]);
  }
}

/* Mean squared quantisation error of the samples under the f32 table c32 (cells as above). */
double kvq_ref_table_mse(const double* z, int64_t n, int L, const float* c32) {
  float t[255];
  kvq_ref_thresholds(c32, L, t);
  double acc = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    int code = 0;
    for (int k = 0; k + 1 < L; ++k)
      if (z[i] > (double)t[k]) ++code;
    const double d = z[i] - (double)c32[code];
    acc += d * d;
  }
  return n > 0 ? acc / (double)n : 0.0;
}
