/*
 * synth.c - seeded synthetic inputs for the DSA / CSA path.
 *
 * This module only draws random numbers and stores them in the dtypes the path consumes
 * (fp32, bf16, MXFP4). It holds none of the method's arithmetic and is the one piece of code
 * shared by the CPU oracle and the GPU path: both read the bytes written here.
 *
 * Generator (counter based, so any element can be regenerated on its own, for any thread count):
 *   splitmix64(x): the SplitMix64 finaliser (Steele, Lea, Flood, "Fast splittable pseudorandom
 *                  number generators", OOPSLA 2014), applied to x + golden-gamma.
 *   stream key   : key = splitmix64(splitmix64(seed) ^ tensor_id)
 *   raw word     : r(i, j) = splitmix64(key + 2*i + j),  j in {0, 1}
 *   uniform      : U(i, j) = (r(i, j) >> 11) * 2^-53  in [0, 1)
 *   normal       : Box-Muller, z(i) = sqrt(-2 ln(1 - U(i,0))) * cos(2 pi U(i,1))
 * Values are formed in fp64 and rounded once (round-to-nearest-even) to the stored dtype.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t splitmix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tensor_id) {
  return splitmix64(splitmix64(seed) ^ tensor_id);
}

static inline double unif(uint64_t key, int64_t i, int j) {
  uint64_t r = splitmix64(key + 2u * (uint64_t)i + (uint64_t)j);
  return (double)(r >> 11) * 0x1.0p-53;
}

static inline double normal(uint64_t key, int64_t i) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = 1.0 - unif(key, i, 0); /* (0, 1] */
  double u2 = unif(key, i, 1);
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

/* fp64 -> bf16 bits with a single round-to-nearest-even (no double rounding through fp32).
 * Normal bf16 range is exact; magnitudes below the smallest normal go through fp32. */
uint16_t synth_bf16_from_double(double x) {
  if (x != x) return 0x7FC0;
  if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
  double ax = fabs(x);
  if (ax < 0x1.0p-126) {
    float f = (float)x; /* subnormal bf16 region: never produced by the workloads */
    uint32_t b;
    memcpy(&b, &f, 4);
    uint32_t lsb = (b >> 16) & 1u;
    b += 0x7FFFu + lsb;
    return (uint16_t)(b >> 16);
  }
  int e;
  double mant = frexp(ax, &e);        /* ax = mant * 2^e, mant in [0.5, 1) */
  double r = nearbyint(ldexp(mant, 8)); /* 8 significant bits, RNE (default rounding mode) */
  double v = ldexp(r, e - 8);
  if (v > 0x1.FEp127) return signbit(x) ? 0xFF80 : 0x7F80; /* overflow -> inf */
  float f = (float)(signbit(x) ? -v : v); /* exact: v has 8 significant bits */
  uint32_t b;
  memcpy(&b, &f, 4);
  return (uint16_t)(b >> 16);
}

void synth_normal_f32(uint64_t seed, uint64_t tensor_id, int64_t start, int64_t count,
                      double scale, float* out) {
  uint64_t key = stream_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = (float)(scale * normal(key, start + i));
}

void synth_normal_bf16(uint64_t seed, uint64_t tensor_id, int64_t start, int64_t count,
                       double scale, uint16_t* out) {
  uint64_t key = stream_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = synth_bf16_from_double(scale * normal(key, start + i));
}

void synth_uniform_f32(uint64_t seed, uint64_t tensor_id, int64_t start, int64_t count,
                       double lo, double hi, float* out) {
  uint64_t key = stream_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = (float)(lo + (hi - lo) * unif(key, start + i, 0));
}

/* Magnitude of e2m1 -> code (0..7) with round-to-nearest-even on the grid
 * {0, 0.5, 1, 1.5, 2, 3, 4, 6}; saturates at 6. "Even" = code with LSB 0. */
static int e2m1_code(double a) {
  if (a < 0.25) return 0;
  if (a == 0.25) return 0;
  if (a < 0.75) return 1;
  if (a <= 1.25) return 2; /* 0.75 -> 1.0 (even), 1.25 -> 1.0 (even) */
  if (a < 1.75) return 3;
  if (a <= 2.5) return 4;  /* 1.75 -> 2.0 (even), 2.5 -> 2.0 (even) */
  if (a < 3.5) return 5;
  if (a <= 5.0) return 6;  /* 3.5 -> 4.0 (even), 5.0 -> 4.0 (even) */
  return 7;
}

/* Quantise one block of 32 fp64 values to MXFP4: shared E8M0 exponent e with
 * 2^e = 2^(floor(log2(amax)) - 2) (so amax / 2^e lies in [4, 8) and the largest
 * magnitudes saturate at 6), then RNE of x / 2^e onto the e2m1 grid. */
void synth_mxfp4_block(const double* x, uint8_t* codes16, uint8_t* scale) {
  double amax = 0.0;
  for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(x[i]));
  int e;
  if (amax == 0.0) {
    e = -127;
  } else {
    int k;
    frexp(amax, &k); /* amax = f * 2^k, f in [0.5, 1): floor(log2 amax) = k - 1 */
    e = k - 1 - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
  }
  *scale = (uint8_t)(e + 127);
  for (int i = 0; i < 32; i += 2) {
    uint8_t nib[2];
    for (int h = 0; h < 2; ++h) {
      double v = ldexp(x[i + h], -e);
      int c = e2m1_code(fabs(v));
      nib[h] = (uint8_t)(c | (v < 0 ? 8 : 0));
    }
    codes16[i / 2] = (uint8_t)(nib[0] | (nib[1] << 4));
  }
}

/* MXFP4 rows of N(0,1)*scale: row r, column d uses element index r*D + d (the same element the
 * bf16 generator would use for a [rows, D] tensor). codes: [rows, D/2]; scales: [rows, D/32]. */
void synth_normal_mxfp4(uint64_t seed, uint64_t tensor_id, int64_t start_row, int64_t rows,
                        int D, double scale, uint8_t* codes, uint8_t* scales) {
  uint64_t key = stream_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double blk[32];
    for (int b = 0; b < D / 32; ++b) {
      for (int i = 0; i < 32; ++i)
        blk[i] = scale * normal(key, (start_row + r) * (int64_t)D + b * 32 + i);
      synth_mxfp4_block(blk, codes + r * (int64_t)(D / 2) + b * 16, scales + r * (int64_t)(D / 32) + b);
    }
  }
}

/* Raw words, for generator self-tests. */
/* |a| -> e4m3 (OCP E4M3FN) code 0..0x7E, round-to-nearest-even, saturating at 448. */
static int e4m3_code(double a) {
  if (a >= 448.0) return 0x7E;
  if (a < ldexp(1.0, -6)) {               /* subnormal grid: multiples of 2^-9 */
    double n = rint(a * 512.0);            /* 0 .. 8; 8 is the smallest normal */
    return (int)n;                          /* code 8 == exponent field 1, mantissa 0 */
  }
  int k;
  frexp(a, &k);                            /* a = f 2^k, f in [0.5, 1) */
  int e = k - 1;                           /* floor(log2 a), -6 .. 8 */
  double n = rint(ldexp(a, 3 - e));        /* 8 .. 16 on the grid 2^(e-3) */
  if (n == 16.0) {
    e += 1;
    n = 8.0;
  }
  if (e > 8 || (e == 8 && n > 14.0)) return 0x7E;
  return ((e + 7) << 3) | ((int)n - 8);
}

/* One MXFP8 block: 32 values -> 32 e4m3 codes + one E8M0 scale (OCP MX: scale
 * 2^(floor(log2 amax) - 8), the largest e4m3 binade, magnitudes saturating at 448). */
void synth_mxfp8_block(const double* x, uint8_t* codes32, uint8_t* scale) {
  double amax = 0.0;
  for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(x[i]));
  int e;
  if (amax == 0.0) {
    e = -127;
  } else {
    int k;
    frexp(amax, &k);
    e = k - 1 - 8;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
  }
  *scale = (uint8_t)(e + 127);
  for (int i = 0; i < 32; ++i) {
    double v = ldexp(x[i], -e);
    codes32[i] = (uint8_t)(e4m3_code(fabs(v)) | (v < 0 ? 0x80 : 0));
  }
}

void synth_normal_mxfp8(uint64_t seed, uint64_t tensor_id, int64_t start_row, int64_t rows,
                        int D, double scale, uint8_t* codes, uint8_t* scales) {
  const uint64_t key = stream_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double blk[32];
    for (int b = 0; b < D / 32; ++b) {
      for (int i = 0; i < 32; ++i) blk[i] = scale * normal(key, (start_row + r) * (int64_t)D + 32 * b + i);
      synth_mxfp8_block(blk, codes + r * (int64_t)D + 32 * b, scales + r * (int64_t)(D / 32) + b);
    }
  }
}

uint64_t synth_splitmix64(uint64_t x) { return splitmix64(x); }
double synth_uniform_at(uint64_t seed, uint64_t tensor_id, int64_t i, int j) {
  return unif(stream_key(seed, tensor_id), i, j);
}
double synth_normal_at(uint64_t seed, uint64_t tensor_id, int64_t i) {
  return normal(stream_key(seed, tensor_id), i);
}
