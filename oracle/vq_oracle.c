/*
 * CPU oracle for the VQ dequantize-and-multiply path.  TEST INFRASTRUCTURE ONLY (see
 * vq_oracle.h): slow, plain and independent of the HIP library.  Built with
 *   gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off
 * so that every float operation below is one IEEE operation rounded to nearest-even,
 * with subnormals kept.
 *
 * Sources on the pages this follows:
 *   - VPTQ guide (aifetchly), "The Information-Theoretic Superiority of Vector
 *     Quantization": a vector of v adjacent weights is replaced by a centroid of a
 *     K-entry codebook, its index costs log2(K) bits.
 *   - VPTQ guide, "2. Multi-Stage Residual Vector Quantization (RVQ)": the decoded
 *     vector is the main centroid plus the residual centroid.
 *   - VPTQ guide, "Step 2" (dequantize: gather both books, add, view as [out, in])
 *     and "Step 3" (forward: y = x W^T + bias).
 *   - Production-VQ post (llms.blog), QuIP# "per-channel scaling": a scale per output
 *     channel multiplies the rebuilt vector.
 */
#define _POSIX_C_SOURCE 200809L
#include "vq_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ---------------------------------------------------------------- number formats */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double val;
  if (e == 0) {
    val = ldexp((double)f, -24); /* subnormal: f * 2^-14 / 2^10 */
  } else if (e == 31) {
    val = f ? NAN : INFINITY;
  } else {
    val = ldexp((double)(1024 + f), e - 15 - 10); /* (1 + f/2^10) * 2^(e-15) */
  }
  return sign ? -val : val;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t b) {
  int sign = (b >> 15) & 1;
  int e = (b >> 7) & 0xff;
  int f = b & 0x7f;
  double val;
  if (e == 0) {
    val = ldexp((double)f, -126 - 7);
  } else if (e == 255) {
    val = f ? NAN : INFINITY;
  } else {
    val = ldexp((double)(128 + f), e - 127 - 7);
  }
  return sign ? -val : val;
}

/* Round |a| to a multiple of the quantum q, ties to an even multiple.  a/q is exact
 * because a carries at most 24 significant bits and q is a power of two. */
static double round_to_quantum_even(double a, double q) {
  double n = a / q;
  double fl = floor(n);
  double fr = n - fl;
  double r;
  if (fr > 0.5) {
    r = fl + 1.0;
  } else if (fr < 0.5) {
    r = fl;
  } else {
    r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
  }
  return r * q;
}

/* Generic RNE to a binary format with `mbits` fraction bits and exponent range
 * [emin, emax] (normal numbers), then encoded. */
static uint16_t encode_rne(double x, int mbits, int emin, int emax, int ebias, int ebits) {
  uint16_t sign = signbit(x) ? (uint16_t)0x8000 : (uint16_t)0;
  uint16_t exp_all_ones = (uint16_t)(((1 << ebits) - 1) << mbits);
  if (isnan(x)) return (uint16_t)(exp_all_ones | (1u << (mbits - 1)));
  double a = fabs(x);
  double maxfin = ldexp(2.0 - ldexp(1.0, -mbits), emax);
  double overflow_mid = ldexp(2.0 - ldexp(1.0, -mbits - 1), emax);
  if (a >= overflow_mid) return (uint16_t)(sign | exp_all_ones); /* tie goes to even = infinity */
  double q;
  if (a < ldexp(1.0, emin)) {
    q = ldexp(1.0, emin - mbits);
  } else {
    int e2;
    frexp(a, &e2); /* a in [2^(e2-1), 2^e2) */
    q = ldexp(1.0, (e2 - 1) - mbits);
  }
  double r = round_to_quantum_even(a, q);
  if (r > maxfin) return (uint16_t)(sign | exp_all_ones);
  if (r == 0.0) return sign;
  if (r < ldexp(1.0, emin)) {
    return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, emin - mbits)));
  }
  int e2;
  double fr = frexp(r, &e2); /* r = fr * 2^e2, fr in [0.5, 1) */
  int E = e2 - 1;
  uint16_t mant = (uint16_t)((fr * 2.0 - 1.0) * ldexp(1.0, mbits));
  return (uint16_t)(sign | (uint16_t)((E + ebias) << mbits) | mant);
}

uint16_t oracle_f64_to_f16_rne(double x) { return encode_rne(x, 10, -14, 15, 15, 5); }
uint16_t oracle_f64_to_bf16_rne(double x) { return encode_rne(x, 7, -126, 127, 127, 8); }

void oracle_f32_to_f16_rne_array(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_f16_rne((double)in[i]);
}
void oracle_f32_to_bf16_rne_array(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_bf16_rne((double)in[i]);
}

/* ---------------------------------------------------------------- layout */

static int valid_desc(int64_t n, int64_t in_features, int v, int bits1, int bits2) {
  if (n < 0 || in_features < 0) return 0;
  if (v < 1 || v > 16) return 0;
  if (bits1 < 1 || bits1 > 16) return 0;
  if (bits2 < 0 || bits2 > 16) return 0;
  return 1;
}

static int64_t num_vectors(int64_t in_features, int v) { return (in_features + v - 1) / v; }

int64_t oracle_row_stride(int64_t in_features, int v, int bits) {
  if (bits == 0) return 0;
  int64_t bits_per_row = num_vectors(in_features, v) * (int64_t)bits;
  return 16 * ((bits_per_row + 127) / 128);
}

int64_t oracle_packed_bytes(int64_t n, int64_t in_features, int v, int bits1, int bits2) {
  if (!valid_desc(n, in_features, v, bits1, bits2)) return -1;
  return n * (oracle_row_stride(in_features, v, bits1) + oracle_row_stride(in_features, v, bits2));
}

/* Bit k of a row is bit (k mod 8) of byte floor(k/8). */
static int get_bit(const uint8_t* row, int64_t k) { return (row[k >> 3] >> (k & 7)) & 1; }
static void set_bit(uint8_t* row, int64_t k) { row[k >> 3] = (uint8_t)(row[k >> 3] | (1u << (k & 7))); }

/* Field j (B bits, LSB first) of a row, read one bit at a time. */
static uint32_t read_field(const uint8_t* row, int64_t j, int bits) {
  uint32_t val = 0;
  for (int q = 0; q < bits; ++q) {
    if (get_bit(row, j * bits + q)) val |= (uint32_t)1 << q;
  }
  return val;
}

int oracle_pack(int64_t n, int64_t in_features, int v, int bits1, int bits2, const uint32_t* idx1,
                const uint32_t* idx2, uint8_t* out, int64_t out_bytes) {
  if (!valid_desc(n, in_features, v, bits1, bits2)) return ORACLE_BAD_ARGS;
  if ((n > 0 && in_features > 0) && (!idx1 || (bits2 > 0 && !idx2) || !out)) return ORACLE_BAD_ARGS;
  int64_t need = oracle_packed_bytes(n, in_features, v, bits1, bits2);
  if (out_bytes < need) return ORACLE_BUFFER_SMALL;
  int64_t nv = num_vectors(in_features, v);
  for (int stream = 1; stream <= 2; ++stream) {
    int bits = stream == 1 ? bits1 : bits2;
    if (bits == 0) continue;
    const uint32_t* idx = stream == 1 ? idx1 : idx2;
    for (int64_t i = 0; i < n * nv; ++i)
      if (idx[i] >> bits) return ORACLE_INDEX_RANGE;
  }
  memset(out, 0, (size_t)need);
  int64_t s1 = oracle_row_stride(in_features, v, bits1);
  int64_t s2 = oracle_row_stride(in_features, v, bits2);
  for (int stream = 1; stream <= 2; ++stream) {
    int bits = stream == 1 ? bits1 : bits2;
    if (bits == 0) continue;
    const uint32_t* idx = stream == 1 ? idx1 : idx2;
    for (int64_t o = 0; o < n; ++o) {
      uint8_t* row = stream == 1 ? out + o * s1 : out + n * s1 + o * s2;
      for (int64_t j = 0; j < nv; ++j) {
        uint32_t val = idx[o * nv + j];
        for (int q = 0; q < bits; ++q)
          if ((val >> q) & 1u) set_bit(row, j * bits + q);
      }
    }
  }
  return ORACLE_OK;
}

int oracle_unpack(int64_t n, int64_t in_features, int v, int bits1, int bits2, const uint8_t* packed,
                  uint32_t* idx1, uint32_t* idx2) {
  if (!valid_desc(n, in_features, v, bits1, bits2)) return ORACLE_BAD_ARGS;
  int64_t nv = num_vectors(in_features, v);
  int64_t s1 = oracle_row_stride(in_features, v, bits1);
  int64_t s2 = oracle_row_stride(in_features, v, bits2);
  int pad_set = 0;
  for (int stream = 1; stream <= 2; ++stream) {
    int bits = stream == 1 ? bits1 : bits2;
    if (bits == 0) continue;
    uint32_t* idx = stream == 1 ? idx1 : idx2;
    int64_t stride = stream == 1 ? s1 : s2;
    for (int64_t o = 0; o < n; ++o) {
      const uint8_t* row = stream == 1 ? packed + o * s1 : packed + n * s1 + o * s2;
      for (int64_t j = 0; j < nv; ++j) idx[o * nv + j] = read_field(row, j, bits);
      for (int64_t k = nv * bits; k < stride * 8; ++k)
        if (get_bit(row, k)) pad_set = 1;
    }
  }
  return pad_set ? ORACLE_PAD_NONZERO : ORACLE_OK;
}

/* ---------------------------------------------------------------- dequant + product */

typedef struct {
  int64_t n, in_features;
  int v, bits1, bits2;
  const uint8_t* packed;
  const uint16_t* cb1;
  const uint16_t* cb2;
  const uint16_t* scale;
  const uint16_t* bias;
  const double* xd; /* [M][in] decoded activations, NULL for dequant-only */
  int64_t M;
  const int64_t* rows;
  int64_t nrows;
  const uint16_t* lat_a; /* affine-lattice decode: A [4][4] fp16 bits, NULL for codebooks */
  const uint16_t* lat_b; /* affine-lattice decode: B [4] fp16 bits */
  float* w_out;  /* dequant-only: [nrows][in] */
  double* y_out; /* forward: [M][nrows] */
  int64_t begin, end;
} job_t;

/* One row of W in fp32, following the decode order: sum the two centroids in fp32,
 * then multiply by the channel scale in fp32. */
static void dequant_row(const job_t* jb, int64_t o, float* wrow) {
  int64_t nv = num_vectors(jb->in_features, jb->v);
  int64_t s1 = oracle_row_stride(jb->in_features, jb->v, jb->bits1);
  int64_t s2 = oracle_row_stride(jb->in_features, jb->v, jb->bits2);
  const uint8_t* row1 = jb->packed + o * s1;
  const uint8_t* row2 = jb->packed + jb->n * s1 + o * s2;
  float s = jb->scale ? (float)oracle_f16_to_f64(jb->scale[o]) : 1.0f;
  for (int64_t j = 0; j < nv; ++j) {
    uint32_t i1 = read_field(row1, j, jb->bits1);
    uint32_t i2 = jb->bits2 ? read_field(row2, j, jb->bits2) : 0;
    for (int t = 0; t < jb->v; ++t) {
      int64_t col = j * jb->v + t;
      if (col >= jb->in_features) break; /* tail lanes of the last vector are dropped */
      float c1 = (float)oracle_f16_to_f64(jb->cb1[(int64_t)i1 * jb->v + t]);
      float w;
      if (jb->bits2) {
        float c2 = (float)oracle_f16_to_f64(jb->cb2[(int64_t)i2 * jb->v + t]);
        w = c1 + c2;
      } else {
        w = c1; /* no residual: no add, so a -0 centroid stays -0 */
      }
      if (jb->scale) w = w * s;
      wrow[col] = w;
    }
  }
}

/* One row of W for the affine lattice (UniSVQ summary, "Mathematical Formulation":
 * Phi(w) = A w + B over integer grid coordinates; "Efficiency": d = 4, 2 bits per
 * coordinate).  The 8-bit field of vector j holds its four 2-bit codes, code u in bits
 * [2u, 2u + 2); the code value itself is the integer coordinate q_u (reading taken: the
 * pages do not say how the integers are stored).  Coordinate t of the vector is
 * B[t] + sum_u A[t][u] q_u, summed in double, where every term (an fp16 value times an
 * integer below 4) and every partial sum is exact, then rounded once to fp32; the
 * channel scale then multiplies it in fp32. */
static void dequant_row_lattice(const job_t* jb, int64_t o, float* wrow) {
  int64_t nv = num_vectors(jb->in_features, 4);
  int64_t stride = oracle_row_stride(jb->in_features, 4, 8);
  const uint8_t* row = jb->packed + o * stride;
  float s = jb->scale ? (float)oracle_f16_to_f64(jb->scale[o]) : 1.0f;
  for (int64_t j = 0; j < nv; ++j) {
    uint32_t field = read_field(row, j, 8);
    int q[4];
    for (int u = 0; u < 4; ++u) q[u] = (int)((field >> (2 * u)) & 3u);
    for (int t = 0; t < 4; ++t) {
      int64_t col = j * 4 + t;
      if (col >= jb->in_features) break; /* tail lanes of the last vector are dropped */
      double acc = oracle_f16_to_f64(jb->lat_b[t]);
      for (int u = 0; u < 4; ++u) acc += oracle_f16_to_f64(jb->lat_a[t * 4 + u]) * (double)q[u];
      float w = (float)acc;
      if (jb->scale) w = w * s;
      wrow[col] = w;
    }
  }
}

static void* worker(void* arg) {
  job_t* jb = (job_t*)arg;
  float* wrow = NULL;
  if (jb->y_out) {
    wrow = (float*)malloc(sizeof(float) * (size_t)(jb->in_features > 0 ? jb->in_features : 1));
    if (!wrow) return (void*)1;
  }
  for (int64_t r = jb->begin; r < jb->end; ++r) {
    int64_t o = jb->rows ? jb->rows[r] : r;
    if (!jb->y_out) {
      if (jb->lat_a)
        dequant_row_lattice(jb, o, jb->w_out + r * jb->in_features);
      else
        dequant_row(jb, o, jb->w_out + r * jb->in_features);
      continue;
    }
    if (jb->lat_a)
      dequant_row_lattice(jb, o, wrow);
    else
      dequant_row(jb, o, wrow);
    double b = jb->bias ? oracle_f16_to_f64(jb->bias[o]) : 0.0;
    for (int64_t m = 0; m < jb->M; ++m) {
      const double* xm = jb->xd + m * jb->in_features;
      double acc = 0.0;
      for (int64_t col = 0; col < jb->in_features; ++col) acc += xm[col] * (double)wrow[col];
      jb->y_out[m * jb->nrows + r] = acc + b;
    }
  }
  free(wrow);
  return NULL;
}

static int run_jobs(job_t* proto, int nthreads) {
  if (nthreads <= 0) {
    long c = sysconf(_SC_NPROCESSORS_ONLN);
    nthreads = c > 0 ? (int)c : 1;
  }
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > proto->nrows) nthreads = proto->nrows > 0 ? (int)proto->nrows : 1;
  job_t jobs[256];
  pthread_t th[256];
  int started[256];
  int64_t per = (proto->nrows + nthreads - 1) / nthreads;
  int rc = ORACLE_OK;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = *proto;
    jobs[t].begin = t * per;
    jobs[t].end = (t + 1) * per < proto->nrows ? (t + 1) * per : proto->nrows;
    started[t] = 0;
    if (jobs[t].begin >= jobs[t].end) continue;
    if (nthreads == 1) {
      if (worker(&jobs[t])) rc = ORACLE_BAD_ARGS;
    } else if (pthread_create(&th[t], NULL, worker, &jobs[t]) == 0) {
      started[t] = 1;
    } else if (worker(&jobs[t])) {
      rc = ORACLE_BAD_ARGS;
    }
  }
  for (int t = 0; t < nthreads; ++t) {
    if (!started[t]) continue;
    void* ret = NULL;
    pthread_join(th[t], &ret);
    if (ret) rc = ORACLE_BAD_ARGS;
  }
  return rc;
}

static int check_rows(int64_t n, const int64_t* rows, int64_t nrows) {
  if (!rows) return nrows == n;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= n) return 0;
  return 1;
}

int oracle_dequant_rows(int64_t n, int64_t in_features, int v, int bits1, int bits2, const uint8_t* packed,
                        const uint16_t* cb1, const uint16_t* cb2, const uint16_t* scale, const int64_t* rows,
                        int64_t nrows, float* w, int nthreads) {
  if (!valid_desc(n, in_features, v, bits1, bits2)) return ORACLE_BAD_ARGS;
  if (!rows) nrows = n;
  if (!check_rows(n, rows, nrows)) return ORACLE_BAD_ARGS;
  if (nrows == 0 || in_features == 0) return ORACLE_OK;
  if (!packed || !cb1 || (bits2 && !cb2) || !w) return ORACLE_BAD_ARGS;
  job_t proto;
  memset(&proto, 0, sizeof proto);
  proto.n = n;
  proto.in_features = in_features;
  proto.v = v;
  proto.bits1 = bits1;
  proto.bits2 = bits2;
  proto.packed = packed;
  proto.cb1 = cb1;
  proto.cb2 = cb2;
  proto.scale = scale;
  proto.rows = rows;
  proto.nrows = nrows;
  proto.w_out = w;
  return run_jobs(&proto, nthreads);
}

int oracle_forward_rows(int64_t n, int64_t in_features, int v, int bits1, int bits2, const uint8_t* packed,
                        const uint16_t* cb1, const uint16_t* cb2, const uint16_t* scale, const uint16_t* bias,
                        const uint16_t* x, int x_is_bf16, int64_t M, const int64_t* rows, int64_t nrows,
                        double* y, int nthreads) {
  if (!valid_desc(n, in_features, v, bits1, bits2) || M < 0) return ORACLE_BAD_ARGS;
  if (!rows) nrows = n;
  if (!check_rows(n, rows, nrows)) return ORACLE_BAD_ARGS;
  if (nrows == 0 || M == 0) return ORACLE_OK;
  if (!y) return ORACLE_BAD_ARGS;
  if (in_features > 0 && (!packed || !cb1 || (bits2 && !cb2) || !x)) return ORACLE_BAD_ARGS;
  double* xd = (double*)malloc(sizeof(double) * (size_t)(M * in_features > 0 ? M * in_features : 1));
  if (!xd) return ORACLE_BAD_ARGS;
  for (int64_t i = 0; i < M * in_features; ++i)
    xd[i] = x_is_bf16 ? oracle_bf16_to_f64(x[i]) : oracle_f16_to_f64(x[i]);
  job_t proto;
  memset(&proto, 0, sizeof proto);
  proto.n = n;
  proto.in_features = in_features;
  proto.v = v;
  proto.bits1 = bits1;
  proto.bits2 = bits2;
  proto.packed = packed;
  proto.cb1 = cb1;
  proto.cb2 = cb2;
  proto.scale = scale;
  proto.bias = bias;
  proto.xd = xd;
  proto.M = M;
  proto.rows = rows;
  proto.nrows = nrows;
  proto.y_out = y;
  int rc = run_jobs(&proto, nthreads);
  free(xd);
  return rc;
}

/* ---------------------------------------------------------------- affine lattice entry points */

int oracle_svq_dequant_rows(int64_t n, int64_t in_features, const uint8_t* packed, const uint16_t* a,
                            const uint16_t* b, const uint16_t* scale, const int64_t* rows, int64_t nrows, float* w,
                            int nthreads) {
  if (n < 0 || in_features < 0) return ORACLE_BAD_ARGS;
  if (!rows) nrows = n;
  if (!check_rows(n, rows, nrows)) return ORACLE_BAD_ARGS;
  if (nrows == 0 || in_features == 0) return ORACLE_OK;
  if (!packed || !a || !b || !w) return ORACLE_BAD_ARGS;
  job_t proto;
  memset(&proto, 0, sizeof proto);
  proto.n = n;
  proto.in_features = in_features;
  proto.v = 4;
  proto.bits1 = 8;
  proto.packed = packed;
  proto.lat_a = a;
  proto.lat_b = b;
  proto.scale = scale;
  proto.rows = rows;
  proto.nrows = nrows;
  proto.w_out = w;
  return run_jobs(&proto, nthreads);
}

int oracle_svq_forward_rows(int64_t n, int64_t in_features, const uint8_t* packed, const uint16_t* a,
                            const uint16_t* b, const uint16_t* scale, const uint16_t* bias, const uint16_t* x,
                            int x_is_bf16, int64_t M, const int64_t* rows, int64_t nrows, double* y, int nthreads) {
  if (n < 0 || in_features < 0 || M < 0) return ORACLE_BAD_ARGS;
  if (!rows) nrows = n;
  if (!check_rows(n, rows, nrows)) return ORACLE_BAD_ARGS;
  if (nrows == 0 || M == 0) return ORACLE_OK;
  if (!y) return ORACLE_BAD_ARGS;
  if (in_features > 0 && (!packed || !a || !b || !x)) return ORACLE_BAD_ARGS;
  double* xd = (double*)malloc(sizeof(double) * (size_t)(M * in_features > 0 ? M * in_features : 1));
  if (!xd) return ORACLE_BAD_ARGS;
  for (int64_t i = 0; i < M * in_features; ++i)
    xd[i] = x_is_bf16 ? oracle_bf16_to_f64(x[i]) : oracle_f16_to_f64(x[i]);
  job_t proto;
  memset(&proto, 0, sizeof proto);
  proto.n = n;
  proto.in_features = in_features;
  proto.v = 4;
  proto.bits1 = 8;
  proto.packed = packed;
  proto.lat_a = a;
  proto.lat_b = b;
  proto.scale = scale;
  proto.bias = bias;
  proto.xd = xd;
  proto.M = M;
  proto.rows = rows;
  proto.nrows = nrows;
  proto.y_out = y;
  int rc = run_jobs(&proto, nthreads);
  free(xd);
  return rc;
}

/* ---------------------------------------------------------------- randomized Hadamard transform */

/* Block of the transform: the largest power of two that divides n, at most 16384. */
int64_t oracle_rht_block(int64_t n) {
  if (n <= 0) return 0;
  int64_t b = 1;
  while (b < 16384 && n % (2 * b) == 0) b *= 2;
  return b;
}

static int popcount64(uint64_t v) {
  int c = 0;
  while (v) {
    v &= v - 1;
    ++c;
  }
  return c;
}

/* Randomized Walsh-Hadamard transform of each row of x (production-VQ post, QuIP#: random
 * orthogonal Hadamard transforms with random signs on the layer's inputs; sub-4-bit
 * lecture, "QuIP#: Incoherence Processing": Hadamard + random signs; UniSVQ summary,
 * "Preprocessing (Randomized Hadamard Transform - RHT)").  With b = oracle_rht_block(n),
 * each block of b columns is transformed on its own (the transform is I kron H_b / sqrt(b)
 * with random signs): forward y = H_b (s . x) / sqrt(b), transpose y = s . (H_b x) / sqrt(b),
 * where H_b[i][j] = (-1)^popcount(i & j) and s_j = -1 when bit j (LSB-first within byte j/8)
 * of signs is set.  Written out as the matrix product, O(b) per output. */
int oracle_rht(int64_t M, int64_t n, const double* x, const uint8_t* signs, int transpose, double* y) {
  if (M < 0 || n < 0 || (M * n > 0 && (!x || !signs || !y))) return ORACLE_BAD_ARGS;
  const int64_t b = oracle_rht_block(n);
  const double inv = b > 0 ? 1.0 / sqrt((double)b) : 0.0;
  for (int64_t m = 0; m < M; ++m) {
    const double* xr = x + m * n;
    double* yr = y + m * n;
    for (int64_t base = 0; base < n; base += b) {
      for (int64_t i = 0; i < b; ++i) {
        double acc = 0.0;
        for (int64_t j = 0; j < b; ++j) {
          double v = xr[base + j];
          if (!transpose && ((signs[(base + j) >> 3] >> ((base + j) & 7)) & 1)) v = -v;
          acc += (popcount64((uint64_t)(i & j)) & 1) ? -v : v;
        }
        acc *= inv;
        if (transpose && ((signs[(base + i) >> 3] >> ((base + i) & 7)) & 1)) acc = -acc;
        yr[base + i] = acc;
      }
    }
  }
  return ORACLE_OK;
}

/* ---------------------------------------------------------------- residual VQ encode */

/*
 * The encode picks, for each v-vector w, the centroid c_k of smallest squared Euclidean
 * distance D_k = sum_t (w_t - c_t)^2 (VPTQ guide, "The Information-Theoretic Superiority of
 * Vector Quantization": q(w) = argmin_k |w - c_k|^2; its "Step 2" quantizer takes
 * torch.cdist and argmin, the first index among equal minima).  Here the minimum is the
 * exact one: ties and near-ties are decided on exact values, never on a rounded distance.
 *
 * Exact values.  w_t is an fp32 value (fp16 / bf16 / fp32 weights, or an fp32 residual) and
 * c_t an fp16 value, so each of w_t^2, w_t c_t and c_t^2 is exact in fp64 (at most 48, 35
 * and 22 significant bits), and (w_t - c_t)^2 = w_t^2 - 2 w_t c_t + c_t^2 exactly.  D_k is
 * therefore an exact sum of fp64 numbers, each an integer multiple of 2^-350 (the lowest
 * bit of w_t^2 for the smallest fp32 subnormal is 2^-298, and a 53-bit significand reaches
 * 52 bits below its leading bit) and below 2^257 in magnitude.  The sum is held as a
 * two's-complement integer in units of 2^-350 in ten 64-bit limbs (640 bits).
 */
#define EXACT_LIMBS 10
#define EXACT_UNIT_EXP (-350)
typedef struct {
  uint64_t limb[EXACT_LIMBS]; /* little-endian, two's complement */
} exact_sum;

/* acc += x (x finite, an integer multiple of 2^-350 below 2^257 in magnitude). */
static void exact_add(exact_sum* acc, double x) {
  if (x == 0.0) return;
  int e;
  const double f = frexp(fabs(x), &e);              /* |x| = f 2^e, 0.5 <= f < 1 */
  uint64_t m = (uint64_t)ldexp(f, 53);              /* exact: f has at most 53 bits */
  int shift = e - 53 - EXACT_UNIT_EXP;              /* |x| = m 2^(shift + unit exponent) */
  while (shift < 0 && (m & 1u) == 0) {              /* drop trailing zero bits */
    m >>= 1;
    ++shift;
  }
  if (shift < 0) abort();                           /* not a multiple of the unit */
  const int li = shift / 64, off = shift % 64;
  uint64_t part[EXACT_LIMBS] = {0};
  const unsigned __int128 wide = (unsigned __int128)m << off;
  part[li] = (uint64_t)wide;
  if (li + 1 < EXACT_LIMBS) part[li + 1] = (uint64_t)(wide >> 64);
  else if ((uint64_t)(wide >> 64) != 0) abort();
  if (x < 0.0) { /* part = -part: complement and add one */
    unsigned carry = 1;
    for (int i = 0; i < EXACT_LIMBS; ++i) {
      const uint64_t c = ~part[i] + carry;
      carry = carry && c == 0;
      part[i] = c;
    }
  }
  unsigned carry = 0;
  for (int i = 0; i < EXACT_LIMBS; ++i) {
    const unsigned __int128 t = (unsigned __int128)acc->limb[i] + part[i] + carry;
    acc->limb[i] = (uint64_t)t;
    carry = (unsigned)(t >> 64);
  }
}

/* Sign of a - b as signed integers: -1, 0 or 1. */
static int exact_cmp(const exact_sum* a, const exact_sum* b) {
  const int na = (int)(a->limb[EXACT_LIMBS - 1] >> 63), nb = (int)(b->limb[EXACT_LIMBS - 1] >> 63);
  if (na != nb) return na ? -1 : 1;
  for (int i = EXACT_LIMBS - 1; i >= 0; --i) {
    if (a->limb[i] != b->limb[i]) return a->limb[i] < b->limb[i] ? -1 : 1;
  }
  return 0;
}

/* D = sum_t (w_t - c_t)^2 exactly, as w_t^2 - 2 w_t c_t + c_t^2 per coordinate. */
static void exact_distance(const double* w, const uint16_t* c, int v, exact_sum* d) {
  memset(d, 0, sizeof *d);
  for (int t = 0; t < v; ++t) {
    const double ct = oracle_f16_to_f64(c[t]);
    exact_add(d, w[t] * w[t]);
    exact_add(d, -2.0 * (w[t] * ct));
    exact_add(d, ct * ct);
  }
}

/* Kind of D_k under IEEE arithmetic on extended values: a NaN coordinate, or the same
 * infinity in w and c at one coordinate (inf - inf), makes it NaN; otherwise any infinite
 * coordinate makes it +inf; otherwise it is finite. */
enum { DIST_FINITE = 0, DIST_INF = 1, DIST_NAN = 2 };
static int distance_kind(const double* w, const uint16_t* c, int v) {
  int inf = 0;
  for (int t = 0; t < v; ++t) {
    const double ct = oracle_f16_to_f64(c[t]);
    if (isnan(w[t]) || isnan(ct)) return DIST_NAN;
    if (isinf(w[t]) && isinf(ct) && (w[t] > 0) == (ct > 0)) return DIST_NAN;
    if (isinf(w[t]) || isinf(ct)) inf = 1;
  }
  return inf ? DIST_INF : DIST_FINITE;
}

/* fp64 approximation of a finite D: fl(fl(w_t - c_t)^2) summed in ascending t.  Every term
 * is >= 0 and none underflows or overflows (w_t - c_t is 0 or at least 2^-149 and below
 * 2^129), so the result is D times a factor within (1 -+ u)^(v + 2), u = 2^-53: the
 * difference, the square and at most v - 1 additions each round once. */
static double approx_distance(const double* w, const uint16_t* c, int v) {
  double d = 0.0;
  for (int t = 0; t < v; ++t) {
    const double diff = w[t] - oracle_f16_to_f64(c[t]);
    d = d + diff * diff;
  }
  return d;
}

/* Nearest centroid of w among k, as defined above: the smallest exact D_k among finite
 * distances, the lowest index among equal ones; with no finite distance the lowest index
 * whose distance is +inf; with every distance NaN, index 0.  The fp64 approximations only
 * select which centroids get an exact evaluation: with rho = 2 (v + 3) u, every exact D_k
 * lies in [a_k (1 - rho), a_k (1 + rho)] (a_k the approximation), so the exact minimum is
 * among the centroids whose lower end is at most the smallest upper end. */
static uint32_t nearest(const double* w, const uint16_t* cb, int64_t k, int v, double* approx) {
  const double rho = 2.0 * (v + 3) * 0x1p-53;
  int64_t first_inf = -1;
  double min_hi = INFINITY;
  int any_finite = 0;
  for (int64_t i = 0; i < k; ++i) {
    const int kind = distance_kind(w, cb + i * v, v);
    if (kind == DIST_FINITE) {
      approx[i] = approx_distance(w, cb + i * v, v);
      const double hi = approx[i] * (1.0 + rho);
      if (hi < min_hi) min_hi = hi;
      any_finite = 1;
    } else {
      approx[i] = NAN;
      if (kind == DIST_INF && first_inf < 0) first_inf = i;
    }
  }
  if (!any_finite) return first_inf >= 0 ? (uint32_t)first_inf : 0u;
  uint32_t best = 0;
  int have = 0;
  exact_sum bd, d;
  for (int64_t i = 0; i < k; ++i) {
    if (!(approx[i] * (1.0 - rho) <= min_hi)) continue; /* also skips the NaN markers */
    exact_distance(w, cb + i * v, v, &d);
    if (!have || exact_cmp(&d, &bd) < 0) { /* increasing i: equal ones keep the lower index */
      bd = d;
      best = (uint32_t)i;
      have = 1;
    }
  }
  return best;
}

/* Two-stage residual VQ encode (VPTQ guide, "Step 2: Multi-Stage Residual Vector Quantizer
 * (RVQ)"): each v-vector of W takes the nearest main centroid, the residual
 * r = w - C1[idx1] (computed in fp32, as the guide's residuals are) takes the nearest
 * residual centroid.  Codebooks are given (the guide's random-sample initialisation and
 * any k-means are outside this).  w: [n][in] as doubles holding fp32 values; in % v == 0;
 * cb1 fp16 [k1][v]; cb2 fp16 [k2][v] or NULL when k2 == 0 (idx2 untouched). */
int oracle_rvq_assign(int64_t n, int64_t in_features, int v, int64_t k1, int64_t k2, const double* w,
                      const uint16_t* cb1, const uint16_t* cb2, uint32_t* idx1, uint32_t* idx2) {
  if (n < 0 || in_features < 0 || v < 1 || v > 16 || k1 < 1 || k2 < 0 || in_features % v != 0) return ORACLE_BAD_ARGS;
  if (n * in_features > 0 && (!w || !cb1 || !idx1 || (k2 > 0 && (!cb2 || !idx2)))) return ORACLE_BAD_ARGS;
  const int64_t nv = in_features / v;
  if (n * nv == 0) return ORACLE_OK;
  double* approx = (double*)malloc((size_t)(k1 > k2 ? k1 : k2) * sizeof(double));
  if (!approx) return ORACLE_BAD_ARGS;
  for (int64_t o = 0; o < n; ++o) {
    for (int64_t j = 0; j < nv; ++j) {
      const double* wv = w + o * in_features + j * v;
      const uint32_t i1 = nearest(wv, cb1, k1, v, approx);
      idx1[o * nv + j] = i1;
      if (k2 > 0) {
        double r[16];
        for (int t = 0; t < v; ++t) r[t] = (double)((float)wv[t] - (float)oracle_f16_to_f64(cb1[(int64_t)i1 * v + t]));
        idx2[o * nv + j] = nearest(r, cb2, k2, v, approx);
      }
    }
  }
  free(approx);
  return ORACLE_OK;
}
