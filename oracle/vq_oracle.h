/*
 * CPU oracle for the VQ dequantize-and-multiply path.  TEST INFRASTRUCTURE ONLY:
 * nothing on the product path may include, link or call this; only tests, the
 * smoke check and the CPU-baseline leg of the benchmark use it.  It shares no code,
 * header, table or constant with the HIP library.
 *
 * What it computes (plain definitions, written out slowly):
 *   - index layout: per output row, each codebook's indices form one LSB-first
 *     bitstream of nv = ceil(in/v) fields of B bits, the row padded with zero bits
 *     to a multiple of 16 bytes; the main stream for all rows comes first, the
 *     residual stream (if any) after it.  The pages are silent on packing (the VPTQ
 *     guide stores whole uint8/int16 tensors, the production-VQ post speaks only of
 *     "a 16-bit uint per 8 weights"); this bit order is the reading taken.
 *   - dequant (VPTQ guide, "Step 2 ... dequantize" and the residual-decode formula
 *     of "2. Multi-Stage Residual Vector Quantization"): w = C1[i1] + C2[i2], summed in
 *     fp32, then times the per-output-channel scale in fp32.
 *   - product (VPTQ guide, "Step 3: Fused Low-Bit VPTQ Linear Layer"): y = x W^T (+ bias),
 *     accumulated in fp64 in ascending column order.
 *   - affine-lattice decode (UniSVQ summary): W's vectors are A q + B over 2-bit integer
 *     codes instead of codebook entries; the same product follows.
 *   - the randomized Hadamard transform of the activations (QuIP# incoherence processing):
 *     the definition as a matrix product.
 *   - the residual VQ encode (VPTQ guide, "Step 2"): nearest main centroid, then nearest
 *     residual centroid of the fp32 residual, ties to the lowest index.
 */
#ifndef VQ_ORACLE_H
#define VQ_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define ORACLE_OK 0
#define ORACLE_BAD_ARGS (-1)
#define ORACLE_BUFFER_SMALL (-2)
#define ORACLE_INDEX_RANGE (-3)
#define ORACLE_PAD_NONZERO 1 /* unpack: a pad bit was set (indices are still written) */

/* Exact decode of IEEE binary16 / bfloat16 bit patterns (values returned in double). */
double oracle_f16_to_f64(uint16_t h);
double oracle_bf16_to_f64(uint16_t b);
/* Round-to-nearest-even of a finite double holding an fp32 value to binary16 / bfloat16 bits. */
uint16_t oracle_f64_to_f16_rne(double x);
uint16_t oracle_f64_to_bf16_rne(double x);
/* The same roundings applied to an fp32 array. */
void oracle_f32_to_f16_rne_array(const float* in, uint16_t* out, int64_t n);
void oracle_f32_to_bf16_rne_array(const float* in, uint16_t* out, int64_t n);

/* Bytes of one row's bitstream for nv fields of `bits` bits (0 if bits == 0). */
int64_t oracle_row_stride(int64_t in_features, int v, int bits);
/* Total packed bytes; -1 on invalid arguments. */
int64_t oracle_packed_bytes(int64_t n, int64_t in_features, int v, int bits1, int bits2);

/* Pack idx1 [n][nv] (and idx2 when bits2 > 0) bit by bit. */
int oracle_pack(int64_t n, int64_t in_features, int v, int bits1, int bits2, const uint32_t* idx1,
                const uint32_t* idx2, uint8_t* out, int64_t out_bytes);
/* Unpack bit by bit; returns ORACLE_PAD_NONZERO when any pad bit is 1. */
int oracle_unpack(int64_t n, int64_t in_features, int v, int bits1, int bits2, const uint8_t* packed,
                  uint32_t* idx1, uint32_t* idx2);

/*
 * Dequantize rows (rows == NULL: all n rows, in order) into w[nrows][in_features] fp32.
 * cb1: fp16 bits [2^bits1][v]; cb2: fp16 bits [2^bits2][v] or NULL when bits2 == 0;
 * scale: fp16 bits [n] or NULL (scale 1, multiply skipped).
 */
int oracle_dequant_rows(int64_t n, int64_t in_features, int v, int bits1, int bits2, const uint8_t* packed,
                        const uint16_t* cb1, const uint16_t* cb2, const uint16_t* scale, const int64_t* rows,
                        int64_t nrows, float* w, int nthreads);

/*
 * y[m][r] (fp64, [M][nrows]) = sum_col x[m][col] * w[row_r][col] (+ bias[row_r]).
 * x: [M][in_features] fp16 bits (x_is_bf16 == 0) or bf16 bits (x_is_bf16 == 1);
 * bias: fp16 bits [n] or NULL.
 */
int oracle_forward_rows(int64_t n, int64_t in_features, int v, int bits1, int bits2, const uint8_t* packed,
                        const uint16_t* cb1, const uint16_t* cb2, const uint16_t* scale, const uint16_t* bias,
                        const uint16_t* x, int x_is_bf16, int64_t M, const int64_t* rows, int64_t nrows,
                        double* y, int nthreads);

/*
 * Affine-lattice layers (UniSVQ summary, "Mathematical Formulation" and "Efficiency"):
 * d = 4, each vector stored as one 8-bit field of four 2-bit codes (code u in bits
 * [2u, 2u+2)), packed like a v = 4, bits1 = 8 index stream with no residual.  Coordinate
 * t of a vector is fl32(B[t] + sum_u A[t][u] * q_u) with q_u the code value, then times
 * the channel scale in fp32.  a: fp16 bits [4][4] (row t, column u); b: fp16 bits [4].
 */
int oracle_svq_dequant_rows(int64_t n, int64_t in_features, const uint8_t* packed, const uint16_t* a,
                            const uint16_t* b, const uint16_t* scale, const int64_t* rows, int64_t nrows, float* w,
                            int nthreads);
int oracle_svq_forward_rows(int64_t n, int64_t in_features, const uint8_t* packed, const uint16_t* a,
                            const uint16_t* b, const uint16_t* scale, const uint16_t* bias, const uint16_t* x,
                            int x_is_bf16, int64_t M, const int64_t* rows, int64_t nrows, double* y, int nthreads);

/*
 * Randomized Walsh-Hadamard transform of the rows of x [M][n] (fp64 in and out): blocks of
 * b = oracle_rht_block(n) columns (the largest power of two dividing n, at most 16384);
 * forward y = H_b (s . x) / sqrt(b), transpose (its inverse) y = s . (H_b x) / sqrt(b), with
 * H_b[i][j] = (-1)^popcount(i & j) and s_j = -1 where bit j of signs (LSB-first) is set.
 */
int64_t oracle_rht_block(int64_t n);
int oracle_rht(int64_t M, int64_t n, const double* x, const uint8_t* signs, int transpose, double* y);

/*
 * Two-stage residual VQ encode with given codebooks: idx1 = nearest main centroid of each
 * v-vector of w, idx2 = nearest residual centroid of r = fl32(w - C1[idx1]); "nearest" is the
 * lowest index of the exact minimum of |w - c|^2 (decided in exact arithmetic, not on a
 * rounded distance).  Non-finite values: a distance is NaN when a coordinate is NaN or holds
 * the same infinity in w and c, else +inf when a coordinate is infinite; finite distances
 * win over +inf, NaN ones are never taken, and index 0 is returned when all are NaN.
 * w: [n][in] doubles holding fp32 values, in % v == 0.
 */
int oracle_rvq_assign(int64_t n, int64_t in_features, int v, int64_t k1, int64_t k2, const double* w,
                      const uint16_t* cb1, const uint16_t* cb2, uint32_t* idx1, uint32_t* idx2);

#ifdef __cplusplus
}
#endif
#endif
