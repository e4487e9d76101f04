/*
 * vq.h -- C ABI of the MI355X (gfx950) VQ dequantize-and-multiply library, libvq.so.
 *
 * The operation (VPTQ guide, aifetchly, "2. Multi-Stage Residual Vector Quantization
 * (RVQ)" and "Step 3: Fused Low-Bit VPTQ Linear Layer"; per-channel scaling as in the
 * QuIP# entry of the production-VQ post, llms.blog):
 *
 *   W^[o, j*v + t] = scale[o] * ( C1[idx1[o, j]][t] + C2[idx2[o, j]][t] ),  t < v
 *   y[m, o]        = sum_col x[m, col] * W^[o, col]  (+ bias[o])
 *
 * for o < N = out_features, col < IN = in_features, j < nv = ceil(IN / v).  The weight
 * matrix is never stored: every call rebuilds W^ on the fly from bit-packed indices
 * into a main codebook C1 of K1 = 2^bits1 fp16 centroids and an optional residual
 * codebook C2 of K2 = 2^bits2 fp16 centroids, each centroid a row of v fp16 values.
 *
 * Packed index layout (VQ_LAYOUT_ROWSTREAM, the layout every call takes):
 *   - row stride of stream b: S_b = 16 * ceil(nv * bits_b / 128) bytes (0 if bits_b == 0);
 *   - stream 1 (idx1) for rows 0..N-1 occupies bytes [0, N*S1), stream 2 (idx2) follows
 *     at [N*S1, N*(S1+S2));
 *   - index j of row o is the unsigned integer in bits [j*B, (j+1)*B) of its row, where
 *     bit k is bit (k mod 8) of byte floor(k/8) (LSB-first, little-endian);
 *   - pad bits are written as zero by vq_pack and ignored by the kernels.
 * When IN is not a multiple of v, the last vector's lanes t with j*v + t >= IN are
 * dropped (the centroid is stored in full, its tail is never used).
 *
 * Slice-bucketed layout (VQ_LAYOUT_BUCKETED): the same indices, regrouped once at load
 * time for the batch-1 decode product of vq_gemv_ws / vq_gemv_noalloc, the only calls
 * that take it.  Defined for v = 8, bits1 = 16 (K1 = 65536), bits2 = 0 or 8, IN a
 * multiple of 8.  The main book is seen as 8 slices of 8192 centroids (slice s =
 * idx1 >> 13); the vectors of row o are cut into chunks of 1024 (chunk c = j / 1024).
 *   - bucket b = (c*8 + s)*N + o holds the vectors j of row o in chunk c whose idx1
 *     lies in slice s, one 32-bit little-endian word each, in an order vq_pack chooses
 *     (deterministically: word k preferably holds an idx1 whose bits [2, 4) equal those
 *     of k, which lines the product's main-book reads up with the LDS banks); any order
 *     gives the same y up to fp32 summation order:
 *       bits [0, 10) j - 1024*c,  bits [10, 23) idx1 & 8191,  bits [23, 31) idx2
 *     (idx2 = 0 without a residual book), bit 31 zero;
 *   - bytes [0, H) hold start[b], b = 0 .. 8*chunks*N, as uint32: bucket b is words
 *     [start[b], start[b+1]); start[0] = 0; H = 4*(8*chunks*N + 1) rounded up to 256,
 *     the rest of it zero;
 *   - the words follow at byte H, buckets in order of b: N * IN/8 words in all.
 * It stores 32 bits per vector where the row stream stores bits1 + bits2 (24 with the
 * residual book): the position travels with each index, so that each slice's CUs read
 * exactly the vectors whose centroids they hold.
 *
 * Numerics.  vq_dequant is exact: in fp32, w = fp32(C1) + fp32(C2) rounded to nearest
 * even, then w * fp32(scale[o]); without a residual book the add is skipped, without a
 * scale the multiply is skipped.  vq_gemv accumulates in fp32 and applies scale[o] once
 * per output; vq_gemm rounds the rebuilt vector to the activation's 16-bit type
 * (bf16 activations: as a bf16 hi + lo pair, ~16 significant bits) and accumulates in
 * fp32 on the matrix cores.  Outputs are rounded to nearest even into y_dtype.
 *
 * Ownership and execution.  The caller allocates and owns every buffer.  Pointers given
 * to vq_dequant / vq_gemv / vq_gemm are DEVICE pointers; `stream` is a hipStream_t
 * (NULL = the default stream).  These three calls validate on the host, enqueue kernels
 * on `stream` and return without synchronising: inputs must stay unchanged until the
 * stream has run them, and y / w must not alias any input.  The library allocates no
 * memory (vq_gemv_ws and vq_assign take their scratch space from the caller;
 * vq_gemv_noalloc uses a fixed array in device memory that the library holds), keeps no
 * pointer after returning and is safe to call from several threads.
 * vq_packed_bytes and vq_pack work on HOST memory and are synchronous.
 *
 * Errors.  Every argument is checked before anything is enqueued; on error nothing is
 * launched and no output is written.  A launch failure reported by the runtime maps to
 * VQ_ERR_HIP.  No C++ exception crosses this interface.
 */
#ifndef VQ_H
#define VQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VQ_ABI_VERSION 1
#define VQ_LAYOUT_ROWSTREAM 1
#define VQ_LAYOUT_BUCKETED 2

typedef enum vq_status {
  VQ_OK = 0,
  VQ_ERR_NULL = -1,         /* a required pointer is NULL */
  VQ_ERR_SHAPE = -2,        /* negative sizes, M out of range */
  VQ_ERR_BITS = -3,         /* v not in 1..16, bits1 not in 1..16, bits2 not in 0..16 */
  VQ_ERR_UNSUPPORTED = -4,  /* valid but not built for the GPU (v, bits, dtype combination), unknown layout */
  VQ_ERR_ALIGN = -5,        /* a device pointer is not aligned as the call requires */
  VQ_ERR_INDEX_RANGE = -6,  /* vq_pack: an index is >= 2^bits */
  VQ_ERR_BUFFER_SIZE = -7,  /* vq_pack: nbytes < vq_packed_bytes; vq_gemv_ws: workspace too small */
  VQ_ERR_HIP = -8           /* the HIP runtime reported an error at launch */
} vq_status;

typedef enum vq_dtype { VQ_F16 = 0, VQ_BF16 = 1, VQ_F32 = 2 } vq_dtype;

/* W is [out_features][in_features]; vectors of v weights run along in_features.
 * bits1 in 1..16 (K1 = 2^bits1), bits2 in 0..16 (0: no residual book); layout =
 * VQ_LAYOUT_ROWSTREAM, or VQ_LAYOUT_BUCKETED where a call says it takes it. */
typedef struct vq_desc {
  int32_t out_features;
  int32_t in_features;
  int32_t v;
  int32_t bits1;
  int32_t bits2;
  int32_t layout;
} vq_desc;

/* VQ_ABI_VERSION of the loaded library. */
int32_t vq_abi_version(void);

/* Static, human-readable name of a status code. */
const char* vq_status_string(vq_status status);

/* Bytes of the packed index buffer for `desc` (bitrate log2(K)/v per book, VPTQ guide
 * "3. Effective Bit-Width Calculation", plus row padding to 16 bytes).  For
 * VQ_LAYOUT_BUCKETED: the prefix table plus 4 bytes per vector (VQ_ERR_UNSUPPORTED where
 * that layout is not defined). */
vq_status vq_packed_bytes(const vq_desc* desc, size_t* nbytes);

/* Pack idx1 [N][nv] (and idx2 [N][nv] when bits2 > 0; must be NULL-free then, ignored
 * otherwise) into `packed` (HOST memory, nbytes >= vq_packed_bytes).  Writes every byte
 * of the packed size, pad bits zero.  VQ_ERR_INDEX_RANGE if any index >= 2^bits, with
 * `packed` untouched.  The pages fix no storage layout (the VPTQ guide's "Step 3" layer
 * keeps whole uint8 / int16 index tensors); this one stores exactly the log2(K) bits per
 * index per book that the guide's "3. Effective Bit-Width Calculation" counts, main and
 * residual indices in separate streams as its residual pipeline keeps them ("2.
 * Multi-Stage Residual Vector Quantization (RVQ)").  With desc->layout ==
 * VQ_LAYOUT_BUCKETED the same indices are written in the slice-bucketed layout above
 * (VQ_ERR_UNSUPPORTED where it is not defined; VQ_ERR_BUFFER_SIZE also if the host runs
 * out of memory for the regrouping, with `packed` then partly written). */
vq_status vq_pack(const vq_desc* desc, const uint32_t* idx1, const uint32_t* idx2, void* packed, size_t nbytes);

/* Rebuild W^ [N][IN] into `w` (device, row-major, w_dtype; fp16 / bf16 outputs are the
 * nearest-even rounding of the exact fp32 value): the VPTQ guide's "Step 2" dequantize
 * (gather both books, add, view as [out, in]) with the per-channel scale.  packed: device, 4-byte aligned;
 * cb1: fp16 [2^bits1][v]; cb2: fp16 [2^bits2][v] (NULL iff bits2 == 0);
 * scale: fp16 [N] or NULL (scale 1).  Codebook and scale pointers must be 2-byte
 * aligned, w aligned to its element size. */
vq_status vq_dequant(const vq_desc* desc, const void* packed, const void* cb1, const void* cb2, const void* scale,
                     void* w, vq_dtype w_dtype, void* stream);

/* Decode-batch product y [M][N] = x [M][IN] * W^T (+ bias), 1 <= M <= 16 (M = 0: no-op):
 * the forward of the VPTQ guide's "Step 3: Fused Low-Bit VPTQ Linear Layer", fused so that
 * W^ is never written, for the memory-bound decode regime of the production-VQ post's
 * "1. Prefill vs. Decode Bottlenecks".
 * The VALU path: each wavefront reduces whole rows; accumulation in fp32.
 * x: device, x_dtype VQ_F16 or VQ_BF16, row-major [M][IN]; bias: fp16 [N] or NULL;
 * y: device, y_dtype VQ_F16, VQ_BF16 or VQ_F32, row-major [M][N].  Other pointers as
 * for vq_dequant.  IN == 0 gives y = bias (or 0). */
vq_status vq_gemv(const vq_desc* desc, const void* packed, const void* cb1, const void* cb2, const void* scale,
                  const void* bias, const void* x, vq_dtype x_dtype, int32_t M, void* y, vq_dtype y_dtype,
                  void* stream);

/* Bytes of device workspace with which vq_gemv_ws runs `desc` at batch M (1..16) with
 * activations of x_dtype on its codebook-sliced path; 0 when the shape does not take
 * that path.  It needs v = 8, bits1 = 16, bits2 = 0 or 8, IN a multiple of 8, and at
 * least 2^22 weight vectors (N * IN / 8) for M < 8 or 2^19 for M >= 8: below that the
 * vq_gemv kernels are as fast.  M = 0 gives 0.  A VQ_LAYOUT_BUCKETED desc has no other
 * path: M = 1 gives its workspace (8 * chunks * N floats and 256 bytes; 0 when IN == 0),
 * M >= 2 VQ_ERR_UNSUPPORTED. */
vq_status vq_gemv_workspace_bytes(const vq_desc* desc, int32_t M, vq_dtype x_dtype, size_t* nbytes);

/* vq_gemv with a caller-owned device workspace, for the 65536-entry main book (VPTQ
 * guide, "Step 3: Fused Low-Bit VPTQ Linear Layer"; the production-VQ post, "Lookup
 * Table (LUT) Overhead vs. Bit-Shifting", on lookups that spill out of fast memory).
 * The book is split into eight 8192-centroid slices, each held in the LDS of the CUs
 * that serve it; the matrix cores form the dot products; per-slice fp32 partial sums
 * go to the workspace and a second kernel adds them in a fixed order, so results are
 * deterministic.  bf16 activations are rewritten as fp16 times a power of two per
 * batch row, chosen so that the row's largest magnitude lands in [2^14, 2^15); every
 * value down to 2^-31 of that magnitude converts exactly, smaller ones round with an
 * absolute error below 2^-39 of it.
 * Same arguments, results (to the vq_gemv tolerance) and errors as vq_gemv, plus:
 *   workspace: NULL (then this is vq_gemv), or device memory, 256-byte aligned, of at
 *     least vq_gemv_workspace_bytes(desc, M, x_dtype) bytes (VQ_ERR_BUFFER_SIZE /
 *     VQ_ERR_ALIGN otherwise).  Its contents need no initialisation and are scratch
 *     after the call; calls that may run at the same time need different workspaces.
 * Shapes without the sliced path, or packed / cb1 / cb2 / x pointers that are not
 * 16-byte aligned, run the vq_gemv kernels and leave the workspace untouched.
 * A VQ_LAYOUT_BUCKETED desc (packed in that layout) runs the batch-1 decode product over
 * it: each slice's workgroups read only their own buckets, so every index is read once;
 * per word, the activation vector, the main and the residual centroid come from LDS and
 * eight packed fp16 dot products accumulate in fp32; partial sums per (chunk, slice,
 * row) are added in a fixed order by the same second kernel.  It takes M = 1 only (M >= 2:
 * VQ_ERR_UNSUPPORTED), requires the workspace (NULL: VQ_ERR_NULL) and 16-byte aligned
 * packed, cb1, cb2 and x (VQ_ERR_ALIGN): there is no other path for that layout. */
vq_status vq_gemv_ws(const vq_desc* desc, const void* packed, const void* cb1, const void* cb2, const void* scale,
                     const void* bias, const void* x, vq_dtype x_dtype, int32_t M, void* y, vq_dtype y_dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/* vq_gemv_ws for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same operation,
 * arguments (without the workspace) and errors as vq_gemv, and on the codebook-sliced path
 * the same kernels and results as vq_gemv_ws, but the workspace is a fixed 16 MiB array in
 * device memory that the library holds on each GPU it runs on until the process ends.
 * It allocates nothing: the array's address is looked up on the first call on each
 * device (with that device current).  Shapes whose sliced-path workspace
 * (vq_gemv_workspace_bytes) exceeds 16 MiB return VQ_ERR_BUFFER_SIZE and launch
 * nothing; shapes without the sliced path run the vq_gemv kernels, which use no
 * workspace.  A VQ_LAYOUT_BUCKETED desc runs its decode product as in vq_gemv_ws.  Every
 * call on one GPU shares that GPU's array: calls that may run at the same time on one GPU
 * (other streams, other threads) race and must not overlap. */
vq_status vq_gemv_noalloc(const vq_desc* desc, const void* packed, const void* cb1, const void* cb2,
                          const void* scale, const void* bias, const void* x, vq_dtype x_dtype, int32_t M, void* y,
                          vq_dtype y_dtype, void* stream);

/* Same operation and arguments as vq_gemv for any M >= 1 (M = 0: no-op), on the matrix
 * cores: rebuilt weight tiles are staged in LDS in the activation's 16-bit type and
 * multiplied with MFMA, fp32 accumulation.  Meant for prefill batches (M >= 32), where the
 * production-VQ post ("1. Prefill vs. Decode Bottlenecks", "Throughput and Concurrency
 * Trade-Offs") places the compute-bound regime and matrix-engine formats. */
vq_status vq_gemm(const vq_desc* desc, const void* packed, const void* cb1, const void* cb2, const void* scale,
                  const void* bias, const void* x, vq_dtype x_dtype, int32_t M, void* y, vq_dtype y_dtype,
                  void* stream);

/* Bytes of device workspace with which vq_gemm_ws runs `desc` at batch M with activations
 * of x_dtype on its gather path: the fp16 copy of bf16 activations with one power of two
 * per batch row, and fp32 partial sums when the K range is split across workgroups.  0
 * when the shape does not take that path or needs no workspace (fp16 activations, no
 * split).  The path needs v = 8, bits1 = 16, bits2 = 0 or 8 and IN a multiple of 8
 * (IN >= 8).  M = 0 gives 0. */
vq_status vq_gemm_workspace_bytes(const vq_desc* desc, int32_t M, vq_dtype x_dtype, size_t* nbytes);

/* vq_gemm with a caller-owned device workspace, for the 65536-entry main book (VPTQ
 * guide, "Step 3: Fused Low-Bit VPTQ Linear Layer"; the production-VQ post, "1. Prefill
 * vs. Decode Bottlenecks" and "Lookup Table (LUT) Overhead vs. Bit-Shifting").  Each
 * lane gathers one weight vector's main centroid from L2, adds its residual centroid in
 * fp16 (the exact sum rounded once to nearest even) and hands the vector to the matrix
 * cores as one column of an fp16 operand; activations stay in LDS.  bf16 activations are
 * first rewritten as fp16 times a power of two per batch row (as in vq_gemv_ws), so the
 * product uses fp16 weights and activations with fp32 accumulation; partial sums of a
 * split K range are added in a fixed order, so results are deterministic.
 * Same arguments, results (to the vq_gemm tolerance) and errors as vq_gemm, plus:
 *   workspace: device memory, 256-byte aligned, of at least
 *     vq_gemm_workspace_bytes(desc, M, x_dtype) bytes (VQ_ERR_BUFFER_SIZE / VQ_ERR_ALIGN
 *     otherwise), or NULL.  Its contents need no initialisation and are scratch after the
 *     call; calls that may run at the same time need different workspaces.
 * Shapes without the gather path, packed / cb1 / cb2 / x pointers that are not 16-byte
 * aligned, or a NULL workspace where one is needed run the vq_gemm kernels. */
vq_status vq_gemm_ws(const vq_desc* desc, const void* packed, const void* cb1, const void* cb2, const void* scale,
                     const void* bias, const void* x, vq_dtype x_dtype, int32_t M, void* y, vq_dtype y_dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Affine-lattice layers (UniSVQ summary, gist.science, "Mathematical Formulation" and
 * "Efficiency"): instead of codebook entries, each 4-vector of W^ is a point of an affine
 * integer grid,
 *
 *   W^[o, 4j + t] = scale[o] * fp32( B[t] + sum_u A[t][u] * q_u(o, j) ),   t, u < 4,
 *
 * with q_u in 0..3 the 2-bit code of coordinate u (the integer grid coordinate itself),
 * A an fp16 [4][4] matrix (row t, column u, row-major) and B an fp16 [4] vector: 20
 * parameters per layer.  The sum is exact before its single rounding to fp32; the scale
 * multiply is one more fp32 rounding (skipped when scale is NULL).  The codes are stored
 * as the row stream of a descriptor with v = 4, bits1 = 8, bits2 = 0: vector j's 8-bit
 * field holds code u in bits [2u, 2u + 2), so vq_pack packs them from idx1[o][j] =
 * q_0 | q_1 << 2 | q_2 << 4 | q_3 << 6, and a row takes 16 * ceil(nv / 16) bytes
 * (2 bits per weight); vq_svq_pack packs them from the coordinates directly.  Any other
 * descriptor gives VQ_ERR_UNSUPPORTED.  As for the codebook calls, lanes of the last
 * vector past IN are dropped.
 */

/* Pack the integer grid coordinates q [N][nv][4] (uint8, each 0..3; nv = ceil(IN / 4),
 * the last vector's lanes past IN included and ignored by the products) of an
 * affine-lattice layer into its row stream (HOST memory, synchronous, nbytes >=
 * vq_packed_bytes(desc)): vector j's byte in row o is q_0 | q_1 << 2 | q_2 << 4 | q_3 << 6,
 * rows padded to 16 bytes with zeros.  desc must be the lattice descriptor (v = 4,
 * bits1 = 8, bits2 = 0; else VQ_ERR_UNSUPPORTED); a coordinate above 3 gives
 * VQ_ERR_INDEX_RANGE with `packed` untouched; other errors as for vq_pack.  The UniSVQ
 * summary gives the grid (w̄ in Z^4, "Mathematical Formulation") and 2 bits per weight
 * ("Efficiency") but no storage; this is the plainest packing of those 2-bit codes. */
vq_status vq_svq_pack(const vq_desc* desc, const uint8_t* q, void* packed, size_t nbytes);

/* Write W^ [N][IN] of an affine-lattice layer into `w` (device, w_dtype; fp16 / bf16 are
 * the nearest-even rounding of the exact fp32 value, which this call reproduces bit for
 * bit).  packed, a, b, scale: device; a, b, scale 2-byte aligned. */
vq_status vq_svq_dequant(const vq_desc* desc, const void* packed, const void* a, const void* b, const void* scale,
                         void* w, vq_dtype w_dtype, void* stream);

/* Decode-batch product y [M][N] = x [M][IN] * W^T (+ bias) of an affine-lattice layer,
 * 0 <= M <= 16, without rebuilding W^: the affine map is applied to the activations
 * (UniSVQ summary, "Efficiency"),
 *   y[m, o] = scale[o] * ( sum_j q(o, j) . (A^T x_mj) + B . sum_j x_mj ) + bias[o],
 * where x_mj are the 4 activations of vector j (zero past IN); the rest is a 2-bit
 * scalar product accumulated in fp32, so results match W^ to the vq_gemv tolerance.
 * packed: device, 16-byte aligned; x: device [M][IN], VQ_F16 or VQ_BF16; y: device
 * [M][N], VQ_F16, VQ_BF16 or VQ_F32; bias: fp16 [N] or NULL.  IN == 0 gives y = bias
 * (or 0).  Errors as for vq_gemv.  From M = 4 the call runs the vq_svq_gemm kernel (same
 * results to the same tolerance). */
vq_status vq_svq_gemv(const vq_desc* desc, const void* packed, const void* a, const void* b, const void* scale,
                      const void* bias, const void* x, vq_dtype x_dtype, int32_t M, void* y, vq_dtype y_dtype,
                      void* stream);

/* Same operation, arguments and tolerance as vq_svq_gemv for any M >= 1 (M = 0: no-op;
 * M up to 128 * 65535), on the matrix cores: the layer is rebuilt tile by tile into LDS
 * in the activation's 16-bit type (bf16: a hi + lo pair) and multiplied with MFMA, fp32
 * accumulation.  Meant for prefill batches (M >= 32). */
vq_status vq_svq_gemm(const vq_desc* desc, const void* packed, const void* a, const void* b, const void* scale,
                      const void* bias, const void* x, vq_dtype x_dtype, int32_t M, void* y, vq_dtype y_dtype,
                      void* stream);

/*
 * Randomized Walsh-Hadamard transform of activations, the incoherence step that runs
 * ahead of (and, transposed, after) a product with incoherence-processed weights
 * (production-VQ post, llms.blog, QuIP#: randomized orthogonal Hadamard transforms on a
 * layer's inputs and outputs; sub-4-bit lecture, "QuIP#: Incoherence Processing": Hadamard
 * plus random signs at O(d log d); UniSVQ summary, "Preprocessing (Randomized Hadamard
 * Transform - RHT)").  For each row of x [M][n] and each block of b = vq_rht_block(n)
 * columns (the largest power of two dividing n, at most 16384):
 *
 *   transpose = 0:  y = H_b (s . x) / sqrt(b)
 *   transpose = 1:  y = s . (H_b x) / sqrt(b)      (the inverse of transpose = 0)
 *
 * with H_b[i][j] = (-1)^popcount(i & j) (Sylvester order) and s_j = -1 where bit j of
 * `signs` is set (bit j is bit j % 8 of byte j / 8).  Computed in fp32.
 * x: device [M][n], VQ_F16, VQ_BF16 or VQ_F32, 16-byte aligned; signs: device, ceil(n / 8)
 * bytes; y: device [M][n], VQ_F16, VQ_BF16 or VQ_F32, aligned to its element; y may be x
 * itself when both have the same type.  n must be a multiple of 16 (VQ_ERR_UNSUPPORTED
 * otherwise); M = 0 or n = 0: no-op.  Errors as for the other calls.
 */
vq_status vq_rht(int32_t M, int32_t n, const void* x, vq_dtype x_dtype, const void* signs, int32_t transpose, void* y,
                 vq_dtype y_dtype, void* stream);

/* The transform's block size for row length n (0 for n <= 0). */
int32_t vq_rht_block(int32_t n);

/* Products with the transform fused ahead of them: y = x~ W^T (+ bias), where x~ is
 * vq_rht(x, signs, transpose = 0) row by row (the incoherence step on a layer's inputs:
 * sub-4-bit lecture, "QuIP#: Incoherence Processing"; UniSVQ summary, "Preprocessing
 * (Randomized Hadamard Transform - RHT)").  vq_gemv_ws_rht takes 1 <= M <= 16 as vq_gemv_ws,
 * vq_gemm_ws_rht any M as vq_gemm_ws.  Where the shape has the workspace path of
 * vq_gemv_ws / vq_gemm_ws (and IN <= 32768), the transform runs in that path's x pass: one
 * workgroup per batch row transforms the row in LDS in fp32 and rewrites it as fp16 times a
 * power of two, in place of vq_rht's own launch (and of the x pass bf16 activations take
 * for M > 2 and in vq_gemm_ws).  Otherwise the call runs vq_rht into the workspace (x~
 * rounded to x_dtype) and then vq_gemv / vq_gemm on it.
 * Arguments as for vq_gemv_ws / vq_gemm_ws, plus signs (device, ceil(IN / 8) bytes, bit j
 * of byte j / 8 set: s_j = -1).  IN must be a multiple of 16 (VQ_ERR_UNSUPPORTED); x must be
 * 16-byte aligned (VQ_ERR_ALIGN).  The workspace is required (NULL: VQ_ERR_NULL): device
 * memory, 256-byte aligned, of at least vq_rht_product_workspace_bytes(desc, M, x_dtype,
 * gemm) bytes, gemm = 0 for vq_gemv_ws_rht and 1 for vq_gemm_ws_rht; contents need no
 * initialisation, calls that may overlap need different workspaces.  Results match
 * vq_gemv / vq_gemm on x~ to their tolerance. */
vq_status vq_rht_product_workspace_bytes(const vq_desc* desc, int32_t M, vq_dtype x_dtype, int32_t gemm,
                                         size_t* nbytes);
vq_status vq_gemv_ws_rht(const vq_desc* desc, const void* packed, const void* cb1, const void* cb2, const void* scale,
                         const void* bias, const void* x, vq_dtype x_dtype, int32_t M, const void* signs, void* y,
                         vq_dtype y_dtype, void* workspace, size_t workspace_bytes, void* stream);
vq_status vq_gemm_ws_rht(const vq_desc* desc, const void* packed, const void* cb1, const void* cb2, const void* scale,
                         const void* bias, const void* x, vq_dtype x_dtype, int32_t M, const void* signs, void* y,
                         vq_dtype y_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Two-stage residual VQ encode with given codebooks (VPTQ guide, "Step 2: Multi-Stage
 * Residual Vector Quantizer (RVQ)": Euclidean distance and argmin, then the same on the
 * residuals; the nearest-centroid rule q(w) = argmin_k |w - c_k|^2 of "The
 * Information-Theoretic Superiority of Vector Quantization"; "2. Multi-Stage Residual
 * Vector Quantization" for the residual).  W [N][IN] is cut into nv = IN / v vectors per
 * row; for each vector w
 *
 *   idx1 = the lowest k of the exact minimum of |w - C1[k]|^2
 *   idx2 = the lowest k of the exact minimum of |r - C2[k]|^2,    r = fp32(w - C1[idx1])
 *
 * decided on exact values (not on a rounded distance), so the result does not depend on
 * an evaluation order.  NaN or infinite values: a distance is NaN when a coordinate is NaN
 * or holds the same infinity in w and c, +inf when a coordinate is infinite; finite
 * distances win over +inf, NaN ones are never taken, and index 0 is returned when all are
 * NaN.  Codebook initialisation (the guide's random samples) and refinement are the
 * caller's.
 * desc: N = out_features, IN = in_features (a multiple of v, else VQ_ERR_UNSUPPORTED),
 *   v, K1 = 2^bits1, K2 = 2^bits2 (bits2 = 0: one stage; idx2 and cb2 ignored), layout
 *   as for the other calls.
 * w: device [N][IN], VQ_F16, VQ_BF16 or VQ_F32, aligned to its element.
 * cb1: device fp16 [K1][v]; cb2: device fp16 [K2][v]; 2-byte aligned.
 * idx1, idx2: device uint32 [N][nv] (the layout vq_pack takes), 4-byte aligned.
 * workspace: device, 256-byte aligned, at least vq_assign_workspace_bytes(desc) bytes
 *   (VQ_ERR_BUFFER_SIZE otherwise); scratch after the call, one per concurrent call.
 * N * IN = 0: no-op.  Errors as for the other calls.
 */
vq_status vq_assign_workspace_bytes(const vq_desc* desc, size_t* nbytes);
vq_status vq_assign(const vq_desc* desc, const void* w, vq_dtype w_dtype, const void* cb1, const void* cb2,
                    uint32_t* idx1, uint32_t* idx2, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VQ_H */
