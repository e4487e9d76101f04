// vq_assign: two-stage residual VQ encode with given codebooks (VPTQ guide, "Step 2:
// Multi-Stage Residual Vector Quantizer (RVQ)"; the nearest-centroid rule of "The
// Information-Theoretic Superiority of Vector Quantization"; the residual of "2.
// Multi-Stage Residual Vector Quantization").  Each v-vector w of W takes
//
//   idx1 = the lowest k of the exact minimum of |w - C1[k]|^2
//   idx2 = the lowest k of the exact minimum of |r - C2[k]|^2,   r = fp32(w - C1[idx1])
//
// Centroids are ranked by d(c) = |c|^2 - 2 w . c, which orders them as the squared distance
// does (|w|^2 is common to all), evaluated in fp64 with one fused multiply-add per term.
// That value is within E = v 2^-53 (|c|^2 + 2 sum_t |w_t c_t|) of the exact one, so a
// centroid whose fp64 value differs from the best one's by more than the two bounds is
// ordered by it.  The fast kernels take only such certain decisions; a vector that meets a
// closer pair (a near tie, or an exact one) is marked (top bit of its index) and the
// fix-up kernel ranks it again with exact comparisons: for fp16 centroids and fp16 / bf16
// / fp32 weights every product c_t^2 and 2 w_t c_t is exact in fp64, and `exact_order`
// adds them exactly in 384-bit fixed point.  Vectors and books holding NaN or infinite
// values are marked too; `nearest_general` ranks their IEEE distances: NaN ones never,
// finite ones before +inf.
//
// Kernels:
//   assign_table_kernel  one thread per centroid: the fp64 record {|c|^2, c_0 .. c_{v-1}}
//                        of each fp16 centroid into the workspace, and per 256 centroids
//                        the largest |c_t| and |c|^2 (infinite if any value is not finite).
//   assign_mfma_table_kernel, assign_mfma_kernel<V>  the main stage for fp16 weights and
//                        books of 256 or more centroids on the matrix cores (below).
//   assign_kernel<V, R, WT, FIRST>  both stages (the residual stage only, after the
//                        matrix-core pass): one lane per R vectors (consecutive lanes on
//                        consecutive vectors), the vectors held in fp64 registers; every
//                        wave walks the whole record table in index order with uniform
//                        (scalar-unit) loads, so each centroid costs V + 1 fp64 FMAs and
//                        one compare per vector, and the rare improvements or near ties
//                        take a branch that the wave skips when none of its lanes needs it.
//   assign_fixup_kernel<V, WT>  one thread per vector: marked vectors are ranked again by
//                        nearest_general (both stages when the main index was marked).
#include "vq_device.h"

namespace {

constexpr int kThreads = 256;
constexpr uint32_t kMark = 0x80000000u;  // index needs the exact ranking (indices are < 2^16)

template <int WT>  // VQ_F16, VQ_BF16, VQ_F32
__device__ __forceinline__ double weight_at(const void* w, int64_t i) {
  if constexpr (WT == VQ_F16) {
    return (double)vqd::f16_to_f32(((const uint16_t*)w)[i]);
  } else if constexpr (WT == VQ_BF16) {
    return (double)vqd::bf16_to_f32(((const uint16_t*)w)[i]);
  } else {
    return (double)((const float*)w)[i];
  }
}

__global__ __launch_bounds__(kThreads) void assign_table_kernel(const uint16_t* __restrict__ cb, int32_t k, int32_t v,
                                                                double* __restrict__ tab, double2* __restrict__ tmax) {
  const int32_t c = blockIdx.x * kThreads + threadIdx.x;
  double cm = 0.0, nm = 0.0;
  if (c < k) {
    double* rec = tab + (size_t)c * (size_t)(v + 1);
    double nc = 0.0;
    bool fin = true;
    for (int t = 0; t < v; ++t) {
      const double ct = (double)vqd::f16_to_f32(cb[(size_t)c * v + t]);
      nc = fma(ct, ct, nc);
      rec[1 + t] = ct;
      fin = fin && __builtin_isfinite(ct);
      cm = fmax(cm, fabs(ct));
    }
    rec[0] = nc;
    nm = nc;
    if (!fin) cm = nm = __builtin_inf();
  }
  __shared__ double2 red[kThreads / 64];
  for (int o = 32; o > 0; o >>= 1) {
    cm = fmax(cm, __shfl_xor(cm, o));
    nm = fmax(nm, __shfl_xor(nm, o));
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_double2(cm, nm);
  __syncthreads();
  if (threadIdx.x == 0) {
    double2 m = red[0];
    for (int i = 1; i < kThreads / 64; ++i) m = make_double2(fmax(m.x, red[i].x), fmax(m.y, red[i].y));
    tmax[blockIdx.x] = m;
  }
}

// Book maxima {largest |c_t|, largest |c|^2} from the per-256-centroid table (uniform loads).
__device__ __forceinline__ double2 book_max(const double2* __restrict__ tmax, int32_t k) {
  const int nb = (k + kThreads - 1) / kThreads;
  double2 m = make_double2(0.0, 0.0);
  for (int i = 0; i < nb; ++i) {
    const double2 b = tmax[i];
    m = make_double2(fmax(m.x, b.x), fmax(m.y, b.y));
  }
  return m;
}

// Bound on |d~(c) - d(c) + d~(c') - d(c')| for every pair of centroids of a book, for one
// vector (S_w = sum |w_t|): twice (V + 2) 2^-53 (|c|^2 + 2 sum_t |w_t c_t|), the latter at
// most ncmax + 2 S_w cmax.  The margins over the V 2^-53 of the error analysis cover the
// rounding of this expression.
template <int V>
__device__ __forceinline__ double pair_bound(double sw, double cmax, double ncmax) {
  return 2.0 * (V + 2) * 0x1p-53 * (ncmax + 2.0 * sw * cmax) * (1.0 + 0x1p-20);
}

// Exact comparison of ranking distances.  For fp16 centroids and weights that are fp32
// values, c_t^2 and 2 w_t c_t are exact fp64 numbers, each an integer multiple of 2^-226
// (the lowest bit of an fp32 subnormal times an fp16 subnormal, times the 53-bit
// significand's span) and below 2^146.  Positive and negative terms are added into two
// unsigned 384-bit integers in units of 2^-226 (six 64-bit limbs; at most 4V <= 64 terms
// stay below 2^152), which are then compared.
constexpr int kUnitExp = -226;

__device__ __forceinline__ void exact_acc(uint64_t (&a)[6], double x) {  // x > 0, as above
  const uint64_t bits = __builtin_bit_cast(uint64_t, x);
  const int sh = (int)(bits >> 52) - 1075 - kUnitExp;  // x = m 2^(sh + kUnitExp), 1 <= sh < 320
  const uint64_t m = (bits & ((1ull << 52) - 1ull)) | (1ull << 52);
  const int q = sh >> 6, r = sh & 63;
  const uint64_t lo = m << r;
  const uint64_t hi = r ? (m >> (64 - r)) : 0ull;
  uint64_t carry = 0;
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const uint64_t add = (j == q) ? lo : ((j == q + 1) ? hi : 0ull);
    const uint64_t t = a[j] + add;
    const uint64_t t2 = t + carry;
    carry = (uint64_t)(t < add) | (uint64_t)(t2 < carry);
    a[j] = t2;
  }
}

// Sign of d(a) - d(b), d(c) = sum_t c_t^2 - 2 w_t c_t, all values finite: -1, 0 or 1.
template <int V>
__device__ __noinline__ int exact_order(const double* w, const double* ca, const double* cb) {
  uint64_t pos[6] = {0, 0, 0, 0, 0, 0}, neg[6] = {0, 0, 0, 0, 0, 0};
  auto put = [&](double x) {
    if (x > 0.0) exact_acc(pos, x);
    else if (x < 0.0) exact_acc(neg, -x);
  };
  for (int t = 0; t < V; ++t) {
    const double a = ca[t], b = cb[t];
    put(a * a);
    put(-(b * b));
    put(-2.0 * (w[t] * a));
    put(2.0 * (w[t] * b));
  }
  for (int j = 5; j >= 0; --j) {
    if (pos[j] != neg[j]) return pos[j] > neg[j] ? 1 : -1;
  }
  return 0;
}

// Nearest centroid for vectors or books with NaN or infinite values (or anything else):
// the distance of a centroid is NaN when a coordinate is NaN or holds the same infinity in
// w and c, +inf when a coordinate is infinite, finite otherwise.  The lowest index of the
// exact smallest finite distance, else the lowest +inf one, else 0.  Finite distances are
// ranked in fp64 with each centroid's own bound and near ones ordered exactly.
template <int V>
__device__ __noinline__ uint32_t nearest_general(const double* w, const double* __restrict__ tab, int32_t k) {
  for (int t = 0; t < V; ++t) {
    if (__builtin_isnan(w[t])) return 0u;
  }
  bool have = false;
  double bd = 0.0, be = 0.0;
  uint32_t bi = 0;
  int32_t first_inf = -1;
  for (int32_t c = 0; c < k; ++c) {
    const double* rec = tab + (size_t)c * (V + 1);
    bool nan = false, inf = false;
    double dot = 0.0, sabs = 0.0;
    for (int t = 0; t < V; ++t) {
      const double ct = rec[1 + t];
      const bool wi = __builtin_isinf(w[t]), ci = __builtin_isinf(ct);
      nan = nan || __builtin_isnan(ct) || (wi && ci && ((w[t] > 0.0) == (ct > 0.0)));
      inf = inf || wi || ci;
      dot = fma(w[t], ct, dot);
      sabs = fma(fabs(w[t]), fabs(ct), sabs);
    }
    if (nan) continue;
    if (inf) {
      if (first_inf < 0) first_inf = c;
      continue;
    }
    const double d = fma(-2.0, dot, rec[0]);
    const double e = (V + 2) * 0x1p-53 * (rec[0] + 2.0 * sabs) * (1.0 + 0x1p-20);
    if (!have || d + e < bd - be) {
      have = true;
      bd = d;
      be = e;
      bi = (uint32_t)c;
    } else if (d - e <= bd + be && exact_order<V>(w, rec + 1, tab + (size_t)bi * (V + 1) + 1) < 0) {
      bd = d;
      be = e;
      bi = (uint32_t)c;
    }
  }
  return have ? bi : (first_inf >= 0 ? (uint32_t)first_inf : 0u);
}

// Lowest index of the exact minimum, for each of the lane's R vectors whose values and
// book are finite (the others are marked).  The record of centroid c + 1 is loaded while
// centroid c is ranked.  Every decision taken is certain: a centroid replaces the best
// only when its fp64 value is below the best's by more than the pair bound T; one within T
// of the best marks the vector instead.  An unmarked result is therefore the exact
// nearest.  The loop keeps lim = best + T (one compare per centroid); T is held in fp32,
// rounded upwards, and is NaN for vectors that are marked from the start.
template <int V, int R>
__device__ __forceinline__ void nearest(const double (&w)[R][V], const double* __restrict__ tab, int32_t k,
                                        const float (&T)[R], uint32_t (&best_i)[R]) {
  double lim[R];
  uint32_t marks = 0;  // bit r: vector r needs the exact ranking
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool ok = T[r] == T[r];
    lim[r] = ok ? __builtin_inf() : -__builtin_inf();
    best_i[r] = 0;
    marks |= ok ? 0u : 1u << r;
  }
  double cur[V + 1];
#pragma unroll
  for (int t = 0; t <= V; ++t) cur[t] = tab[t];  // uniform: the same record for every lane
  for (int32_t c = 0; c < k; ++c) {
    const double* nrec = tab + (size_t)min(c + 1, k - 1) * (V + 1);
    double nxt[V + 1];
#pragma unroll
    for (int t = 0; t <= V; ++t) nxt[t] = nrec[t];
    double d[R];
    bool look = false;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      double dot = fma(w[r][0], cur[1], 0.0);
#pragma unroll
      for (int t = 1; t < V; ++t) dot = fma(w[r][t], cur[1 + t], dot);
      d[r] = fma(-2.0, dot, cur[0]);
      look |= d[r] <= lim[r];
    }
    if (__any(look)) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (d[r] <= lim[r]) {
          const double t = (double)T[r];
          if (d[r] < lim[r] - 2.0 * t) {  // below best - T
            lim[r] = d[r] + t;
            best_i[r] = (uint32_t)c;
          } else {
            marks |= 1u << r;
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t <= V; ++t) cur[t] = nxt[t];
  }
#pragma unroll
  for (int r = 0; r < R; ++r) best_i[r] |= (marks >> r) & 1u ? kMark : 0u;
}

// Per-vector pair bound: NaN (marked from the start) for vectors or books with non-finite
// values, else the bound of `pair_bound` rounded up to fp32.
template <int V, int R>
__device__ __forceinline__ void walk_setup(const double (&w)[R][V], double2 bm, float (&T)[R]) {
  const bool book_ok = bm.x < __builtin_inf() && bm.y < __builtin_inf();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    double sw = 0.0;
    bool fin = book_ok;
#pragma unroll
    for (int t = 0; t < V; ++t) {
      sw += fabs(w[r][t]);
      fin = fin && __builtin_isfinite(w[r][t]);
    }
    T[r] = fin ? __double2float_ru(pair_bound<V>(sw, bm.x, bm.y)) : __builtin_nanf("");
  }
}

template <int V, int R, int WT, bool FIRST>
__global__ __launch_bounds__(kThreads) void assign_kernel(const void* __restrict__ w, int64_t nvec,
                                                          const double* __restrict__ tab1,
                                                          const double2* __restrict__ tmax1, int32_t k1,
                                                          const double* __restrict__ tab2,
                                                          const double2* __restrict__ tmax2, int32_t k2,
                                                          uint32_t* __restrict__ idx1, uint32_t* __restrict__ idx2) {
  const int64_t base = (int64_t)blockIdx.x * (kThreads * R) + threadIdx.x;
  double wv[R][V];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t g = min(base + (int64_t)r * kThreads, nvec - 1);  // lanes past the end rank a copy
#pragma unroll
    for (int t = 0; t < V; ++t) wv[r][t] = weight_at<WT>(w, g * V + t);
  }
  float T[R];
  uint32_t i1[R];
  if constexpr (FIRST) {
    walk_setup<V, R>(wv, book_max(tmax1, k1), T);
    nearest<V, R>(wv, tab1, k1, T, i1);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t g = base + (int64_t)r * kThreads;
      if (g < nvec) idx1[g] = i1[r];
    }
    if (k2 == 0) return;
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) i1[r] = idx1[min(base + (int64_t)r * kThreads, nvec - 1)];
  }
  // residual in fp32, held exactly in fp64 (a marked main index is ranked again, both
  // stages, by the fix-up kernel; its residual here only has to be a valid one)
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const double* rec = tab1 + (size_t)(i1[r] & ~kMark) * (V + 1);
#pragma unroll
    for (int t = 0; t < V; ++t) wv[r][t] = (double)((float)wv[r][t] - (float)rec[1 + t]);
  }
  walk_setup<V, R>(wv, book_max(tmax2, k2), T);
  uint32_t i2[R];
  nearest<V, R>(wv, tab2, k2, T, i2);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t g = base + (int64_t)r * kThreads;
    if (g < nvec) idx2[g] = i2[r];
  }
}

// ---------------------------------------------------------------------------------------
// Matrix-core pass for stage 1 with fp16 weights.  The matrix cores form, for 32 centroids
// x 32 vectors at a time, the fp32 half-distance h = |c|^2 / 2 - w . c
// (v_mfma_f32_32x32x16_f16 with A = -c, B = w, C = fl32(|c|^2 / 2), K = 16 holding v <= 16
// coordinates and zeros).  Each product of two fp16 values is exact in fp32, so h differs
// from the exact half-distance by at most E = (v + 2) 2^-23 (S_w Cmax + NCmax / 2), with
// S_w = sum |w_t| and Cmax, NCmax the largest |c_t| and |c|^2 of the book (the sum of
// v + 1 terms with at most 2^-23 relative error per addition, and the rounding of C).  If
// k* is the exact nearest centroid and m the smallest h seen so far, then h(k*) <= m + 2E
// at every point of the walk.  Each lane therefore keeps a threshold thr = min over seen
// tiles of (tile minimum + delta), delta = 4 (v + 2) 2^-23 (S_w Cmax + NCmax / 2) (twice
// the bound, which also covers the rounding of thr itself), and ranks every centroid with
// h <= thr in fp64 with the same near-tie rule as the walk above (exact comparison within
// the fp64 bound); k* is always among them.  A 32x32 block costs one MFMA, eight
// three-way minima and a compare; the fp64 ranking runs only where a block holds a
// candidate (a new running minimum or a near tie), about one block in eight for 65536
// centroids.  Vectors with NaN or infinite values, and every vector of a book holding
// such values, skip the candidates and take nearest_general on the fp64 records at the
// end.  The matrix cores must multiply fp16 subnormals exactly (they do on gfx950; a
// book of subnormals is among the tests).
//
// Work split: 256 threads = 4 wavefronts; a wavefront owns kGroups groups of 32 vectors
// (B operands in registers for the whole walk); lanes l and l + 32 share vector l % 32
// (coordinates 0 .. 7 and 8 .. 15 of the B operand, and rows 4 .. 7 of every 8 in the
// output), and combine their results at the end.  The book is staged through LDS in chunks of
// kChunk centroids, double-buffered, one barrier per chunk.

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kChunk = 512;                                // centroids per LDS chunk
constexpr int kTile = 32;                                  // centroids per MFMA tile
constexpr int kGroups = 4;                                 // 32-vector groups per wavefront
constexpr int kMfmaVectors = (kThreads / 64) * kGroups * 32;  // vectors per workgroup

struct MfmaTable {
  const uint16_t* a16;  // [kp][KB][8] fp16: -c, zero padded
  const float* cf;      // [kp] fl32(|c|^2 / 2), +inf on padding rows
  const float2* bmax;   // [nbmax] per-256-centroid {max |c_t|, max |c|^2}
  int32_t nbmax, kp;
};

// Smallest of the 16 values of an MFMA result; NaN if any of them is NaN (IEEE minimum,
// which propagates NaN and so needs no quieting of its inputs).
__device__ __forceinline__ float min16(const f32x16_t& d) {
  auto mn = [](float a, float b) { return __builtin_elementwise_minimum(a, b); };
  const float m0 = mn(mn(d[0], d[1]), d[2]);
  const float m1 = mn(mn(d[3], d[4]), d[5]);
  const float m2 = mn(mn(d[6], d[7]), d[8]);
  const float m3 = mn(mn(d[9], d[10]), d[11]);
  const float m4 = mn(mn(d[12], d[13]), d[14]);
  return mn(mn(mn(m0, m1), mn(m2, m3)), mn(m4, d[15]));
}

template <int KB>
__global__ __launch_bounds__(kThreads) void assign_mfma_table_kernel(const uint16_t* __restrict__ cb, int32_t k,
                                                                     int32_t kp, int32_t v,
                                                                     uint16_t* __restrict__ a16,
                                                                     float* __restrict__ cf,
                                                                     float2* __restrict__ bmax) {
  __shared__ float2 red[kThreads / 64];
  const int32_t c = blockIdx.x * kThreads + threadIdx.x;  // grid covers kp exactly
  float cm = 0.f, nm = 0.f;
  uint16_t* row = a16 + (size_t)c * (KB * 8);
  if (c < k) {
    double nc = 0.0;
    for (int t = 0; t < KB * 8; ++t) {
      uint16_t hbits = 0;
      if (t < v) {
        hbits = cb[(size_t)c * v + t];
        const double ct = (double)vqd::f16_to_f32(hbits);
        nc = fma(ct, ct, nc);
        cm = fmaxf(cm, fabsf((float)ct));
        hbits ^= 0x8000u;  // -c
      }
      row[t] = hbits;
    }
    cf[c] = (float)(nc * 0.5);
    nm = (float)nc;
    if (!(cm <= __builtin_inff()) || !(nm <= __builtin_inff())) cm = nm = __builtin_inff();  // NaN: rank all
  } else {
    for (int t = 0; t < KB * 8; ++t) row[t] = 0;
    cf[c] = __builtin_inff();
  }
  for (int o = 32; o > 0; o >>= 1) {
    cm = fmaxf(cm, __shfl_xor(cm, o));
    nm = fmaxf(nm, __shfl_xor(nm, o));
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = make_float2(cm, nm);
  __syncthreads();
  if (threadIdx.x == 0) {
    float2 m = red[0];
    for (int i = 1; i < kThreads / 64; ++i) m = make_float2(fmaxf(m.x, red[i].x), fmaxf(m.y, red[i].y));
    bmax[blockIdx.x] = m;
  }
}

// The lane's whole vector in fp64: coordinates 8 h .. 8 h + 7 from its own B operand, the
// others from the partner lane (l ^ 32).  Every lane of the wave must call this.
template <int V>
__device__ __forceinline__ void gather_vector(const half8_t& bv, int h, double (&wv)[V]) {
  const uint4 own = __builtin_bit_cast(uint4, bv);
  uint4 oth;
  oth.x = (uint32_t)__shfl_xor((int)own.x, 32);
  oth.y = (uint32_t)__shfl_xor((int)own.y, 32);
  oth.z = (uint32_t)__shfl_xor((int)own.z, 32);
  oth.w = (uint32_t)__shfl_xor((int)own.w, 32);
#pragma unroll
  for (int t = 0; t < V; ++t) {
    const uint4 u = ((t >> 3) == h) ? own : oth;
    const int e = t & 7;
    const uint32_t word = e < 2 ? u.x : e < 4 ? u.y : e < 6 ? u.z : u.w;
    wv[t] = (double)vqd::f16_to_f32((e & 1) ? (word >> 16) : (word & 0xFFFFu));
  }
}

template <int V>
__global__ __launch_bounds__(kThreads) void assign_mfma_kernel(const uint16_t* __restrict__ w, int64_t nvec,
                                                               const uint16_t* __restrict__ a16,
                                                               const float* __restrict__ cf,
                                                               const float2* __restrict__ bmax, int32_t nbmax,
                                                               int32_t kp, int32_t k1,
                                                               uint32_t* __restrict__ idx1) {
  constexpr int KB = (V + 7) / 8;     // 8-wide K blocks
  constexpr int R = kGroups;
  constexpr int kAWords = kChunk * KB;  // uint4 (8 fp16) per (centroid, K block)
  __shared__ uint4 sa[2][kAWords];
  __shared__ float4 sc[2][kChunk / 4];
  __shared__ float2 sred[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, col = lane & 31;

  // book maxima
  float cmax = 0.f, ncmax = 0.f;
  for (int i = tid; i < nbmax; i += kThreads) {
    const float2 m = bmax[i];
    cmax = fmaxf(cmax, m.x);
    ncmax = fmaxf(ncmax, m.y);
  }
  for (int o = 32; o > 0; o >>= 1) {
    cmax = fmaxf(cmax, __shfl_xor(cmax, o));
    ncmax = fmaxf(ncmax, __shfl_xor(ncmax, o));
  }
  if (lane == 0) sred[wave] = make_float2(cmax, ncmax);

  // B operands: lane (col, h) holds coordinates 8 h .. 8 h + 7 of vector col of each group
  const int64_t vbase = (int64_t)blockIdx.x * kMfmaVectors + (int64_t)wave * (R * 32) + col;
  half8_t b[R];
  float swp[R];
  bool fast[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint16_t* wp = w + min(vbase + r * 32, nvec - 1) * V;  // lanes past the end rank a copy
    float sw = 0.f;
    bool fin = true;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int t = 8 * h + q;
      const uint16_t hv = t < V ? wp[t] : (uint16_t)0;
      b[r][q] = __builtin_bit_cast(_Float16, hv);
      sw += fabsf(vqd::f16_to_f32(hv));
      fin = fin && (hv & 0x7C00u) != 0x7C00u;
    }
    swp[r] = sw + __shfl_xor(sw, 32);
    fast[r] = fin && __shfl_xor((int)fin, 32);
  }
  __syncthreads();
  cmax = fmaxf(fmaxf(sred[0].x, sred[1].x), fmaxf(sred[2].x, sred[3].x));
  ncmax = fmaxf(fmaxf(sred[0].y, sred[1].y), fmaxf(sred[2].y, sred[3].y));
  const bool book_ok = cmax < __builtin_inff() && ncmax < __builtin_inff();
  float thr[R], tb[R];
  double best[R];
  uint32_t bi[R];
  uint32_t marks = 0;  // bit r: vector r needs the exact ranking
#pragma unroll
  for (int r = 0; r < R; ++r) {
    // vectors or books with non-finite values are marked from the start; their threshold
    // of -inf keeps them out of the candidate ranking (but for NaN / -inf entries, whose
    // result is discarded anyway)
    const bool ok = fast[r] && book_ok;
    thr[r] = ok ? __builtin_inff() : -__builtin_inff();
    best[r] = __builtin_inf();
    bi[r] = 0;
    marks |= ok ? 0u : 1u << r;
    // the fp64 pair bound (|c_t| is exact in fp32; |c|^2 and the sum of |w_t| are rounded,
    // hence the margins), held in fp32 rounded upwards
    tb[r] = __double2float_ru(
        pair_bound<V>((double)swp[r] * (1.0 + 0x1p-18), (double)cmax, (double)ncmax * (1.0 + 0x1p-20)));
  }
  // the fp32 threshold margin, computed where used
  auto delta = [&](int r) { return (4.f * (V + 2) * 0x1p-23f) * (swp[r] * cmax + 0.5f * ncmax) + 0x1p-100f; };

  // chunk staging: thread tid copies A words tid, tid + 256, ... and C quad tid (< kChunk / 4)
  constexpr int kAPer = kAWords / kThreads;
  static_assert(kAPer == 2 || kAPer == 4, "chunk staging takes two or four words per thread");
  uint4 ra0, ra1, ra2, ra3;  // staging registers (ra2, ra3 for two K blocks)
  float4 rc;
  const uint4* ga = (const uint4*)a16;
  const float4* gc = (const float4*)cf;
  const int nch = kp / kChunk;
#pragma unroll
  for (int i = 0; i < kAPer; ++i) sa[0][tid + i * kThreads] = ga[tid + i * kThreads];
  if (tid < kChunk / 4) sc[0][tid] = gc[tid];
  __syncthreads();
  for (int ch = 0; ch < nch; ++ch) {
    const int buf = ch & 1;
    // next chunk (the last one again at the end) into registers while this one is walked
    const size_t nx = (size_t)min(ch + 1, nch - 1);
    ra0 = ga[nx * kAWords + tid];
    ra1 = ga[nx * kAWords + tid + kThreads];
    if constexpr (kAPer == 4) {
      ra2 = ga[nx * kAWords + tid + 2 * kThreads];
      ra3 = ga[nx * kAWords + tid + 3 * kThreads];
    }
    rc = gc[nx * (kChunk / 4) + (tid & (kChunk / 4 - 1))];
    for (int tt = 0; tt < kChunk / kTile; ++tt) {
      const int c0 = tt * kTile;
      // A operand: row c0 + col, coordinates 8 h .. 8 h + 7 (zero past the book's K blocks)
      half8_t a = __builtin_bit_cast(half8_t, sa[buf][(c0 + col) * KB + (KB == 2 ? h : 0)]);
      if constexpr (KB == 1) a = h ? half8_t{} : a;
      f32x16_t cv;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 f = sc[buf][(c0 + 8 * g + 4 * h) >> 2];
        cv[4 * g] = f.x;
        cv[4 * g + 1] = f.y;
        cv[4 * g + 2] = f.z;
        cv[4 * g + 3] = f.w;
      }
      float tmin[R];
      bool any = false;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const f32x16_t d = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b[r], cv, 0, 0, 0);
        tmin[r] = min16(d);
        any |= !(tmin[r] > thr[r]);
      }
      if (__any(any)) {
        // a tile holds candidates: tighten the thresholds, rank the candidates in fp64
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const bool trig = !(tmin[r] > thr[r]);
          if (__any(trig)) {
            const f32x16_t d = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b[r], cv, 0, 0, 0);
            double wv[V];
            gather_vector<V>(b[r], h, wv);
            if (trig) {  // (fp64 candidates ranked in increasing index order)
              thr[r] = fminf(thr[r], tmin[r] + delta(r));
              const double T = (double)tb[r];
              uint32_t cand = 0;
#pragma unroll
              for (int q = 0; q < 16; ++q) cand |= (d[q] > thr[r] ? 0u : 1u) << q;
              while (cand) {
                const int q = __builtin_ctz(cand);
                cand &= cand - 1;
                const int ci = c0 + 8 * (q >> 2) + 4 * h + (q & 3);  // row of the chunk
                const int32_t k = ch * kChunk + ci;
                if (k < k1) {
                  // the fp64 ranking, on the centroid's fp16 values from the chunk in LDS
                  double nc = 0.0, dot = 0.0;
#pragma unroll
                  for (int kb = 0; kb < KB; ++kb) {
                    const uint4 u = sa[buf][ci * KB + kb];
                    const uint32_t words[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                      const int t = kb * 8 + e;
                      if (t < V) {
                        const uint32_t neg = (e & 1) ? (words[e >> 1] >> 16) : (words[e >> 1] & 0xFFFFu);
                        const double ct = (double)vqd::f16_to_f32(neg ^ 0x8000u);
                        nc = fma(ct, ct, nc);
                        dot = fma(wv[t], ct, dot);
                      }
                    }
                  }
                  const double dd = fma(-2.0, dot, nc);
                  if (dd < best[r] - T) {  // certainly nearer
                    best[r] = dd;
                    bi[r] = (uint32_t)k;
                  } else if (dd <= best[r] + T) {  // too close to tell in fp64
                    marks |= 1u << r;
                  }
                }
              }
            }
          }
        }
      }
    }
    sa[buf ^ 1][tid] = ra0;
    sa[buf ^ 1][tid + kThreads] = ra1;
    if constexpr (kAPer == 4) {
      sa[buf ^ 1][tid + 2 * kThreads] = ra2;
      sa[buf ^ 1][tid + 3 * kThreads] = ra3;
    }
    if (tid < kChunk / 4) sc[buf ^ 1][tid] = rc;
    __syncthreads();
  }
  // lanes l and l + 32 hold the same vector: the certainly smaller distance, else a mark
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const double ob = __shfl_xor(best[r], 32);
    const uint32_t oi = (uint32_t)__shfl_xor((int)bi[r], 32);
    const uint32_t om = (uint32_t)__shfl_xor((int)marks, 32);
    const double T = (double)tb[r];
    uint32_t pick = bi[r], m = ((marks | om) >> r) & 1u ? kMark : 0u;
    if (ob < best[r] - T) {
      pick = oi;
    } else if (!(ob > best[r] + T)) {
      m = kMark;
    }
    const int64_t g = vbase + r * 32;
    if (h == 0 && g < nvec) idx1[g] = pick | m;
  }
}

// Marked vectors ranked again with exact comparisons: the main stage when its index is
// marked (then the residual stage too, from the new residual), else the residual stage
// when that index is marked.
template <int V, int WT>
__global__ __launch_bounds__(kThreads) void assign_fixup_kernel(const void* __restrict__ w, int64_t nvec,
                                                                const double* __restrict__ tab1, int32_t k1,
                                                                const double* __restrict__ tab2, int32_t k2,
                                                                uint32_t* __restrict__ idx1,
                                                                uint32_t* __restrict__ idx2) {
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (g >= nvec) return;
  uint32_t i1 = idx1[g];
  uint32_t i2 = k2 ? idx2[g] : 0u;
  if (!((i1 | i2) & kMark)) return;
  double wv[V];
  for (int t = 0; t < V; ++t) wv[t] = weight_at<WT>(w, g * V + t);
  const bool redo1 = (i1 & kMark) != 0;
  if (redo1) {
    i1 = nearest_general<V>(wv, tab1, k1);
    idx1[g] = i1;
  }
  if (k2 && (redo1 || (i2 & kMark))) {
    const double* rec = tab1 + (size_t)i1 * (V + 1);
    for (int t = 0; t < V; ++t) wv[t] = (double)((float)wv[t] - (float)rec[1 + t]);
    idx2[g] = nearest_general<V>(wv, tab2, k2);
  }
}

template <int V>
vq_status launch_v(const void* w, vq_dtype w_dtype, int64_t nvec, const double* tab1, const double2* tmax1, int32_t k1,
                   const double* tab2, const double2* tmax2, int32_t k2, uint32_t* idx1, uint32_t* idx2,
                   const MfmaTable* mt, hipStream_t s) {
  constexpr int R = V <= 4 ? 4 : 2;
  const int64_t blocks = (nvec + (int64_t)kThreads * R - 1) / ((int64_t)kThreads * R);
  if (blocks > 0x7FFFFFFF) return VQ_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)blocks), block(kThreads);
  if (mt) {
    const int64_t mblocks = (nvec + kMfmaVectors - 1) / kMfmaVectors;
    if (mblocks > 0x7FFFFFFF) return VQ_ERR_UNSUPPORTED;
    hipLaunchKernelGGL((assign_mfma_kernel<V>), dim3((unsigned)mblocks), dim3(kThreads), 0, s, (const uint16_t*)w,
                       nvec, mt->a16, mt->cf, mt->bmax, mt->nbmax, mt->kp, k1, idx1);
    if (k2) {
      hipLaunchKernelGGL((assign_kernel<V, R, VQ_F16, false>), grid, block, 0, s, w, nvec, tab1, tmax1, k1, tab2, tmax2, k2,
                         idx1, idx2);
    }
  } else if (w_dtype == VQ_F16) {
    hipLaunchKernelGGL((assign_kernel<V, R, VQ_F16, true>), grid, block, 0, s, w, nvec, tab1, tmax1, k1, tab2, tmax2, k2,
                       idx1, idx2);
  } else if (w_dtype == VQ_BF16) {
    hipLaunchKernelGGL((assign_kernel<V, R, VQ_BF16, true>), grid, block, 0, s, w, nvec, tab1, tmax1, k1, tab2, tmax2, k2,
                       idx1, idx2);
  } else {
    hipLaunchKernelGGL((assign_kernel<V, R, VQ_F32, true>), grid, block, 0, s, w, nvec, tab1, tmax1, k1, tab2, tmax2, k2,
                       idx1, idx2);
  }
  const dim3 fgrid((unsigned)((nvec + kThreads - 1) / kThreads));
  if (w_dtype == VQ_F16) {
    hipLaunchKernelGGL((assign_fixup_kernel<V, VQ_F16>), fgrid, block, 0, s, w, nvec, tab1, k1, tab2, k2, idx1, idx2);
  } else if (w_dtype == VQ_BF16) {
    hipLaunchKernelGGL((assign_fixup_kernel<V, VQ_BF16>), fgrid, block, 0, s, w, nvec, tab1, k1, tab2, k2, idx1, idx2);
  } else {
    hipLaunchKernelGGL((assign_fixup_kernel<V, VQ_F32>), fgrid, block, 0, s, w, nvec, tab1, k1, tab2, k2, idx1, idx2);
  }
  return VQ_OK;
}

}  // namespace

namespace {

// Workspace layout: the fp64 records of both books, their per-256-centroid maxima, then
// (K1 >= 256) the matrix-core tables of the main book, each part 256-byte aligned.
struct WsLayout {
  size_t tab, tmax1, tmax2, a16, cf, bmax, total;
  int32_t kp;
  bool mfma;
};

inline size_t up256(size_t b) { return (b + 255) & ~(size_t)255; }

WsLayout ws_layout(const vq_desc& d) {
  WsLayout l{};
  const size_t k1 = (size_t)1 << d.bits1, k2 = d.bits2 ? (size_t)1 << d.bits2 : 0;
  l.tab = 0;
  size_t off = up256((k1 + k2) * (size_t)(d.v + 1) * sizeof(double));
  l.tmax1 = off;
  off += up256((k1 + kThreads - 1) / kThreads * sizeof(double2));
  l.tmax2 = off;
  off += up256((k2 + kThreads - 1) / kThreads * sizeof(double2));
  l.mfma = d.bits1 >= 8;
  if (l.mfma) {
    const int kb = (d.v + 7) / 8;
    l.kp = (int32_t)((k1 + kChunk - 1) / kChunk * kChunk);
    l.a16 = off;
    off += up256((size_t)l.kp * kb * 16);
    l.cf = off;
    off += up256((size_t)l.kp * sizeof(float));
    l.bmax = off;
    off += up256((size_t)(l.kp / kThreads) * sizeof(float2));
  }
  l.total = off;
  return l;
}

}  // namespace

namespace vqi {

size_t assign_workspace(const vq_desc& d) { return ws_layout(d).total; }

vq_status launch_assign(const vq_desc& d, const void* w, vq_dtype w_dtype, const uint16_t* cb1, const uint16_t* cb2,
                        uint32_t* idx1, uint32_t* idx2, void* workspace, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const WsLayout l = ws_layout(d);
  const int32_t k1 = 1 << d.bits1, k2 = d.bits2 ? 1 << d.bits2 : 0;
  char* ws = (char*)workspace;
  double* tab1 = (double*)(ws + l.tab);
  double* tab2 = tab1 + (size_t)k1 * (d.v + 1);
  double2* tmax1 = (double2*)(ws + l.tmax1);
  double2* tmax2 = (double2*)(ws + l.tmax2);
  hipLaunchKernelGGL(assign_table_kernel, dim3((k1 + kThreads - 1) / kThreads), dim3(kThreads), 0, s, cb1, k1, d.v,
                     tab1, tmax1);
  if (k2) {
    hipLaunchKernelGGL(assign_table_kernel, dim3((k2 + kThreads - 1) / kThreads), dim3(kThreads), 0, s, cb2, k2, d.v,
                       tab2, tmax2);
  }
  MfmaTable mt{};
  const MfmaTable* mtp = nullptr;
  if (l.mfma && w_dtype == VQ_F16) {
    mt.a16 = (const uint16_t*)(ws + l.a16);
    mt.cf = (const float*)(ws + l.cf);
    mt.bmax = (const float2*)(ws + l.bmax);
    mt.kp = l.kp;
    mt.nbmax = l.kp / kThreads;
    if (d.v > 8) {
      hipLaunchKernelGGL(assign_mfma_table_kernel<2>, dim3(mt.nbmax), dim3(kThreads), 0, s, cb1, k1, l.kp, d.v,
                         (uint16_t*)mt.a16, (float*)mt.cf, (float2*)mt.bmax);
    } else {
      hipLaunchKernelGGL(assign_mfma_table_kernel<1>, dim3(mt.nbmax), dim3(kThreads), 0, s, cb1, k1, l.kp, d.v,
                         (uint16_t*)mt.a16, (float*)mt.cf, (float2*)mt.bmax);
    }
    mtp = &mt;
  }
  const int64_t nvec = (int64_t)d.out_features * (d.in_features / d.v);
  vq_status st = VQ_OK;
  switch (d.v) {
#define VQ_ASSIGN_CASE(V)                                                        \
  case V:                                                                        \
    st = launch_v<V>(w, w_dtype, nvec, tab1, tmax1, k1, tab2, tmax2, k2, idx1, idx2, mtp, s); \
    break;
    VQ_ASSIGN_CASE(1)
    VQ_ASSIGN_CASE(2)
    VQ_ASSIGN_CASE(3)
    VQ_ASSIGN_CASE(4)
    VQ_ASSIGN_CASE(5)
    VQ_ASSIGN_CASE(6)
    VQ_ASSIGN_CASE(7)
    VQ_ASSIGN_CASE(8)
    VQ_ASSIGN_CASE(9)
    VQ_ASSIGN_CASE(10)
    VQ_ASSIGN_CASE(11)
    VQ_ASSIGN_CASE(12)
    VQ_ASSIGN_CASE(13)
    VQ_ASSIGN_CASE(14)
    VQ_ASSIGN_CASE(15)
    VQ_ASSIGN_CASE(16)
#undef VQ_ASSIGN_CASE
    default:
      return VQ_ERR_UNSUPPORTED;
  }
  if (st != VQ_OK) return st;
  return hipGetLastError() == hipSuccess ? VQ_OK : VQ_ERR_HIP;
}

}  // namespace vqi
