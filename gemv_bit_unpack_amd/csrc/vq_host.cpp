// Host side of libvq: descriptor and argument validation, the index packer and the
// exported C entry points.  Everything here runs on the CPU; the kernels live in the
// .hip units and are reached through the launch_* functions.
#include <algorithm>
#include <atomic>
#include <cstring>
#include <new>
#include <thread>
#include <vector>

#include "vq_internal.h"

namespace vqi {

vq_status check_desc(const vq_desc* d) {
  if (!d) return VQ_ERR_NULL;
  if (d->v < 1 || d->v > 16) return VQ_ERR_BITS;
  if (d->bits1 < 1 || d->bits1 > 16) return VQ_ERR_BITS;
  if (d->bits2 < 0 || d->bits2 > 16) return VQ_ERR_BITS;
  if (d->out_features < 0 || d->in_features < 0) return VQ_ERR_SHAPE;
  if (d->layout != VQ_LAYOUT_ROWSTREAM) return VQ_ERR_UNSUPPORTED;
  return VQ_OK;
}

vq_status check_desc_any(const vq_desc* d) {
  if (d && d->layout == VQ_LAYOUT_BUCKETED) {
    vq_desc rs = *d;
    rs.layout = VQ_LAYOUT_ROWSTREAM;
    const vq_status st = check_desc(&rs);
    if (st != VQ_OK) return st;
    return bucketed_gemv_shape_ok(*d) ? VQ_OK : VQ_ERR_UNSUPPORTED;
  }
  return check_desc(d);
}

static bool valid_x_dtype(vq_dtype t) { return t == VQ_F16 || t == VQ_BF16; }
static bool valid_out_dtype(vq_dtype t) { return t == VQ_F16 || t == VQ_BF16 || t == VQ_F32; }
static size_t dtype_size(vq_dtype t) { return t == VQ_F32 ? 4 : 2; }

vq_status prepare_product(const vq_desc* desc, const void* packed, const void* cb1, const void* cb2,
                          const void* scale, const void* bias, const void* x, vq_dtype x_dtype, int32_t m, void* y,
                          vq_dtype y_dtype, int32_t max_m, ProductArgs* a) {
  vq_status st = check_desc(desc);
  if (st != VQ_OK) return st;
  if (m < 0 || (max_m > 0 && m > max_m)) return VQ_ERR_SHAPE;
  if (!valid_x_dtype(x_dtype) || !valid_out_dtype(y_dtype)) return VQ_ERR_UNSUPPORTED;
  const vq_desc& d = *desc;
  std::memset(a, 0, sizeof *a);
  a->n = d.out_features;
  a->in_features = d.in_features;
  a->v = d.v;
  a->bits1 = d.bits1;
  a->bits2 = d.bits2;
  a->m = m;
  a->x_dtype = x_dtype;
  a->y_dtype = y_dtype;
  if (d.out_features == 0 || m == 0) return VQ_OK;  // nothing to compute
  if (!y) return VQ_ERR_NULL;
  if (!aligned(y, dtype_size(y_dtype))) return VQ_ERR_ALIGN;
  if (bias && !aligned(bias, 2)) return VQ_ERR_ALIGN;
  if (scale && !aligned(scale, 2)) return VQ_ERR_ALIGN;
  if (d.in_features > 0) {
    if (!packed || !cb1 || !x || (d.bits2 > 0 && !cb2)) return VQ_ERR_NULL;
    if (!aligned(packed, 4)) return VQ_ERR_ALIGN;
    if (!aligned(cb1, 2) || !aligned(x, 2) || (d.bits2 > 0 && !aligned(cb2, 2))) return VQ_ERR_ALIGN;
  }
  const int64_t s1 = row_stride(d.in_features, d.v, d.bits1);
  const int64_t s2 = row_stride(d.in_features, d.v, d.bits2);
  a->nv = (int32_t)num_vectors(d.in_features, d.v);
  a->s1_words = (int32_t)(s1 / 4);
  a->s2_words = (int32_t)(s2 / 4);
  a->packed1 = (const uint32_t*)packed;
  a->packed2 = d.bits2 > 0 ? (const uint32_t*)((const uint8_t*)packed + (size_t)d.out_features * (size_t)s1) : nullptr;
  a->cb1 = (const uint16_t*)cb1;
  a->cb2 = d.bits2 > 0 ? (const uint16_t*)cb2 : nullptr;
  a->scale = (const uint16_t*)scale;
  a->bias = (const uint16_t*)bias;
  a->x = (const uint16_t*)x;
  a->y = y;
  return VQ_OK;
}

// Products over the slice-bucketed layout (vq_gemv_ws, vq_gemv_noalloc): M = 1, 16-byte
// aligned packed / cb1 / cb2 / x.  packed1 = the prefix table, packed2 = the bucket words.
static vq_status prepare_bucketed(const vq_desc* desc, const void* packed, const void* cb1, const void* cb2,
                                  const void* scale, const void* bias, const void* x, vq_dtype x_dtype, int32_t m,
                                  void* y, vq_dtype y_dtype, ProductArgs* a) {
  vq_status st = check_desc_any(desc);
  if (st != VQ_OK) return st;
  if (m < 0 || m > 16) return VQ_ERR_SHAPE;
  if (!valid_x_dtype(x_dtype) || !valid_out_dtype(y_dtype)) return VQ_ERR_UNSUPPORTED;
  const vq_desc& d = *desc;
  std::memset(a, 0, sizeof *a);
  a->n = d.out_features;
  a->in_features = d.in_features;
  a->v = d.v;
  a->bits1 = d.bits1;
  a->bits2 = d.bits2;
  a->m = m;
  a->x_dtype = x_dtype;
  a->y_dtype = y_dtype;
  if (d.out_features == 0 || m == 0) return VQ_OK;
  if (m != 1) return VQ_ERR_UNSUPPORTED;
  if (!y) return VQ_ERR_NULL;
  if (!aligned(y, dtype_size(y_dtype))) return VQ_ERR_ALIGN;
  if ((bias && !aligned(bias, 2)) || (scale && !aligned(scale, 2))) return VQ_ERR_ALIGN;
  if (d.in_features > 0) {
    if (!packed || !cb1 || !x || (d.bits2 > 0 && !cb2)) return VQ_ERR_NULL;
    if (!aligned(packed, 16) || !aligned(cb1, 16) || !aligned(x, 16) || (d.bits2 > 0 && !aligned(cb2, 16)))
      return VQ_ERR_ALIGN;
  }
  a->nv = (int32_t)(d.in_features / 8);
  a->packed1 = (const uint32_t*)packed;
  a->packed2 = packed ? (const uint32_t*)((const uint8_t*)packed + bucketed_header_bytes(d)) : nullptr;
  a->cb1 = (const uint16_t*)cb1;
  a->cb2 = d.bits2 > 0 ? (const uint16_t*)cb2 : nullptr;
  a->scale = (const uint16_t*)scale;
  a->bias = (const uint16_t*)bias;
  a->x = (const uint16_t*)x;
  a->y = y;
  return VQ_OK;
}

// Order of the words inside one bucket.  The product hands word k of a bucket to lane
// k mod 64, and each word costs three 16-byte LDS reads (the activation vector, the main
// centroid, the residual centroid).  LDS serves such a read in one pass when lanes
// 4q .. 4q + 3 of every 16-lane group read entries whose column (entry mod 16) lies in
// 4q .. 4q + 3, rows free; the product's slice starts on a column-0 entry, so a main
// centroid's column is idx1 mod 16.  The words are therefore dealt so that word k holds,
// where the bucket's mix of indices allows, an index with idx1 mod 16 == k mod 16 (first
// pass), else one in the same group of four columns (second pass), else any left over
// (third pass), each pass in the words' order.  Only one of the three reads can be lined
// up this way: the main-book read, from the largest table.
namespace {
void align_bucket(uint32_t* w, uint32_t n, std::vector<uint32_t>& tmp) {
  if (n <= 1) return;
  tmp.assign(w, w + n);
  std::vector<uint32_t> q[16];
  for (uint32_t i = 0; i < n; ++i) q[(tmp[i] >> 10) & 15u].push_back(tmp[i]);
  uint32_t head[16] = {0};
  auto take = [&](uint32_t col, uint32_t& out) {
    if (head[col] < q[col].size()) {
      out = q[col][head[col]++];
      return true;
    }
    return false;
  };
  std::vector<uint8_t> filled(n, 0);
  for (uint32_t k = 0; k < n; ++k) filled[k] = take(k & 15u, w[k]);
  for (uint32_t k = 0; k < n; ++k) {
    if (filled[k]) continue;
    const uint32_t base = k & 12u;
    for (uint32_t c = 0; c < 4 && !filled[k]; ++c) filled[k] = take(base + ((k + c) & 3u), w[k]);
  }
  uint32_t col = 0;
  for (uint32_t k = 0; k < n; ++k) {
    if (filled[k]) continue;
    while (!take(col, w[k])) ++col;
    filled[k] = 1;
  }
}
}  // namespace

// The slice-bucketed layout of idx1 / idx2 (vq.h): bucket sizes, their prefix table, each
// row's vectors dropped into their buckets, then every bucket's words ordered for the LDS
// (buckets in parallel threads; the result does not depend on their number).  Throws
// std::bad_alloc when host memory runs out, in this thread or a worker.
static void pack_bucketed(const vq_desc& d, const uint32_t* idx1, const uint32_t* idx2, uint8_t* out) {
  const int64_t n = d.out_features;
  const int64_t nv = num_vectors(d.in_features, 8);
  const int64_t chunks = bucketed_chunks(d);
  const size_t nb = (size_t)(8 * chunks) * (size_t)n;
  uint32_t* start = (uint32_t*)out;
  uint32_t* words = (uint32_t*)(out + bucketed_header_bytes(d));
  auto bucket = [&](int64_t o, int64_t j, uint32_t i1) {
    return (size_t)((j / kBucketChunk) * 8 + (i1 >> 13)) * (size_t)n + (size_t)o;
  };
  std::vector<uint32_t> next(nb + 1, 0u);
  for (int64_t o = 0; o < n; ++o)
    for (int64_t j = 0; j < nv; ++j) ++next[bucket(o, j, idx1[o * nv + j]) + 1];
  for (size_t b = 0; b < nb; ++b) next[b + 1] += next[b];
  std::memcpy(start, next.data(), (nb + 1) * sizeof(uint32_t));
  for (int64_t o = 0; o < n; ++o) {
    for (int64_t j = 0; j < nv; ++j) {
      const uint32_t i1 = idx1[o * nv + j];
      const uint32_t i2 = d.bits2 > 0 ? idx2[o * nv + j] : 0u;
      words[next[bucket(o, j, i1)]++] = (uint32_t)(j % kBucketChunk) | ((i1 & 8191u) << 10) | (i2 << 23);
    }
  }
  const unsigned hw = std::thread::hardware_concurrency();
  const int64_t nthreads = std::max<int64_t>(1, std::min<int64_t>({(int64_t)(hw ? hw : 1), 16, (n + 63) / 64}));
  std::atomic<bool> failed{false};
  auto work = [&](int64_t t0) {
    try {  // an exception must not leave a worker thread
      std::vector<uint32_t> tmp;
      for (size_t b = (size_t)t0; b < nb; b += (size_t)nthreads)
        align_bucket(words + start[b], start[b + 1] - start[b], tmp);
    } catch (...) {
      failed.store(true);
    }
  };
  std::vector<std::thread> pool;
  int64_t started = 1;  // work shares 1 .. started - 1 run in threads
  try {
    for (; started < nthreads; ++started) pool.emplace_back(work, started);
  } catch (...) {  // no more threads: this one takes the shares that did not start
  }
  work(0);
  for (int64_t t = started; t < nthreads; ++t) work(t);
  for (auto& th : pool) th.join();
  if (failed.load()) throw std::bad_alloc();
}

// Affine-lattice calls: the descriptor must be the lattice stream (v = 4, bits1 = 8, no
// residual).  m < 0 marks the dequant (no x, y checked by the caller); max_m > 0 bounds M.
static vq_status prepare_svq(const vq_desc* desc, const void* packed, const void* a, const void* b,
                             const void* scale, const void* bias, const void* x, vq_dtype x_dtype, int32_t m,
                             void* y, vq_dtype y_dtype, int32_t max_m, SvqArgs* p) {
  vq_status st = check_desc(desc);
  if (st != VQ_OK) return st;
  const vq_desc& d = *desc;
  if (d.v != 4 || d.bits1 != 8 || d.bits2 != 0) return VQ_ERR_UNSUPPORTED;
  if (max_m > 0 && m > max_m) return VQ_ERR_SHAPE;
  if (m >= 0 && !valid_x_dtype(x_dtype)) return VQ_ERR_UNSUPPORTED;
  if (!valid_out_dtype(y_dtype)) return VQ_ERR_UNSUPPORTED;
  std::memset(p, 0, sizeof *p);
  p->n = d.out_features;
  p->in_features = d.in_features;
  p->nv = (int32_t)num_vectors(d.in_features, 4);
  p->stride = (int32_t)row_stride(d.in_features, 4, 8);
  p->m = m < 0 ? 0 : m;
  p->x_dtype = x_dtype;
  p->y_dtype = y_dtype;
  if (d.out_features == 0 || m == 0) return VQ_OK;
  if (m < 0 && d.in_features == 0) return VQ_OK;
  if (!y) return VQ_ERR_NULL;
  if (!aligned(y, dtype_size(y_dtype))) return VQ_ERR_ALIGN;
  if ((scale && !aligned(scale, 2)) || (bias && !aligned(bias, 2))) return VQ_ERR_ALIGN;
  if (d.in_features > 0) {
    if (!packed || !a || !b || (m > 0 && !x)) return VQ_ERR_NULL;
    // the product reads up to 16 code bytes per load
    if ((m > 0 && !aligned(packed, 16)) || !aligned(a, 2) || !aligned(b, 2) || (m > 0 && !aligned(x, 2)))
      return VQ_ERR_ALIGN;
  }
  p->packed = (const uint8_t*)packed;
  p->a = (const uint16_t*)a;
  p->b = (const uint16_t*)b;
  p->scale = (const uint16_t*)scale;
  p->bias = (const uint16_t*)bias;
  p->x = (const uint16_t*)x;
  p->y = y;
  p->x_vec4 = (m > 0 && d.in_features % 4 == 0 && aligned(x, 8)) ? 1 : 0;
  return VQ_OK;
}

// Appends `bits`-bit fields LSB-first into a row of 32-bit little-endian words.
struct BitWriter {
  uint8_t* row;
  uint64_t acc = 0;
  int nacc = 0;
  size_t pos = 0;
  void put(uint32_t value, int bits) {
    acc |= (uint64_t)value << nacc;
    nacc += bits;
    while (nacc >= 8) {
      row[pos++] = (uint8_t)(acc & 0xFF);
      acc >>= 8;
      nacc -= 8;
    }
  }
  void flush() {
    if (nacc > 0) row[pos++] = (uint8_t)(acc & 0xFF);
    acc = 0;
    nacc = 0;
  }
};

}  // namespace vqi

using namespace vqi;

extern "C" {

int32_t vq_abi_version(void) { return VQ_ABI_VERSION; }

const char* vq_status_string(vq_status status) {
  switch (status) {
    case VQ_OK: return "VQ_OK";
    case VQ_ERR_NULL: return "VQ_ERR_NULL: a required pointer is NULL";
    case VQ_ERR_SHAPE: return "VQ_ERR_SHAPE: invalid sizes or M out of range";
    case VQ_ERR_BITS: return "VQ_ERR_BITS: v or index bit width out of range";
    case VQ_ERR_UNSUPPORTED: return "VQ_ERR_UNSUPPORTED: combination not supported";
    case VQ_ERR_ALIGN: return "VQ_ERR_ALIGN: pointer misaligned";
    case VQ_ERR_INDEX_RANGE: return "VQ_ERR_INDEX_RANGE: index >= 2^bits";
    case VQ_ERR_BUFFER_SIZE: return "VQ_ERR_BUFFER_SIZE: packed buffer too small";
    case VQ_ERR_HIP: return "VQ_ERR_HIP: HIP runtime error";
  }
  return "unknown vq_status";
}

vq_status vq_packed_bytes(const vq_desc* desc, size_t* nbytes) {
  vq_status st = check_desc_any(desc);
  if (st != VQ_OK) return st;
  if (!nbytes) return VQ_ERR_NULL;
  *nbytes = packed_size(*desc);
  return VQ_OK;
}

vq_status vq_pack(const vq_desc* desc, const uint32_t* idx1, const uint32_t* idx2, void* packed, size_t nbytes) {
  vq_status st = check_desc_any(desc);
  if (st != VQ_OK) return st;
  const vq_desc& d = *desc;
  const size_t need = packed_size(d);
  const int64_t nv = num_vectors(d.in_features, d.v);
  const size_t count = (size_t)d.out_features * (size_t)nv;
  if (need > 0 || count > 0) {
    if (!packed || !idx1 || (d.bits2 > 0 && !idx2)) return VQ_ERR_NULL;
  }
  if (nbytes < need) return VQ_ERR_BUFFER_SIZE;
  for (int stream = 0; stream < 2; ++stream) {
    const int bits = stream == 0 ? d.bits1 : d.bits2;
    if (bits == 0) continue;
    const uint32_t* idx = stream == 0 ? idx1 : idx2;
    const uint32_t limit = (uint32_t)1 << bits;
    for (size_t i = 0; i < count; ++i)
      if (idx[i] >= limit) return VQ_ERR_INDEX_RANGE;
  }
  if (need == 0) return VQ_OK;
  uint8_t* out = (uint8_t*)packed;
  std::memset(out, 0, need);
  if (d.layout == VQ_LAYOUT_BUCKETED) {
    try {
      pack_bucketed(d, idx1, idx2, out);
    } catch (...) {  // host memory for the regrouping ran out: no exception crosses the ABI
      return VQ_ERR_BUFFER_SIZE;
    }
    return VQ_OK;
  }
  const int64_t s1 = row_stride(d.in_features, d.v, d.bits1);
  const int64_t s2 = row_stride(d.in_features, d.v, d.bits2);
  for (int stream = 0; stream < 2; ++stream) {
    const int bits = stream == 0 ? d.bits1 : d.bits2;
    if (bits == 0) continue;
    const uint32_t* idx = stream == 0 ? idx1 : idx2;
    uint8_t* base = stream == 0 ? out : out + (size_t)d.out_features * (size_t)s1;
    const int64_t stride = stream == 0 ? s1 : s2;
    for (int64_t o = 0; o < d.out_features; ++o) {
      BitWriter w{base + (size_t)o * (size_t)stride};
      const uint32_t* r = idx + (size_t)o * (size_t)nv;
      for (int64_t j = 0; j < nv; ++j) w.put(r[j], bits);
      w.flush();
    }
  }
  return VQ_OK;
}

vq_status vq_svq_pack(const vq_desc* desc, const uint8_t* q, void* packed, size_t nbytes) {
  vq_status st = check_desc(desc);
  if (st != VQ_OK) return st;
  const vq_desc& d = *desc;
  if (d.v != 4 || d.bits1 != 8 || d.bits2 != 0) return VQ_ERR_UNSUPPORTED;
  const size_t need = packed_size(d);
  const int64_t nv = num_vectors(d.in_features, 4);
  const size_t count = (size_t)d.out_features * (size_t)nv * 4;
  if ((need > 0 || count > 0) && (!packed || !q)) return VQ_ERR_NULL;
  if (nbytes < need) return VQ_ERR_BUFFER_SIZE;
  for (size_t i = 0; i < count; ++i)
    if (q[i] > 3) return VQ_ERR_INDEX_RANGE;
  if (need == 0) return VQ_OK;
  uint8_t* out = (uint8_t*)packed;
  std::memset(out, 0, need);
  const int64_t stride = row_stride(d.in_features, 4, 8);  // one byte per vector
  for (int64_t o = 0; o < d.out_features; ++o) {
    for (int64_t j = 0; j < nv; ++j) {
      const uint8_t* c = q + ((size_t)o * (size_t)nv + (size_t)j) * 4;
      out[(size_t)o * (size_t)stride + (size_t)j] = (uint8_t)(c[0] | (c[1] << 2) | (c[2] << 4) | (c[3] << 6));
    }
  }
  return VQ_OK;
}

vq_status vq_dequant(const vq_desc* desc, const void* packed, const void* cb1, const void* cb2, const void* scale,
                     void* w, vq_dtype w_dtype, void* stream) {
  vq_status st = check_desc(desc);
  if (st != VQ_OK) return st;
  if (!valid_out_dtype(w_dtype)) return VQ_ERR_UNSUPPORTED;
  const vq_desc& d = *desc;
  if (d.out_features == 0 || d.in_features == 0) return VQ_OK;
  if (!packed || !cb1 || !w || (d.bits2 > 0 && !cb2)) return VQ_ERR_NULL;
  if (!aligned(packed, 4) || !aligned(cb1, 2) || (d.bits2 > 0 && !aligned(cb2, 2)) || (scale && !aligned(scale, 2)) ||
      !aligned(w, dtype_size(w_dtype)))
    return VQ_ERR_ALIGN;
  return launch_dequant(d, packed, cb1, d.bits2 > 0 ? cb2 : nullptr, scale, w, w_dtype, stream);
}

vq_status vq_gemv(const vq_desc* desc, const void* packed, const void* cb1, const void* cb2, const void* scale,
                  const void* bias, const void* x, vq_dtype x_dtype, int32_t M, void* y, vq_dtype y_dtype,
                  void* stream) {
  ProductArgs a;
  vq_status st = prepare_product(desc, packed, cb1, cb2, scale, bias, x, x_dtype, M, y, y_dtype, 16, &a);
  if (st != VQ_OK) return st;
  if (a.n == 0 || a.m == 0) return VQ_OK;
  return launch_gemv(a, stream);
}

vq_status vq_gemv_workspace_bytes(const vq_desc* desc, int32_t M, vq_dtype x_dtype, size_t* nbytes) {
  if (!nbytes) return VQ_ERR_NULL;
  vq_status st = check_desc_any(desc);
  if (st != VQ_OK) return st;
  if (M < 0 || M > 16) return VQ_ERR_SHAPE;
  if (x_dtype != VQ_F16 && x_dtype != VQ_BF16) return VQ_ERR_UNSUPPORTED;
  if (desc->layout == VQ_LAYOUT_BUCKETED) {
    if (M > 1) return VQ_ERR_UNSUPPORTED;
    *nbytes = (M == 0 || desc->in_features == 0 || desc->out_features == 0) ? 0 : bucketed_gemv_workspace(*desc);
    return VQ_OK;
  }
  *nbytes = sliced_gemv_workspace(*desc, M, x_dtype);
  return VQ_OK;
}

vq_status vq_gemv_ws(const vq_desc* desc, const void* packed, const void* cb1, const void* cb2, const void* scale,
                     const void* bias, const void* x, vq_dtype x_dtype, int32_t M, void* y, vq_dtype y_dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
  ProductArgs a;
  if (desc && desc->layout == VQ_LAYOUT_BUCKETED) {
    vq_status st = prepare_bucketed(desc, packed, cb1, cb2, scale, bias, x, x_dtype, M, y, y_dtype, &a);
    if (st != VQ_OK) return st;
    if (a.n == 0 || a.m == 0) return VQ_OK;
    if (a.in_features == 0) return launch_gemv(a, stream);  // y = bias or 0: no index is read
    if (!workspace) return VQ_ERR_NULL;
    if (workspace_bytes < bucketed_gemv_workspace(*desc)) return VQ_ERR_BUFFER_SIZE;
    if (!aligned(workspace, 256)) return VQ_ERR_ALIGN;
    return launch_gemv_bucketed(a, workspace, stream);
  }
  vq_status st = prepare_product(desc, packed, cb1, cb2, scale, bias, x, x_dtype, M, y, y_dtype, 16, &a);
  if (st != VQ_OK) return st;
  if (a.n == 0 || a.m == 0) return VQ_OK;
  const size_t need = sliced_gemv_workspace(*desc, a.m, a.x_dtype);
  if (workspace && need > 0) {
    if (workspace_bytes < need) return VQ_ERR_BUFFER_SIZE;
    if (!aligned(workspace, 256)) return VQ_ERR_ALIGN;
    if (sliced_gemv_pointers_ok(a)) return launch_gemv_sliced(a, workspace, stream);
  }
  return launch_gemv(a, stream);
}

vq_status vq_gemv_noalloc(const vq_desc* desc, const void* packed, const void* cb1, const void* cb2,
                          const void* scale, const void* bias, const void* x, vq_dtype x_dtype, int32_t M, void* y,
                          vq_dtype y_dtype, void* stream) {
  ProductArgs a;
  if (desc && desc->layout == VQ_LAYOUT_BUCKETED) {
    vq_status st = prepare_bucketed(desc, packed, cb1, cb2, scale, bias, x, x_dtype, M, y, y_dtype, &a);
    if (st != VQ_OK) return st;
    if (a.n == 0 || a.m == 0) return VQ_OK;
    if (a.in_features == 0) return launch_gemv(a, stream);
    if (bucketed_gemv_workspace(*desc) > static_scratch_bytes()) return VQ_ERR_BUFFER_SIZE;
    void* ws = nullptr;
    st = static_scratch(&ws);
    if (st != VQ_OK) return st;
    return launch_gemv_bucketed(a, ws, stream);
  }
  vq_status st = prepare_product(desc, packed, cb1, cb2, scale, bias, x, x_dtype, M, y, y_dtype, 16, &a);
  if (st != VQ_OK) return st;
  if (a.n == 0 || a.m == 0) return VQ_OK;
  const size_t need = sliced_gemv_workspace(*desc, a.m, a.x_dtype);
  if (need == 0 || !sliced_gemv_pointers_ok(a)) return launch_gemv(a, stream);  // no workspace used
  if (need > static_scratch_bytes()) return VQ_ERR_BUFFER_SIZE;
  void* ws = nullptr;
  st = static_scratch(&ws);
  if (st != VQ_OK) return st;
  return launch_gemv_sliced(a, ws, stream);
}

vq_status vq_svq_dequant(const vq_desc* desc, const void* packed, const void* a, const void* b, const void* scale,
                         void* w, vq_dtype w_dtype, void* stream) {
  SvqArgs p;
  vq_status st = prepare_svq(desc, packed, a, b, scale, nullptr, nullptr, VQ_F16, -1, w, w_dtype, 0, &p);
  if (st != VQ_OK) return st;
  if (p.n == 0 || p.in_features == 0) return VQ_OK;
  return launch_svq_dequant(p, w, w_dtype, stream);
}

vq_status vq_svq_gemv(const vq_desc* desc, const void* packed, const void* a, const void* b, const void* scale,
                      const void* bias, const void* x, vq_dtype x_dtype, int32_t M, void* y, vq_dtype y_dtype,
                      void* stream) {
  if (M < 0) return VQ_ERR_SHAPE;
  SvqArgs p;
  vq_status st = prepare_svq(desc, packed, a, b, scale, bias, x, x_dtype, M, y, y_dtype, 16, &p);
  if (st != VQ_OK) return st;
  if (p.n == 0 || p.m == 0) return VQ_OK;
  return launch_svq_gemv(p, stream);
}

vq_status vq_svq_gemm(const vq_desc* desc, const void* packed, const void* a, const void* b, const void* scale,
                      const void* bias, const void* x, vq_dtype x_dtype, int32_t M, void* y, vq_dtype y_dtype,
                      void* stream) {
  if (M < 0) return VQ_ERR_SHAPE;
  if (M > 0 && ((int64_t)M + 127) / 128 > 65535) return VQ_ERR_SHAPE;  // grid rows of 128-row batch chunks
  SvqArgs p;
  vq_status st = prepare_svq(desc, packed, a, b, scale, bias, x, x_dtype, M, y, y_dtype, 0, &p);
  if (st != VQ_OK) return st;
  if (p.n == 0 || p.m == 0) return VQ_OK;
  return launch_svq_gemm(p, stream);
}

int32_t vq_rht_block(int32_t n) { return rht_block(n); }

vq_status vq_rht(int32_t M, int32_t n, const void* x, vq_dtype x_dtype, const void* signs, int32_t transpose, void* y,
                 vq_dtype y_dtype, void* stream) {
  if (M < 0 || n < 0) return VQ_ERR_SHAPE;
  if (!valid_out_dtype(x_dtype) || !valid_out_dtype(y_dtype)) return VQ_ERR_UNSUPPORTED;
  if (transpose != 0 && transpose != 1) return VQ_ERR_UNSUPPORTED;
  if (M == 0 || n == 0) return VQ_OK;
  if (rht_block(n) < 16) return VQ_ERR_UNSUPPORTED;  // n must be a multiple of 16
  if (!x || !signs || !y) return VQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, dtype_size(y_dtype))) return VQ_ERR_ALIGN;
  return launch_rht(M, n, x, x_dtype, (const uint8_t*)signs, transpose, y, y_dtype, stream);
}

vq_status vq_assign_workspace_bytes(const vq_desc* desc, size_t* nbytes) {
  if (!nbytes) return VQ_ERR_NULL;
  const vq_status st = check_desc(desc);
  if (st != VQ_OK) return st;
  *nbytes = assign_workspace(*desc);
  return VQ_OK;
}

vq_status vq_assign(const vq_desc* desc, const void* w, vq_dtype w_dtype, const void* cb1, const void* cb2,
                    uint32_t* idx1, uint32_t* idx2, void* workspace, size_t workspace_bytes, void* stream) {
  const vq_status st = check_desc(desc);
  if (st != VQ_OK) return st;
  const vq_desc& d = *desc;
  if (w_dtype != VQ_F16 && w_dtype != VQ_BF16 && w_dtype != VQ_F32) return VQ_ERR_UNSUPPORTED;
  if (d.in_features % d.v != 0) return VQ_ERR_UNSUPPORTED;
  if ((int64_t)d.out_features * d.in_features == 0) return VQ_OK;
  if (!w || !cb1 || !idx1 || !workspace || (d.bits2 > 0 && (!cb2 || !idx2))) return VQ_ERR_NULL;
  if (workspace_bytes < assign_workspace(d)) return VQ_ERR_BUFFER_SIZE;
  if (!aligned(workspace, 256) || !aligned(w, dtype_size(w_dtype)) || !aligned(cb1, 2) || !aligned(idx1, 4) ||
      (d.bits2 > 0 && (!aligned(cb2, 2) || !aligned(idx2, 4))))
    return VQ_ERR_ALIGN;
  return launch_assign(d, w, w_dtype, (const uint16_t*)cb1, d.bits2 > 0 ? (const uint16_t*)cb2 : nullptr, idx1,
                       d.bits2 > 0 ? idx2 : nullptr, workspace, stream);
}

vq_status vq_gemm(const vq_desc* desc, const void* packed, const void* cb1, const void* cb2, const void* scale,
                  const void* bias, const void* x, vq_dtype x_dtype, int32_t M, void* y, vq_dtype y_dtype,
                  void* stream) {
  ProductArgs a;
  vq_status st = prepare_product(desc, packed, cb1, cb2, scale, bias, x, x_dtype, M, y, y_dtype, 0, &a);
  if (st != VQ_OK) return st;
  if (a.n == 0 || a.m == 0) return VQ_OK;
  return launch_gemm(a, stream);
}

vq_status vq_gemm_workspace_bytes(const vq_desc* desc, int32_t M, vq_dtype x_dtype, size_t* nbytes) {
  if (!nbytes) return VQ_ERR_NULL;
  vq_status st = check_desc(desc);
  if (st != VQ_OK) return st;
  if (M < 0) return VQ_ERR_SHAPE;
  if (x_dtype != VQ_F16 && x_dtype != VQ_BF16) return VQ_ERR_UNSUPPORTED;
  *nbytes = M == 0 ? 0 : gather_gemm_workspace(*desc, M, x_dtype);
  return VQ_OK;
}

vq_status vq_gemm_ws(const vq_desc* desc, const void* packed, const void* cb1, const void* cb2, const void* scale,
                     const void* bias, const void* x, vq_dtype x_dtype, int32_t M, void* y, vq_dtype y_dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
  ProductArgs a;
  vq_status st = prepare_product(desc, packed, cb1, cb2, scale, bias, x, x_dtype, M, y, y_dtype, 0, &a);
  if (st != VQ_OK) return st;
  if (a.n == 0 || a.m == 0) return VQ_OK;
  if (gather_gemm_shape_ok(*desc, a.m, a.x_dtype) && gather_gemm_pointers_ok(a)) {
    const size_t need = gather_gemm_workspace(*desc, a.m, a.x_dtype);
    if (need == 0) return launch_gemm_gather(a, nullptr, stream);
    if (workspace) {
      if (workspace_bytes < need) return VQ_ERR_BUFFER_SIZE;
      if (!aligned(workspace, 256)) return VQ_ERR_ALIGN;
      return launch_gemm_gather(a, workspace, stream);
    }
  }
  return launch_gemm(a, stream);
}

// Workspace of the transform-fused products: the fused path's (x pass, partial sums) or,
// without it, the transformed activations [M][IN] for the separate transform.
static size_t rht_product_bytes(const vq_desc& d, int32_t m, vq_dtype x_dtype, bool gemm) {
  if (m <= 0 || d.in_features == 0) return 0;
  const size_t fused = gemm ? gather_gemm_rht_workspace(d, m, x_dtype) : sliced_gemv_rht_workspace(d, m, x_dtype);
  const size_t sep = ((size_t)m * (size_t)d.in_features * 2 + 255) / 256 * 256;
  return fused > sep ? fused : sep;
}

vq_status vq_rht_product_workspace_bytes(const vq_desc* desc, int32_t M, vq_dtype x_dtype, int32_t gemm,
                                         size_t* nbytes) {
  if (!nbytes) return VQ_ERR_NULL;
  vq_status st = check_desc(desc);
  if (st != VQ_OK) return st;
  if (gemm != 0 && gemm != 1) return VQ_ERR_UNSUPPORTED;
  if (M < 0 || (!gemm && M > 16)) return VQ_ERR_SHAPE;
  if (x_dtype != VQ_F16 && x_dtype != VQ_BF16) return VQ_ERR_UNSUPPORTED;
  if (desc->in_features % 16 != 0) return VQ_ERR_UNSUPPORTED;
  *nbytes = rht_product_bytes(*desc, M, x_dtype, gemm != 0);
  return VQ_OK;
}

static vq_status rht_product(bool gemm, const vq_desc* desc, const void* packed, const void* cb1, const void* cb2,
                             const void* scale, const void* bias, const void* x, vq_dtype x_dtype, int32_t M,
                             const void* signs, void* y, vq_dtype y_dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
  ProductArgs a;
  vq_status st = prepare_product(desc, packed, cb1, cb2, scale, bias, x, x_dtype, M, y, y_dtype, gemm ? 0 : 16, &a);
  if (st != VQ_OK) return st;
  if (a.in_features % 16 != 0) return VQ_ERR_UNSUPPORTED;
  if (a.n == 0 || a.m == 0) return VQ_OK;
  if (a.in_features == 0) return gemm ? launch_gemm(a, stream) : launch_gemv(a, stream);  // y = bias
  if (!signs || !workspace) return VQ_ERR_NULL;
  if (!aligned(x, 16)) return VQ_ERR_ALIGN;
  const size_t need = rht_product_bytes(*desc, a.m, a.x_dtype, gemm);
  if (workspace_bytes < need) return VQ_ERR_BUFFER_SIZE;
  if (!aligned(workspace, 256)) return VQ_ERR_ALIGN;
  const uint8_t* sg = (const uint8_t*)signs;
  if (gemm) {
    if (gather_gemm_rht_workspace(*desc, a.m, a.x_dtype) > 0 && gather_gemm_pointers_ok(a))
      return launch_gemm_gather(a, workspace, stream, sg);
  } else {
    if (sliced_gemv_rht_workspace(*desc, a.m, a.x_dtype) > 0 && sliced_gemv_pointers_ok(a))
      return launch_gemv_sliced(a, workspace, stream, sg);
  }
  // no fused path: the transform into the workspace, then the plain product on it
  st = launch_rht(a.m, a.in_features, a.x, a.x_dtype, sg, 0, workspace, a.x_dtype, stream);
  if (st != VQ_OK) return st;
  ProductArgs at = a;
  at.x = (const uint16_t*)workspace;
  return gemm ? launch_gemm(at, stream) : launch_gemv(at, stream);
}

vq_status vq_gemv_ws_rht(const vq_desc* desc, const void* packed, const void* cb1, const void* cb2, const void* scale,
                         const void* bias, const void* x, vq_dtype x_dtype, int32_t M, const void* signs, void* y,
                         vq_dtype y_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return rht_product(false, desc, packed, cb1, cb2, scale, bias, x, x_dtype, M, signs, y, y_dtype, workspace,
                     workspace_bytes, stream);
}

vq_status vq_gemm_ws_rht(const vq_desc* desc, const void* packed, const void* cb1, const void* cb2, const void* scale,
                         const void* bias, const void* x, vq_dtype x_dtype, int32_t M, const void* signs, void* y,
                         vq_dtype y_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return rht_product(true, desc, packed, cb1, cb2, scale, bias, x, x_dtype, M, signs, y, y_dtype, workspace,
                     workspace_bytes, stream);
}

}  // extern "C"
