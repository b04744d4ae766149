// layout.hip -- the data-movement kernels of libsprms around the fused shard
// path: the AllGather + unpad that follows it, and the two regroupings in
// front of a row-parallel o_proj (FlashComm2's ODP all-to-all and DSA-CP's
// head-to-token exchange).  What each computes is stated in include/sprms.h
// with the passages that define it.
//
// All three are pure copies, bound by HBM bandwidth: every byte is read once
// and written once, with non-temporal accesses of 16 bytes per lane (4 or 8
// when rows are not a multiple of 16 bytes).  One workgroup moves one
// destination row; the grids are rows x (ranks written), far more than the
// 256 compute units.  On one GPU the sources of "other ranks" are local
// buffers; on a node they would be peer-mapped memory and each rank would
// write only its own destination (the rank field of the descriptors).
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "common.h"
#include "sprms.h"

namespace {

using namespace sprms;

// ------------------------------------------------------------ row copy

// B-byte accesses (B = 16, 8 or 4): loads through a row descriptor or from a
// per-lane global address, stores through the destination row's descriptor.
typedef __attribute__((address_space(1))) const u32x4 global_u32x4;
typedef __attribute__((address_space(1))) const u32x2 global_u32x2;
typedef __attribute__((address_space(1))) const uint32_t global_u32;

template <int B>
struct Access;

template <>
struct Access<16> {
  using T = u32x4;
  static __device__ T load(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kLoadPolicy);
  }
  static __device__ T load(const char* p) { return __builtin_nontemporal_load((global_u32x4*)p); }
  static __device__ void store(T v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kStorePolicy);
  }
};

template <>
struct Access<8> {
  using T = u32x2;
  static __device__ T load(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kLoadPolicy);
  }
  static __device__ T load(const char* p) { return __builtin_nontemporal_load((global_u32x2*)p); }
  static __device__ void store(T v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kStorePolicy);
  }
};

template <>
struct Access<4> {
  using T = uint32_t;
  static __device__ T load(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kLoadPolicy);
  }
  static __device__ T load(const char* p) { return __builtin_nontemporal_load((global_u32*)p); }
  static __device__ void store(T v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kStorePolicy);
  }
};

// Accesses each lane keeps in flight: all loads of an iteration are issued
// before its first store.  With one access per lane a wavefront waits a full
// memory latency per KiB; two keep twice the bytes moving (about +10% of
// HBM bandwidth on the regroup at H = 5120 and 7168; more brings nothing).
constexpr int kInFlight = 2;

// Copies one destination row of `bytes` bytes; load(off) fetches byte offset
// off of the row's source.
template <int B, typename Load>
__device__ __forceinline__ void copy_row(uint32_t bytes, rsrc_t dst, Load load) {
  using A = Access<B>;
  const uint32_t step = blockDim.x * B;
  for (uint32_t off0 = threadIdx.x * B; off0 < bytes; off0 += step * kInFlight) {
    typename A::T v[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) {
      const uint32_t off = off0 + k * step;
      if (off < bytes) v[k] = load(off);
    }
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) {
      const uint32_t off = off0 + k * step;
      if (off < bytes) A::store(v[k], dst, off);
    }
  }
}

// ------------------------------------------------------------ all-gather

struct GArgs {
  const char* src[kMaxTp];     // shard q's [S][H] output
  const char* ssrc[kMaxTp];    // shard q's [S][scale_row_bytes] scales (or all null)
  char* out;                   // [T][H]
  char* out_scale;             // [T][scale_row_bytes] or null
  int64_t S;
  uint32_t row_bytes;          // bytes of one output row
  uint32_t scale_row_bytes;    // 0 when there are no scales
  uint32_t scale_words;        // scale rows copied as 4-byte words (length and addresses allow it)
};

// One workgroup per gathered row t: shard q = t / S, row s = t - q*S, copied
// unchanged with non-temporal 16-byte (or 8-byte) accesses.  The source and
// destination descriptors cover exactly one row.
template <int B>
__global__ void __launch_bounds__(kMaxThreads) gather_kernel(const GArgs a) {
  const int64_t t = blockIdx.x;
  const int q = static_cast<int>(t / a.S);
  const int64_t s = t - static_cast<int64_t>(q) * a.S;
  const rsrc_t src = row_rsrc(a.src[q] + s * a.row_bytes, a.row_bytes);
  const rsrc_t dst = row_rsrc(a.out + t * a.row_bytes, a.row_bytes);
  copy_row<B>(a.row_bytes, dst, [&](uint32_t off) { return Access<B>::load(src, off); });
  if (a.scale_row_bytes) {
    const rsrc_t ssrc = row_rsrc(a.ssrc[q] + s * a.scale_row_bytes, a.scale_row_bytes);
    const rsrc_t sdst = row_rsrc(a.out_scale + t * a.scale_row_bytes, a.scale_row_bytes);
    // A scale row is a few bytes; neighbouring rows belong to neighbouring
    // workgroups, so the accesses go through L2 (policy 0), where the rows
    // of one cache line meet, instead of streaming a DRAM sector each.
    if (a.scale_words) {  // whole words: no partial-word writes
      for (uint32_t off = threadIdx.x * 4; off < a.scale_row_bytes; off += blockDim.x * 4) {
        const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(ssrc, off, 0, kCachedPolicy);
        __builtin_amdgcn_raw_buffer_store_b32(v, sdst, off, 0, kCachedPolicy);
      }
    } else {
      for (uint32_t off = threadIdx.x; off < a.scale_row_bytes; off += blockDim.x) {
        const uint8_t v = __builtin_amdgcn_raw_buffer_load_b8(ssrc, off, 0, kCachedPolicy);
        __builtin_amdgcn_raw_buffer_store_b8(v, sdst, off, 0, kCachedPolicy);
      }
    }
  }
}

// ------------------------------------------------------- FlashComm2 regroup

struct FArgs {
  const char* src[kMaxTp];  // rank q's [N][C]
  char* dst[kMaxTp];        // rank r's [N/odp][odp*C]
  int32_t odp;
  int32_t seg_rows;         // N / G
  int32_t dst_rows;         // N / odp
  int32_t first_rank;       // rank written by blocks [0, dst_rows)
  uint32_t piece;           // C * element size, bytes
};

// One workgroup per destination row: blockIdx.x = (r - first_rank) *
// dst_rows + t.  Rank r = g*odp + j; row t lies in its k-th segment (source
// segment j + k*odp, row u of it) and is the odp source rows of that token
// side by side.  A row draws on odp source buffers, so the loads address
// memory per lane; the store goes through the row's descriptor.
template <int B>
__global__ void __launch_bounds__(kMaxThreads) fc2_regroup_kernel(const FArgs a) {
  const int64_t b = blockIdx.x;
  const int rr = static_cast<int>(b / a.dst_rows);
  const int r = a.first_rank + rr;
  const int t = static_cast<int>(b - static_cast<int64_t>(rr) * a.dst_rows);
  const int g = r / a.odp, j = r - g * a.odp;
  const int k = t / a.seg_rows, u = t - k * a.seg_rows;
  const int64_t n = static_cast<int64_t>(j + k * a.odp) * a.seg_rows + u;  // source token
  const uint32_t row_bytes = a.piece * static_cast<uint32_t>(a.odp);
  const rsrc_t dst = row_rsrc(a.dst[r] + static_cast<int64_t>(t) * row_bytes, row_bytes);
  copy_row<B>(row_bytes, dst, [&](uint32_t off) {
    const uint32_t i = off / a.piece;  // sender i of the ODP group
    return Access<B>::load(a.src[g * a.odp + static_cast<int>(i)] + n * a.piece + (off - i * a.piece));
  });
}

// ------------------------------------------------ DSA-CP head-to-token exchange

struct DArgs {
  const char* src[kMaxTp];  // rank p's [S][tp*D]
  char* dst[kMaxTp];        // rank q's [tp*S][D]
  int64_t S;
  int32_t tp;
  int32_t first_rank;       // rank written by blocks [0, tp*S)
  uint32_t piece;           // D * element size, bytes
};

// One workgroup per destination row t of rank q: token s = t - p*S of rank
// p = t / S, head block q, which is one contiguous piece of the source row.
template <int B>
__global__ void __launch_bounds__(kMaxThreads) dsacp_kernel(const DArgs a) {
  const int64_t rows = static_cast<int64_t>(a.tp) * a.S;
  const int64_t b = blockIdx.x;
  const int qq = static_cast<int>(b / rows);
  const int q = a.first_rank + qq;
  const int64_t t = b - static_cast<int64_t>(qq) * rows;
  const int p = static_cast<int>(t / a.S);
  const int64_t s = t - static_cast<int64_t>(p) * a.S;
  const rsrc_t src = row_rsrc(a.src[p] + (s * a.tp + q) * a.piece, a.piece);
  const rsrc_t dst = row_rsrc(a.dst[q] + t * a.piece, a.piece);
  copy_row<B>(a.piece, dst, [&](uint32_t off) { return Access<B>::load(src, off); });
}

// Threads for rows of `bytes` moved `width` bytes per access, kInFlight
// accesses per lane: whole wavefronts, at most one workgroup's worth.
int row_threads(size_t bytes, int width) {
  const size_t lanes = (bytes / static_cast<size_t>(width) + kInFlight - 1) / kInFlight;
  size_t nt = (lanes + 63) / 64 * 64;
  return static_cast<int>(nt > static_cast<size_t>(kMaxThreads) ? kMaxThreads : nt);
}

// Every written destination: non-NULL, aligned, clear of every source and of
// the other written destinations.
int check_copy_sets(const char* what_src, const void* const* src, int nsrc, size_t src_n,
                    const char* what_dst, void* const* dst, int first, int ndst, size_t dst_n,
                    uintptr_t align) {
  for (int q = 0; q < nsrc; ++q) {
    if (!src[q]) return fail(SP_ERR_NULL, "%s[%d] is NULL", what_src, q);
    if (misaligned(src[q], align)) return fail(SP_ERR_ALIGN, "%s[%d] is not %d-byte aligned", what_src, q, (int)align);
  }
  for (int r = first; r < first + ndst; ++r) {
    if (!dst[r]) return fail(SP_ERR_NULL, "%s[%d] is NULL", what_dst, r);
    if (misaligned(dst[r], align)) return fail(SP_ERR_ALIGN, "%s[%d] is not %d-byte aligned", what_dst, r, (int)align);
    for (int q = 0; q < nsrc; ++q)
      if (overlap(dst[r], dst_n, src[q], src_n))
        return fail(SP_ERR_SHAPE, "%s[%d] overlaps %s[%d]", what_dst, r, what_src, q);
    for (int q = first; q < first + ndst; ++q)
      if (q != r && overlap(dst[r], dst_n, dst[q], dst_n))
        return fail(SP_ERR_SHAPE, "%s[%d] overlaps %s[%d]", what_dst, r, what_dst, q);
  }
  return SP_OK;
}

}  // namespace

// ------------------------------------------------------------------ C ABI

extern "C" {

int sp_all_gather_unpad(const sp_gather_problem* g, const void* const* shards,
                        const void* const* shard_scales, void* out, void* out_scale,
                        void* stream) {
  if (!g) return fail(SP_ERR_NULL, "gather descriptor is NULL");
  if (g->tp < 1 || g->tp > kMaxTp) return fail(SP_ERR_SHAPE, "tp=%d outside [1, %d]", g->tp, kMaxTp);
  const int64_t S = g->shard_rows, H = g->hidden, T = g->num_tokens;
  if (S < 0 || S > INT32_MAX) return fail(SP_ERR_SHAPE, "shard_rows=%lld outside [0, 2^31)", (long long)S);
  if (H < 8 || H > kMaxHidden || H % 8 != 0)
    return fail(SP_ERR_SHAPE, "hidden=%lld must be a multiple of 8 in [8, %d]", (long long)H, kMaxHidden);
  if (T < 0 || T > g->tp * S || T > INT32_MAX)
    return fail(SP_ERR_SHAPE, "num_tokens=%lld outside [0, tp*S=%lld]", (long long)T, (long long)(g->tp * S));
  const size_t row_bytes = row_bytes_of(g->dtype, H);
  if (row_bytes == 0) return fail(SP_ERR_DTYPE, "dtype=%d unknown", g->dtype);
  if (g->dtype == SP_FP4_E2M1 && H % 16 != 0)
    return fail(SP_ERR_SHAPE, "hidden=%lld must be a multiple of 16 for e2m1 rows", (long long)H);
  const int64_t sb = g->scale_row_bytes;
  if (sb < 0 || sb > 65536)
    return fail(SP_ERR_SHAPE, "scale_row_bytes=%lld outside [0, 65536]", (long long)sb);
  if (T == 0) return SP_OK;
  if (!shards || !out) return fail(SP_ERR_NULL, "shards and out must be non-NULL");
  if ((shard_scales == nullptr) != (out_scale == nullptr) || (shard_scales == nullptr) != (sb == 0))
    return fail(SP_ERR_NULL, "shard_scales, out_scale and scale_row_bytes must be all given or all none");
  // 16-byte accesses when rows are a multiple of 16 bytes, else 8-byte ones;
  // every row start must be aligned to the access width
  const int B = row_bytes % 16 == 0 ? 16 : 8;
  const uintptr_t amask = static_cast<uintptr_t>(B - 1);
  if (reinterpret_cast<uintptr_t>(out) & amask)
    return fail(SP_ERR_ALIGN, "out %p is not %d-byte aligned", out, B);
  if (out_scale && sb == 4 && (reinterpret_cast<uintptr_t>(out_scale) & 3u))
    return fail(SP_ERR_ALIGN, "out_scale %p is not 4-byte aligned", out_scale);
  const size_t out_n = static_cast<size_t>(T) * row_bytes;
  const size_t out_scale_n = static_cast<size_t>(T * sb), shard_n = static_cast<size_t>(S) * row_bytes,
               shard_scale_n = static_cast<size_t>(S * sb);
  // nothing written may be read by the call or written twice
  if (overlap(out, out_n, out_scale, out_scale_n)) return fail(SP_ERR_SHAPE, "out overlaps out_scale");
  GArgs ga;
  memset(&ga, 0, sizeof ga);
  for (int q = 0; q < g->tp; ++q) {
    if (!shards[q]) return fail(SP_ERR_NULL, "shards[%d] is NULL", q);
    if (reinterpret_cast<uintptr_t>(shards[q]) & amask)
      return fail(SP_ERR_ALIGN, "shards[%d] %p is not %d-byte aligned", q, shards[q], B);
    if (overlap(out, out_n, shards[q], shard_n)) return fail(SP_ERR_SHAPE, "out overlaps shards[%d]", q);
    if (overlap(out_scale, out_scale_n, shards[q], shard_n))
      return fail(SP_ERR_SHAPE, "out_scale overlaps shards[%d]", q);
    ga.src[q] = static_cast<const char*>(shards[q]);
    if (shard_scales) {
      if (!shard_scales[q]) return fail(SP_ERR_NULL, "shard_scales[%d] is NULL", q);
      if (sb == 4 && (reinterpret_cast<uintptr_t>(shard_scales[q]) & 3u))
        return fail(SP_ERR_ALIGN, "shard_scales[%d] is not 4-byte aligned", q);
      if (overlap(out_scale, out_scale_n, shard_scales[q], shard_scale_n))
        return fail(SP_ERR_SHAPE, "out_scale overlaps shard_scales[%d]", q);
      if (overlap(out, out_n, shard_scales[q], shard_scale_n))
        return fail(SP_ERR_SHAPE, "out overlaps shard_scales[%d]", q);
      ga.ssrc[q] = static_cast<const char*>(shard_scales[q]);
    }
  }
  ga.out = static_cast<char*>(out);
  ga.out_scale = static_cast<char*>(out_scale);
  ga.S = S;
  ga.row_bytes = static_cast<uint32_t>(row_bytes);
  ga.scale_row_bytes = static_cast<uint32_t>(sb);
  bool words = sb % 4 == 0 && !misaligned(out_scale, 4);
  for (int q = 0; words && shard_scales && q < g->tp; ++q) words = !misaligned(shard_scales[q], 4);
  ga.scale_words = words ? 1u : 0u;
  const int nt = row_threads(row_bytes, B);
  void* args[] = {&ga};
  const void* fn = B == 16 ? reinterpret_cast<const void*>(&gather_kernel<16>)
                           : reinterpret_cast<const void*>(&gather_kernel<8>);
  hipError_t err = hipLaunchKernel(fn, dim3(static_cast<unsigned>(T)), dim3(static_cast<unsigned>(nt)), args,
                                   0, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(SP_ERR_HIP, "gather launch failed: %s", hipGetErrorString(err));
  return SP_OK;
}

int sp_fc2_regroup(const sp_fc2_problem* f, const void* const* src, void* const* dst, void* stream) {
  if (!f) return fail(SP_ERR_NULL, "fc2 descriptor is NULL");
  const int G = f->global_tp, P = f->otp;
  if (G < 2 || G > kMaxTp) return fail(SP_ERR_SHAPE, "global_tp=%d outside [2, %d]", G, kMaxTp);
  if (P < 1 || P >= G || G % P != 0)
    return fail(SP_ERR_SHAPE, "otp=%d must divide global_tp=%d and be smaller", P, G);
  if (f->rank < -1 || f->rank >= G) return fail(SP_ERR_SHAPE, "rank=%d outside [-1, %d)", f->rank, G);
  const size_t e = elt_size(f->dtype);
  if (e == 0) return fail(SP_ERR_DTYPE, "dtype=%d unsupported", f->dtype);
  const int64_t N = f->tokens, C = f->cols;
  if (N < 0 || N % G != 0 || N > INT32_MAX)
    return fail(SP_ERR_SHAPE, "tokens=%lld must be a multiple of %d below 2^31", (long long)N, G);
  const int odp = G / P;
  if (C < 1 || C > (1ll << 30) / (static_cast<int64_t>(e) * odp) || (C * static_cast<int64_t>(e)) % 4 != 0)
    return fail(SP_ERR_SHAPE, "cols=%lld: rows must be a multiple of 4 bytes and at most 1 GiB", (long long)C);
  const int first = f->rank < 0 ? 0 : f->rank, nranks = f->rank < 0 ? G : 1;
  const int64_t rows = static_cast<int64_t>(nranks) * (N / odp);
  if (rows > static_cast<int64_t>(UINT32_MAX)) return fail(SP_ERR_SHAPE, "too many rows for one grid");
  if (N == 0) return SP_OK;
  if (!src || !dst) return fail(SP_ERR_NULL, "src and dst must be non-NULL");
  const size_t piece = static_cast<size_t>(C) * e;
  const int B = piece % 16 == 0 ? 16 : 4;
  const size_t src_n = static_cast<size_t>(N) * piece, dst_n = static_cast<size_t>(N / odp) * piece * odp;
  int rc = check_copy_sets("src", src, G, src_n, "dst", dst, first, nranks, dst_n, static_cast<uintptr_t>(B));
  if (rc != SP_OK) return rc;
  const int nt = row_threads(piece * odp, B);
  if (rows * nt > static_cast<int64_t>(UINT32_MAX))
    return fail(SP_ERR_SHAPE, "%lld rows x %d threads exceed the dispatch limit", (long long)rows, nt);
  FArgs fa;
  memset(&fa, 0, sizeof fa);
  for (int q = 0; q < G; ++q) fa.src[q] = static_cast<const char*>(src[q]);
  for (int r = first; r < first + nranks; ++r) fa.dst[r] = static_cast<char*>(dst[r]);
  fa.odp = odp;
  fa.seg_rows = static_cast<int32_t>(N / G);
  fa.dst_rows = static_cast<int32_t>(N / odp);
  fa.first_rank = first;
  fa.piece = static_cast<uint32_t>(piece);
  void* args[] = {&fa};
  const void* fn = B == 16 ? reinterpret_cast<const void*>(&fc2_regroup_kernel<16>)
                           : reinterpret_cast<const void*>(&fc2_regroup_kernel<4>);
  hipError_t err = hipLaunchKernel(fn, dim3(static_cast<unsigned>(rows)), dim3(static_cast<unsigned>(nt)), args,
                                   0, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(SP_ERR_HIP, "fc2 regroup launch failed: %s", hipGetErrorString(err));
  return SP_OK;
}

int sp_dsacp_heads_to_tokens(const sp_dsacp_problem* f, const void* const* attn, void* const* out,
                             void* stream) {
  if (!f) return fail(SP_ERR_NULL, "dsacp descriptor is NULL");
  const int tp = f->tp;
  if (tp < 1 || tp > kMaxTp) return fail(SP_ERR_SHAPE, "tp=%d outside [1, %d]", tp, kMaxTp);
  if (f->rank < -1 || f->rank >= tp) return fail(SP_ERR_SHAPE, "rank=%d outside [-1, %d)", f->rank, tp);
  if (f->reserved != 0) return fail(SP_ERR_UNSUPPORTED, "reserved field must be 0");
  const size_t e = elt_size(f->dtype);
  if (e == 0) return fail(SP_ERR_DTYPE, "dtype=%d unsupported", f->dtype);
  const int64_t S = f->shard_rows, D = f->head_cols;
  // bound S before multiplying, so that tp*S cannot wrap past the check
  if (S < 0 || S > INT32_MAX / tp) return fail(SP_ERR_SHAPE, "shard_rows=%lld: need 0 <= tp*S < 2^31", (long long)S);
  if (D < 1 || D > (1ll << 30) / (static_cast<int64_t>(e) * tp) || (D * static_cast<int64_t>(e)) % 4 != 0)
    return fail(SP_ERR_SHAPE, "head_cols=%lld: rows must be a multiple of 4 bytes and at most 1 GiB", (long long)D);
  const int first = f->rank < 0 ? 0 : f->rank, nranks = f->rank < 0 ? tp : 1;
  const int64_t rows = static_cast<int64_t>(nranks) * tp * S;
  if (rows > static_cast<int64_t>(UINT32_MAX)) return fail(SP_ERR_SHAPE, "too many rows for one grid");
  if (S == 0) return SP_OK;
  if (!attn || !out) return fail(SP_ERR_NULL, "attn and out must be non-NULL");
  const size_t piece = static_cast<size_t>(D) * e;
  const int B = piece % 16 == 0 ? 16 : 4;
  const size_t n = static_cast<size_t>(S) * tp * piece;  // bytes of every attn and out buffer
  int rc = check_copy_sets("attn", attn, tp, n, "out", out, first, nranks, n, static_cast<uintptr_t>(B));
  if (rc != SP_OK) return rc;
  const int nt = row_threads(piece, B);
  if (rows * nt > static_cast<int64_t>(UINT32_MAX))
    return fail(SP_ERR_SHAPE, "%lld rows x %d threads exceed the dispatch limit", (long long)rows, nt);
  DArgs da;
  memset(&da, 0, sizeof da);
  for (int p = 0; p < tp; ++p) da.src[p] = static_cast<const char*>(attn[p]);
  for (int q = first; q < first + nranks; ++q) da.dst[q] = static_cast<char*>(out[q]);
  da.S = S;
  da.tp = tp;
  da.first_rank = first;
  da.piece = static_cast<uint32_t>(piece);
  void* args[] = {&da};
  const void* fn = B == 16 ? reinterpret_cast<const void*>(&dsacp_kernel<16>)
                           : reinterpret_cast<const void*>(&dsacp_kernel<4>);
  hipError_t err = hipLaunchKernel(fn, dim3(static_cast<unsigned>(rows)), dim3(static_cast<unsigned>(nt)), args,
                                   0, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(SP_ERR_HIP, "dsacp exchange launch failed: %s", hipGetErrorString(err));
  return SP_OK;
}

}  // extern "C"
