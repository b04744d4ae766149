// sprms.hip -- libsprms: fused ReduceScatter-reduce + deepstack/residual add +
// RMSNorm (+bias) + optional output quantisation (e4m3 with a static or
// per-token scale, or block-scaled MXFP8 / MXFP4) for one rank's token shard,
// written for MI355X (gfx950, CDNA4).
//
// What is computed is stated in include/sprms.h, with the passages of the
// pages that define it.  This file is the fused kernel family and its
// host-side validation and dispatch behind the C ABI; the layout kernels
// (gather, regroupings) are in layout.hip, the producer GEMM in gemm.hip, the
// error channel and host-only helpers in abi.cpp.
//
// Kernel design (HBM-bandwidth bound: about one flop per byte and no dense
// contraction, so no MFMA):
//   * one workgroup per shard row; the row is split into 8-element vectors
//     (16 B of bf16) and thread t owns vectors t, t+NT, ..., so each load or
//     store instruction of a wavefront covers 1 KiB of contiguous memory.
//     Rows of up to 8192 elements use one vector per thread (up to 1024
//     threads); longer rows use 4 or 8 vectors per thread within 512 threads;
//   * all row data moves through buffer instructions on per-row descriptors
//     held in scalar registers; the streamed data (partials, deepstack,
//     residual, outputs) is marked non-temporal, the gain and bias are
//     cached (every row re-reads them from L2);
//   * every load of the row is issued before the first add when the loads
//     fit the register budget (otherwise partials come in groups of 2-4);
//     the fp32 sum stays in registers and nothing is re-read;
//   * the updated residual is stored as soon as the sum is known, which
//     spreads the write traffic over the kernel;
//   * the sum of squares (and, for per-token FP8 without bias, max |z*w|) is
//     reduced with DPP row operations inside the wavefront, then across
//     wavefronts through LDS with one barrier; with a bias the per-token max
//     needs y, so a second LDS step follows;
//   * output conversion uses gfx950's v_cvt_pk_bf16_f32 / v_cvt_pk_fp8_f32
//     (OCP e4m3fn), after an explicit clamp to +-448 that keeps NaN as NaN;
//     maxima use v_maximum3_f32, which propagates NaN; block scaling takes the
//     32-element max across a quad of lanes (DPP), an E8M0 exponent from
//     v_frexp_exp, exact v_ldexp scaling and v_cvt_scalef32_pk_fp4_f32 for
//     e2m1;
//   * padding rows (s >= valid_rows) only store zeros.
// Rows are independent and there is no reuse across rows except the gain and
// bias vectors (a few KiB, served from each XCD's L2), so the workgroup ->
// row mapping needs no XCD-aware swizzle.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "common.h"
#include "sprms.h"

namespace {

using namespace sprms;

constexpr int kVec = 8;  // elements per thread-vector
// Workgroup size bounds: one 8-element vector per thread allows a
// 1024-thread workgroup (rows of up to 8192 elements); more vectors per
// thread hold more registers and are limited to 512 threads.
constexpr int kMaxThreadsMultiVec = 512;
constexpr int kMaxWaves = kMaxThreads / 64;

template <int VPT>
constexpr int max_threads() {
  return VPT == 1 ? kMaxThreads : kMaxThreadsMultiVec;
}

enum OutMode { OM_BF16 = 0, OM_F32 = 1, OM_FP8_STATIC = 2, OM_FP8_DYN = 3, OM_MX_FP8 = 4, OM_MX_FP4 = 5 };
constexpr int kMxBlock = 32;  // elements per block scale (4 lanes x 8 elements)
// Largest byte span the partials may cover (beyond any device's memory); it
// keeps every offset computed from the descriptor far from int64 overflow.
constexpr int64_t kMaxSpanBytes = int64_t(1) << 47;

struct KArgs {
  const void* partials;   // [tp][S][H]
  const void* residual;   // this shard's residual rows (block tp_rank already applied)
  void* residual_out;     // [S][H]; equals residual for in-place
  const void* weight;     // [H]
  const void* bias;       // [H] or nullptr
  const void* deepstack;  // this shard's deepstack rows or nullptr
  void* out;              // [S][H]
  void* out_scale;        // static: [1] f32 (read); dynamic: [S] f32, MX: [S][H/32] bytes (written)
  int64_t plane;          // elements between partial q's row and partial q+1's row
  int32_t H;
  int32_t nvec;           // H / 8
  int32_t valid;          // rows [0, valid) are real tokens
  int32_t tp;
  float eps;
  float pscale;           // factor applied to every partial before the sum
};

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <int DT>
struct Vec;

// 8 bf16 = one 16-byte access
template <>
struct Vec<SP_BF16> {
  using raw = u32x4;
  static constexpr int kBytes = 16;
  template <int POL>
  static __device__ __forceinline__ raw load(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POL);
  }
  static __device__ __forceinline__ void add(const raw& v, float (&f)[kVec]) {
    f[0] += bf16_lo(v.x); f[1] += bf16_hi(v.x);
    f[2] += bf16_lo(v.y); f[3] += bf16_hi(v.y);
    f[4] += bf16_lo(v.z); f[5] += bf16_hi(v.z);
    f[6] += bf16_lo(v.w); f[7] += bf16_hi(v.w);
  }
  // f += c * v with one rounding (c = 1 gives exactly f + v)
  static __device__ __forceinline__ void add_scaled(const raw& v, float c, float (&f)[kVec]) {
    f[0] = fmaf(c, bf16_lo(v.x), f[0]); f[1] = fmaf(c, bf16_hi(v.x), f[1]);
    f[2] = fmaf(c, bf16_lo(v.y), f[2]); f[3] = fmaf(c, bf16_hi(v.y), f[3]);
    f[4] = fmaf(c, bf16_lo(v.z), f[4]); f[5] = fmaf(c, bf16_hi(v.z), f[5]);
    f[6] = fmaf(c, bf16_lo(v.w), f[6]); f[7] = fmaf(c, bf16_hi(v.w), f[7]);
  }
  static __device__ __forceinline__ void unpack(const raw& v, float (&f)[kVec]) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  }
  static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, const float (&f)[kVec]) {
    u32x4 o = {pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]),
               pack_bf16(f[6], f[7])};
    __builtin_amdgcn_raw_buffer_store_b128(o, r, off, 0, kStorePolicy);
  }
  static __device__ __forceinline__ void store_zero(rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{0, 0, 0, 0}, r, off, 0, kStorePolicy);
  }
};

// 8 f32 = two 16-byte accesses
template <>
struct Vec<SP_F32> {
  struct raw {
    u32x4 a, b;
  };
  static constexpr int kBytes = 32;
  template <int POL>
  static __device__ __forceinline__ raw load(rsrc_t r, uint32_t off) {
    return raw{__builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POL),
               __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, POL)};
  }
  static __device__ __forceinline__ void add(const raw& v, float (&f)[kVec]) {
    f[0] += __uint_as_float(v.a.x); f[1] += __uint_as_float(v.a.y);
    f[2] += __uint_as_float(v.a.z); f[3] += __uint_as_float(v.a.w);
    f[4] += __uint_as_float(v.b.x); f[5] += __uint_as_float(v.b.y);
    f[6] += __uint_as_float(v.b.z); f[7] += __uint_as_float(v.b.w);
  }
  // f += c * v with one rounding (c = 1 gives exactly f + v)
  static __device__ __forceinline__ void add_scaled(const raw& v, float c, float (&f)[kVec]) {
    f[0] = fmaf(c, __uint_as_float(v.a.x), f[0]); f[1] = fmaf(c, __uint_as_float(v.a.y), f[1]);
    f[2] = fmaf(c, __uint_as_float(v.a.z), f[2]); f[3] = fmaf(c, __uint_as_float(v.a.w), f[3]);
    f[4] = fmaf(c, __uint_as_float(v.b.x), f[4]); f[5] = fmaf(c, __uint_as_float(v.b.y), f[5]);
    f[6] = fmaf(c, __uint_as_float(v.b.z), f[6]); f[7] = fmaf(c, __uint_as_float(v.b.w), f[7]);
  }
  static __device__ __forceinline__ void unpack(const raw& v, float (&f)[kVec]) {
    f[0] = __uint_as_float(v.a.x); f[1] = __uint_as_float(v.a.y);
    f[2] = __uint_as_float(v.a.z); f[3] = __uint_as_float(v.a.w);
    f[4] = __uint_as_float(v.b.x); f[5] = __uint_as_float(v.b.y);
    f[6] = __uint_as_float(v.b.z); f[7] = __uint_as_float(v.b.w);
  }
  static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, const float (&f)[kVec]) {
    u32x4 lo = {__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                __float_as_uint(f[3])};
    u32x4 hi = {__float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]),
                __float_as_uint(f[7])};
    __builtin_amdgcn_raw_buffer_store_b128(lo, r, off, 0, kStorePolicy);
    __builtin_amdgcn_raw_buffer_store_b128(hi, r, off + 16, 0, kStorePolicy);
  }
  static __device__ __forceinline__ void store_zero(rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{0, 0, 0, 0}, r, off, 0, kStorePolicy);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{0, 0, 0, 0}, r, off + 16, 0, kStorePolicy);
  }
};

// Largest of a and b, NaN if either is NaN (v_maximum3_f32); fmaxf would
// return the number and drop the NaN.
__device__ __forceinline__ float nan_max(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Saturation to +-448 for numbers; a NaN stays a NaN (fminf/fmaxf alone would
// turn it into -448, a plausible-looking finite code).
__device__ __forceinline__ float sat_e4m3(float t) {
  return t == t ? fminf(fmaxf(t, -448.0f), 448.0f) : __builtin_nanf("");
}

// v_cvt_pk_fp8_f32 encodes a NaN as 0xFF (measured on gfx950, also for the
// positive quiet NaN); the NaN code here is 0x7F, the one torch's
// float8_e4m3fn cast writes.  Numbers are saturated to +-448 (0x7E / 0xFE)
// before the conversion, so a 0xFF byte can only be a NaN: clear bit 7 of
// every 0xFF byte of a packed word (x = ~w has a zero byte exactly there;
// (x & 0x7F) + 0x7F sets bit 7 of a byte unless its low bits are zero, with
// no carry out of the byte).
__device__ __forceinline__ uint32_t nan_code_7f(uint32_t w) {
  const uint32_t x = ~w;
  const uint32_t ff_bytes = ~(((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x | 0x7F7F7F7Fu);
  return w ^ ff_bytes;
}

// 8 fp32 -> 8 OCP e4m3fn codes (little-endian byte order = element order),
// saturated first so the conversion never sees an out-of-range number.
__device__ __forceinline__ u32x2 pack_e4m3(const float (&t)[kVec]) {
  float c[kVec];
#pragma unroll
  for (int k = 0; k < kVec; ++k) c[k] = sat_e4m3(t[k]);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], lo, true);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[4], c[5], 0, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(c[6], c[7], hi, true);
  return u32x2{nan_code_7f(static_cast<uint32_t>(lo)), nan_code_7f(static_cast<uint32_t>(hi))};
}

__device__ __forceinline__ void store_e4m3(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kStorePolicy);
}

// 8 fp32 -> 8 OCP e2m1 codes in one dword (element k in bits 4k..4k+3),
// clamped to +-6 first; v_cvt_scalef32_pk_fp4_f32 with a unit scale.
__device__ __forceinline__ uint32_t pack_e2m1(const float (&t)[kVec]) {
  float c[kVec];
#pragma unroll
  for (int k = 0; k < kVec; ++k) c[k] = fminf(fmaxf(t[k], -6.0f), 6.0f);
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, c[0], c[1], 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, c[2], c[3], 1.0f, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, c[4], c[5], 1.0f, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, c[6], c[7], 1.0f, 3);
  return r;
}

__device__ __forceinline__ void store_e2m1(rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kStorePolicy);
}

// ------------------------------------------------------------- reductions

// DPP move within a wavefront (row = 16 lanes); all controls used here read
// a valid lane, so bound_ctrl / masks never substitute the old value.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;   // row_ror:4
constexpr int kRowRor8 = 0x128;   // row_ror:8

__device__ __forceinline__ float lane_read(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over the 64 lanes, same fixed order in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<kQuadSwap1>(v);
  v += dpp<kQuadSwap2>(v);
  v += dpp<kRowRor4>(v);
  v += dpp<kRowRor8>(v);  // every lane now holds its 16-lane row total
  return (lane_read(v, 0) + lane_read(v, 16)) + (lane_read(v, 32) + lane_read(v, 48));
}

// Max over the 4 lanes of a quad (lanes 4b..4b+3), in every lane of it; NaN
// if any of them holds NaN.
__device__ __forceinline__ float quad_max(float v) {
  v = nan_max(v, dpp<kQuadSwap1>(v));
  return nan_max(v, dpp<kQuadSwap2>(v));
}

// Max over the 64 lanes, NaN if any lane holds NaN.
__device__ __forceinline__ float wave_max(float v) {
  v = nan_max(v, dpp<kQuadSwap1>(v));
  v = nan_max(v, dpp<kQuadSwap2>(v));
  v = nan_max(v, dpp<kRowRor4>(v));
  v = nan_max(v, dpp<kRowRor8>(v));
  return nan_max(nan_max(lane_read(v, 0), lane_read(v, 16)), nan_max(lane_read(v, 32), lane_read(v, 48)));
}

// ----------------------------------------------------------------- kernel

// One shard row s, processed by the whole workgroup.
template <int PT, int AT, int OM, int TP, int VPT>
__device__ __forceinline__ void process_row(const KArgs& a, const int64_t s, float (&red)[3][kMaxWaves]) {
  using VP = Vec<PT>;
  using VA = Vec<AT>;
  constexpr int kOutBytes = OM == OM_F32 ? 32 : OM == OM_BF16 ? 16 : OM == OM_MX_FP4 ? 4 : 8;  // per 8 elements
  constexpr bool kMx = OM == OM_MX_FP8 || OM == OM_MX_FP4;

  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int nw = nt >> 6;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int64_t row = s * a.H;  // element index of the row's first element
  const uint32_t rowA = static_cast<uint32_t>(a.H) * (VA::kBytes / kVec);
  const uint32_t rowO = static_cast<uint32_t>(a.H) * kOutBytes / kVec;

  // Lanes past the end of the row (only when NT*VPT*8 > H) load a valid
  // vector of the row and discard it; they store nothing and add 0.
  uint32_t vec[VPT];
  bool live[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int j = tid + i * nt;
    live[i] = j < a.nvec;
    vec[i] = static_cast<uint32_t>(live[i] ? j : a.nvec - 1);
  }

  const rsrc_t r_res_out = row_rsrc(static_cast<char*>(a.residual_out) + row * (VA::kBytes / kVec), rowA);
  const rsrc_t r_out = row_rsrc(static_cast<char*>(a.out) + row * kOutBytes / kVec, rowO);

  if (s >= a.valid) {  // padding row: zeros only, no input is read
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      if (!live[i]) continue;
      VA::store_zero(r_res_out, vec[i] * VA::kBytes);
      if constexpr (OM == OM_BF16) Vec<SP_BF16>::store_zero(r_out, vec[i] * 16);
      if constexpr (OM == OM_F32) Vec<SP_F32>::store_zero(r_out, vec[i] * 32);
      if constexpr (OM == OM_FP8_STATIC || OM == OM_FP8_DYN || OM == OM_MX_FP8)
        store_e4m3(r_out, vec[i] * 8, u32x2{0, 0});
      if constexpr (OM == OM_MX_FP4) store_e2m1(r_out, vec[i] * 4, 0u);
      if constexpr (kMx) {
        if ((tid & 3) == 0) {  // one scale byte per block of 32 = per quad of lanes
          const rsrc_t r_sc = row_rsrc(static_cast<uint8_t*>(a.out_scale) + s * (a.H / kMxBlock),
                                       static_cast<uint32_t>(a.H / kMxBlock));
          __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(0), r_sc, vec[i] / 4, 0, kStorePolicy);
        }
      }
    }
    if constexpr (OM == OM_FP8_DYN) {
      if (tid == 0) static_cast<float*>(a.out_scale)[s] = 0.0f;
    }
    return;
  }

  const bool has_ds = a.deepstack != nullptr;
  const bool has_bias = a.bias != nullptr;
  const rsrc_t r_w = row_rsrc(a.weight, rowA);
  const rsrc_t r_b = row_rsrc(a.bias, rowA);
  const rsrc_t r_res = row_rsrc(static_cast<const char*>(a.residual) + row * (VA::kBytes / kVec), rowA);
  const rsrc_t r_ds = row_rsrc(static_cast<const char*>(a.deepstack) + row * (VA::kBytes / kVec), rowA);
  const uint32_t rowP = static_cast<uint32_t>(a.H) * (VP::kBytes / kVec);
  const char* p0 = static_cast<const char*>(a.partials) + row * (VP::kBytes / kVec);
  const int64_t planeB = a.plane * (VP::kBytes / kVec);

  float z[VPT][kVec];
#pragma unroll
  for (int i = 0; i < VPT; ++i)
#pragma unroll
    for (int k = 0; k < kVec; ++k) z[i][k] = 0.0f;

  // Gain and bias first: vmcnt counts loads and stores in issue order, so the
  // oldest loads can be waited for without waiting for later stores.
  typename VA::raw rw[VPT], rb[VPT];
#pragma unroll
  for (int i = 0; i < VPT; ++i) rw[i] = VA::template load<kCachedPolicy>(r_w, vec[i] * VA::kBytes);
  if (has_bias) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) rb[i] = VA::template load<kCachedPolicy>(r_b, vec[i] * VA::kBytes);
  }
  float static_scale = 1.0f;
  if constexpr (OM == OM_FP8_STATIC) static_scale = static_cast<const float*>(a.out_scale)[0];

  if constexpr (TP > 0) {
    // ---- every load of the row in flight before the first add
    typename VP::raw rp[TP][VPT];
    typename VA::raw rd[VPT], rr[VPT];
#pragma unroll
    for (int q = 0; q < TP; ++q) {
      const rsrc_t r_p = row_rsrc(p0 + q * planeB, rowP);
#pragma unroll
      for (int i = 0; i < VPT; ++i) rp[q][i] = VP::template load<kLoadPolicy>(r_p, vec[i] * VP::kBytes);
    }
    if (has_ds) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) rd[i] = VA::template load<kLoadPolicy>(r_ds, vec[i] * VA::kBytes);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) rr[i] = VA::template load<kLoadPolicy>(r_res, vec[i] * VA::kBytes);
    // sum of the (scaled) partials in ascending rank order, then deepstack, then residual
#pragma unroll
    for (int q = 0; q < TP; ++q)
#pragma unroll
      for (int i = 0; i < VPT; ++i) VP::add_scaled(rp[q][i], a.pscale, z[i]);
    if (has_ds) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) VA::add(rd[i], z[i]);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) VA::add(rr[i], z[i]);
  } else {
    // ---- runtime tp (or too many loads for registers): G partials in
    // flight at a time, ascending rank order; the rest loaded at use
    constexpr int kRegsP = PT == SP_F32 ? 8 : 4;
    constexpr int G = (64 / (VPT * kRegsP)) >= 4 ? 4 : (64 / (VPT * kRegsP)) >= 2 ? 2 : 1;
    for (int q0 = 0; q0 < a.tp; q0 += G) {
      typename VP::raw rp[G][VPT];
      const int g = a.tp - q0 < G ? a.tp - q0 : G;
#pragma unroll
      for (int k = 0; k < G; ++k)
        if (k < g) {
          const rsrc_t r_p = row_rsrc(p0 + (q0 + k) * planeB, rowP);
#pragma unroll
          for (int i = 0; i < VPT; ++i) rp[k][i] = VP::template load<kLoadPolicy>(r_p, vec[i] * VP::kBytes);
        }
#pragma unroll
      for (int k = 0; k < G; ++k)
        if (k < g) {
#pragma unroll
          for (int i = 0; i < VPT; ++i) VP::add_scaled(rp[k][i], a.pscale, z[i]);
        }
    }
    if (has_ds) {
#pragma unroll
      for (int i = 0; i < VPT; ++i)
        VA::add(VA::template load<kLoadPolicy>(r_ds, vec[i] * VA::kBytes), z[i]);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i)
      VA::add(VA::template load<kLoadPolicy>(r_res, vec[i] * VA::kBytes), z[i]);
  }

  // ---- store the updated residual once, as soon as it is known
#pragma unroll
  for (int i = 0; i < VPT; ++i)
    if (live[i]) VA::store(r_res_out, vec[i] * VA::kBytes, z[i]);

  // ---- zw = z * w; per-thread sum of z^2 and max |zw|
  float ss = 0.0f, amax = 0.0f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    float w[kVec];
    VA::unpack(rw[i], w);
    float part = 0.0f, m = 0.0f;
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
      part += z[i][k] * z[i][k];
      z[i][k] *= w[k];
      m = nan_max(m, fabsf(z[i][k]));
    }
    if (live[i]) {
      ss += part;
      amax = nan_max(amax, m);
    }
  }

  // ---- block reduction: DPP inside the wavefront, LDS across wavefronts
  constexpr bool kFusedMax = (OM == OM_FP8_DYN);
  ss = wave_sum(ss);
  if constexpr (kFusedMax) amax = wave_max(amax);
  if (lane == 0) {
    red[0][wave] = ss;
    if constexpr (kFusedMax) red[1][wave] = amax;
  }
  __syncthreads();
  ss = 0.0f;
  amax = 0.0f;
  for (int w = 0; w < nw; ++w) {
    ss += red[0][w];
    if constexpr (kFusedMax) amax = nan_max(amax, red[1][w]);
  }
  const float rstd = 1.0f / sqrtf(ss / static_cast<float>(a.H) + a.eps);

  // ---- y = zw * rstd (+ b)
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
#pragma unroll
    for (int k = 0; k < kVec; ++k) z[i][k] *= rstd;
    if (has_bias) VA::add(rb[i], z[i]);
  }

  if constexpr (OM == OM_BF16 || OM == OM_F32) {
    using VO = Vec<OM == OM_BF16 ? SP_BF16 : SP_F32>;
#pragma unroll
    for (int i = 0; i < VPT; ++i)
      if (live[i]) VO::store(r_out, vec[i] * VO::kBytes, z[i]);
  } else if constexpr (kMx) {
    // block of 32 = the 8-element vectors of one quad of lanes; rows hold
    // whole blocks (H % 32 == 0), so a quad is entirely live or entirely not
    constexpr int kEmax = OM == OM_MX_FP8 ? 8 : 2;
    const rsrc_t r_sc = row_rsrc(static_cast<uint8_t*>(a.out_scale) + s * (a.H / kMxBlock),
                                 static_cast<uint32_t>(a.H / kMxBlock));
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      float m = 0.0f;
#pragma unroll
      for (int k = 0; k < kVec; ++k) m = nan_max(m, fabsf(z[i][k]));
      m = quad_max(m);
      // a block holding a NaN takes the E8M0 NaN byte 0xFF (the whole block
      // reads as NaN); its elements become the e4m3 NaN code, or 0 in e2m1,
      // which has no NaN code
      const bool nan_block = m != m;
      // floor(log2 m) = frexp exponent - 1 (exact, subnormals included)
      int e = m > 0.0f ? __builtin_amdgcn_frexp_expf(m) - 1 - kEmax : -127;
      e = e < -127 ? -127 : (e > 127 ? 127 : e);
      constexpr float kNanElt = OM == OM_MX_FP8 ? __builtin_nanf("") : 0.0f;
      float t[kVec];
#pragma unroll
      for (int k = 0; k < kVec; ++k) t[k] = nan_block ? kNanElt : __builtin_ldexpf(z[i][k], -e);
      if (live[i]) {
        if constexpr (OM == OM_MX_FP8) store_e4m3(r_out, vec[i] * 8, pack_e4m3(t));
        else store_e2m1(r_out, vec[i] * 4, pack_e2m1(t));
        if ((tid & 3) == 0)
          __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(nan_block ? 0xFF : e + 127), r_sc,
                                               vec[i] / 4, 0, kStorePolicy);
      }
    }
  } else {
    float inv;
    if constexpr (OM == OM_FP8_STATIC) {
      inv = 1.0f / static_scale;
    } else {
      // max |y|: without bias, rounding is monotone so max|zw*rstd| equals
      // max|zw| * rstd exactly; with bias it needs a pass over y.  A NaN
      // anywhere in the row makes it NaN (a NaN z makes rstd NaN).
      float ymax;
      if (!has_bias) {
        ymax = amax * rstd;
      } else {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < VPT; ++i)
          if (live[i]) {
#pragma unroll
            for (int k = 0; k < kVec; ++k) m = nan_max(m, fabsf(z[i][k]));
          }
        m = wave_max(m);
        if (lane == 0) red[2][wave] = m;
        __syncthreads();
        ymax = 0.0f;
        for (int w = 0; w < nw; ++w) ymax = nan_max(ymax, red[2][w]);
      }
      // a NaN scale is stored as the positive quiet NaN; its reciprocal is
      // NaN, so every code of the row is the NaN code; a zero row (scale 0)
      // gets zero codes
      float scale = ymax / 448.0f;
      if (scale != scale) scale = __builtin_nanf("");
      if (tid == 0) static_cast<float*>(a.out_scale)[s] = scale;
      inv = scale == 0.0f ? 0.0f : 1.0f / scale;
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      float t[kVec];
#pragma unroll
      for (int k = 0; k < kVec; ++k) t[k] = z[i][k] * inv;
      if (live[i]) store_e4m3(r_out, vec[i] * 8, pack_e4m3(t));
    }
  }
}

// PT: partial dtype, AT: activation dtype, OM: output mode,
// TP: number of partials (0 = runtime, loaded in groups),
// VPT: 8-element vectors per thread.  One workgroup per shard row.
template <int PT, int AT, int OM, int TP, int VPT>
__global__ void __launch_bounds__(max_threads<VPT>()) sprms_kernel(const KArgs a) {
  __shared__ float red[3][kMaxWaves];
  process_row<PT, AT, OM, TP, VPT>(a, blockIdx.x, red);
}

// --------------------------------------------------------------- dispatch

using KFn = void (*)(KArgs);

// A compile-time partial count (every load in flight at once) is used while
// the row's loads fit in the register budget of the workgroup size (about 96
// VGPRs at 1024 threads, 112 at 512); otherwise the grouped path.
template <int PT, int AT, int TP, int VPT>
constexpr int fixed_tp() {
  constexpr int rp = PT == SP_F32 ? 8 : 4, ra = AT == SP_F32 ? 8 : 4;
  constexpr int budget = VPT == 1 ? 96 : 112;
  return (TP * VPT * rp + 4 * VPT * ra <= budget) ? TP : 0;
}

template <int PT, int AT, int OM, int TP>
KFn pick_vpt(int vpt) {
  switch (vpt) {
    case 1: return &sprms_kernel<PT, AT, OM, fixed_tp<PT, AT, TP, 1>(), 1>;
    case 2: return &sprms_kernel<PT, AT, OM, fixed_tp<PT, AT, TP, 2>(), 2>;
    case 4: return &sprms_kernel<PT, AT, OM, fixed_tp<PT, AT, TP, 4>(), 4>;
    case 8: return &sprms_kernel<PT, AT, OM, fixed_tp<PT, AT, TP, 8>(), 8>;
  }
  return nullptr;
}

template <int PT, int AT, int OM>
KFn pick_tp(int tp, int vpt) {
  switch (tp) {
    case 2: return pick_vpt<PT, AT, OM, 2>(vpt);
    case 4: return pick_vpt<PT, AT, OM, 4>(vpt);
    case 8: return pick_vpt<PT, AT, OM, 8>(vpt);
    case 16: return pick_vpt<PT, AT, OM, 16>(vpt);
    default: return pick_vpt<PT, AT, OM, 0>(vpt);
  }
}

template <int PT, int AT>
KFn pick_om(int om, int tp, int vpt) {
  switch (om) {
    case OM_BF16: return pick_tp<PT, AT, OM_BF16>(tp, vpt);
    case OM_F32: return pick_tp<PT, AT, OM_F32>(tp, vpt);
    case OM_FP8_STATIC: return pick_tp<PT, AT, OM_FP8_STATIC>(tp, vpt);
    case OM_FP8_DYN: return pick_tp<PT, AT, OM_FP8_DYN>(tp, vpt);
    case OM_MX_FP8: return pick_tp<PT, AT, OM_MX_FP8>(tp, vpt);
    case OM_MX_FP4: return pick_tp<PT, AT, OM_MX_FP4>(tp, vpt);
  }
  return nullptr;
}

KFn pick_kernel(int pt, int at, int om, int tp, int vpt) {
  if (pt == SP_BF16 && at == SP_BF16) return pick_om<SP_BF16, SP_BF16>(om, tp, vpt);
  if (pt == SP_F32 && at == SP_F32) return pick_om<SP_F32, SP_F32>(om, tp, vpt);
  if (pt == SP_BF16 && at == SP_F32) return pick_om<SP_BF16, SP_F32>(om, tp, vpt);
  if (pt == SP_F32 && at == SP_BF16) return pick_om<SP_F32, SP_BF16>(om, tp, vpt);
  return nullptr;
}

// Threads per row: one 8-element vector per thread while the row has at most
// 1024 vectors (H <= 8192), else 4 or 8 vectors per thread within 512
// threads; rounded up to whole wavefronts.
void launch_shape(int nvec, int* vpt, int* nt) {
  const int v = nvec <= kMaxThreads ? 1 : (nvec + 3) / 4 <= kMaxThreadsMultiVec ? 4 : 8;
  int n = (nvec + v - 1) / v;
  n = (n + 63) / 64 * 64;
  *vpt = v;
  *nt = n;
}

// ------------------------------------------------------------ host checks

// bytes of out_scale per row, per quant mode (static: one f32 for the tensor)
size_t scale_row_bytes_of(int quant_mode, int64_t H) {
  if (quant_mode == SP_QUANT_DYNAMIC_TOKEN) return 4;
  if (quant_mode == SP_QUANT_MX_BLOCK) return static_cast<size_t>(H) / kMxBlock;
  return 0;
}

struct Plan {
  int64_t valid;
  int64_t roff;  // first residual row used
  int64_t doff;  // first deepstack row used
};

int check(const sp_problem* p, const void* partials, const void* residual, const void* weight,
          const void* bias, float eps, int quant_mode, const void* deepstack, const void* out,
          const void* out_scale, Plan* plan) {
  if (!p) return fail(SP_ERR_NULL, "problem descriptor is NULL");
  if (p->tp < 1 || p->tp > 64) return fail(SP_ERR_SHAPE, "tp=%d outside [1, 64]", p->tp);
  if (p->tp_rank < 0 || p->tp_rank >= p->tp)
    return fail(SP_ERR_SHAPE, "tp_rank=%d outside [0, tp=%d)", p->tp_rank, p->tp);
  const int64_t S = p->shard_rows, H = p->hidden, tp = p->tp;
  if (S < 0 || S > INT32_MAX) return fail(SP_ERR_SHAPE, "shard_rows=%lld outside [0, 2^31)", (long long)S);
  if (H < 8 || H > kMaxHidden || H % 8 != 0)
    return fail(SP_ERR_SHAPE, "hidden=%lld must be a multiple of 8 in [8, %d]", (long long)H, kMaxHidden);
  if (p->num_tokens < 0 || p->num_tokens > tp * S)
    return fail(SP_ERR_SHAPE, "num_tokens=%lld outside [0, tp*S=%lld]", (long long)p->num_tokens,
                (long long)(tp * S));
  if (p->residual_rows != S && p->residual_rows != tp * S)
    return fail(SP_ERR_SHAPE, "residual_rows=%lld is neither S=%lld nor tp*S=%lld",
                (long long)p->residual_rows, (long long)S, (long long)(tp * S));
  if (deepstack == nullptr && p->deepstack_rows != 0)
    return fail(SP_ERR_SHAPE, "deepstack is NULL but deepstack_rows=%lld", (long long)p->deepstack_rows);
  if (deepstack != nullptr && p->deepstack_rows != S && p->deepstack_rows != tp * S)
    return fail(SP_ERR_SHAPE, "deepstack_rows=%lld is neither S=%lld nor tp*S=%lld",
                (long long)p->deepstack_rows, (long long)S, (long long)(tp * S));
  if (p->partial_dtype != SP_F32 && p->partial_dtype != SP_BF16)
    return fail(SP_ERR_DTYPE, "partial_dtype=%d must be SP_F32 or SP_BF16", p->partial_dtype);
  if (p->act_dtype != SP_F32 && p->act_dtype != SP_BF16)
    return fail(SP_ERR_DTYPE, "act_dtype=%d must be SP_F32 or SP_BF16", p->act_dtype);
  if (quant_mode == SP_QUANT_NONE) {
    if (p->out_dtype != SP_BF16 && p->out_dtype != SP_F32)
      return fail(SP_ERR_DTYPE, "out_dtype=%d must be SP_BF16 or SP_F32 without quantisation", p->out_dtype);
  } else if (quant_mode == SP_QUANT_STATIC_TENSOR || quant_mode == SP_QUANT_DYNAMIC_TOKEN) {
    if (p->out_dtype != SP_FP8_E4M3)
      return fail(SP_ERR_DTYPE, "out_dtype=%d must be SP_FP8_E4M3 with quant_mode=%d", p->out_dtype, quant_mode);
  } else if (quant_mode == SP_QUANT_MX_BLOCK) {
    if (p->out_dtype != SP_FP8_E4M3 && p->out_dtype != SP_FP4_E2M1)
      return fail(SP_ERR_DTYPE, "out_dtype=%d must be SP_FP8_E4M3 or SP_FP4_E2M1 with block scaling",
                  p->out_dtype);
    if (H % kMxBlock != 0)
      return fail(SP_ERR_SHAPE, "hidden=%lld must be a multiple of %d with block scaling", (long long)H,
                  kMxBlock);
  } else {
    return fail(SP_ERR_UNSUPPORTED,
                "quant_mode=%d unsupported (dynamic per-tensor scaling is not shard-local)", quant_mode);
  }
  if (!(eps >= 0.0f) || eps == __builtin_inff()) return fail(SP_ERR_SHAPE, "eps must be finite and >= 0");
  if (p->flags != 0 && p->flags != SP_FLAG_VALID_ROWS_ONLY)
    return fail(SP_ERR_UNSUPPORTED, "flags=%d unsupported", p->flags);
  if (!(p->partial_scale == p->partial_scale) || p->partial_scale == __builtin_inff() ||
      p->partial_scale == -__builtin_inff())
    return fail(SP_ERR_SHAPE, "partial_scale must be finite");
  if (p->partial_stride != 0 && p->partial_stride < S * H)
    return fail(SP_ERR_SHAPE, "partial_stride=%lld is below S*H=%lld (partials would overlap)",
                (long long)p->partial_stride, (long long)(S * H));
  if (S > 0) {
    if (!partials || !residual || !weight || !out)
      return fail(SP_ERR_NULL, "partials, residual, weight and out must be non-NULL");
    if (quant_mode != SP_QUANT_NONE && !out_scale)
      return fail(SP_ERR_NULL, "out_scale must be non-NULL with quant_mode=%d", quant_mode);
  }
  const void* dev[] = {partials, residual, weight, bias, deepstack, p->residual_out};
  for (const void* d : dev)
    if (d && misaligned(d)) return fail(SP_ERR_ALIGN, "device pointer %p is not 16-byte aligned", d);
  // out: the width of one lane's store (8 elements) -- 16 bytes for bf16 and
  // f32, 8 for e4m3, 4 for packed e2m1 -- so that an e4m3 out may start at any
  // row of a gathered tensor whose rows are a multiple of 8 bytes
  const uintptr_t out_align = p->out_dtype == SP_FP8_E4M3 ? 8 : p->out_dtype == SP_FP4_E2M1 ? 4 : 16;
  if (out && misaligned(out, out_align))
    return fail(SP_ERR_ALIGN, "out %p is not %d-byte aligned", out, static_cast<int>(out_align));
  // partials span (tp-1)*stride + S*H elements: no overflow, at most 2^47 bytes
  const int64_t stride = p->partial_stride ? p->partial_stride : S * H;
  const int64_t pe = static_cast<int64_t>(elt_size(p->partial_dtype));
  int64_t span_elems, span_bytes;
  if (__builtin_mul_overflow(tp - 1, stride, &span_elems) ||
      __builtin_add_overflow(span_elems, S * H, &span_elems) ||
      __builtin_mul_overflow(span_elems, pe, &span_bytes) || span_bytes > kMaxSpanBytes)
    return fail(SP_ERR_SHAPE, "partials of tp=%lld with partial_stride=%lld span more than 2^47 bytes",
                (long long)tp, (long long)stride);
  // (stride * pe) % 16, in a form that cannot overflow: with tp = 1 the span
  // check above leaves the stride unbounded
  if (((stride % 16) * pe) % 16 != 0)
    return fail(SP_ERR_ALIGN, "partial_stride=%lld elements is not a multiple of 16 bytes",
                (long long)stride);
  if (out_scale && quant_mode != SP_QUANT_MX_BLOCK && (reinterpret_cast<uintptr_t>(out_scale) & 3u))
    return fail(SP_ERR_ALIGN, "out_scale %p is not 4-byte aligned", out_scale);

  const int64_t r = p->tp_rank;
  int64_t v = p->num_tokens - r * S;
  v = v < 0 ? 0 : (v > S ? S : v);
  plan->valid = v;
  plan->roff = (p->residual_rows == tp * S) ? r * S : 0;
  plan->doff = (deepstack && p->deepstack_rows == tp * S) ? r * S : 0;

  // No byte written by the call may be read by it or written twice: other
  // workgroups may still be reading what one of them writes.  The one
  // exception is the in-place update of the residual rows in use.
  const size_t ae = elt_size(p->act_dtype);
  const size_t row_a = static_cast<size_t>(H) * ae;
  const char* res_used = static_cast<const char*>(residual) + plan->roff * row_a;
  const void* res_written = p->residual_out ? p->residual_out : res_used;
  const bool in_place = res_written == res_used;
  struct Span {
    const char* name;
    const void* p;
    size_t n;
  };
  const Span ins[] = {
      {"partials", partials, static_cast<size_t>(span_bytes)},
      {"weight", weight, row_a},
      {"bias", bias, bias ? row_a : 0},
      {"deepstack", deepstack, deepstack ? static_cast<size_t>(p->deepstack_rows) * row_a : 0},
      {"residual", residual, static_cast<size_t>(p->residual_rows) * row_a},
      {"the static scale", out_scale, quant_mode == SP_QUANT_STATIC_TENSOR ? sizeof(float) : 0},
  };
  const int64_t written_rows = (p->flags & SP_FLAG_VALID_ROWS_ONLY) ? plan->valid : S;
  const Span outs[] = {
      {in_place ? "the residual updated in place" : "residual_out", res_written,
       static_cast<size_t>(written_rows) * row_a},
      {"out", out, static_cast<size_t>(written_rows) * row_bytes_of(p->out_dtype, H)},
      {"out_scale", out_scale, static_cast<size_t>(written_rows) * scale_row_bytes_of(quant_mode, H)},
  };
  constexpr int kResidualIn = 4;  // ins[] entry of the residual
  for (int o = 0; o < 3; ++o) {
    for (int k = 0; k < 6; ++k) {
      if (o == 0 && in_place && k == kResidualIn) continue;
      if (overlap(outs[o].p, outs[o].n, ins[k].p, ins[k].n))
        return fail(SP_ERR_SHAPE, "%s overlaps %s", outs[o].name, ins[k].name);
    }
    for (int o2 = o + 1; o2 < 3; ++o2)
      if (overlap(outs[o].p, outs[o].n, outs[o2].p, outs[o2].n))
        return fail(SP_ERR_SHAPE, "%s overlaps %s", outs[o].name, outs[o2].name);
  }
  return SP_OK;
}

}  // namespace

// ------------------------------------------------------------------ C ABI

extern "C" {

int sp_validate(const sp_problem* p, const void* partials, const void* residual, const void* weight,
                const void* bias, float eps, int quant_mode, const void* deepstack, const void* out,
                const void* out_scale) {
  Plan plan;
  return check(p, partials, residual, weight, bias, eps, quant_mode, deepstack, out, out_scale, &plan);
}

int sp_reduce_add_rmsnorm(const sp_problem* p, const void* partials, void* residual,
                          const void* weight, const void* bias, float eps, int quant_mode,
                          const void* deepstack, void* out, void* out_scale, void* stream) {
  Plan plan;
  int rc = check(p, partials, residual, weight, bias, eps, quant_mode, deepstack, out, out_scale, &plan);
  if (rc != SP_OK) return rc;
  // rows to launch: all S rows, or only the valid ones (padding rows untouched)
  const int64_t launch_rows = (p->flags & SP_FLAG_VALID_ROWS_ONLY) ? plan.valid : p->shard_rows;
  if (launch_rows == 0) return SP_OK;

  const int64_t H = p->hidden;
  const size_t ae = elt_size(p->act_dtype);
  KArgs ka;
  ka.partials = partials;
  ka.residual = static_cast<const char*>(residual) + plan.roff * H * ae;
  ka.residual_out = p->residual_out ? p->residual_out : static_cast<char*>(residual) + plan.roff * H * ae;
  ka.weight = weight;
  ka.bias = bias;
  ka.deepstack = deepstack ? static_cast<const char*>(deepstack) + plan.doff * H * ae : nullptr;
  ka.out = out;
  ka.out_scale = out_scale;
  // with one partial the stride addresses nothing (and is not bounded by the span check)
  ka.plane = p->tp == 1 ? 0 : p->partial_stride ? p->partial_stride : p->shard_rows * H;
  ka.H = static_cast<int32_t>(H);
  ka.nvec = static_cast<int32_t>(H / kVec);
  ka.valid = static_cast<int32_t>(plan.valid);
  ka.tp = p->tp;
  ka.eps = eps;
  ka.pscale = p->partial_scale == 0.0f ? 1.0f : p->partial_scale;

  const int om = quant_mode == SP_QUANT_STATIC_TENSOR   ? OM_FP8_STATIC
                 : quant_mode == SP_QUANT_DYNAMIC_TOKEN ? OM_FP8_DYN
                 : quant_mode == SP_QUANT_MX_BLOCK      ? (p->out_dtype == SP_FP4_E2M1 ? OM_MX_FP4 : OM_MX_FP8)
                 : p->out_dtype == SP_BF16              ? OM_BF16
                                                        : OM_F32;
  int vpt, nt;
  launch_shape(ka.nvec, &vpt, &nt);
  if (nt > (vpt == 1 ? kMaxThreads : kMaxThreadsMultiVec) || nt % 64 != 0)  // launch bounds, LDS
    return fail(SP_ERR_UNSUPPORTED, "no launch shape for hidden=%lld", (long long)H);
  KFn fn = pick_kernel(p->partial_dtype, p->act_dtype, om, p->tp, vpt);
  if (!fn) return fail(SP_ERR_UNSUPPORTED, "no kernel for this dtype / mode combination");
  void* args[] = {&ka};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(static_cast<unsigned>(launch_rows)),
                                 dim3(static_cast<unsigned>(nt)), args, 0,
                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(SP_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return SP_OK;
}

}  // extern "C"
