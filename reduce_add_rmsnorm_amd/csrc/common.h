// common.h -- pieces shared by the translation units of libsprms (sprms.hip,
// layout.hip, gemm.hip, abi.cpp): the buffer-descriptor row I/O used by every
// kernel, the size limits, and the host-side error channel and pointer checks
// behind the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "sprms.h"

namespace sprms {

constexpr int kMaxThreads = 1024;  // largest workgroup any kernel here launches
constexpr int kMaxHidden = 32768;  // longest row of the fused path, elements
constexpr int kMaxTp = 64;         // most ranks a layout call addresses

// ------------------------------------------------------------ element I/O
//
// Row data moves through buffer instructions.  A resource descriptor covers
// exactly one row of one tensor (its base is uniform per workgroup, so it
// lives in scalar registers); the per-lane operand is a 32-bit byte offset
// inside the row, and the hardware range check against the row length
// turns a stray offset into a dropped access instead of a fault.

// Cache policy of the streamed (read-once / write-once) row data, as the
// buffer instruction's cache-policy bits on gfx950: bit 0 sc0, bit 1 nt,
// bit 4 sc1.  Data re-read by every row (gain, bias) uses policy 0.
#ifndef SPRMS_STREAM_LOAD_POLICY
#define SPRMS_STREAM_LOAD_POLICY 2
#endif
#ifndef SPRMS_STREAM_STORE_POLICY
#define SPRMS_STREAM_STORE_POLICY 2
#endif
constexpr int kLoadPolicy = SPRMS_STREAM_LOAD_POLICY;
constexpr int kStorePolicy = SPRMS_STREAM_STORE_POLICY;
constexpr int kCachedPolicy = 0;

// word 3 of a gfx9-family buffer descriptor: 32-bit data format, raw
// (stride 0) addressing with the range check against num_records
constexpr int kRsrcWord3 = 0x00020000;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
using rsrc_t = __amdgpu_buffer_rsrc_t;

__device__ __forceinline__ rsrc_t row_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           kRsrcWord3);
}

// ------------------------------------------------------------ host side

// Records a message for sp_last_error() (per host thread) and returns code.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// bytes of one element; 0 for e2m1 (two per byte) and unknown types
inline size_t elt_size(int dt) {
  return dt == SP_F32 ? 4 : dt == SP_BF16 ? 2 : dt == SP_FP8_E4M3 ? 1 : 0;
}

// bytes of one row of H elements (e2m1: two per byte); 0 for an unknown type
inline size_t row_bytes_of(int dt, int64_t H) {
  if (dt == SP_FP4_E2M1) return static_cast<size_t>(H) / 2;
  return static_cast<size_t>(H) * elt_size(dt);
}

inline bool misaligned(const void* ptr, uintptr_t align = 16) {
  return (reinterpret_cast<uintptr_t>(ptr) & (align - 1)) != 0;
}

// [a, a+an) and [b, b+bn) share a byte (empty or NULL ranges never do)
inline bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  if (!a || !b || an == 0 || bn == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bn && b0 < a0 + an;
}

}  // namespace sprms
