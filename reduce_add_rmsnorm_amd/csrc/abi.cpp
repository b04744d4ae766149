// abi.cpp -- the host-only parts of libsprms's C ABI: the per-thread error
// channel every entry point reports through, the status strings, and the
// shard-geometry helper.  No device code.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "common.h"
#include "sprms.h"

namespace sprms {

namespace {
thread_local char g_last_error[512] = "no error";
}  // namespace

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

const char* last_error() { return g_last_error; }

}  // namespace sprms

using sprms::fail;

extern "C" {

int sp_shard_geometry(int64_t num_tokens, int64_t num_tokens_pad, int32_t tp, int32_t rank,
                      int64_t* shard_rows, int64_t* local_start, int64_t* valid_rows) {
  if (!shard_rows || !local_start || !valid_rows) return fail(SP_ERR_NULL, "output pointer is NULL");
  if (tp < 1 || rank < 0 || rank >= tp) return fail(SP_ERR_SHAPE, "rank=%d outside [0, tp=%d)", rank, tp);
  if (num_tokens < 0 || num_tokens_pad < 0 || num_tokens > num_tokens_pad)
    return fail(SP_ERR_SHAPE, "need 0 <= num_tokens <= num_tokens_pad");
  if (num_tokens_pad % tp != 0) return fail(SP_ERR_SHAPE, "num_tokens_pad is not a multiple of tp");
  const int64_t S = num_tokens_pad / tp;
  const int64_t start = static_cast<int64_t>(rank) * S;
  int64_t v = num_tokens - start;
  v = v < 0 ? 0 : (v > S ? S : v);
  *shard_rows = S;
  *local_start = start;
  *valid_rows = v;
  return SP_OK;
}

const char* sp_error_string(int status) {
  switch (status) {
    case SP_OK: return "success";
    case SP_ERR_NULL: return "a required pointer is NULL";
    case SP_ERR_SHAPE: return "inconsistent sizes, rank or row counts";
    case SP_ERR_DTYPE: return "unsupported dtype combination";
    case SP_ERR_ALIGN: return "device pointer not aligned as the call requires";
    case SP_ERR_UNSUPPORTED: return "unsupported quantisation mode, flag or reserved field";
    case SP_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

const char* sp_last_error(void) { return sprms::last_error(); }

}  // extern "C"
