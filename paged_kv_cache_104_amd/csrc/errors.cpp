// Error reporting and descriptor validation of the C ABI.
#include <cmath>
#include <cstdio>
#include <cstring>

#include "pkv_internal.h"

namespace pkv {

static thread_local char g_msg[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_msg[0] = '\0'; }

int check_desc(const pkv_cache_desc* c) {
  if (!c) return fail(PKV_E_INVAL, "cache descriptor is NULL");
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0)
    return fail(PKV_E_INVAL, "num_blocks (%d) and num_kv_heads (%d) must be positive",
                c->num_blocks, c->num_kv_heads);
  if (c->block_size != 8 && c->block_size != 16 && c->block_size != 32)
    return fail(PKV_E_UNSUPPORTED, "block_size %d not built (8, 16, 32)", c->block_size);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(PKV_E_UNSUPPORTED, "head_dim %d not built (64, 128)", c->head_dim);
  if (c->kv_dtype != PKV_F32 && c->kv_dtype != PKV_BF16 && c->kv_dtype != PKV_FP8_E4M3)
    return fail(PKV_E_INVAL, "unknown kv_dtype %d", c->kv_dtype);
  if (c->kv_dtype == PKV_FP8_E4M3) {
    if (!(c->k_scale > 0.f) || !(c->v_scale > 0.f) || !std::isfinite(c->k_scale) ||
        !std::isfinite(c->v_scale))
      return fail(PKV_E_INVAL, "fp8 pool needs finite positive k_scale / v_scale");
  } else if (c->k_scale != 1.f || c->v_scale != 1.f) {
    return fail(PKV_E_INVAL, "k_scale / v_scale must be 1 for a %s pool", dtype_name(c->kv_dtype));
  }
  // 64-bit block stride x num_blocks must fit the address space comfortably
  return PKV_OK;
}

}  // namespace pkv

extern "C" const char* pkv_last_error(void) { return pkv::g_msg; }
extern "C" const char* pkv_version(void) { return "pagedkv 0.1 (gfx950)"; }
