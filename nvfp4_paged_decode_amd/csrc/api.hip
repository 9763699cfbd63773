// C ABI of libkvfp4: argument validation and dispatch.  Declarations and
// the contract (layouts, ownership, errors) are in include/kvfp4.h.
#include <float.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <mutex>

#include "common.hpp"
#include "kvfp4.h"

namespace {

thread_local char g_msg[512] = "";

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

int32_t ok() {
  g_msg[0] = '\0';
  return KVFP4_OK;
}

bool geometry_valid(const kvfp4_geometry* g) {
  if (!g) return false;
  if (g->num_kv_tensors != 1 && g->num_kv_tensors != 2) return false;
  if (g->page_size <= 0 || g->num_kv_heads <= 0 || g->head_dim <= 0) return false;
  if (g->head_dim % 16 != 0) return false;
  long long e = (long long)g->num_kv_tensors * g->page_size * g->num_kv_heads * g->head_dim;
  return e <= (1LL << 28);  // a page's bf16 bytes stay within a 32-bit offset
}

int32_t check_geometry(const kvfp4_geometry* g) {
  if (!g) return fail(KVFP4_ERR_INVALID_ARG, "geometry is NULL");
  if (!geometry_valid(g))
    return fail(KVFP4_ERR_INVALID_ARG,
                "invalid geometry (num_kv_tensors=%d page_size=%d num_kv_heads=%d head_dim=%d): "
                "need num_kv_tensors in {1,2}, positive sizes, head_dim %% 16 == 0",
                g->num_kv_tensors, g->page_size, g->num_kv_heads, g->head_dim);
  return KVFP4_OK;
}

int32_t check_scales(const kvfp4_geometry* g, const float* gs) {
  if (!gs) return fail(KVFP4_ERR_INVALID_ARG, "global_scale is NULL");
  for (int t = 0; t < g->num_kv_tensors; ++t) {
    float v = gs[t];
    if (!(v > 0.0f) || !isfinite(v) || (double)v * 2688.0 > (double)FLT_MAX)
      return fail(KVFP4_ERR_INVALID_ARG,
                  "global_scale[%d] = %g: must be finite, > 0 and <= FLT_MAX / 2688", t, (double)v);
  }
  return KVFP4_OK;
}

kvfp4::Geom to_geom(const kvfp4_geometry* g) {
  return kvfp4::Geom{g->num_kv_tensors, g->page_size, g->num_kv_heads, g->head_dim};
}

std::atomic<int> g_cus[64];

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int c = g_cus[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0) {
    (void)hipGetLastError();
    n = 256;
  }
  g_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Split-K scratch of the allocation-free decode entry point (one copy per
// device, allocated with the library's code object and held until the
// process ends).  In host code `scratch` names a host-side stand-in; the
// device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = size_t(96) << 20;
std::atomic<void*> g_scratch_addr[64];
std::mutex g_scratch_mu;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of `scratch` on the current device, looked up on the
// first call there (with that device current) and kept.
int32_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVFP4_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64)
    return fail(KVFP4_ERR_UNSUPPORTED, "device %d: the scratch table covers devices 0-63", dev);
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return fail(KVFP4_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                    hipGetErrorString(e));
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return KVFP4_OK;
}

int32_t check_codec(const kvfp4_geometry* g, const void* from, int32_t from_pages,
                    const int32_t* src, const void* to, int32_t to_pages, const int32_t* dst,
                    int32_t num_pages, const float* gs, const char* from_name,
                    const char* to_name) {
  int32_t st = check_geometry(g);
  if (st) return st;
  if (num_pages < 0) return fail(KVFP4_ERR_INVALID_ARG, "num_pages = %d < 0", num_pages);
  if (from_pages < 0 || to_pages < 0)
    return fail(KVFP4_ERR_INVALID_ARG, "pool page counts must be >= 0 (%d, %d)", from_pages,
                to_pages);
  if (num_pages == 0) return KVFP4_OK;
  if (!from) return fail(KVFP4_ERR_INVALID_ARG, "%s is NULL", from_name);
  if (!to) return fail(KVFP4_ERR_INVALID_ARG, "%s is NULL", to_name);
  if (from == to) return fail(KVFP4_ERR_INVALID_ARG, "%s and %s alias", from_name, to_name);
  if (!src && num_pages > from_pages)
    return fail(KVFP4_ERR_INVALID_ARG, "num_pages %d > %s pages %d with identity slots",
                num_pages, from_name, from_pages);
  if (!dst && num_pages > to_pages)
    return fail(KVFP4_ERR_INVALID_ARG, "num_pages %d > %s pages %d with identity slots",
                num_pages, to_name, to_pages);
  return check_scales(g, gs);
}

}  // namespace

namespace {

long long rope_ext_bytes(const kvfp4_geometry* g, const kvfp4_rope_layout* r) {
  const long long n = (long long)g->page_size * g->num_kv_heads * r->rope_dims;
  if (r->mode == KVFP4_ROPE_BF16) return 2 * n;
  if (r->mode == KVFP4_ROPE_2FP4) return n / 2 + n / 16;
  return 0;
}

bool rope_valid(const kvfp4_geometry* g, const kvfp4_rope_layout* r) {
  return geometry_valid(g) && r && r->rope_dims > 0 && r->rope_dims % 16 == 0 &&
         r->rope_dims <= g->head_dim &&
         (r->mode == KVFP4_ROPE_NVFP4 || r->mode == KVFP4_ROPE_BF16 ||
          r->mode == KVFP4_ROPE_2FP4);
}

int32_t check_rope(const kvfp4_geometry* g, const kvfp4_rope_layout* r) {
  if (!r) return fail(KVFP4_ERR_INVALID_ARG, "rope layout is NULL");
  if (!rope_valid(g, r))
    return fail(KVFP4_ERR_INVALID_ARG,
                "invalid rope layout (rope_dims=%d mode=%d): need rope_dims a positive multiple "
                "of 16 <= head_dim and mode KVFP4_ROPE_NVFP4, _BF16 or _2FP4",
                r->rope_dims, r->mode);
  const long long base = to_geom(g).packed_bytes();
  if (base % 16 != 0 || rope_ext_bytes(g, r) % 16 != 0)
    return fail(KVFP4_ERR_UNSUPPORTED,
                "rope layouts need the plain slot (%lld B) and the extension (%lld B) to be "
                "multiples of 16 bytes", base, rope_ext_bytes(g, r));
  return KVFP4_OK;
}

kvfp4::Geom rope_geom(const kvfp4_geometry* g, const kvfp4_rope_layout* r) {
  kvfp4::Geom k = to_geom(g);
  k.stride = k.packed_bytes() + rope_ext_bytes(g, r);
  return k;
}

}  // namespace

extern "C" {

size_t kvfp4_hot_page_bytes(const kvfp4_geometry* g) {
  if (!geometry_valid(g)) return 0;
  return (size_t)to_geom(g).hot_bytes();
}

size_t kvfp4_packed_page_bytes(const kvfp4_geometry* g) {
  if (!geometry_valid(g)) return 0;
  return (size_t)to_geom(g).packed_bytes();
}

int32_t kvfp4_quantize_pages(const kvfp4_geometry* g, const void* hot_pool,
                             int32_t hot_pool_pages, const int32_t* src_slots, void* packed_pool,
                             int32_t packed_pool_pages, const int32_t* dst_slots,
                             int32_t num_pages, const float* global_scale, void* stream) {
  int32_t st = check_codec(g, hot_pool, hot_pool_pages, src_slots, packed_pool,
                           packed_pool_pages, dst_slots, num_pages, global_scale, "hot_pool",
                           "packed_pool");
  if (st) return st;
  if (num_pages == 0) return ok();
  hipError_t e = kvfp4::launch_quantize(to_geom(g), hot_pool, hot_pool_pages, src_slots,
                                        packed_pool, packed_pool_pages, dst_slots, num_pages,
                                        global_scale, (hipStream_t)stream);
  if (e != hipSuccess) return fail(KVFP4_ERR_HIP, "quantize launch: %s", hipGetErrorString(e));
  return ok();
}

int32_t kvfp4_dequantize_pages(const kvfp4_geometry* g, const void* packed_pool,
                               int32_t packed_pool_pages, const int32_t* src_slots,
                               void* hot_pool, int32_t hot_pool_pages, const int32_t* dst_slots,
                               int32_t num_pages, const float* global_scale, void* stream) {
  int32_t st = check_codec(g, packed_pool, packed_pool_pages, src_slots, hot_pool,
                           hot_pool_pages, dst_slots, num_pages, global_scale, "packed_pool",
                           "hot_pool");
  if (st) return st;
  if (num_pages == 0) return ok();
  hipError_t e = kvfp4::launch_dequantize(to_geom(g), packed_pool, packed_pool_pages, src_slots,
                                          hot_pool, hot_pool_pages, dst_slots, num_pages,
                                          global_scale, (hipStream_t)stream);
  if (e != hipSuccess) return fail(KVFP4_ERR_HIP, "dequantize launch: %s", hipGetErrorString(e));
  return ok();
}

int32_t kvfp4_sort_page_list(const int32_t* key, const int32_t* other, int32_t num_pages,
                             int32_t* key_out, int32_t* other_out, void* stream) {
  if (num_pages < 0) return fail(KVFP4_ERR_INVALID_ARG, "num_pages = %d < 0", num_pages);
  if (num_pages == 0) return ok();
  if (!key || !key_out)
    return fail(KVFP4_ERR_INVALID_ARG, "NULL key list (key=%p key_out=%p)", (const void*)key,
                (void*)key_out);
  if ((other == nullptr) != (other_out == nullptr))
    return fail(KVFP4_ERR_INVALID_ARG, "other and other_out must both be given or both be NULL");
  const uintptr_t n4 = (uintptr_t)num_pages * sizeof(int32_t);
  auto overlap = [n4](const void* a, const void* b) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return a && b && x < y + n4 && y < x + n4;
  };
  if (overlap(key_out, key) || overlap(key_out, other) || overlap(other_out, key) ||
      overlap(other_out, other) || overlap(key_out, other_out))
    return fail(KVFP4_ERR_INVALID_ARG, "sort outputs overlap each other or the inputs");
  hipError_t e = kvfp4::launch_sort_pages(key, other, num_pages, key_out, other_out,
                                          (hipStream_t)stream);
  if (e != hipSuccess) return fail(KVFP4_ERR_HIP, "sort launch: %s", hipGetErrorString(e));
  return ok();
}

size_t kvfp4_packed_page_bytes_rope(const kvfp4_geometry* g, const kvfp4_rope_layout* rope) {
  if (!rope_valid(g, rope)) return 0;
  return (size_t)(to_geom(g).packed_bytes() + rope_ext_bytes(g, rope));
}

int32_t kvfp4_quantize_pages_rope(const kvfp4_geometry* g, const kvfp4_rope_layout* rope,
                                  const void* hot_pool, int32_t hot_pool_pages,
                                  const int32_t* src_slots, void* packed_pool,
                                  int32_t packed_pool_pages, const int32_t* dst_slots,
                                  int32_t num_pages, const float* global_scale, void* stream) {
  int32_t st = check_codec(g, hot_pool, hot_pool_pages, src_slots, packed_pool,
                           packed_pool_pages, dst_slots, num_pages, global_scale, "hot_pool",
                           "packed_pool");
  if (st) return st;
  st = check_rope(g, rope);
  if (st) return st;
  if (num_pages == 0) return ok();
  const kvfp4::Geom k = rope_geom(g, rope);
  hipError_t e = kvfp4::launch_quantize(k, hot_pool, hot_pool_pages, src_slots, packed_pool,
                                        packed_pool_pages, dst_slots, num_pages, global_scale,
                                        (hipStream_t)stream);
  if (e == hipSuccess)
    e = kvfp4::launch_rope_encode(k, rope->rope_dims, rope->mode, k.packed_bytes(), hot_pool,
                                  hot_pool_pages, src_slots, packed_pool, packed_pool_pages,
                                  dst_slots, num_pages, global_scale, (hipStream_t)stream);
  if (e != hipSuccess) return fail(KVFP4_ERR_HIP, "quantize launch: %s", hipGetErrorString(e));
  return ok();
}

int32_t kvfp4_dequantize_pages_rope(const kvfp4_geometry* g, const kvfp4_rope_layout* rope,
                                    const void* packed_pool, int32_t packed_pool_pages,
                                    const int32_t* src_slots, void* hot_pool,
                                    int32_t hot_pool_pages, const int32_t* dst_slots,
                                    int32_t num_pages, const float* global_scale, void* stream) {
  int32_t st = check_codec(g, packed_pool, packed_pool_pages, src_slots, hot_pool,
                           hot_pool_pages, dst_slots, num_pages, global_scale, "packed_pool",
                           "hot_pool");
  if (st) return st;
  st = check_rope(g, rope);
  if (st) return st;
  if (num_pages == 0) return ok();
  const kvfp4::Geom k = rope_geom(g, rope);
  hipError_t e = kvfp4::launch_dequantize(k, packed_pool, packed_pool_pages, src_slots, hot_pool,
                                          hot_pool_pages, dst_slots, num_pages, global_scale,
                                          (hipStream_t)stream);
  if (e == hipSuccess)
    e = kvfp4::launch_rope_decode(k, rope->rope_dims, rope->mode, k.packed_bytes(), packed_pool,
                                  packed_pool_pages, src_slots, hot_pool, hot_pool_pages,
                                  dst_slots, num_pages, global_scale, (hipStream_t)stream);
  if (e != hipSuccess) return fail(KVFP4_ERR_HIP, "dequantize launch: %s", hipGetErrorString(e));
  return ok();
}

int32_t kvfp4_append_quantize(const kvfp4_geometry* g, const void* rows, int32_t rows_dtype,
                              int32_t num_tokens, const int32_t* token_slots,
                              const int32_t* token_rows, void* packed_pool,
                              int32_t packed_pool_pages, const float* global_scale,
                              void* stream) {
  int32_t st = check_geometry(g);
  if (st) return st;
  if (rows_dtype != KVFP4_ROWS_BF16 && rows_dtype != KVFP4_ROWS_FP8_E4M3)
    return fail(KVFP4_ERR_INVALID_ARG, "rows_dtype = %d is not KVFP4_ROWS_BF16 or "
                "KVFP4_ROWS_FP8_E4M3", rows_dtype);
  if (num_tokens < 0) return fail(KVFP4_ERR_INVALID_ARG, "num_tokens = %d < 0", num_tokens);
  if (packed_pool_pages < 0)
    return fail(KVFP4_ERR_INVALID_ARG, "packed_pool_pages = %d < 0", packed_pool_pages);
  if (num_tokens == 0) return ok();
  if (!rows) return fail(KVFP4_ERR_INVALID_ARG, "rows is NULL");
  if (!token_slots) return fail(KVFP4_ERR_INVALID_ARG, "token_slots is NULL");
  if (!token_rows) return fail(KVFP4_ERR_INVALID_ARG, "token_rows is NULL");
  if (!packed_pool) return fail(KVFP4_ERR_INVALID_ARG, "packed_pool is NULL");
  if (((uintptr_t)rows & 15u) != 0)
    return fail(KVFP4_ERR_INVALID_ARG, "rows must be 16-byte aligned");
  const long long per_token = (long long)g->num_kv_tensors * g->num_kv_heads * g->head_dim;
  if (per_token / 8 * num_tokens >= (1LL << 31))
    return fail(KVFP4_ERR_INVALID_ARG, "num_tokens %d x %lld values per token is too large",
                num_tokens, per_token);
  st = check_scales(g, global_scale);
  if (st) return st;
  hipError_t e = kvfp4::launch_append(to_geom(g), rows, rows_dtype == KVFP4_ROWS_FP8_E4M3,
                                      num_tokens, token_slots, token_rows,
                                      packed_pool, packed_pool_pages, global_scale,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return fail(KVFP4_ERR_HIP, "append launch: %s", hipGetErrorString(e));
  return ok();
}

int32_t kvfp4_gather_dequantize(const kvfp4_geometry* g, const void* packed_pool,
                                int32_t packed_pool_pages, const int32_t* token_slots,
                                const int32_t* token_rows, int32_t num_tokens, void* out,
                                int32_t out_dtype, const float* global_scale, void* stream) {
  int32_t st = check_geometry(g);
  if (st) return st;
  if (out_dtype != KVFP4_ROWS_BF16 && out_dtype != KVFP4_ROWS_FP8_E4M3)
    return fail(KVFP4_ERR_INVALID_ARG, "out_dtype = %d is not KVFP4_ROWS_BF16 or "
                "KVFP4_ROWS_FP8_E4M3", out_dtype);
  if (num_tokens < 0) return fail(KVFP4_ERR_INVALID_ARG, "num_tokens = %d < 0", num_tokens);
  if (packed_pool_pages < 0)
    return fail(KVFP4_ERR_INVALID_ARG, "packed_pool_pages = %d < 0", packed_pool_pages);
  if (num_tokens == 0) return ok();
  if (!packed_pool) return fail(KVFP4_ERR_INVALID_ARG, "packed_pool is NULL");
  if (!token_slots) return fail(KVFP4_ERR_INVALID_ARG, "token_slots is NULL");
  if (!token_rows) return fail(KVFP4_ERR_INVALID_ARG, "token_rows is NULL");
  if (!out) return fail(KVFP4_ERR_INVALID_ARG, "out is NULL");
  const bool fp8 = out_dtype == KVFP4_ROWS_FP8_E4M3;
  if (((uintptr_t)out & (fp8 ? 7u : 15u)) != 0)
    return fail(KVFP4_ERR_INVALID_ARG, "out must be %d-byte aligned", fp8 ? 8 : 16);
  const long long per_token = (long long)g->num_kv_tensors * g->num_kv_heads * g->head_dim;
  if (per_token / 8 * num_tokens >= (1LL << 31))
    return fail(KVFP4_ERR_INVALID_ARG, "num_tokens %d x %lld values per token is too large",
                num_tokens, per_token);
  st = check_scales(g, global_scale);
  if (st) return st;
  hipError_t e = kvfp4::launch_gather(to_geom(g), packed_pool, packed_pool_pages, token_slots,
                                      token_rows, num_tokens, out, fp8, global_scale,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return fail(KVFP4_ERR_HIP, "gather launch: %s", hipGetErrorString(e));
  return ok();
}

static int32_t check_decode_shape(const kvfp4_geometry* g, int32_t batch, int32_t num_q_heads,
                                  int32_t v_dim, int32_t max_seq_len_hint) {
  int32_t st = check_geometry(g);
  if (st) return st;
  if (batch < 0) return fail(KVFP4_ERR_INVALID_ARG, "batch = %d < 0", batch);
  if (num_q_heads <= 0 || num_q_heads % g->num_kv_heads != 0)
    return fail(KVFP4_ERR_INVALID_ARG, "num_q_heads = %d must be a positive multiple of %d",
                num_q_heads, g->num_kv_heads);
  if (v_dim <= 0 || v_dim > g->head_dim)
    return fail(KVFP4_ERR_INVALID_ARG, "v_dim = %d must be in [1, head_dim=%d]", v_dim,
                g->head_dim);
  if (g->num_kv_tensors == 2 && v_dim != g->head_dim)
    return fail(KVFP4_ERR_INVALID_ARG, "v_dim = %d must equal head_dim with separate K and V",
                v_dim);
  if (max_seq_len_hint < 0)
    return fail(KVFP4_ERR_INVALID_ARG, "max_seq_len_hint = %d < 0", max_seq_len_hint);
  if (g->head_dim > 576)
    return fail(KVFP4_ERR_UNSUPPORTED, "head_dim %d > 576 has no decode kernel", g->head_dim);
  return KVFP4_OK;
}

size_t kvfp4_decode_workspace_bytes(const kvfp4_geometry* g, int32_t batch, int32_t num_q_heads,
                                    int32_t v_dim, int32_t max_seq_len_hint) {
  if (check_decode_shape(g, batch, num_q_heads, v_dim, max_seq_len_hint)) return 0;
  return kvfp4::plan_decode(to_geom(g), batch, num_q_heads, v_dim, max_seq_len_hint,
                            device_cus())
      .workspace_bytes;
}

}  // extern "C"

namespace {

// Validation and launch of one decode call: on the caller's workspace
// (`workspace`, `workspace_bytes`), or with `scratch` set on the library's
// scratch array (the allocation-free entry point; the workspace arguments
// are then ignored).
int32_t decode_call(const kvfp4_geometry* g, const void* packed_pool, int32_t packed_pool_pages,
                    const float* global_scale, const void* q, int32_t batch,
                    int32_t num_q_heads, int32_t v_dim, const int32_t* block_table,
                    int32_t max_pages_per_seq, const int32_t* seq_lens,
                    int32_t max_seq_len_hint, float softmax_scale, void* out, float* lse,
                    void* workspace, size_t workspace_bytes, bool scratch, void* stream);

}  // namespace

extern "C" {

int32_t kvfp4_paged_decode_attention(const kvfp4_geometry* g, const void* packed_pool,
                                     int32_t packed_pool_pages, const float* global_scale,
                                     const void* q, int32_t batch, int32_t num_q_heads,
                                     int32_t v_dim, const int32_t* block_table,
                                     int32_t max_pages_per_seq, const int32_t* seq_lens,
                                     int32_t max_seq_len_hint, float softmax_scale, void* out,
                                     float* lse, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  return decode_call(g, packed_pool, packed_pool_pages, global_scale, q, batch, num_q_heads,
                     v_dim, block_table, max_pages_per_seq, seq_lens, max_seq_len_hint,
                     softmax_scale, out, lse, workspace, workspace_bytes, false, stream);
}

int32_t kvfp4_paged_decode_attention_noalloc(const kvfp4_geometry* g, const void* packed_pool,
                                             int32_t packed_pool_pages, const float* global_scale,
                                             const void* q, int32_t batch, int32_t num_q_heads,
                                             int32_t v_dim, const int32_t* block_table,
                                             int32_t max_pages_per_seq, const int32_t* seq_lens,
                                             int32_t max_seq_len_hint, float softmax_scale,
                                             void* out, float* lse, void* stream) {
  return decode_call(g, packed_pool, packed_pool_pages, global_scale, q, batch, num_q_heads,
                     v_dim, block_table, max_pages_per_seq, seq_lens, max_seq_len_hint,
                     softmax_scale, out, lse, nullptr, 0, true, stream);
}

}  // extern "C"

namespace {

int32_t decode_call(const kvfp4_geometry* g, const void* packed_pool, int32_t packed_pool_pages,
                    const float* global_scale, const void* q, int32_t batch,
                    int32_t num_q_heads, int32_t v_dim, const int32_t* block_table,
                    int32_t max_pages_per_seq, const int32_t* seq_lens,
                    int32_t max_seq_len_hint, float softmax_scale, void* out, float* lse,
                    void* workspace, size_t workspace_bytes, bool scratch, void* stream) {
  int32_t st = check_decode_shape(g, batch, num_q_heads, v_dim, max_seq_len_hint);
  if (st) return st;
  if (batch == 0) return ok();
  if (!packed_pool || !q || !block_table || !seq_lens || !out)
    return fail(KVFP4_ERR_INVALID_ARG,
                "NULL required pointer (packed_pool=%p q=%p block_table=%p seq_lens=%p out=%p)",
                packed_pool, q, block_table, seq_lens, out);
  if (packed_pool_pages <= 0)
    return fail(KVFP4_ERR_INVALID_ARG, "packed_pool_pages = %d <= 0", packed_pool_pages);
  if (max_pages_per_seq <= 0)
    return fail(KVFP4_ERR_INVALID_ARG, "max_pages_per_seq = %d <= 0", max_pages_per_seq);
  if (!isfinite(softmax_scale))
    return fail(KVFP4_ERR_INVALID_ARG, "softmax_scale is not finite");
  st = check_scales(g, global_scale);
  if (st) return st;
  kvfp4::Geom geom = to_geom(g);
  kvfp4::DecodePlan plan =
      kvfp4::plan_decode(geom, batch, num_q_heads, v_dim, max_seq_len_hint, device_cus());
  if (scratch) {
    if (plan.workspace_bytes > kScratchBytes)
      return fail(KVFP4_ERR_WORKSPACE,
                  "these sizes need %zu bytes of split-K scratch, more than the %zu bytes the "
                  "allocation-free entry point holds; call kvfp4_paged_decode_attention with "
                  "a workspace instead", plan.workspace_bytes, kScratchBytes);
    if (((uintptr_t)q & 15) != 0)
      return fail(KVFP4_ERR_INVALID_ARG, "q must be 16-byte aligned");
    int32_t sst = scratch_address(&workspace);
    if (sst) return sst;
    workspace_bytes = kScratchBytes;
  }
  if (workspace_bytes < plan.workspace_bytes || (plan.workspace_bytes > 0 && !workspace))
    return fail(KVFP4_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes,
                plan.workspace_bytes);
  if (plan.workspace_bytes > 0 && ((uintptr_t)workspace & 15) != 0)
    return fail(KVFP4_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (((uintptr_t)q & 15) != 0)
    return fail(KVFP4_ERR_INVALID_ARG, "q must be 16-byte aligned");
  kvfp4::DecodeArgs a{};
  a.g = geom;
  a.pool = (const uint8_t*)packed_pool;
  a.pool_pages = packed_pool_pages;
  a.gs_k = global_scale[0];
  a.gs_v = g->num_kv_tensors == 2 ? global_scale[1] : global_scale[0];
  a.q = (const uint16_t*)q;
  a.batch = batch;
  a.hq = num_q_heads;
  a.v_dim = v_dim;
  a.block_table = block_table;
  a.max_pages = max_pages_per_seq;
  a.seq_lens = seq_lens;
  a.softmax_scale = softmax_scale;
  a.out = (uint16_t*)out;
  a.lse = lse;
  a.splits = plan.splits;
  a.pages_per_split = plan.pages_per_split;
  a.nwg = plan.nwg;
  // pads need P nwg < 2^31 (P <= batch * max_pages_per_seq)
  a.seg_pad = (long long)batch * max_pages_per_seq * plan.nwg < (1LL << 31) ? plan.seg_pad : 0;
  size_t partials = plan.kernel == 0 ? (size_t)batch * num_q_heads * plan.splits
                                     : (size_t)(plan.nwg + batch) * num_q_heads;
  if (plan.kernel == 0) {  // generic kernel: fp32 partial outputs
    a.ws_o = (float*)workspace;
    a.ws_ml = a.ws_o + partials * v_dim;
  } else {  // balanced kernels: fp16 partial outputs (v_dim is even)
    a.ws_oh = (uint16_t*)workspace;
    a.ws_ml = reinterpret_cast<float*>(a.ws_oh + partials * v_dim);
  }
  a.ws_idx = reinterpret_cast<int32_t*>(a.ws_ml + partials * 2);
  hipError_t e = kvfp4::launch_decode(plan, a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(KVFP4_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* kvfp4_status_string(int32_t status) {
  switch (status) {
    case KVFP4_OK: return "ok";
    case KVFP4_ERR_INVALID_ARG: return "invalid argument";
    case KVFP4_ERR_UNSUPPORTED: return "unsupported geometry";
    case KVFP4_ERR_WORKSPACE: return "workspace too small";
    case KVFP4_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* kvfp4_last_error_message(void) { return g_msg; }

}  // extern "C"
