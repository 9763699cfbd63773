// Shared device helpers and internal launcher declarations for libkvfp4.
//
// Everything here is gfx950 (CDNA4) code: wave64, 64 KiB LDS per workgroup,
// MFMA / packed-16-bit VALU.  Host-visible entry points live in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace kvfp4 {

constexpr int kBlock = 16;  // values per NVFP4 block (one E4M3 scale each)

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Page geometry as the kernels see it.
struct Geom {
  int nt;  // KV tensors per page (2: K,V; 1: MLA latent)
  int T;   // tokens per page
  int H;   // KV heads
  int D;   // head dim (multiple of 16)
  long long stride = 0;  // bytes between packed slots; 0: packed_bytes()
  __host__ __device__ long long page_stride() const { return stride ? stride : packed_bytes(); }
  __host__ __device__ long long elems() const { return (long long)nt * T * H * D; }
  __host__ __device__ long long hot_bytes() const { return 2 * elems(); }
  __host__ __device__ long long data_bytes() const { return elems() / 2; }
  __host__ __device__ long long scale_bytes() const { return elems() / kBlock; }
  __host__ __device__ long long packed_bytes() const { return data_bytes() + scale_bytes(); }
  __host__ __device__ int blocks_per_tensor() const { return T * H * (D / kBlock); }
};

// 4 floats as fp16 (round to nearest even), packed for one 8-byte store,
// and back.  The unpack works on the two 32-bit words with shifts: a
// bit_cast of a vector element (w.y) to a 2 x fp16 vector compiled to a
// copy of the low pair here.
__device__ inline u32x2 pack_f16x4(f32x4 v) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 lo = {(_Float16)v.x, (_Float16)v.y}, hi = {(_Float16)v.z, (_Float16)v.w};
  return (u32x2){__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}
__device__ inline uint16_t f16_bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
__device__ inline float f16_value(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ inline f32x4 unpack_f16x4(u32x2 w) {
  return (f32x4){f16_value((uint16_t)(w.x & 0xFFFFu)), f16_value((uint16_t)(w.x >> 16)),
                 f16_value((uint16_t)(w.y & 0xFFFFu)), f16_value((uint16_t)(w.y >> 16))};
}

// OCP E4M3FN value of a scale byte (NaN for 0x7F / 0xFF), as fp32 (exact).
__device__ inline float e4m3_to_float(uint32_t code) {
  uint32_t e = (code >> 3) & 0xF, m = code & 7;
  float v;
  if (e == 0) {
    v = (float)m * 0x1p-9f;
  } else {
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  }
  if ((code & 0x7F) == 0x7F) v = __uint_as_float(0x7FC00000u);
  return (code & 0x80) ? -v : v;
}

// fp32 value of an E2M1 magnitude code 0..7: {0, .5, 1, 1.5, 2, 3, 4, 6}.
__device__ inline float e2m1_mag_to_float(uint32_t m) {
  uint32_t bits = (m << 22) + (126u << 23);
  bits = m >= 2 ? bits : (m == 1 ? 0x3F000000u : 0u);
  return __uint_as_float(bits);
}

// bf16 bits of a finite fp64 value, rounded to nearest even once.  When v
// is the rounded head of an exact value v + e (|e| below half an fp64 ulp
// of v), tie_bias is the sign of e relative to v: +1 if the exact magnitude
// is above |v|, -1 if below, 0 if v is exact.  It only matters when v lies
// exactly halfway between two bf16 values.
__device__ inline uint32_t bf16_rne_from_f64(double v, int tie_bias = 0) {
  uint64_t b = (uint64_t)__double_as_longlong(v);
  uint32_t sign = (uint32_t)(b >> 63) << 15;
  int ex = (int)((b >> 52) & 0x7FF);
  if (ex == 0) return sign;  // zero (fp64 subnormals cannot occur here)
  uint64_t m53 = (b & ((1ull << 52) - 1)) | (1ull << 52);
  int e = ex - 1023;
  int shift = 45;                     // keep 8 significant bits
  uint32_t base;
  if (e >= -126) {
    base = (uint32_t)(e + 127) << 7;  // exponent field; the kept value adds
    // m53 >> 45 is in [128, 256): subtract the implicit bit via base
    base -= 128;
  } else {
    shift += (-126 - e);              // bf16 subnormal: fewer kept bits
    base = 0;
  }
  if (shift > 60) return sign;        // below half the smallest subnormal
  uint64_t keep = m53 >> shift;
  uint64_t rem = m53 & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  keep += (rem > half || (rem == half && (tie_bias > 0 || (tie_bias == 0 && (keep & 1))))) ? 1 : 0;
  uint32_t bits = base + (uint32_t)keep;
  if (bits >= 0x7F80u) bits = 0x7F80u;  // overflow to inf
  return sign | bits;
}

// Wave-level inclusive prefix sum of an int over 64 lanes, on DPP lane
// moves (no LDS round trips): a Hillis-Steele scan within each row of 16
// lanes (row_shr 1, 2, 4, 8), then the row totals, row_bcast:15 adding lane
// 15 of each row to the next row (rows 1 and 3) and row_bcast:31 adding
// lane 31 to rows 2 and 3.  A lane whose source lies outside its row, or
// whose row the mask leaves out, adds 0.
__device__ inline int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// ---------------------------------------------------------------------------
// Internal launchers (host side).  All validate nothing: the C ABI did.
// ---------------------------------------------------------------------------
hipError_t launch_quantize(const Geom& g, const void* hot, int hot_pages, const int32_t* src,
                           void* packed, int packed_pages, const int32_t* dst, int num_pages,
                           const float* gs, hipStream_t stream);
hipError_t launch_dequantize(const Geom& g, const void* packed, int packed_pages,
                             const int32_t* src, void* hot, int hot_pages, const int32_t* dst,
                             int num_pages, const float* gs, hipStream_t stream);

hipError_t launch_append(const Geom& g, const void* rows, bool fp8, int num_tokens,
                         const int32_t* slots, const int32_t* page_rows, void* packed,
                         int packed_pages, const float* gs, hipStream_t stream);

hipError_t launch_gather(const Geom& g, const void* packed, int packed_pages, const int32_t* slots,
                         const int32_t* page_rows, int num_tokens, void* out, bool fp8,
                         const float* gs, hipStream_t stream);

hipError_t launch_rope_encode(const Geom& g, int rope_dims, int mode, long long ext_off,
                              const void* hot, int hot_pages, const int32_t* src, void* packed,
                              int packed_pages, const int32_t* dst, int num_pages, const float* gs,
                              hipStream_t stream);
hipError_t launch_rope_decode(const Geom& g, int rope_dims, int mode, long long ext_off,
                              const void* packed, int packed_pages, const int32_t* src, void* hot,
                              int hot_pages, const int32_t* dst, int num_pages, const float* gs,
                              hipStream_t stream);

hipError_t launch_sort_pages(const int32_t* key, const int32_t* other, int num_pages,
                             int32_t* key_out, int32_t* other_out, hipStream_t stream);

// Raises a kernel's dynamic-LDS limit once per device (the setting is
// idempotent; doing it once keeps it out of launches a caller may be
// capturing into a graph).  `done` is that kernel's own device bitmask.
inline hipError_t allow_lds_once(std::atomic<unsigned long long>& done, const void* kernel,
                                 size_t bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = dev < 64 ? 1ull << dev : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

struct DecodeArgs {
  Geom g;
  const uint8_t* pool;
  int pool_pages;
  float gs_k, gs_v;
  const uint16_t* q;
  int batch, hq, v_dim;
  const int32_t* block_table;
  int max_pages;
  const int32_t* seq_lens;
  float softmax_scale;
  uint16_t* out;
  float* lse;
  // split-K plan.  Generic kernel: `splits` fixed page ranges per sequence,
  // partials [batch][hq][splits].  Balanced kernels: `nwg` workgroups over
  // the batch's concatenated pages, partials [nwg + batch][hq].
  int splits;
  int pages_per_split;
  int nwg;
  int seg_pad;           // balanced kernels: pages of a segment pad (0: none)
  float* ws_o;           // generic kernel: partial outputs, v_dim floats each
  // balanced kernels: partial outputs divided by their sum, v_dim fp16 each
  // (a weighted average of value rows: |o / l| <= 2688, which fp16 holds)
  uint16_t* ws_oh;
  float* ws_ml;          // partial (max, sum), scores in log2 units
  // Balanced kernels: the first and last workgroup whose range holds pages
  // of sequence b ([batch][2], written for every sequence with pages), then
  // the length of the split (pages and pads); the merge reads these instead
  // of rescanning.
  int32_t* ws_idx;
};

// Which decode kernel a shape uses, and how it splits the context.
struct DecodePlan {
  int kernel;            // 0 = generic, 1 = GQA VALU, 2 = MLA MFMA, 3 = GQA MFMA
  int splits;            // generic kernel
  int pages_per_split;   // generic kernel
  int nwg;               // balanced kernels
  int seg_pad;           // balanced kernels: pages of a segment pad
  size_t workspace_bytes;
};

DecodePlan plan_decode(const Geom& g, int batch, int hq, int v_dim, int max_seq_len_hint,
                       int num_cus);
hipError_t launch_decode(const DecodePlan& plan, const DecodeArgs& a, hipStream_t stream);

}  // namespace kvfp4
