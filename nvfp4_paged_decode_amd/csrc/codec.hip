// NVFP4 page codec: bf16 hot pages <-> packed NVFP4 pages.
//
// "KV Cache Compression in TensorRT LLM", NVFP4 Cold-Page Compression / How
// It Works: a batch of pages is encoded into one fixed-size block per page
// on the way out and decoded on the way back.  Both kernels are pure
// streaming maps (HBM-bound): one lane owns one 16-value block, so a wave
// reads 2 KiB of bf16 contiguously and writes 512 data bytes + 64 scale
// bytes contiguously; pages are found through the slot arrays.
//
// Exactness.  The block scale is E4M3(amax / (6 gs)) and an element code is
// E2M1(|x| / (sb gs)), both rounded once from the exact quotient.  Instead
// of dividing, each workgroup builds, per tensor, the exact rounding
// thresholds of both steps in fp64 (every threshold mid * 6 gs or
// mu * sb * gs has at most 31 significant bits, so fp64 holds it exactly)
// and turns each into an integer threshold on bf16 magnitude bit patterns
// with directed rounding: for a bf16 magnitude v, "v > M" equals
// "bits(v) > bits(RD(M))" and "v >= M" equals "bits(v) > bits(RU(M)) - 1".
// A code is then the number of thresholds its input exceeds, found by
// binary search: 7 steps over 126 E4M3 thresholds per block, 3 steps over 7
// E2M1 thresholds per element, two elements per packed 16-bit instruction.
// Ties go to the even code because even-code boundaries use the strict and
// odd-code boundaries the non-strict comparison.
#include "common.hpp"

namespace kvfp4 {

namespace {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr uint32_t kPad = 0x7FFFu;  // above every finite bf16 magnitude

// LDS threshold tables, one set per tensor.
struct QuantLds {
  uint16_t e4m3[2][128];     // scale thresholds (126 used)
  uint16_t e2m1[2][128][8];  // element thresholds per scale code (7 used)
};

__device__ inline void build_tables(QuantLds& s, int nt, float gs0, float gs1) {
  const double mu[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  for (int i = threadIdx.x; i < nt * 128; i += blockDim.x) {
    int t = i >> 7, j = i & 127;
    double gs = t == 0 ? (double)gs0 : (double)gs1;
    // E4M3 midpoint between codes j and j+1, times 6 gs (exact in fp64).
    uint32_t th = kPad;
    if (j < 126) {
      double mid = 0.5 * ((double)e4m3_to_float(j) + (double)e4m3_to_float(j + 1));
      th = gt_threshold(mid * 6.0 * gs, (j & 1) == 0);
    }
    s.e4m3[t][j] = (uint16_t)th;
    double sb = (double)e4m3_to_float(j);
    for (int k = 0; k < 8; ++k) {
      uint32_t v = kPad;
      if (k < 7 && j >= 1 && j <= 126) v = gt_threshold(mu[k] * sb * gs, (k & 1) == 0);
      s.e2m1[t][j][k] = (uint16_t)v;
    }
  }
}

// Number of the 128 sorted scale thresholds that amax exceeds.
__device__ inline uint32_t scale_code(const uint16_t* th, uint32_t amax) {
  uint32_t pos = 0;
#pragma unroll
  for (uint32_t step = 64; step >= 1; step >>= 1) pos += (amax > th[pos + step - 1]) ? step : 0;
  return pos;
}

__device__ inline u16x2 as_u16x2(uint32_t x) { return __builtin_bit_cast(u16x2, x); }
__device__ inline s16x2 as_s16x2(uint32_t x) { return __builtin_bit_cast(s16x2, x); }
__device__ inline uint32_t as_u32(u16x2 x) { return __builtin_bit_cast(uint32_t, x); }
__device__ inline uint32_t as_u32(s16x2 x) { return __builtin_bit_cast(uint32_t, x); }

// 0xFFFF in each half whose magnitude v exceeds the threshold t (both < 0x8000).
__device__ inline uint32_t gt_mask(uint32_t t, uint32_t v) {
  return as_u32(as_s16x2(as_u32(as_u16x2(t) - as_u16x2(v))) >> (s16x2){15, 15});
}
__device__ inline uint32_t gt_bit(uint32_t t, uint32_t v) {
  return as_u32(as_u16x2(as_u32(as_u16x2(t) - as_u16x2(v))) >> (u16x2){15, 15});
}
__device__ inline uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) { return (m & a) | (~m & b); }

// Two elements (one dword of bf16) -> two nibbles in bits 3:0 and 19:16.
__device__ inline uint32_t encode_pair(uint32_t raw, const uint32_t T[7]) {
  uint32_t v = raw & 0x7FFF7FFFu;
  uint32_t m1 = gt_mask(T[3], v);
  uint32_t m2 = gt_mask(bfi(m1, T[5], T[1]), v);
  uint32_t ta = bfi(m1, T[4], T[0]);
  uint32_t tb = bfi(m1, T[6], T[2]);
  uint32_t b0 = gt_bit(bfi(m2, tb, ta), v);
  uint32_t code = (m1 & 0x00040004u) | (m2 & 0x00020002u) | b0;
  return code | ((raw >> 12) & 0x00080008u);
}

__global__ __launch_bounds__(kThreads) void quantize_kernel(
    Geom g, const uint8_t* __restrict__ hot, int hot_pages, const int32_t* __restrict__ src,
    uint8_t* __restrict__ packed, int packed_pages, const int32_t* __restrict__ dst,
    long long total_blocks, float gs0, float gs1) {
  __shared__ QuantLds s;
  build_tables(s, g.nt, gs0, gs1);
  __syncthreads();

  const long long bpp = (long long)g.elems() / kBlock;  // blocks per page
  const int bpt = g.blocks_per_tensor();
  const long long stride = (long long)gridDim.x * kThreads;
  for (long long blk = (long long)blockIdx.x * kThreads + threadIdx.x; blk < total_blocks;
       blk += stride) {
    long long page = blk / bpp;
    int bip = (int)(blk - page * bpp);
    int ss = src ? src[page] : (int)page;
    int ds = dst ? dst[page] : (int)page;
    if (ss < 0 || ss >= hot_pages || ds < 0 || ds >= packed_pages) continue;
    int t = bip >= bpt ? 1 : 0;
    const u32x4* in = reinterpret_cast<const u32x4*>(hot + (long long)ss * g.hot_bytes() +
                                                     (long long)bip * 32);
    u32x4 a = __builtin_nontemporal_load(in);
    u32x4 b = __builtin_nontemporal_load(in + 1);
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    // block amax over 16 magnitudes, two per packed max
    u16x2 mx = as_u16x2(w[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = __builtin_elementwise_max(mx, as_u16x2(w[i] & 0x7FFF7FFFu));
    uint32_t amax = mx.x > mx.y ? mx.x : mx.y;
    uint32_t sc = scale_code(s.e4m3[t], amax);
    const u32x4 trow = *reinterpret_cast<const u32x4*>(s.e2m1[t][sc]);
    uint32_t th16[8] = {trow.x & 0xFFFF, trow.x >> 16, trow.y & 0xFFFF, trow.y >> 16,
                        trow.z & 0xFFFF, trow.z >> 16, trow.w & 0xFFFF, trow.w >> 16};
    uint32_t T[7];
#pragma unroll
    for (int k = 0; k < 7; ++k) T[k] = th16[k] | (th16[k] << 16);
    uint32_t by[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t n = encode_pair(w[i], T);
      by[i] = (n | (n >> 12)) & 0xFFu;
    }
    u32x2 o;
    o.x = by[0] | (by[1] << 8) | (by[2] << 16) | (by[3] << 24);
    o.y = by[4] | (by[5] << 8) | (by[6] << 16) | (by[7] << 24);
    uint8_t* pp = packed + (long long)ds * g.packed_bytes();
    __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(pp + (long long)bip * 8));
    pp[g.data_bytes() + bip] = (uint8_t)sc;
  }
}

// bf16 bits of (+-) cs * gs, rounded once, for |cs * gs| in fp32's normal
// range and an exactly representable product error (gs >= 2^-96): the fp32
// product is taken to round-to-odd (sticky last bit) and then rounded to
// bf16, which equals rounding the exact product once.
__device__ inline uint32_t bf16_of_product(float cs, float gs) {
  float p = __fmul_rn(cs, gs);
  float err = __fmaf_rn(cs, gs, -p);
  uint32_t pb = __float_as_uint(p);
  bool inexact = err != 0.0f;
  bool away = inexact && ((err < 0.0f) != (p < 0.0f));  // |p| > |exact|
  pb = pb - (away ? 1u : 0u);
  pb = pb | (inexact ? 1u : 0u);
  return (pb + 0x7FFFu + ((pb >> 16) & 1u)) >> 16;
}

template <bool kTinyScale>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(
    Geom g, const uint8_t* __restrict__ packed, int packed_pages, const int32_t* __restrict__ src,
    uint8_t* __restrict__ hot, int hot_pages, const int32_t* __restrict__ dst,
    long long total_blocks, float gs0, float gs1) {
  const long long bpp = (long long)g.elems() / kBlock;
  const int bpt = g.blocks_per_tensor();
  const long long stride = (long long)gridDim.x * kThreads;
  for (long long blk = (long long)blockIdx.x * kThreads + threadIdx.x; blk < total_blocks;
       blk += stride) {
    long long page = blk / bpp;
    int bip = (int)(blk - page * bpp);
    int ss = src ? src[page] : (int)page;
    int ds = dst ? dst[page] : (int)page;
    if (ss < 0 || ss >= packed_pages || ds < 0 || ds >= hot_pages) continue;
    float gs = bip >= bpt ? gs1 : gs0;
    const uint8_t* pp = packed + (long long)ss * g.packed_bytes();
    u32x2 d = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(pp + (long long)bip * 8));
    float sb = e4m3_to_float(pp[g.data_bytes() + bip]);
    uint32_t h[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t word = i < 8 ? d.x : d.y;
      uint32_t nib = (word >> (4 * (i & 7))) & 0xF;
      float cs = e2m1_mag_to_float(nib & 7) * sb;  // exact: <= 6 significant bits
      uint32_t sign = (nib & 8) << 12;
      if (kTinyScale) {
        h[i] = bf16_rne_from_f64((double)cs * (double)gs) ^ sign;
      } else {
        h[i] = bf16_of_product(cs, gs) ^ sign;
      }
    }
    u32x4 o0 = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    u32x4 o1 = {h[8] | (h[9] << 16), h[10] | (h[11] << 16), h[12] | (h[13] << 16),
                h[14] | (h[15] << 16)};
    u32x4* out = reinterpret_cast<u32x4*>(hot + (long long)ds * g.hot_bytes() + (long long)bip * 32);
    __builtin_nontemporal_store(o0, out);
    __builtin_nontemporal_store(o1, out + 1);
  }
}

int grid_for(long long total_blocks) {
  long long wgs = (total_blocks + kThreads - 1) / kThreads;
  // enough workgroups to cover 256 CUs several times; each then loops
  long long cap = 256LL * 16;
  return (int)(wgs < cap ? wgs : cap);
}

}  // namespace

hipError_t launch_quantize(const Geom& g, const void* hot, int hot_pages, const int32_t* src,
                           void* packed, int packed_pages, const int32_t* dst, int num_pages,
                           const float* gs, hipStream_t stream) {
  long long total = (long long)num_pages * (g.elems() / kBlock);
  if (total == 0) return hipSuccess;
  float gs1 = g.nt > 1 ? gs[1] : gs[0];
  hipLaunchKernelGGL(quantize_kernel, dim3(grid_for(total)), dim3(kThreads), 0, stream, g,
                     (const uint8_t*)hot, hot_pages, src, (uint8_t*)packed, packed_pages, dst,
                     total, gs[0], gs1);
  return hipGetLastError();
}

hipError_t launch_dequantize(const Geom& g, const void* packed, int packed_pages,
                             const int32_t* src, void* hot, int hot_pages, const int32_t* dst,
                             int num_pages, const float* gs, hipStream_t stream) {
  long long total = (long long)num_pages * (g.elems() / kBlock);
  if (total == 0) return hipSuccess;
  float gs1 = g.nt > 1 ? gs[1] : gs[0];
  bool tiny = gs[0] < 0x1p-96f || gs1 < 0x1p-96f;
  if (tiny) {
    hipLaunchKernelGGL(dequantize_kernel<true>, dim3(grid_for(total)), dim3(kThreads), 0, stream,
                       g, (const uint8_t*)packed, packed_pages, src, (uint8_t*)hot, hot_pages, dst,
                       total, gs[0], gs1);
  } else {
    hipLaunchKernelGGL(dequantize_kernel<false>, dim3(grid_for(total)), dim3(kThreads), 0, stream,
                       g, (const uint8_t*)packed, packed_pages, src, (uint8_t*)hot, hot_pages, dst,
                       total, gs[0], gs1);
  }
  return hipGetLastError();
}

}  // namespace kvfp4
