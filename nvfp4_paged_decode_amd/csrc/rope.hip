// RoPE-part storage variants of the cold-page codec ("KV Cache Compression
// in TensorRT LLM", How It Works / The RoPE part of K): the position-encoded
// last R dims of every tensor-0 (K, or MLA latent) head row are either kept
// at their original bf16 precision or stored as two FP4 layers, the second
// encoding the first one's rounding error (2FP4).
//
// The page keeps the base layout -- every value NVFP4-encoded, written by the
// base encoder -- and appends one extension region [T][H][R]: bf16 values,
// or the second layer's data [T][H][R/2] then its scales [T][H][R/16].
// These kernels run after the base kernels on the same stream: the encoder
// reads the first layer the base encoder just wrote, and the decoder
// overwrites the RoPE dims the base decoder just wrote.
//
// Exactness of 2FP4: x (bf16) minus the first layer's value D1 (at most 30
// significant bits, within a few binades of x when it is not zero) is exact
// in fp64, but the residual has up to ~40 significant bits, so its scale and
// element codes are decided by comparisons with exact fp64 thresholds (the
// rounding midpoints times 6 gs, or times sb gs), never by a rounded
// quotient alone.  D1 + D2 can need more than 53 bits: the sum is formed
// with an exact two-sum and rounded to bf16 once, the error term breaking
// exact ties.
#include "common.hpp"

namespace kvfp4 {
namespace {

constexpr int kThreads = 256;

struct RopeGeom {
  int R;              // RoPE dims per tensor-0 head row
  long long ext_off;  // byte offset of the extension region in a page
};

__device__ inline int page_slot_r(const int32_t* slots, int i, int pool_pages) {
  int s = slots ? __builtin_amdgcn_readfirstlane(slots[i]) : i;
  return (s >= 0 && s < pool_pages) ? s : -1;
}

__device__ inline void page_range_r(int num_pages, int& p0, int& p1) {
  p0 = (int)((long long)blockIdx.x * num_pages / gridDim.x);
  p1 = (int)((long long)(blockIdx.x + 1) * num_pages / gridDim.x);
}

// Exact value of nibble n (sign bit 3) under scale code sc and tensor scale gs.
__device__ inline double nib_value(uint32_t n, uint32_t sc, double gs) {
  const double v = (double)e2m1_mag_to_float(n & 7u) * (double)e4m3_to_float(sc) * gs;
  return (n & 8u) ? -v : v;
}

// Nearest-even E4M3 code of amax / (6 gs) for an exact amax: estimate from
// the fp64 quotient, then settle against the exact midpoints either side.
__device__ inline uint32_t residual_scale_code(double amax, double gs) {
  const double q = amax / (6.0 * gs);
  int c;
  if (!(q > 0.0)) {
    c = 0;
  } else if (q >= 448.0) {
    c = 126;
  } else if (q < 0x1p-6) {
    c = (int)rint(q * 512.0);
  } else {
    int E;
    (void)frexp(q, &E);
    const int e = E - 1;
    c = ((e + 7) << 3) + (int)rint(ldexp(q, -e) * 8.0) - 8;
    if (c > 126) c = 126;
  }
  // the exact code is within one of the estimate
  if (c > 0) {
    const double lo = 0.5 * ((double)e4m3_to_float(c - 1) + (double)e4m3_to_float(c)) * 6.0 * gs;
    if (amax < lo || (amax == lo && (c & 1))) --c;
  }
  if (c < 126) {
    const double hi = 0.5 * ((double)e4m3_to_float(c) + (double)e4m3_to_float(c + 1)) * 6.0 * gs;
    if (amax > hi || (amax == hi && ((c + 1) & 1) == 0)) ++c;
  }
  return (uint32_t)c;
}

// E2M1 magnitude code of |r| / (sb gs) by exact comparisons with the seven
// midpoints; at a midpoint, the even code.
__device__ inline uint32_t residual_code(double a, double sbgs) {
  const double mu[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
  uint32_t c = 0;
#pragma unroll
  for (int k = 0; k < 7; ++k) {
    const double th = mu[k] * sbgs;  // exact
    // past midpoint k the code is k + 1; at it, k + 1 only if that is even
    c += (a > th || (a == th && (k & 1))) ? 1u : 0u;
  }
  return c;
}

// One lane per half block of the RoPE dims (R/8 per row, two per block,
// adjacent lanes): reads 8 bf16 inputs and the first layer's 4 data bytes
// and scale byte, writes the extension's bf16 copy or second layer.
template <int kMode>
__global__ __launch_bounds__(kThreads) void rope_encode_kernel(
    Geom g, RopeGeom rg, const uint8_t* __restrict__ hot, int hot_pages,
    const int32_t* __restrict__ src, uint8_t* __restrict__ packed, int packed_pages,
    const int32_t* __restrict__ dst, int num_pages, float gs0) {
  const int hpr = rg.R / 8;                 // half-blocks per row (even)
  const int rows = g.T * g.H;               // tensor-0 rows per page
  const int hpp = rows * hpr;
  const long long data_bytes = g.data_bytes();
  const double gs = (double)gs0;
  int p0, p1;
  page_range_r(num_pages, p0, p1);
  for (int p = p0; p < p1; ++p) {
    const int ss = page_slot_r(src, p, hot_pages);
    const int ds = page_slot_r(dst, p, packed_pages);
    if (ss < 0 || ds < 0) continue;
    const uint8_t* in = hot + (long long)ss * g.hot_bytes();
    uint8_t* page = packed + (long long)ds * g.page_stride();
    uint8_t* ext = page + rg.ext_off;
    // the loop bound is uniform: every lane runs the body (DPP partner)
    for (int h0 = 0; h0 < hpp; h0 += kThreads) {
      const int hb = h0 + (int)threadIdx.x;
      const bool live = hb < hpp;
      const int row = live ? hb / hpr : 0, k = live ? hb - row * hpr : 0;
      // first element of this half block in tensor 0's [T][H][D] order
      const long long e0 = (long long)row * g.D + (g.D - rg.R) + 8 * k;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (live) x = *reinterpret_cast<const u32x4*>(in + 2 * e0);
      if (kMode == 1) {
        if (live)
          *reinterpret_cast<u32x4*>(ext + 16 * ((long long)row * hpr + k)) = x;
        continue;
      }
      uint32_t w1 = 0u, s1 = 0u;
      if (live) {
        w1 = *reinterpret_cast<const uint32_t*>(page + e0 / 2);
        s1 = page[data_bytes + e0 / 16];
      }
      const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
      double r[8];
      double amax = 0.0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t xb = (xs[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
        const double xv = (double)__uint_as_float(xb << 16);
        const double d1 = nib_value((w1 >> (4 * i)) & 0xFu, s1, gs);
        double ri = xv - d1;                  // exact
        if (ri == 0.0) ri = copysign(0.0, xv);  // a zero residual keeps x's sign
        r[i] = ri;
        amax = fmax(amax, fabs(ri));
      }
      // the partner lane holds the other half of the block
      const long long ab = __double_as_longlong(amax);
      const int lo = __builtin_amdgcn_mov_dpp((int)(ab & 0xFFFFFFFF), 0xB1, 0xF, 0xF, true);
      const int hi = __builtin_amdgcn_mov_dpp((int)(ab >> 32), 0xB1, 0xF, 0xF, true);
      const double other =
          __longlong_as_double(((long long)(uint32_t)hi << 32) | (long long)(uint32_t)lo);
      amax = fmax(amax, other);
      const uint32_t sc = residual_scale_code(amax, gs);
      const double sbgs = (double)e4m3_to_float(sc) * gs;
      uint32_t word = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t mag = sc == 0u ? 0u : residual_code(fabs(r[i]), sbgs);
        const uint32_t nib = (signbit(r[i]) ? 8u : 0u) | mag;
        word |= nib << (4 * i);
      }
      if (!live) continue;
      const long long idx = (long long)row * hpr + k;  // half block in [T][H][R/8]
      *reinterpret_cast<uint32_t*>(ext + 4 * idx) = word;
      if ((k & 1) == 0) ext[(long long)rows * rg.R / 2 + idx / 2] = (uint8_t)sc;
    }
  }
}

// Overwrites the RoPE dims of decoded tensor-0 rows: the kept bf16 values,
// or bf16_RNE(D1 + D2) from both layers.
template <int kMode>
__global__ __launch_bounds__(kThreads) void rope_decode_kernel(
    Geom g, RopeGeom rg, const uint8_t* __restrict__ packed, int packed_pages,
    const int32_t* __restrict__ src, uint8_t* __restrict__ hot, int hot_pages,
    const int32_t* __restrict__ dst, int num_pages, float gs0) {
  const int hpr = rg.R / 8;
  const int rows = g.T * g.H;
  const int hpp = rows * hpr;
  const long long data_bytes = g.data_bytes();
  const double gs = (double)gs0;
  int p0, p1;
  page_range_r(num_pages, p0, p1);
  for (int p = p0; p < p1; ++p) {
    const int ss = page_slot_r(src, p, packed_pages);
    const int ds = page_slot_r(dst, p, hot_pages);
    if (ss < 0 || ds < 0) continue;
    const uint8_t* page = packed + (long long)ss * g.page_stride();
    const uint8_t* ext = page + rg.ext_off;
    uint8_t* out = hot + (long long)ds * g.hot_bytes();
    for (int hb = (int)threadIdx.x; hb < hpp; hb += kThreads) {
      const int row = hb / hpr, k = hb - row * hpr;
      const long long e0 = (long long)row * g.D + (g.D - rg.R) + 8 * k;
      const long long idx = (long long)row * hpr + k;
      u32x4 o;
      if (kMode == 1) {
        o = *reinterpret_cast<const u32x4*>(ext + 16 * idx);
      } else {
        const uint32_t w1 = *reinterpret_cast<const uint32_t*>(page + e0 / 2);
        const uint32_t s1 = page[data_bytes + e0 / 16];
        const uint32_t w2 = *reinterpret_cast<const uint32_t*>(ext + 4 * idx);
        const uint32_t s2 = ext[(long long)rows * rg.R / 2 + idx / 2];
        uint32_t b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double a = nib_value((w1 >> (4 * i)) & 0xFu, s1, gs);
          const double c = nib_value((w2 >> (4 * i)) & 0xFu, s2, gs);
          // two-sum: s + err == a + c exactly
          const double s = a + c;
          const double bb = s - a;
          const double err = (a - (s - bb)) + (c - bb);
          const int bias = err == 0.0 ? 0 : ((err > 0.0) == (s > 0.0) ? 1 : -1);
          b[i] = bf16_rne_from_f64(s, bias);
        }
        o = (u32x4){b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16),
                    b[6] | (b[7] << 16)};
      }
      *reinterpret_cast<u32x4*>(out + 2 * e0) = o;
    }
  }
}

// One workgroup per page (no per-workgroup table to amortize); with fewer
// workgroups than pages some would take one page more while the rest wait.
// Past the cap each walks a contiguous run, the runs differing by at most one.
int rope_grid(int num_pages) { return num_pages < 65536 ? num_pages : 65536; }

}  // namespace

hipError_t launch_rope_encode(const Geom& g, int rope_dims, int mode, long long ext_off,
                              const void* hot, int hot_pages, const int32_t* src, void* packed,
                              int packed_pages, const int32_t* dst, int num_pages, const float* gs,
                              hipStream_t stream) {
  if (num_pages == 0 || mode == 0) return hipSuccess;
  const RopeGeom rg{rope_dims, ext_off};
  auto kernel = mode == 1 ? rope_encode_kernel<1> : rope_encode_kernel<2>;
  hipLaunchKernelGGL(kernel, dim3(rope_grid(num_pages)), dim3(kThreads), 0, stream, g, rg,
                     (const uint8_t*)hot, hot_pages, src, (uint8_t*)packed, packed_pages, dst,
                     num_pages, gs[0]);
  return hipGetLastError();
}

hipError_t launch_rope_decode(const Geom& g, int rope_dims, int mode, long long ext_off,
                              const void* packed, int packed_pages, const int32_t* src, void* hot,
                              int hot_pages, const int32_t* dst, int num_pages, const float* gs,
                              hipStream_t stream) {
  if (num_pages == 0 || mode == 0) return hipSuccess;
  const RopeGeom rg{rope_dims, ext_off};
  auto kernel = mode == 1 ? rope_decode_kernel<1> : rope_decode_kernel<2>;
  hipLaunchKernelGGL(kernel, dim3(rope_grid(num_pages)), dim3(kThreads), 0, stream, g, rg,
                     (const uint8_t*)packed, packed_pages, src, (uint8_t*)hot, hot_pages, dst,
                     num_pages, gs[0]);
  return hipGetLastError();
}

}  // namespace kvfp4
