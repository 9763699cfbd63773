// NVFP4 page codec: bf16 hot pages <-> packed NVFP4 pages.
//
// "KV Cache Compression in TensorRT LLM", NVFP4 Cold-Page Compression / How
// It Works: a batch of pages is encoded into one fixed-size block per page
// on the way out and decoded on the way back.  Both kernels are streaming
// maps: one lane owns half a 16-value block, so every wave instruction
// moves one contiguous run (1 KiB of bf16, 256 packed bytes), and each lane
// keeps several half-blocks in flight.
// Each workgroup owns a contiguous run of pages and walks them block by
// block; a page's slot is read once per page (scalar), and all loads and
// stores go through per-page buffer resources, so no per-lane 64-bit
// address arithmetic is needed.
//
// Exactness, encoder.  The block scale is E4M3(amax / (6 gs)) and an
// element code is E2M1(|x| / (sb gs)), each rounded once from the exact
// quotient.  Every workgroup first builds, per tensor, the exact rounding
// thresholds of both steps in fp64 (a threshold mid * 6 gs or mu * sb * gs
// has at most 31 significant bits, so fp64 holds it exactly) and turns each
// into an integer threshold on bf16 magnitude bit patterns by directed
// rounding: for a bf16 magnitude v, "v > M" equals "bits(v) > bits(RD(M))"
// and "v >= M" equals "bits(v) > bits(RU(M)) - 1".  A code is the number of
// thresholds its input exceeds.  Ties go to the even code because
// even-code boundaries use the strict and odd-code boundaries the
// non-strict comparison.
//  - scale: an fp64 estimate of amax / (6 gs), truncated to E4M3, is the
//    exact code or one below it; one threshold comparison decides.
//  - elements: a 3-step binary search over the 7 thresholds, two elements
//    per packed 16-bit instruction; selects are multiply-adds by 0/1.
//
// Exactness, decoder.  For a given tensor scale the result depends only on
// the scale code (128) and the magnitude code (8): every workgroup builds
// that table once, each entry rounded to bf16 once from the exact fp64
// product, stored as 8 low bytes then 8 high bytes per scale code; an
// element is then two byte lookups (v_perm) plus its sign bit.
#include "common.hpp"

namespace kvfp4 {

namespace {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr uint32_t kPad = 0x7FFFu;  // above every finite bf16 magnitude
constexpr int kRsrcFlags = 0x00020000;
constexpr int kNoStore = 0x7FFFFFF0;  // buffer offset past every page: store dropped

__device__ inline u16x2 as_u16x2(uint32_t x) { return __builtin_bit_cast(u16x2, x); }
__device__ inline uint32_t as_u32(u16x2 x) { return __builtin_bit_cast(uint32_t, x); }
__device__ inline uint32_t pk_sub(uint32_t a, uint32_t b) { return as_u32(as_u16x2(a) - as_u16x2(b)); }
__device__ inline uint32_t pk_mad(uint32_t a, uint32_t b, uint32_t c) {
  return as_u32(as_u16x2(a) * as_u16x2(b) + as_u16x2(c));
}
__device__ inline uint32_t pk_shr15(uint32_t a) { return as_u32(as_u16x2(a) >> (u16x2){15, 15}); }
// 1 in each 16-bit half where the magnitude v exceeds threshold t (both < 0x8000)
__device__ inline uint32_t gt_bit(uint32_t t, uint32_t v) { return pk_shr15(pk_sub(t, v)); }

// Pages [p0, p1) of this workgroup.
__device__ inline void page_range(int num_pages, int& p0, int& p1) {
  p0 = (int)((long long)blockIdx.x * num_pages / gridDim.x);
  p1 = (int)((long long)(blockIdx.x + 1) * num_pages / gridDim.x);
}

// This workgroup's contiguous run [u0, u1) of num_units work units.
__device__ inline void unit_range(long long num_units, long long& u0, long long& u1) {
  u0 = (long long)blockIdx.x * num_units / gridDim.x;
  u1 = (long long)(blockIdx.x + 1) * num_units / gridDim.x;
}

__device__ inline int page_slot(const int32_t* slots, int i, int pool_pages) {
  int s = slots ? __builtin_amdgcn_readfirstlane(slots[i]) : i;
  return (s >= 0 && s < pool_pages) ? s : -1;
}

// ---------------------------------------------------------------------------
// Encoder
// ---------------------------------------------------------------------------

struct QuantLds {
  uint16_t e4m3[2][128];  // scale thresholds (126 used)
  // per tensor and scale code, the element thresholds T0..T6 in the form
  // the encoder consumes, each in both 16-bit halves: {T0, T1, T3, T5 - T1},
  // {T4 - T0, T2 - T0, (T6 - T4) - (T2 - T0), 0} (differences mod 2^16)
  u32x4 thr[2][128][2];
  double inv6gs[2];       // 1 / (6 gs) per tensor, for the scale estimate
};

__device__ inline uint32_t dup_half(uint32_t x) { return (x & 0xFFFFu) | (x << 16); }

// Directed rounding of a positive fp64 normal x to a bf16 bit pattern: the
// largest bf16 <= x (up = false) or the smallest bf16 >= x (up = true), with
// +inf / the largest finite value past the range.  For non-negative values
// bf16 bit patterns order like the values, so an exact fp64 threshold M
// becomes an integer threshold t on magnitude bits: v > t <=> value > M is
// t = down(M); value >= M is t = up(M) - 1.  Written without branches (the
// encoders build their tables on every workgroup's path): x = m 2^(e - 52);
// the bf16 step at x is 2^(max(e, -126) - 7), and a shift past m's 53 bits
// leaves 0 with m as the remainder, so capping the shift at 63 changes
// nothing.
__device__ __forceinline__ uint32_t bf16_bits_directed_normal(double x, bool up) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const int e = (int)(b >> 52) - 1023;
  const uint64_t m = (b & ((1ull << 52) - 1)) | (1ull << 52);
  const int eb = e > -126 ? e : -126;
  const int sh = 45 + (eb - e) < 63 ? 45 + (eb - e) : 63;
  const uint64_t k = (m >> sh) + ((up && (m & ((1ull << sh) - 1)) != 0) ? 1u : 0u);
  const long long bits = ((long long)(eb + 126) << 7) + (long long)k;
  const long long cap = up ? 0x7F80 : 0x7F7F;
  return (uint32_t)(bits < cap ? bits : cap);
}
// The encoder's tables for tensors [t0, t0 + tn) (tn <= 2): per scale code
// j, the scale threshold (the E4M3 midpoint between codes j and j + 1, times
// 6 gs, strict for even j) and the seven element thresholds (E2M1 midpoints
// times the code's scale times gs, strict for even k), as integer
// thresholds on bf16 magnitude bits.  Each code's eight thresholds are
// computed by two threads, four each and without branches; then each code's
// seven element thresholds are turned into its two rows.  Fixed trip counts
// (a thread-strided loop here made the compiler keep the buffer descriptors
// in VGPRs); forced inline (as a call it spilled through scratch).  Ends
// with a barrier.
struct QuantRaw {
  uint16_t t[2][128][8];  // element thresholds T0..T6 per tensor and code
};
__device__ __forceinline__ void build_quant_tables_items(QuantLds& s, QuantRaw& r, int t0, int tn,
                                                         float gs0, float gs1) {
  static_assert(kThreads == 256, "two threads per scale code of two tensors");
  if (threadIdx.x < 2) s.inv6gs[threadIdx.x] = 1.0 / (6.0 * (double)(threadIdx.x ? gs1 : gs0));
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = (int)threadIdx.x + q * kThreads;
    if (i < tn * 256) {
      const int t = t0 + (i >> 8), j = (i >> 1) & 127, h = i & 1;
      const double gs = t == 0 ? (double)gs0 : (double)gs1;
      const double sb = (double)e4m3_to_float(j);
      // the E4M3 midpoint between codes j and j + 1, times 6
      const double mid6 = 3.0 * (sb + (double)e4m3_to_float(j + 1 < 127 ? j + 1 : 126));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int k = 4 * h + c;  // k < 7: E2M1 midpoint mu_k times sb; k == 7: mid6
        const double mu = h == 0 ? 0.25 + 0.5 * c : (c == 0 ? 2.5 : (c == 1 ? 3.5 : 5.0));
        const double M = (k == 7 ? mid6 : mu * sb) * gs;
        const bool strict = k == 7 ? (j & 1) == 0 : (k & 1) == 0;
        const bool valid = k == 7 ? j < 126 : (j >= 1 && j <= 126);
        const uint32_t d = bf16_bits_directed_normal(valid ? M : 1.0, !strict);
        const uint32_t th = valid ? (strict ? d : d - 1u) : kPad;
        uint16_t* at = k == 7 ? &s.e4m3[t][j] : &r.t[t][j][k];
        *at = (uint16_t)th;
      }
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < tn * 128) {
    const int t = t0 + ((int)threadIdx.x >> 7), j = (int)threadIdx.x & 127;
    uint32_t T[7];
#pragma unroll
    for (int k = 0; k < 7; ++k) T[k] = r.t[t][j][k];
    const uint32_t d51 = (T[5] - T[1]) & 0xFFFFu, d40 = (T[4] - T[0]) & 0xFFFFu;
    const uint32_t d20 = (T[2] - T[0]) & 0xFFFFu;
    const uint32_t dd = (((T[6] - T[4]) & 0xFFFFu) - d20) & 0xFFFFu;
    s.thr[t][j][0] = (u32x4){dup_half(T[0]), dup_half(T[1]), dup_half(T[3]), dup_half(d51)};
    s.thr[t][j][1] = (u32x4){dup_half(d40), dup_half(d20), dup_half(dd), 0u};
  }
  __syncthreads();
}

// E4M3 code of amax / (6 gs): the truncation of an fp64 estimate (error
// far below E4M3's spacing, and no overflow for any valid gs) is the exact
// code or one below it; the exact threshold decides.  Both the normal and
// the subnormal candidate are computed and one is selected (no branch).
__device__ inline uint32_t scale_code(const uint16_t* th, uint32_t amax_bits, double inv6gs) {
  const double q = (double)__uint_as_float(amax_bits << 16) * inv6gs;
  const uint32_t hi = (uint32_t)((uint64_t)__double_as_longlong(q) >> 32);
  const int e = (int)(hi >> 20) - 1016;  // E4M3 exponent field for normal codes
  const int cn = (e << 3) | (int)((hi >> 17) & 7);
  const uint32_t c_norm = (uint32_t)(cn > 126 ? 126 : cn);
  const uint32_t c_sub = (uint32_t)fmin(q * 512.0, 7.0);  // subnormal codes: m * 2^-9
  const uint32_t cand = e >= 1 ? c_norm : c_sub;
  return cand + (amax_bits > th[cand] ? 1u : 0u);
}

// Two elements (one dword of bf16) -> two nibbles in bits 3:0 and 19:16.
// T[k]: threshold k in both halves; D51 = T5 - T1, D40 = T4 - T0,
// D20 = T2 - T0, DD = (T6 - T4) - (T2 - T0), all per half.
struct Thr {
  uint32_t T0, T1, T3, D51, D40, D20, DD;
};

// The sequence is written out instruction by instruction so that the
// compiler keeps the 0/1 multiply-add selects (v_pk_mad_u16) instead of
// expanding them into per-half masks.  k15 holds 15 in both halves, k8 the
// sign-bit mask 0x00080008.
__device__ inline uint32_t encode_pair(uint32_t raw, const Thr& t, uint32_t k15, uint32_t k8) {
  const uint32_t v = raw & 0x7FFF7FFFu;
  uint32_t code, b1, b2, d, u, w;
  asm volatile(
      "v_pk_sub_u16 %[d], %[T3], %[v]\n\t"
      "v_pk_lshrrev_b16 %[b1], %[k15], %[d]\n\t"           // b1 = v > T3
      "v_pk_mad_u16 %[u], %[b1], %[D51], %[T1]\n\t"        // T5 or T1
      "v_pk_sub_u16 %[d], %[u], %[v]\n\t"
      "v_pk_lshrrev_b16 %[b2], %[k15], %[d]\n\t"           // b2
      "v_pk_mad_u16 %[u], %[b1], %[D40], %[T0]\n\t"        // T4 or T0
      "v_pk_mad_u16 %[w], %[b1], %[DD], %[D20]\n\t"        // T6-T4 or T2-T0
      "v_pk_mad_u16 %[u], %[b2], %[w], %[u]\n\t"           // T6, T4, T2 or T0
      "v_pk_sub_u16 %[d], %[u], %[v]\n\t"
      "v_pk_lshrrev_b16 %[d], %[k15], %[d]\n\t"            // b3
      "v_lshl_or_b32 %[d], %[b2], 1, %[d]\n\t"
      "v_lshl_or_b32 %[code], %[b1], 2, %[d]\n\t"
      "v_lshrrev_b32 %[w], 12, %[raw]\n\t"
      "v_and_or_b32 %[code], %[w], %[k8], %[code]"         // sign bits
      : [code] "=&v"(code), [b1] "=&v"(b1), [b2] "=&v"(b2), [d] "=&v"(d), [u] "=&v"(u),
        [w] "=&v"(w)
      : [v] "v"(v), [raw] "v"(raw), [T0] "v"(t.T0), [T1] "v"(t.T1), [T3] "v"(t.T3),
        [D51] "v"(t.D51), [D40] "v"(t.D40), [D20] "v"(t.D20), [DD] "v"(t.DD), [k15] "v"(k15),
        [k8] "v"(k8));
  return code;
}

// Cache-policy bits of the codec's streaming loads and stores.  Each input
// line is read by one load instruction and never again, so those loads are
// non-temporal (nt).  The page decoder's stores (bf16 pages, 4 bytes out
// for each byte in) are non-temporal too: with the page list in slot order
// and calls back to back it took 234.5 against 249.9 us per call with them
// (a single call after a cache flush: 241 against 221 us, the cached stores
// then draining after the kernel).  The encoder's data words are stored
// non-temporal (back to back: Llama-3-8B pages 256.5 against 262.2 us, MLA
// pages 312.6 against 327.7 us) and its scale bytes default: byte stores,
// four to a line from different waves, made non-temporal cost 28 us on MLA
// pages.
#ifndef KVFP4_CODEC_LOAD_AUX
#define KVFP4_CODEC_LOAD_AUX 2
#endif
// The decoder's scale bytes are the exception: the four waves of a
// workgroup each read a quarter of the same 128-byte line, so the line is
// kept in cache for the later ones.
#ifndef KVFP4_CODEC_SCALE_LOAD_AUX
#define KVFP4_CODEC_SCALE_LOAD_AUX 0
#endif
#ifndef KVFP4_CODEC_STORE_AUX
#define KVFP4_CODEC_STORE_AUX 0
#endif
#ifndef KVFP4_DEQUANT_STORE_AUX
#define KVFP4_DEQUANT_STORE_AUX 2
#endif
#ifndef KVFP4_QUANT_DATA_STORE_AUX
#define KVFP4_QUANT_DATA_STORE_AUX 2
#endif
// One lane's half block (8 bf16 values in `a`) of tensor t -> the block's
// E4M3 scale code (identical in both lanes of the pair) and the 4 data bytes
// of its 8 nibbles.  The other half of the block must sit in lane ^ 1.
__device__ inline void encode_half(const QuantLds& s, const u32x4& a, int t, uint32_t& sc,
                                   uint32_t& word) {
  const uint32_t k15 = 0x000F000Fu, k8 = 0x00080008u;
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
  u16x2 mx = __builtin_elementwise_max(as_u16x2(w[0] & 0x7FFF7FFFu), as_u16x2(w[1] & 0x7FFF7FFFu));
  mx = __builtin_elementwise_max(mx, as_u16x2(w[2] & 0x7FFF7FFFu));
  mx = __builtin_elementwise_max(mx, as_u16x2(w[3] & 0x7FFF7FFFu));
  uint32_t amax = mx.x > mx.y ? mx.x : mx.y;
  // the partner lane holds the other half of the block
  const uint32_t other = (uint32_t)__builtin_amdgcn_mov_dpp((int)amax, 0xB1, 0xF, 0xF, true);
  amax = amax > other ? amax : other;
  sc = scale_code(s.e4m3[t], amax, s.inv6gs[t]);
  const u32x4 ra = s.thr[t][sc][0], rb = s.thr[t][sc][1];
  Thr th;
  th.T0 = ra.x;
  th.T1 = ra.y;
  th.T3 = ra.z;
  th.D51 = ra.w;
  th.D40 = rb.x;
  th.D20 = rb.y;
  th.DD = rb.z;
  // pairs (0,1),(2,3) -> nibbles e0..e3; pairs (4,5),(6,7) -> e4..e7
  const uint32_t n0 = encode_pair(w[0], th, k15, k8) | (encode_pair(w[1], th, k15, k8) << 8);
  const uint32_t n1 = encode_pair(w[2], th, k15, k8) | (encode_pair(w[3], th, k15, k8) << 8);
  const uint32_t h0w = n0 | (n0 >> 12), h1w = n1 | (n1 >> 12);
  word = __builtin_amdgcn_perm(h1w, h0w, 0x05040100u);
}

#ifndef KVFP4_QUANT_UNROLL
#define KVFP4_QUANT_UNROLL 8
#endif
#ifndef KVFP4_DEQUANT_UNROLL
#define KVFP4_DEQUANT_UNROLL 16
#endif
#ifndef KVFP4_CODEC_GRID
#define KVFP4_CODEC_GRID 65536
#endif
constexpr int kQuantUnroll = KVFP4_QUANT_UNROLL;    // half-blocks in flight per lane
constexpr int kDequantUnroll = KVFP4_DEQUANT_UNROLL;

// One round of a page: the kThreads x kQuantUnroll half-blocks from h0.  A
// lane owns half a block (8 values): 16 contiguous input bytes, 4 output
// bytes; the two halves of a block sit in adjacent lanes.
template <typename Rsrc>
__device__ inline void encode_round(const QuantLds& s, Rsrc rin, Rsrc rout, int h0, int hpp,
                                    int bpt, int data_bytes) {
  u32x4 a[kQuantUnroll];
#pragma unroll
  for (int u = 0; u < kQuantUnroll; ++u) {
    // out-of-range half-blocks read zero (buffer bounds) and store nothing
    a[u] = __builtin_amdgcn_raw_buffer_load_b128(rin, (h0 + u * kThreads + (int)threadIdx.x) * 16, 0,
                                                 KVFP4_CODEC_LOAD_AUX);
  }
#pragma unroll
  for (int u = 0; u < kQuantUnroll; ++u) {
    const int hb = h0 + u * kThreads + (int)threadIdx.x;
    const int blk = hb >> 1;
    const int t = blk >= bpt ? 1 : 0;
    uint32_t sc, word;
    encode_half(s, a[u], t, sc, word);
    // half-blocks past the page and the odd lane's copy of the scale byte
    // are given an offset past the buffer: the store is dropped
    const bool in = hb < hpp;
    __builtin_amdgcn_raw_buffer_store_b32(word, rout, in ? hb * 4 : kNoStore, 0,
                                          KVFP4_QUANT_DATA_STORE_AUX);
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, rout,
                                         in && (hb & 1) == 0 ? data_bytes + blk : kNoStore, 0,
                                         KVFP4_CODEC_STORE_AUX);
  }
}

constexpr int kQuantRound = kThreads * kQuantUnroll;  // half-blocks of a round

// Workgroups take runs of whole pages (see grid_for).
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    Geom g, const uint8_t* __restrict__ hot, int hot_pages, const int32_t* __restrict__ src,
    uint8_t* __restrict__ packed, int packed_pages, const int32_t* __restrict__ dst,
    int num_pages, float gs0, float gs1) {
  __shared__ QuantLds s;
  __shared__ QuantRaw raw;
  build_quant_tables_items(s, raw, 0, g.nt, gs0, gs1);
  const int hpp = (int)(g.elems() / 8);  // half-blocks per page
  const int bpt = g.blocks_per_tensor();
  const int data_bytes = (int)g.data_bytes();
  int p0, p1;
  page_range(num_pages, p0, p1);
  for (int p = p0; p < p1; ++p) {
    const int ss = page_slot(src, p, hot_pages);
    const int ds = page_slot(dst, p, packed_pages);
    if (ss < 0 || ds < 0) continue;
    const uint8_t* in = hot + (long long)ss * g.hot_bytes();
    uint8_t* out = packed + (long long)ds * g.page_stride();
    auto rin = __builtin_amdgcn_make_buffer_rsrc((void*)in, (short)0, (int)g.hot_bytes(), kRsrcFlags);
    auto rout = __builtin_amdgcn_make_buffer_rsrc((void*)out, (short)0, (int)g.packed_bytes(), kRsrcFlags);
    for (int h0 = 0; h0 < hpp; h0 += kQuantRound) encode_round(s, rin, rout, h0, hpp, bpt, data_bytes);
  }
}

// Pages of whole rounds: the work unit is one round of one page, units in
// list order (unit u: page u / rounds, round u % rounds), dealt to the grid
// in grid-stride order.  The workgroups running at once then cover a few
// hundred consecutive pages' rounds instead of a few thousand pages each
// read from its start, and with the list in slot order they read one
// contiguous stretch of the pool.
__global__ __launch_bounds__(kThreads) void quantize_rounds_kernel(
    Geom g, const uint8_t* __restrict__ hot, int hot_pages, const int32_t* __restrict__ src,
    uint8_t* __restrict__ packed, int packed_pages, const int32_t* __restrict__ dst,
    int num_pages, float gs0, float gs1) {
  __shared__ QuantLds s;
  __shared__ QuantRaw raw;
  const int hpp = (int)(g.elems() / 8);
  const int bpt = g.blocks_per_tensor();
  const int data_bytes = (int)g.data_bytes();
  const int rounds = hpp / kQuantRound;
  const int units = num_pages * rounds;
  {
    // the launcher checks hpp % kQuantRound == 0 and that units fit an int;
    // a workgroup with a single unit builds the tables of its round's
    // tensors only (one, when a tensor is whole rounds).  Back to back on
    // Llama-3-8B pages: 242.8 against 255.6 us with every tensor's tables
    // built one code per thread; a single flushed call 234.6 against 249.2.
    int t0 = 0, tn = g.nt;
    if (units <= (int)gridDim.x) {
      const int b0 = (((int)blockIdx.x % rounds) * kQuantRound) >> 1;  // the round's blocks
      const int b1 = b0 + kQuantRound / 2 - 1;
      t0 = b0 >= bpt ? 1 : 0;
      tn = (b1 >= bpt ? 1 : 0) - t0 + 1;
    }
    build_quant_tables_items(s, raw, t0, tn, gs0, gs1);
  }
  for (int un = blockIdx.x; un < units; un += gridDim.x) {
    const int p = un / rounds, h0 = (un - p * rounds) * kQuantRound;
    const int ss = page_slot(src, p, hot_pages);
    const int ds = page_slot(dst, p, packed_pages);
    if (ss < 0 || ds < 0) continue;
    const uint8_t* in = hot + (long long)ss * g.hot_bytes();
    uint8_t* out = packed + (long long)ds * g.page_stride();
    auto rin = __builtin_amdgcn_make_buffer_rsrc((void*)in, (short)0, (int)g.hot_bytes(), kRsrcFlags);
    auto rout = __builtin_amdgcn_make_buffer_rsrc((void*)out, (short)0, (int)g.packed_bytes(), kRsrcFlags);
    encode_round(s, rin, rout, h0, hpp, bpt, data_bytes);
  }
}

// Append: token i's rows (all tensors and heads, [n_t][H][D]) go to row
// token_rows[i] of packed slot token_slots[i].  A lane owns half a block as
// above; consecutive lanes walk the tokens' rows, so the input is read
// contiguously.  Only the token's own data and scale bytes are written.
// kFp8: the input is OCP E4M3FN bytes instead of bf16.  Every finite E4M3
// value is a bf16 value, so the codes are widened to bf16 exactly (the
// gfx950 convert with scale 1) and encoded like bf16 input.
// Large appends (prefill) keep 4 half-blocks in flight per lane; a decode
// step's few tokens spread one half-block a lane over more workgroups,
// which measured faster (latency, not bandwidth, bounds them).
constexpr int kAppendUnroll = 4;
constexpr long long kAppendSmall = 256LL * kThreads;  // half-blocks: one per lane below this
// Each workgroup builds its own threshold tables (about 2.5k fp64
// roundings): with 1024 workgroups that work hides behind the first loads,
// with 4096 it measured 5.5 us of extra time.
#ifndef KVFP4_APPEND_GRID
#define KVFP4_APPEND_GRID 1024
#endif

struct AppendIn {
  u32x4 a;        // 8 values as bf16 pairs
  int slot, row;  // destination; slot -1 for lanes past the end
  uint32_t t, k;  // tensor, half-block within the tensor row
};

template <bool kFp8>
__device__ inline void append_load(AppendIn& in, uint32_t gi, uint32_t total, uint32_t hpt,
                                   uint32_t hd8, const uint8_t* rows, const int32_t* slots,
                                   const int32_t* page_rows) {
  const bool live = gi < total;
  const uint32_t tok = live ? gi / hpt : 0u;
  const uint32_t j = gi - tok * hpt;
  in.t = j >= hd8 ? 1u : 0u;
  in.k = j - in.t * hd8;
  in.slot = live ? slots[tok] : -1;
  in.row = live ? page_rows[tok] : -1;
  if constexpr (kFp8) {
    u32x2 c = {0u, 0u};
    if (live) c = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(rows) + gi);
    in.a.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, false));
    in.a.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, true));
    in.a.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, false));
    in.a.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, true));
  } else {
    in.a = (u32x4){0u, 0u, 0u, 0u};
    if (live) in.a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rows) + gi);
  }
}

template <bool kFp8, int kUnroll>
__global__ __launch_bounds__(kThreads) void append_kernel(
    Geom g, const uint8_t* __restrict__ rows, int num_tokens, const int32_t* __restrict__ slots,
    const int32_t* __restrict__ page_rows, uint8_t* __restrict__ packed, int packed_pages,
    float gs0, float gs1) {
  __shared__ QuantLds s;
  __shared__ QuantRaw raw;
  // The C ABI bounds num_tokens * half-blocks per token below 2^31.
  const uint32_t hd8 = (uint32_t)(g.H * g.D / 8);     // half-blocks per tensor row (even)
  const uint32_t hpt = (uint32_t)g.nt * hd8;           // half-blocks per token
  const uint32_t total = hpt * (uint32_t)num_tokens;
  const int data_bytes = (int)g.data_bytes();
  const int page_bytes = (int)g.packed_bytes();
  constexpr uint32_t chunk = kThreads * kUnroll;
  const uint32_t stride = gridDim.x * chunk;
  const uint32_t first = blockIdx.x * chunk;
  // the first inputs are requested before the tables are built, so that
  // their latency hides behind the table arithmetic
  AppendIn in[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u)
    append_load<kFp8>(in[u], first + u * kThreads + threadIdx.x, total, hpt, hd8, rows, slots,
                      page_rows);
  build_quant_tables_items(s, raw, 0, g.nt, gs0, gs1);
  // the loop bound is uniform over the workgroup: every lane runs the body,
  // since the DPP exchange needs both halves of a block
  for (uint32_t base = first; base < total; base += stride) {
    if (base != first) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        append_load<kFp8>(in[u], base + u * kThreads + threadIdx.x, total, hpt, hd8, rows, slots,
                          page_rows);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      uint32_t sc, word;
      encode_half(s, in[u].a, (int)in[u].t, sc, word);
      // lanes past the end, bad slots and bad rows store nothing
      const bool ok = in[u].slot >= 0 && in[u].slot < packed_pages && in[u].row >= 0 &&
                      in[u].row < g.T;
      if (!ok) continue;
      uint8_t* page = packed + (long long)in[u].slot * page_bytes;
      auto rout = __builtin_amdgcn_make_buffer_rsrc((void*)page, (short)0, page_bytes, kRsrcFlags);
      const int hb = (int)((in[u].t * (uint32_t)g.T + (uint32_t)in[u].row) * hd8 + in[u].k);
      __builtin_amdgcn_raw_buffer_store_b32(word, rout, hb * 4, 0, KVFP4_CODEC_STORE_AUX);
      if ((in[u].k & 1u) == 0u)
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sc, rout, data_bytes + (hb >> 1), 0,
                                             KVFP4_CODEC_STORE_AUX);
    }
  }
}

// ---------------------------------------------------------------------------
// Decoder
// ---------------------------------------------------------------------------

struct DequantLds {
  // per tensor and scale code: 8 low bytes then 8 high bytes of the bf16
  // results for magnitude codes 0..7
  uint32_t row[2][128][4];
};

__device__ inline void build_dequant_table(DequantLds& s, int nt, float gs0, float gs1) {
  uint8_t* bytes = reinterpret_cast<uint8_t*>(&s.row[0][0][0]);
  for (int i = threadIdx.x; i < nt * 128 * 8; i += blockDim.x) {
    const int t = i >> 10, j = (i >> 3) & 127, c = i & 7;
    const double gs = t == 0 ? (double)gs0 : (double)gs1;
    // exact: <= 2 + 4 + 24 significant bits
    const double v = (double)e2m1_mag_to_float(c) * (double)e4m3_to_float(j) * gs;
    uint32_t b16 = (j == 127) ? 0x7FC0u : bf16_rne_from_f64(v);
    uint8_t* r = bytes + ((t * 128 + j) * 16);
    r[c] = (uint8_t)(b16 & 0xFF);
    r[8 + c] = (uint8_t)(b16 >> 8);
  }
}

// Four elements (selector bytes: bit 3 sign, bits 2:0 magnitude code) ->
// bf16 pairs (e0, e1), (e2, e3).
__device__ inline void lookup4(uint32_t sel, const u32x4& row, uint32_t& o0, uint32_t& o1) {
  const uint32_t m = sel & 0x07070707u;
  const uint32_t lo = __builtin_amdgcn_perm(row.y, row.x, m);
  uint32_t hi = __builtin_amdgcn_perm(row.w, row.z, m);
  hi |= (sel & 0x08080808u) << 4;  // sign into bit 7 of the high byte
  o0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  o1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// Eight nibbles of one data word -> four bf16 pairs in element order.
__device__ inline void decode8(uint32_t w, const u32x4& row, uint32_t sign_flip, uint32_t* o) {
  const uint32_t x = w & 0x0F0F0F0Fu;         // elements 0 2 4 6
  const uint32_t y = (w >> 4) & 0x0F0F0F0Fu;  // elements 1 3 5 7
  const uint32_t s0 = __builtin_amdgcn_perm(y, x, 0x05010400u) ^ sign_flip;  // 0 1 2 3
  const uint32_t s1 = __builtin_amdgcn_perm(y, x, 0x07030602u) ^ sign_flip;  // 4 5 6 7
  lookup4(s0, row, o[0], o[1]);
  lookup4(s1, row, o[2], o[3]);
}

__global__ __launch_bounds__(kThreads) void dequantize_kernel(
    Geom g, const uint8_t* __restrict__ packed, int packed_pages, const int32_t* __restrict__ src,
    uint8_t* __restrict__ hot, int hot_pages, const int32_t* __restrict__ dst, int num_pages,
    int parts, float gs0, float gs1) {
  __shared__ DequantLds s;
  build_dequant_table(s, g.nt, gs0, gs1);
  __syncthreads();
  // A lane owns half a block: 4 data bytes + the block's scale byte in,
  // 16 contiguous output bytes.  A work unit is one of `parts` equal runs
  // of a page's half-blocks (the whole page when parts is 1).
  const int hpp = (int)(g.elems() / 8);
  const int bpt = g.blocks_per_tensor();
  const int data_bytes = (int)g.data_bytes();
  long long u0, u1;
  unit_range((long long)num_pages * parts, u0, u1);
  for (long long un = u0; un < u1; ++un) {
    const int p = (int)(un / parts), part = (int)(un - (long long)p * parts);
    const int hlo = (int)((long long)part * hpp / parts);
    const int hhi = (int)((long long)(part + 1) * hpp / parts);
    const int ss = page_slot(src, p, packed_pages);
    const int ds = page_slot(dst, p, hot_pages);
    if (ss < 0 || ds < 0) continue;
    const uint8_t* in = packed + (long long)ss * g.page_stride();
    uint8_t* out = hot + (long long)ds * g.hot_bytes();
    // the unit's data words, and the scale bytes of its blocks (a block cut
    // by the unit boundary is read by both units): half-blocks past the
    // unit fall outside these ranges and read zero without touching memory,
    // so the data loads need no per-lane condition.  The scale loads keep
    // theirs: without it all 32 loads of a round issue at once and the
    // kernel needs 78 VGPRs (6 waves a SIMD instead of 8), measured slower.
    const int slo = hlo >> 1, shi = (hhi + 1) >> 1;
    auto rdat = __builtin_amdgcn_make_buffer_rsrc((void*)(in + 4LL * hlo), (short)0, 4 * (hhi - hlo),
                                                  kRsrcFlags);
    auto rsc = __builtin_amdgcn_make_buffer_rsrc((void*)(in + data_bytes + slo), (short)0, shi - slo,
                                                 kRsrcFlags);
    auto rout = __builtin_amdgcn_make_buffer_rsrc((void*)out, (short)0, (int)g.hot_bytes(), kRsrcFlags);
    for (int h0 = hlo; h0 < hhi; h0 += kThreads * kDequantUnroll) {
      uint32_t dw[kDequantUnroll], code[kDequantUnroll];
#pragma unroll
      for (int u = 0; u < kDequantUnroll; ++u) {
        const int hb = h0 + u * kThreads + (int)threadIdx.x;
        dw[u] = __builtin_amdgcn_raw_buffer_load_b32(rdat, (hb - hlo) * 4, 0, KVFP4_CODEC_LOAD_AUX);
        code[u] = hb < hhi ? __builtin_amdgcn_raw_buffer_load_b8(rsc, (hb >> 1) - slo, 0,
                                                                 KVFP4_CODEC_SCALE_LOAD_AUX)
                           : 0u;
      }
#pragma unroll
      for (int u = 0; u < kDequantUnroll; ++u) {
        const int hb = h0 + u * kThreads + (int)threadIdx.x;
        const int t = (hb >> 1) >= bpt ? 1 : 0;
        const u32x4 row = *reinterpret_cast<const u32x4*>(s.row[t][code[u] & 127]);
        const uint32_t flip = (code[u] & 0x80u) ? 0x08080808u : 0u;  // negative E4M3 scale
        uint32_t o[4];
        decode8(dw[u], row, flip, o);
        if (hb < hhi)
          __builtin_amdgcn_raw_buffer_store_b128((u32x4){o[0], o[1], o[2], o[3]}, rout, hb * 16, 0,
                                                 KVFP4_DEQUANT_STORE_AUX);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Gather: rows of packed pages -> a contiguous bf16 or FP8 workspace
// ---------------------------------------------------------------------------

// E4M3FN code of an exact non-negative value: nearest finite value, ties to
// the even code, saturating at 448.  Subnormal codes are m * 2^-9 (m = 0..8,
// and m = 8 is the first normal code); a normal value 2^e (1 + m/8) has code
// (e + 7) * 8 + m, so a mantissa rounded up to 8 carries into the exponent.
// Every step is exact in fp64 and rint rounds ties to even.
__device__ inline uint32_t e4m3_code_rne(double v) {
  if (!(v > 0.0)) return 0u;
  if (v >= 448.0) return 126u;
  if (v < 0x1p-6) return (uint32_t)rint(v * 512.0);
  int E;
  (void)frexp(v, &E);  // v in [2^(E-1), 2^E)
  const int e = E - 1;
  const uint32_t m = (uint32_t)rint(ldexp(v, -e) * 8.0) - 8u;  // 0..8
  const uint32_t code = (uint32_t)((e + 7) << 3) + m;
  return code > 126u ? 126u : code;
}

struct GatherFp8Lds {
  // per tensor and scale code: the E4M3 codes of magnitude codes 0..7
  uint32_t row[2][128][2];
};

__device__ inline void build_fp8_table(GatherFp8Lds& s, int nt, float gs0, float gs1) {
  uint8_t* bytes = reinterpret_cast<uint8_t*>(&s.row[0][0][0]);
  for (int i = threadIdx.x; i < nt * 128 * 8; i += blockDim.x) {
    const int t = i >> 10, j = (i >> 3) & 127, c = i & 7;
    const double gs = t == 0 ? (double)gs0 : (double)gs1;
    const double v = (double)e2m1_mag_to_float(c) * (double)e4m3_to_float(j) * gs;  // exact
    bytes[(t * 128 + j) * 8 + c] = (uint8_t)(j == 127 ? 0x7Fu : e4m3_code_rne(v));
  }
}

// Eight nibbles of one data word -> eight E4M3 bytes in element order.
__device__ inline void decode8_fp8(uint32_t w, const u32x2& row, uint32_t sign_flip,
                                   uint32_t& o0, uint32_t& o1) {
  const uint32_t x = w & 0x0F0F0F0Fu;
  const uint32_t y = (w >> 4) & 0x0F0F0F0Fu;
  const uint32_t s0 = __builtin_amdgcn_perm(y, x, 0x05010400u) ^ sign_flip;
  const uint32_t s1 = __builtin_amdgcn_perm(y, x, 0x07030602u) ^ sign_flip;
  o0 = __builtin_amdgcn_perm(row.y, row.x, s0 & 0x07070707u) | ((s0 & 0x08080808u) << 4);
  o1 = __builtin_amdgcn_perm(row.y, row.x, s1 & 0x07070707u) | ((s1 & 0x08080808u) << 4);
}

union GatherLds {
  DequantLds b;
  GatherFp8Lds f;
};

// A lane owns half a block of an output row: it reads the 4 data bytes and
// the scale byte from the token's page and writes 16 bytes (bf16) or 8
// bytes (FP8) of the output, which is read-contiguous across lanes.  The
// slot and row loads come first, then the page loads that depend on them,
// then the lookup tables are built while those are in flight.
template <bool kFp8, int kUnroll>
__global__ __launch_bounds__(kThreads) void gather_kernel(
    Geom g, const uint8_t* __restrict__ packed, int packed_pages, const int32_t* __restrict__ slots,
    const int32_t* __restrict__ page_rows, int num_tokens, uint8_t* __restrict__ out, float gs0,
    float gs1) {
  __shared__ GatherLds s;
  // The C ABI bounds num_tokens * half-blocks per token below 2^31.
  const uint32_t hd8 = (uint32_t)(g.H * g.D / 8);
  const uint32_t hpt = (uint32_t)g.nt * hd8;
  const uint32_t total = hpt * (uint32_t)num_tokens;
  const int data_bytes = (int)g.data_bytes();
  const int page_bytes = (int)g.packed_bytes();
  constexpr uint32_t chunk = kThreads * kUnroll;
  const uint32_t stride = gridDim.x * chunk;
  const uint32_t first = blockIdx.x * chunk;
  bool tables = false;
  for (uint32_t base = first; base < total; base += stride) {
    uint32_t dw[kUnroll], code[kUnroll];
    bool ok[kUnroll];
    int slot[kUnroll], row[kUnroll];
    uint32_t t[kUnroll], k[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t gi = base + u * kThreads + threadIdx.x;
      const bool live = gi < total;
      const uint32_t tok = live ? gi / hpt : 0u;
      const uint32_t j = gi - tok * hpt;
      t[u] = j >= hd8 ? 1u : 0u;
      k[u] = j - t[u] * hd8;
      slot[u] = live ? slots[tok] : -1;
      row[u] = live ? page_rows[tok] : -1;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      ok[u] = slot[u] >= 0 && slot[u] < packed_pages && row[u] >= 0 && row[u] < g.T;
      const uint8_t* page = packed + (long long)(ok[u] ? slot[u] : 0) * page_bytes;
      auto rin = __builtin_amdgcn_make_buffer_rsrc((void*)page, (short)0, ok[u] ? page_bytes : 0,
                                                   kRsrcFlags);
      const int hb = (int)((t[u] * (uint32_t)g.T + (uint32_t)(ok[u] ? row[u] : 0)) * hd8 + k[u]);
      dw[u] = __builtin_amdgcn_raw_buffer_load_b32(rin, hb * 4, 0, 0);
      code[u] = __builtin_amdgcn_raw_buffer_load_b8(rin, data_bytes + (hb >> 1), 0, 0);
    }
    if (!tables) {
      if constexpr (kFp8)
        build_fp8_table(s.f, g.nt, gs0, gs1);
      else
        build_dequant_table(s.b, g.nt, gs0, gs1);
      __syncthreads();
      tables = true;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t gi = base + u * kThreads + threadIdx.x;
      if (gi >= total) continue;
      const uint32_t flip = (code[u] & 0x80u) ? 0x08080808u : 0u;  // negative E4M3 scale
      if constexpr (kFp8) {
        const u32x2 r8 = *reinterpret_cast<const u32x2*>(s.f.row[t[u]][code[u] & 127]);
        uint32_t o0, o1;
        decode8_fp8(dw[u], r8, flip, o0, o1);
        if (!ok[u]) o0 = o1 = 0u;  // a bad slot or row gives a zero row
        *reinterpret_cast<u32x2*>(out + (size_t)gi * 8) = (u32x2){o0, o1};
      } else {
        const u32x4 r16 = *reinterpret_cast<const u32x4*>(s.b.row[t[u]][code[u] & 127]);
        uint32_t o[4];
        decode8(dw[u], r16, flip, o);
        if (!ok[u]) o[0] = o[1] = o[2] = o[3] = 0u;
        *reinterpret_cast<u32x4*>(out + (size_t)gi * 16) = (u32x4){o[0], o[1], o[2], o[3]};
      }
    }
  }
}

// Small calls: at least one workgroup per page (or work unit) up to one per
// CU.  Grouping a call's few small pages into one workgroup runs them one
// after another: 16 pages of 16 tokens (8 KiB of bf16 each) took 44 us to
// encode in a single workgroup.
constexpr long long kFillGrid = 256;
long long fill_grid(long long grid, long long units) {
  const long long fill = units < kFillGrid ? units : kFillGrid;
  return grid < fill ? fill : grid;
}

int grid_for(const Geom& g, int num_pages, long long target_bytes) {
  // Encoder: a workgroup takes at most ppw whole pages, ppw = the pages in
  // about target_bytes of bf16: fewer workgroups than that would leave some
  // with one page more while the rest wait for them (4800 Llama-3-8B-shaped
  // pages over 4096 workgroups took 23% longer than over 4800), more would
  // repeat each workgroup's table build over little data.  Measured: about
  // 320 KiB (MLA pages one a workgroup encoded 6% slower than four; two or
  // four workgroups per Llama-3-8B-shaped page were no faster).  Past the
  // cap the runs grow, still differing by at most one page.
  long long ppw = target_bytes / g.hot_bytes();
  if (ppw < 1) ppw = 1;
  long long grid = ((long long)num_pages + ppw - 1) / ppw;
  grid = fill_grid(grid, num_pages);
  const long long cap = KVFP4_CODEC_GRID;
  return (int)(grid < cap ? grid : cap);
}

}  // namespace

hipError_t launch_quantize(const Geom& g, const void* hot, int hot_pages, const int32_t* src,
                           void* packed, int packed_pages, const int32_t* dst, int num_pages,
                           const float* gs, hipStream_t stream) {
  if (num_pages == 0) return hipSuccess;
  float gs1 = g.nt > 1 ? gs[1] : gs[0];
  const long long hpp = g.elems() / 8;
  if (hpp % kQuantRound == 0 && (long long)num_pages * (hpp / kQuantRound) <= INT32_MAX) {
    // Pages of whole rounds: one round per workgroup.  Measured on 4096
    // Llama-3-8B-shaped pages taken in slot order, steady state: 253.7 us
    // against 285.2 us with a page per workgroup (isolated calls: 249.7
    // against 249.1 us; two rounds a workgroup: 259 / 234 us).  MLA pages
    // (2.25 rounds) keep whole pages: partial rounds idle lanes and the
    // tables are built for less work (332.5 against 329.3 us steady).
    const long long units = (long long)num_pages * (hpp / kQuantRound);
    const long long grid = units < KVFP4_CODEC_GRID ? units : KVFP4_CODEC_GRID;
    hipLaunchKernelGGL(quantize_rounds_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, g,
                       (const uint8_t*)hot, hot_pages, src, (uint8_t*)packed, packed_pages, dst,
                       num_pages, gs[0], gs1);
  } else {
    hipLaunchKernelGGL(quantize_kernel, dim3(grid_for(g, num_pages, 320LL << 10)), dim3(kThreads),
                       0, stream, g, (const uint8_t*)hot, hot_pages, src, (uint8_t*)packed,
                       packed_pages, dst, num_pages, gs[0], gs1);
  }
  return hipGetLastError();
}

hipError_t launch_append(const Geom& g, const void* rows, bool fp8, int num_tokens,
                         const int32_t* slots, const int32_t* page_rows, void* packed,
                         int packed_pages, const float* gs, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const float gs1 = g.nt > 1 ? gs[1] : gs[0];
  const long long hb = (long long)g.nt * g.H * g.D / 8 * num_tokens;
  const bool small = hb <= kAppendSmall;
  const int unroll = small ? 1 : kAppendUnroll;
  long long grid = (hb + kThreads * unroll - 1) / (kThreads * unroll);
  if (grid > KVFP4_APPEND_GRID) grid = KVFP4_APPEND_GRID;
  auto kernel = fp8 ? (small ? append_kernel<true, 1> : append_kernel<true, kAppendUnroll>)
                    : (small ? append_kernel<false, 1> : append_kernel<false, kAppendUnroll>);
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, g,
                     (const uint8_t*)rows, num_tokens, slots, page_rows, (uint8_t*)packed,
                     packed_pages, gs[0], gs1);
  return hipGetLastError();
}

hipError_t launch_dequantize(const Geom& g, const void* packed, int packed_pages,
                             const int32_t* src, void* hot, int hot_pages, const int32_t* dst,
                             int num_pages, const float* gs, hipStream_t stream) {
  if (num_pages == 0) return hipSuccess;
  float gs1 = g.nt > 1 ? gs[1] : gs[0];
  // Decoder: its table is cheap, so the work unit is about one round of
  // loads (kThreads x kDequantUnroll half-blocks, 64 KiB of bf16 out): a
  // larger page is split into that many equal runs, smaller pages are
  // grouped whole.  Measured on 4096 Llama-3-8B-shaped pages in a random
  // slot order (4 runs a page): 241.5-242 us against 250.5-251.5 us with
  // one page a workgroup; runs of a quarter of that were slower (305-310
  // us), the table build dominating.
  const long long hpp = g.elems() / 8;
  const long long unit = (long long)kThreads * kDequantUnroll;
  int parts = 1;
  long long grid;
  if (hpp >= unit) {
    parts = (int)((hpp + unit - 1) / unit);
    grid = (long long)num_pages * parts;
  } else {
    const long long ppw = unit / hpp;
    grid = fill_grid(((long long)num_pages + ppw - 1) / ppw, num_pages);
  }
  if (grid > KVFP4_CODEC_GRID) grid = KVFP4_CODEC_GRID;
  hipLaunchKernelGGL(dequantize_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, g,
                     (const uint8_t*)packed, packed_pages, src, (uint8_t*)hot, hot_pages, dst,
                     num_pages, parts, gs[0], gs1);
  return hipGetLastError();
}

hipError_t launch_gather(const Geom& g, const void* packed, int packed_pages, const int32_t* slots,
                         const int32_t* page_rows, int num_tokens, void* out, bool fp8,
                         const float* gs, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const float gs1 = g.nt > 1 ? gs[1] : gs[0];
  const long long hb = (long long)g.nt * g.H * g.D / 8 * num_tokens;
  const bool small = hb <= kAppendSmall;
  const int unroll = small ? 1 : 4;
  long long grid = (hb + kThreads * unroll - 1) / (kThreads * unroll);
  if (grid > KVFP4_APPEND_GRID) grid = KVFP4_APPEND_GRID;
  auto kernel = fp8 ? (small ? gather_kernel<true, 1> : gather_kernel<true, 4>)
                    : (small ? gather_kernel<false, 1> : gather_kernel<false, 4>);
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, g,
                     (const uint8_t*)packed, packed_pages, slots, page_rows, num_tokens,
                     (uint8_t*)out, gs[0], gs1);
  return hipGetLastError();
}

}  // namespace kvfp4
