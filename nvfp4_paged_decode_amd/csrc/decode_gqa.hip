// Paged NVFP4 decode attention, GQA fast path (head_dim 128, page size a
// multiple of 16 up to 64, up to 8 KV heads, query groups of 1, 2 or 4) on
// VALU.
//
// "Accelerating Long-Context and Agentic Inference with NVFP4 KV Cache",
// NVFP4 KV Decode Attention Kernel Implementation / Figure 3: packed K/V
// and their E4M3 block scales are read straight from the cache, converted
// to bf16 pairs in registers, the products run on bf16 inputs with fp32
// accumulation, and the tensor scales act as scalars on the two products.
// Decode is memory-read-bound (same page, Path 3: Decode), so this kernel
// is organised around reading every packed byte once, coalesced.
//
// Mapping.  A workgroup has one wave per KV head.  In a wave, lane
// (s = lane/8, c = lane%8) owns the 16-value block c of its head (one
// NVFP4 block: 8 data bytes + 1 scale byte per row) for token stream s:
// stream s takes rows s, s+8, s+16, ... of every page, so one load
// instruction reads 8 rows x 64 contiguous bytes.  Each lane keeps its
// block of every query of the group in registers as bf16 pairs.
//   scores:  dot2 over the lane's 16 values (E2M1 codes decoded exactly by
//            the hardware converter with scale 1.0), times the block's
//            E4M3 scale, summed over the 8 lanes of a stream by DPP;
//   softmax: online per stream, one rescale per page at most;
//   P.V:     rows are taken in pairs so that dot2 runs along the token
//            axis: (p_r sv_r, p_r' sv_r') . (c_r[d], c_r'[d]), where sv is
//            the value block scale; accumulation in fp32.
// The 8 streams of a wave are merged at the end of each sequence segment.
//
// Work split.  The pages of all sequences, concatenated in batch order,
// are cut into `nwg` equal contiguous ranges, one per workgroup (balanced
// whatever the length mix).  A workgroup writes one partial per sequence
// it touches, into slot (workgroup + sequence), which is unique because
// ranges are monotone; merge_balanced_kernel combines the partials.
#include "common.hpp"
#include "decode_plan.hpp"

namespace kvfp4 {

namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kD = 128;

__device__ inline bf16x2 as_bf16x2(uint32_t x) { return __builtin_bit_cast(bf16x2, x); }

// E2M1 codes of byte `sel` of w -> two exact bf16 values (scale 1.0 is a
// power of two, which the converter applies exactly).
__device__ inline uint32_t fp4x2_to_bf16x2(uint32_t w, int sel) {
  bf16x2 v;
  switch (sel) {
    case 0: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0); break;
    case 1: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1); break;
    case 2: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2); break;
    default: v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3); break;
  }
  return __builtin_bit_cast(uint32_t, v);
}

// Value of an E4M3FN scale byte (OCP E4M3FN is gfx950's fp8 format; the
// conversion to fp32 is exact).
__device__ inline float scale_value(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

__device__ inline float dpp_sum8(float v) {
  // sum over the 8 lanes of a stream: xor 1, xor 2 (quad_perm), then the
  // half-row mirror pairs lane i with 7-i
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  return v;
}

// Running-max sentinel: finite, so exp2(s - m) needs no special cases
// (an invalid row has s = -inf and gives 0; the first real row resets m).
constexpr float kNoMax = -1e30f;

// One lane's share of two rows of a page (rows s + 16 j and s + 16 j + 8 of
// stream s): its 16-value block of K and of V, and the two block scales.
struct Pair {
  u32x2 k0, k1, v0, v1;
  uint32_t ks0, ks1, vs0, vs1;
  bool ok0, ok1;
};

// Where pair k of a wave's work (pages [p_lo, p_hi) of one sequence) lives.
struct PairSource {
  const uint8_t* pool;
  const int32_t* bt_row;     // block_table row of the sequence
  long long page_bytes;
  int pool_pages, L, T, H, pairs_per_page, h, s, c;
  long long p_lo;
  int npairs;
};

__device__ inline void load_pair(Pair& q, const PairSource& src, int k, const Geom& g) {
  q.ok0 = q.ok1 = false;
  q.k0 = q.k1 = q.v0 = q.v1 = (u32x2){0u, 0u};
  q.ks0 = q.ks1 = q.vs0 = q.vs1 = 0u;
  if (k >= src.npairs) return;
  const long long pg = src.p_lo + k / src.pairs_per_page;
  const int j = k % src.pairs_per_page;
  const int slot = src.bt_row[pg];
  if (slot < 0 || slot >= src.pool_pages) return;
  int n_valid = src.L - (int)pg * src.T;
  if (n_valid > src.T) n_valid = src.T;
  const uint8_t* page = src.pool + (long long)slot * src.page_bytes;
  const long long H = src.H;
  const uint8_t* kdat = page;
  const uint8_t* vdat = page + (long long)src.T * H * (kD / 2);
  const uint8_t* ksc = page + g.data_bytes();
  const uint8_t* vsc = ksc + (long long)src.T * H * (kD / 16);
  const int row0 = src.s + 16 * j, row1 = row0 + 8;
  const long long r0 = (long long)row0 * H + src.h, r1 = (long long)row1 * H + src.h;
  if (row0 < n_valid) {
    q.ok0 = true;
    q.k0 = *reinterpret_cast<const u32x2*>(kdat + r0 * 64 + src.c * 8);
    q.v0 = *reinterpret_cast<const u32x2*>(vdat + r0 * 64 + src.c * 8);
    q.ks0 = ksc[r0 * 8 + src.c];
    q.vs0 = vsc[r0 * 8 + src.c];
  }
  if (row1 < n_valid) {
    q.ok1 = true;
    q.k1 = *reinterpret_cast<const u32x2*>(kdat + r1 * 64 + src.c * 8);
    q.v1 = *reinterpret_cast<const u32x2*>(vdat + r1 * 64 + src.c * 8);
    q.ks1 = ksc[r1 * 8 + src.c];
    q.vs1 = vsc[r1 * 8 + src.c];
  }
}

template <int G>
struct Stream {
  uint32_t q[G][8];  // block c of the G queries, bf16 pairs
  float acc[G][16];
  float m[G], l[G];
};

// Score of one row for every query of the group, summed over the stream.
template <int G>
__device__ inline void row_scores(const Stream<G>& st, u32x2 kw, uint32_t kscale, bool ok,
                                  float qscale, float out[G]) {
  uint32_t kc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) kc[j] = fp4x2_to_bf16x2(j < 4 ? kw.x : kw.y, j & 3);
  const float ks = scale_value(kscale) * qscale;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    float p = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      p = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(st.q[i][j]), as_bf16x2(kc[j]), p, false);
    p = dpp_sum8(p * ks);
    out[i] = ok ? p : -INFINITY;
  }
}

template <int G>
__device__ inline void process_pair(Stream<G>& st, const Pair& pr, float qscale) {
  float s0[G], s1[G];
  row_scores<G>(st, pr.k0, pr.ks0, pr.ok0, qscale, s0);
  row_scores<G>(st, pr.k1, pr.ks1, pr.ok1, qscale, s1);
  // online softmax: rescale only when some running maximum grows
  float mt[G];
  bool grew = false;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    mt[i] = fmaxf(st.m[i], fmaxf(s0[i], s1[i]));
    grew |= mt[i] > st.m[i];
  }
  if (__builtin_amdgcn_ballot_w64(grew)) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float alpha = __builtin_amdgcn_exp2f(st.m[i] - mt[i]);
      st.l[i] *= alpha;
#pragma unroll
      for (int d = 0; d < 16; ++d) st.acc[i][d] *= alpha;
      st.m[i] = mt[i];
    }
  }
  // P.V along the token axis: (p0 sv0, p1 sv1) . (c0[d], c1[d])
  uint32_t va[8], vb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    va[j] = fp4x2_to_bf16x2(j < 4 ? pr.v0.x : pr.v0.y, j & 3);
    vb[j] = fp4x2_to_bf16x2(j < 4 ? pr.v1.x : pr.v1.y, j & 3);
  }
  const float sv0 = scale_value(pr.vs0), sv1 = scale_value(pr.vs1);
  uint32_t pp[G];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const float p0 = __builtin_amdgcn_exp2f(s0[i] - st.m[i]);
    const float p1 = __builtin_amdgcn_exp2f(s1[i] - st.m[i]);
    st.l[i] += p0 + p1;
    bf16x2 w = {(__bf16)(p0 * sv0), (__bf16)(p1 * sv1)};
    pp[i] = __builtin_bit_cast(uint32_t, w);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t lo = __builtin_amdgcn_perm(vb[j], va[j], 0x05040100u);  // element 2j
    const uint32_t hi = __builtin_amdgcn_perm(vb[j], va[j], 0x07060302u);  // element 2j+1
#pragma unroll
    for (int i = 0; i < G; ++i) {
      st.acc[i][2 * j] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pp[i]), as_bf16x2(lo), st.acc[i][2 * j], false);
      st.acc[i][2 * j + 1] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pp[i]), as_bf16x2(hi), st.acc[i][2 * j + 1], false);
    }
  }
}

constexpr int kPrefetch = 4;  // row pairs in flight per lane

template <int G>
__global__ __launch_bounds__(512) void decode_gqa_kernel(DecodeArgs a) {
  const Geom g = a.g;
  const int h = threadIdx.x >> 6;  // wave = KV head
  const int lane = threadIdx.x & 63;
  const int s = lane >> 3, c = lane & 7;
  const int w = blockIdx.x, nwg = gridDim.x;
  const float qscale = a.softmax_scale * a.gs_k * kLog2e;

  BalancedRange rng;
  balanced_range(a, w, nwg, rng);
  long long seq_start = rng.start_first;
  for (int b = rng.b_first; b < a.batch && seq_start < rng.p_end; ++b) {
    const int L = clamped_len(a, b);
    const int npages = (L + g.T - 1) / g.T;
    const long long first = seq_start;
    seq_start += npages;
    const long long p_lo = rng.p_begin > first ? rng.p_begin - first : 0;
    const long long p_hi = rng.p_end - first < npages ? rng.p_end - first : npages;
    if (p_lo >= p_hi) continue;

    Stream<G> st;
    const uint32_t* qrow = reinterpret_cast<const uint32_t*>(a.q) +
                           (((long long)b * a.hq + (long long)h * G) * kD + c * 16) / 2;
#pragma unroll
    for (int i = 0; i < G; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) st.q[i][j] = qrow[i * (kD / 2) + j];
      st.m[i] = kNoMax;
      st.l[i] = 0.f;
#pragma unroll
      for (int d = 0; d < 16; ++d) st.acc[i][d] = 0.f;
    }
    PairSource src;
    src.pool = a.pool;
    src.bt_row = a.block_table + (long long)b * a.max_pages;
    src.page_bytes = g.packed_bytes();
    src.pool_pages = a.pool_pages;
    src.L = L;
    src.T = g.T;
    src.H = g.H;
    src.pairs_per_page = g.T / 16;
    src.h = h;
    src.s = s;
    src.c = c;
    src.p_lo = p_lo;
    src.npairs = (int)(p_hi - p_lo) * src.pairs_per_page;

    Pair ring[kPrefetch];
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) load_pair(ring[k], src, k, g);
    for (int k0 = 0; k0 < src.npairs; k0 += kPrefetch) {
#pragma unroll
      for (int j = 0; j < kPrefetch; ++j) {
        if (k0 + j < src.npairs) {
          const Pair cur = ring[j];
          load_pair(ring[j], src, k0 + j + kPrefetch, g);
          process_pair<G>(st, cur, qscale);
        }
      }
    }
    // merge the 8 streams of this wave (lanes differing in bits 3..5)
#pragma unroll
    for (int off = 8; off < 64; off <<= 1) {
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const float mo = __shfl_xor(st.m[i], off);
        const float lo = __shfl_xor(st.l[i], off);
        const float mn = fmaxf(st.m[i], mo);
        const float fa = __builtin_amdgcn_exp2f(st.m[i] - mn);
        const float fb = __builtin_amdgcn_exp2f(mo - mn);
        st.l[i] = st.l[i] * fa + lo * fb;
#pragma unroll
        for (int d = 0; d < 16; ++d) {
          const float ao = __shfl_xor(st.acc[i][d], off);
          st.acc[i][d] = st.acc[i][d] * fa + ao * fb;
        }
        st.m[i] = mn;
      }
    }
    if (s == 0) {
      const long long slotp = (long long)w + b;  // unique partial slot
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const long long head = (long long)h * G + i;
        float* o = a.ws_o + (slotp * a.hq + head) * kD + c * 16;
#pragma unroll
        for (int d = 0; d < 16; d += 4)
          *reinterpret_cast<float4*>(o + d) =
              make_float4(st.acc[i][d], st.acc[i][d + 1], st.acc[i][d + 2], st.acc[i][d + 3]);
        if (c == 0) {
          a.ws_ml[(slotp * a.hq + head) * 2] = st.m[i];
          a.ws_ml[(slotp * a.hq + head) * 2 + 1] = st.l[i];
        }
      }
    }
  }
}

template <int G>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_gqa_kernel<G>), dim3(a.nwg), dim3(64 * a.g.H), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

bool gqa_supported(const Geom& g, int hq, int v_dim) {
  if (g.nt != 2 || g.D != kD || v_dim != kD) return false;
  if (g.H < 1 || g.H > 8) return false;
  if (g.T != 16 && g.T != 32 && g.T != 64) return false;
  int G = hq / g.H;
  return G == 1 || G == 2 || G == 4;
}

hipError_t launch_decode_gqa(const DecodeArgs& a, hipStream_t stream) {
  switch (a.hq / a.g.H) {
    case 1: return launch_g<1>(a, stream);
    case 2: return launch_g<2>(a, stream);
    case 4: return launch_g<4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvfp4
