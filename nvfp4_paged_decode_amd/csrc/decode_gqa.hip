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
//            axis: (p_r, p_r') . (v_r[d], v_r'[d]) in fp16 with fp32
//            accumulation.  A value v = c sv (E2M1 code times the block's
//            E4M3 scale: at most 6 significant bits, in [2^-10, 2688]) is
//            exact in fp16; p is rounded to fp16 once, and the denominator
//            sums those same rounded values.
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
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

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

// E2M1 codes of byte `sel` of w -> two exact fp16 values.
__device__ inline f16x2 fp4x2_to_f16x2(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  }
}

// Value of an E4M3FN scale byte (OCP E4M3FN is gfx950's fp8 format; the
// conversion to fp32 is exact).
__device__ inline float scale_value(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

// v[i] += value of v[i] in lane (lane ^ 1), (lane ^ 2), then the half-row
// mirror (lane i <-> 7 - i): the sum over the 8 lanes of a stream.  Each
// step runs over all values before the next, so DPP reads never wait on
// the VALU write just before them.
template <int N>
__device__ inline void dpp_sum8(float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    v[i] += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v[i]), 0xB1, 0xF, 0xF, true));
#pragma unroll
  for (int i = 0; i < N; ++i)
    v[i] += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v[i]), 0x4E, 0xF, 0xF, true));
#pragma unroll
  for (int i = 0; i < N; ++i)
    v[i] += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v[i]), 0x141, 0xF, 0xF, true));
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
// Loads go through buffer resources whose size covers only the page's
// valid rows, so rows past the sequence end read as zero and are never
// fetched from memory.
struct PairSource {
  const uint8_t* pool;
  const int32_t* bt_row;     // block_table row of the sequence
  long long page_bytes, data_bytes;
  int pool_pages, L, T, H, pairs_per_page, s;
  long long p_lo;
  int npairs;
  uint32_t lane_data, lane_scale;  // this lane's byte offsets for row s
};

// Loads one lane's share of pair j of page `pg` (an index into the
// sequence's page-table row; pages at or past `pg_end` read as empty).
// The page's slot comes from a register (readlane), never from a memory
// load issued behind the data loads, so waiting for it never drains the
// data loads in flight.
// Unconditional: out-of-range rows come back as zero from the buffer
// resource, so no branch surrounds the loads.
__device__ inline void load_pair(Pair& q, const PairSource& src, int slot_vec, long long c0,
                                 long long pg, long long pg_end, int j) {
  // page-table entries of pages c0 .. c0+63 sit one per lane in slot_vec
  int slot = -1;
  if (pg < pg_end) slot = __builtin_amdgcn_readlane(slot_vec, (int)(pg - c0));
  int n_valid = src.L - (int)pg * src.T;
  if (n_valid > src.T) n_valid = src.T;
  if (slot < 0 || slot >= src.pool_pages) n_valid = 0;
  n_valid = __builtin_amdgcn_readfirstlane(n_valid);
  const uint8_t* page = src.pool + (long long)(n_valid > 0 ? slot : 0) * src.page_bytes;
  const int rowbytes = src.H * (kD / 2), rowscale = src.H * (kD / 16);
  const uint8_t* vdat = page + (long long)src.T * rowbytes;
  const uint8_t* ksc = page + src.data_bytes;
  const uint8_t* vsc = ksc + (long long)src.T * rowscale;
  auto rk = __builtin_amdgcn_make_buffer_rsrc((void*)page, (short)0, n_valid * rowbytes, 0x00020000);
  auto rv = __builtin_amdgcn_make_buffer_rsrc((void*)vdat, (short)0, n_valid * rowbytes, 0x00020000);
  auto rks = __builtin_amdgcn_make_buffer_rsrc((void*)ksc, (short)0, n_valid * rowscale, 0x00020000);
  auto rvs = __builtin_amdgcn_make_buffer_rsrc((void*)vsc, (short)0, n_valid * rowscale, 0x00020000);
  const int so0 = 16 * j * rowbytes, so1 = so0 + 8 * rowbytes;
  const int ss0 = 16 * j * rowscale, ss1 = ss0 + 8 * rowscale;
  q.k0 = __builtin_amdgcn_raw_buffer_load_b64(rk, src.lane_data, so0, 0);
  q.k1 = __builtin_amdgcn_raw_buffer_load_b64(rk, src.lane_data, so1, 0);
  q.v0 = __builtin_amdgcn_raw_buffer_load_b64(rv, src.lane_data, so0, 0);
  q.v1 = __builtin_amdgcn_raw_buffer_load_b64(rv, src.lane_data, so1, 0);
  q.ks0 = __builtin_amdgcn_raw_buffer_load_b8(rks, src.lane_scale, ss0, 0);
  q.ks1 = __builtin_amdgcn_raw_buffer_load_b8(rks, src.lane_scale, ss1, 0);
  q.vs0 = __builtin_amdgcn_raw_buffer_load_b8(rvs, src.lane_scale, ss0, 0);
  q.vs1 = __builtin_amdgcn_raw_buffer_load_b8(rvs, src.lane_scale, ss1, 0);
  q.ok0 = src.s + 16 * j < n_valid;
  q.ok1 = src.s + 16 * j + 8 < n_valid;
}

template <int G>
struct Stream {
  uint32_t q[G][8];  // block c of the G queries, bf16 pairs
  float acc[G][16];
  float m[G], l[G];
};

// Rare path: a running maximum grew; rescale the stream's state.
template <int G>
__device__ inline void rescale(Stream<G>& st, const float (&mt)[G]) {
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const float alpha = __builtin_amdgcn_exp2f(st.m[i] - mt[i]);
    st.l[i] *= alpha;
#pragma unroll
    for (int d = 0; d < 16; ++d) st.acc[i][d] *= alpha;
    st.m[i] = mt[i];
  }
}

template <int G>
__device__ inline void process_pair(Stream<G>& st, const Pair& pr, float qscale) {
  // scores of both rows for every query of the group
  float sc[2 * G];
  {
    uint32_t k0[8], k1[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      k0[j] = fp4x2_to_bf16x2(j < 4 ? pr.k0.x : pr.k0.y, j & 3);
      k1[j] = fp4x2_to_bf16x2(j < 4 ? pr.k1.x : pr.k1.y, j & 3);
    }
    const float ks0 = scale_value(pr.ks0) * qscale, ks1 = scale_value(pr.ks1) * qscale;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      float p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(st.q[i][j]), as_bf16x2(k0[j]), p0, false);
        p1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(st.q[i][j]), as_bf16x2(k1[j]), p1, false);
      }
      sc[i] = p0 * ks0;
      sc[G + i] = p1 * ks1;
    }
  }
  dpp_sum8<2 * G>(sc);
#pragma unroll
  for (int i = 0; i < G; ++i) {
    sc[i] = pr.ok0 ? sc[i] : -INFINITY;
    sc[G + i] = pr.ok1 ? sc[G + i] : -INFINITY;
  }
  // online softmax: rescale only when some running maximum grows
  float mt[G];
  bool grew = false;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    mt[i] = fmaxf(st.m[i], fmaxf(sc[i], sc[G + i]));
    grew |= mt[i] > st.m[i];
  }
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(grew) != 0, 0)) rescale<G>(st, mt);
  // P.V along the token axis: (p0, p1) . (v0[d], v1[d]), v = c sv exact
  // in fp16
  const _Float16 sv0 = (_Float16)scale_value(pr.vs0), sv1 = (_Float16)scale_value(pr.vs1);
  const f16x2 s0 = {sv0, sv0}, s1 = {sv1, sv1};
  uint32_t va[8], vb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    va[j] = __builtin_bit_cast(uint32_t, fp4x2_to_f16x2(j < 4 ? pr.v0.x : pr.v0.y, j & 3) * s0);
    vb[j] = __builtin_bit_cast(uint32_t, fp4x2_to_f16x2(j < 4 ? pr.v1.x : pr.v1.y, j & 3) * s1);
  }
  f16x2 pp[G];
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const _Float16 p0 = (_Float16)__builtin_amdgcn_exp2f(sc[i] - st.m[i]);
    const _Float16 p1 = (_Float16)__builtin_amdgcn_exp2f(sc[G + i] - st.m[i]);
    st.l[i] += (float)p0 + (float)p1;
    pp[i] = (f16x2){p0, p1};
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t lo = __builtin_amdgcn_perm(vb[j], va[j], 0x05040100u);  // element 2j
    const uint32_t hi = __builtin_amdgcn_perm(vb[j], va[j], 0x07060302u);  // element 2j+1
#pragma unroll
    for (int i = 0; i < G; ++i) {
      st.acc[i][2 * j] = __builtin_amdgcn_fdot2(pp[i], __builtin_bit_cast(f16x2, lo), st.acc[i][2 * j], false);
      st.acc[i][2 * j + 1] = __builtin_amdgcn_fdot2(pp[i], __builtin_bit_cast(f16x2, hi), st.acc[i][2 * j + 1], false);
    }
  }
}

template <int G, int PPP>  // PPP: row pairs per page (page size / 16)
__global__ __launch_bounds__(512) void decode_gqa_kernel(DecodeArgs a) {
  const Geom g = a.g;
  const int h = threadIdx.x >> 6;  // wave = KV head
  const int lane = threadIdx.x & 63;
  const int s = lane >> 3, c = lane & 7;
  const int nwg = gridDim.x, w = split_index(blockIdx.x, nwg);  // position in the split
  const float qscale = a.softmax_scale * a.gs_k * kLog2e;

  BalancedRange rng;
  balanced_range(a, w, nwg, rng);
  note_total(a, w, rng.ptot);
  long long seq_start = rng.start_first;
  for (int b = rng.b_first; b < a.batch && seq_start < rng.p_end; ++b) {
    const int L = seq_len(a, rng, b);
    const int npages = (L + g.T - 1) / g.T;
    const long long first = seq_first_page(rng, b, seq_start);
    seq_start = first + npages;
    const long long p_lo = rng.p_begin > first ? rng.p_begin - first : 0;
    const long long p_hi = rng.p_end - first < npages ? rng.p_end - first : npages;
    if (p_lo >= p_hi) continue;
    note_segment(a, w, b, p_lo, p_hi, npages);

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
    src.data_bytes = g.data_bytes();
    src.pool_pages = a.pool_pages;
    src.L = L;
    src.T = g.T;
    src.H = g.H;
    src.pairs_per_page = g.T / 16;
    src.s = s;
    src.p_lo = p_lo;
    src.npairs = (int)(p_hi - p_lo) * src.pairs_per_page;
    src.lane_data = (uint32_t)((s * g.H + h) * (kD / 2) + c * 8);
    src.lane_scale = (uint32_t)((s * g.H + h) * (kD / 16) + c);

    // Two page buffers: while one page is processed the next one is in
    // flight (a page is 64 rows x 144 bytes per wave for a 64-row page).
    // Pages go in chunks of 64 whose page-table entries are read once.
    for (long long c0 = p_lo; c0 < p_hi; c0 += 64) {
      const long long ce = c0 + 64 < p_hi ? c0 + 64 : p_hi;
      const int slot_vec = (c0 + lane < ce) ? src.bt_row[c0 + lane] : -1;
      Pair A[PPP], B[PPP];
#pragma unroll
      for (int j = 0; j < PPP; ++j) load_pair(A[j], src, slot_vec, c0, c0, ce, j);
      for (long long pg = c0; pg < ce; pg += 2) {
#pragma unroll
        for (int j = 0; j < PPP; ++j) load_pair(B[j], src, slot_vec, c0, pg + 1, ce, j);
#pragma unroll
        for (int j = 0; j < PPP; ++j) process_pair<G>(st, A[j], qscale);
#pragma unroll
        for (int j = 0; j < PPP; ++j) load_pair(A[j], src, slot_vec, c0, pg + 2, ce, j);
        if (pg + 1 < ce) {
#pragma unroll
          for (int j = 0; j < PPP; ++j) process_pair<G>(st, B[j], qscale);
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
        // the partial output divided by its sum, in fp16
        uint16_t* o = a.ws_oh + (slotp * a.hq + head) * kD + c * 16;
        const float il = st.l[i] > 0.f ? 1.f / st.l[i] : 0.f;
#pragma unroll
        for (int d = 0; d < 16; d += 4)
          *reinterpret_cast<u32x2*>(o + d) = pack_f16x4(
              (f32x4){st.acc[i][d], st.acc[i][d + 1], st.acc[i][d + 2], st.acc[i][d + 3]} * il);
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
  const dim3 grid(a.nwg), block(64 * a.g.H);
  switch (a.g.T) {
    case 16: hipLaunchKernelGGL((decode_gqa_kernel<G, 1>), grid, block, 0, stream, a); break;
    case 32: hipLaunchKernelGGL((decode_gqa_kernel<G, 2>), grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL((decode_gqa_kernel<G, 4>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
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
