// Paged NVFP4 decode attention: split-K plan, the generic kernel, and the
// cross-workgroup merge.
//
// "Accelerating Long-Context and Agentic Inference with NVFP4 KV Cache",
// Path 3: Decode and NVFP4 KV Decode Attention Kernel Implementation /
// Figure 3: the kernel reads packed NVFP4 K/V and their E4M3 block scales,
// dequantizes in registers, and applies the per-tensor K and V scales as
// scalars on the two products (here: gs_K is folded into the softmax scale,
// gs_V multiplies the merged output).  No standalone dequantization pass.
//
// Split-K.  A sequence's pages are cut into `splits` contiguous ranges of
// `pages_per_split` pages; each (sequence, split) workgroup writes an
// unnormalized partial (o, m, l) with scores in log2 units, and
// merge_kernel combines them: M = max m_s, L = sum l_s 2^(m_s - M),
// out = gs_V * sum o_s 2^(m_s - M) / L, lse = (M + log2 L) ln 2.
#include "common.hpp"
#include "decode_plan.hpp"

namespace kvfp4 {

hipError_t launch_decode_gqa(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_gqa_mfma(const DecodeArgs& a, hipStream_t stream);
bool gqa_supported(const Geom& g, int hq, int v_dim);
bool gqa_mfma_supported(const Geom& g, int hq, int v_dim);
bool mla_supported(const Geom& g, int hq, int v_dim);

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kGenThreads = 256;
constexpr int kGenHeads = 16;   // query heads per workgroup
constexpr int kGenTile = 8;     // tokens per LDS tile
constexpr int kMaxD = 576;

// Generic decode: one workgroup per (split, kv head x 16-query-head chunk,
// sequence).  Thread (qh = tid / 16, r = tid % 16) keeps query head qh's
// elements r, r+16, ... in registers and the matching accumulator slice.
// Correct for every supported geometry (D <= 576); the shape-specialised
// kernels are the fast paths.  DMAX (64, 128, 256 or 576) bounds D so that
// the per-thread loops run D / 16 steps, not 36.
// Staging: a thread takes whole 16-value blocks of the tile (8 data bytes
// and the scale byte in two loads) and writes their 16 exact values c * sb
// to LDS in fp32.
template <int DMAX>
__global__ __launch_bounds__(kGenThreads) void decode_generic_kernel(DecodeArgs a) {
  constexpr int NI = DMAX / 16;
  const Geom g = a.g;
  const int split = blockIdx.x;
  const int b = blockIdx.z;
  const int G = a.hq / g.H;
  const int nqc = (G + kGenHeads - 1) / kGenHeads;
  const int h = blockIdx.y / nqc;
  const int qc = blockIdx.y % nqc;
  const int tid = threadIdx.x;
  const int qh = tid >> 4, r = tid & 15;
  const int head = h * G + qc * kGenHeads + qh;  // query head of this thread
  const bool active = (qc * kGenHeads + qh) < G;

  __shared__ float ks[kGenTile][DMAX + 1];
  __shared__ float vs[kGenTile][DMAX + 1];
  __shared__ int s_slot[kGenTile];

  const int D = g.D, Dv = a.v_dim;
  const int nd = D / 16, nv = (Dv + 15) / 16;
  float qreg[NI];
  float acc[NI];
  const float qscale = a.softmax_scale * a.gs_k * kLog2e;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    int d = r + 16 * i;
    float v = 0.f;
    if (active && i < nd && d < D)
      v = __uint_as_float((uint32_t)a.q[((long long)b * a.hq + head) * D + d] << 16);
    qreg[i] = v * qscale;
    acc[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  int L = a.seq_lens[b];
  const int cap = a.max_pages * g.T;
  if (L > cap) L = cap;
  if (L < 0) L = 0;
  const int t_begin = split * a.pages_per_split * g.T;
  int t_end = t_begin + a.pages_per_split * g.T;
  // the plan is sized from the caller's length hint; the last split takes
  // whatever lies beyond it, so a longer sequence is still attended in full
  if (t_end > L || split == a.splits - 1) t_end = L;

  const long long page_bytes = g.packed_bytes(), data_bytes = g.data_bytes();
  const long long row_data = D / 2, row_scale = D / 16;
  const int units = (g.nt == 2 ? 2 : 1) * kGenTile * nd;  // (tensor, token, block) units
  for (int t0 = t_begin; t0 < t_end; t0 += kGenTile) {
    __syncthreads();  // the previous tile's reads are done
    if (tid < kGenTile) {
      const int tok = t0 + tid;
      int slot = -1;
      if (tok < t_end) {
        slot = a.block_table[(long long)b * a.max_pages + tok / g.T];
        if (slot < 0 || slot >= a.pool_pages) slot = -1;
      }
      s_slot[tid] = slot;
    }
    __syncthreads();
    for (int u = tid; u < units; u += kGenThreads) {
      const int tensor = u / (kGenTile * nd);
      const int rem = u - tensor * kGenTile * nd;
      const int tt = rem / nd, blk = rem - tt * nd;
      const int slot = s_slot[tt];
      float vals[16];
      if (slot >= 0) {
        const uint8_t* page = a.pool + (long long)slot * page_bytes;
        const long long row = ((long long)tensor * g.T + (t0 + tt) % g.T) * g.H + h;
        const uint8_t* dp = page + row * row_data + 8 * blk;
        const uint32_t w0 = (uint32_t)dp[0] | ((uint32_t)dp[1] << 8) | ((uint32_t)dp[2] << 16) |
                            ((uint32_t)dp[3] << 24);
        const uint32_t w1 = (uint32_t)dp[4] | ((uint32_t)dp[5] << 8) | ((uint32_t)dp[6] << 16) |
                            ((uint32_t)dp[7] << 24);
        const float sb = e4m3_to_float(page[data_bytes + row * row_scale + blk]);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint32_t nib = ((e < 8 ? w0 : w1) >> (4 * (e & 7))) & 0xFu;
          const float v = e2m1_mag_to_float(nib & 7u) * sb;
          vals[e] = (nib & 8u) ? -v : v;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) vals[e] = 0.f;
      }
      float* dst = tensor == 0 ? &ks[tt][16 * blk] : &vs[tt][16 * blk];
#pragma unroll
      for (int e = 0; e < 16; ++e) dst[e] = vals[e];
      if (g.nt == 1) {  // MLA-style latent: the values are its prefix
        float* vd = &vs[tt][16 * blk];
#pragma unroll
        for (int e = 0; e < 16; ++e) vd[e] = (16 * blk + e < Dv) ? vals[e] : 0.f;
      }
    }
    __syncthreads();
    float s[kGenTile];
#pragma unroll
    for (int tt = 0; tt < kGenTile; ++tt) {
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if (i < nd) p += qreg[i] * ks[tt][r + 16 * i];
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) p += __shfl_xor(p, off, 16);
      // tokens past the sequence and tokens of an out-of-range page take no
      // part in the softmax
      s[tt] = (t0 + tt < t_end && s_slot[tt] >= 0) ? p : -INFINITY;
    }
    float mt = m;
#pragma unroll
    for (int tt = 0; tt < kGenTile; ++tt) mt = fmaxf(mt, s[tt]);
    float alpha = (m == -INFINITY) ? 0.f : exp2f(m - mt);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < NI; ++i) acc[i] *= alpha;
#pragma unroll
    for (int tt = 0; tt < kGenTile; ++tt) {
      float p = (s[tt] == -INFINITY) ? 0.f : exp2f(s[tt] - mt);
      l += p;
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if (i < nv && r + 16 * i < Dv) acc[i] += p * vs[tt][r + 16 * i];
    }
    m = mt;
  }
  if (!active) return;
  long long base = (((long long)b * a.hq + head) * a.splits + split);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    int d = r + 16 * i;
    if (i < nv && d < Dv) a.ws_o[base * Dv + d] = acc[i];
  }
  if (r == 0) {
    a.ws_ml[base * 2] = m;
    a.ws_ml[base * 2 + 1] = l;
  }
}

constexpr int kMergeThreads = 128;

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(DecodeArgs a) {
  const int head = blockIdx.x, b = blockIdx.y;
  const long long base = ((long long)b * a.hq + head) * a.splits;
  float M = -INFINITY;
  for (int s = 0; s < a.splits; ++s) M = fmaxf(M, a.ws_ml[(base + s) * 2]);
  float Lsum = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    float ms = a.ws_ml[(base + s) * 2];
    if (ms != -INFINITY) Lsum += a.ws_ml[(base + s) * 2 + 1] * exp2f(ms - M);
  }
  const float inv = (Lsum > 0.f) ? a.gs_v / Lsum : 0.f;
  for (int d = threadIdx.x; d < a.v_dim; d += kMergeThreads) {
    float o = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      float ms = a.ws_ml[(base + s) * 2];
      if (ms != -INFINITY) o += a.ws_o[(base + s) * a.v_dim + d] * exp2f(ms - M);
    }
    o *= inv;
    uint32_t u = __float_as_uint(o);
    uint32_t bf = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    a.out[((long long)b * a.hq + head) * a.v_dim + d] = (uint16_t)bf;
  }
  if (threadIdx.x == 0 && a.lse) {
    float v = (Lsum > 0.f) ? (M + log2f(Lsum)) * 0.6931471805599453f : -INFINITY;
    a.lse[(long long)b * a.hq + head] = v;
  }
}

__device__ inline uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

constexpr int kMergeBatch = 8;  // slots whose partials a group requests at once
// Threads of the balanced merge.  Rows of at most 128 columns: 256 (8
// groups of 32 threads request 64 slots per round, so a sequence split over
// up to 64 workgroups is merged after one round of partial loads), or 128
// when the batch's sequences have few holders (32 slots per round; fewer
// threads, less to combine).  Wider rows (MLA): one wave of 64.  The
// launcher below picks one.
constexpr int kBalMergeWide = 64, kBalMergeNarrow = 256, kBalMergeNarrowFew = 128;

// Merge for the balanced kernels: sequence b's partials sit in slots w + b
// for the workgroups w whose page ranges overlap b's pages, w_lo..w_hi
// (recorded by the decode kernel with the length of the split).  One
// workgroup per (head, sequence), two rounds of global reads: the
// sequence's length, slot range and the split's length together, then
// every partial at once.  Loads are unconditional, from slot and column
// indices clamped into range, and whether a slot holds a partial is decided
// after they are all issued: loads under a condition become branches that
// wait for each load before the next.  Slots are split over G thread
// groups (G = threads / (v_dim / 4) when v_dim is small, else 1); a group
// folds its slots with a running maximum, kMergeBatch of them per round of
// loads, and the groups combine through LDS.  VEC (v_dim % 4 == 0, 16-byte
// aligned partials, 8-byte aligned out): a thread owns 4 columns;
// otherwise one column per thread, G = 1.
template <bool VEC, int K4, int kMergeThreads, int kCols>
__global__ __launch_bounds__(kMergeThreads) void merge_balanced_kernel(DecodeArgs a) {
  static_assert(!VEC || K4 * 4 * kMergeThreads >= kCols, "v_dim up to kCols");
  const int head = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  __shared__ float s_m[kMergeThreads], s_l[kMergeThreads];
  __shared__ f32x4 s_acc[kMergeThreads];
  const long long row = (long long)b * a.hq + head;
  const int nwg = a.nwg;
  // first round: all three requested before any is used
  const int L = clamped_len(a, b);
  int w_lo = a.ws_idx[2 * b], w_hi = a.ws_idx[2 * b + 1];
  const long long ptot = a.ws_idx[2 * a.batch];
  // the decode kernel wrote the range for every sequence with pages (and
  // nothing for the others, nor anything at all for a batch without pages:
  // those get an empty range, so a zero output and lse -inf); clamp anyway
  w_lo = w_lo < 0 ? 0 : (w_lo > nwg - 1 ? nwg - 1 : w_lo);
  w_hi = w_hi < w_lo ? w_lo : (w_hi > nwg - 1 ? nwg - 1 : w_hi);
  if (L == 0 || ptot <= 0) w_hi = w_lo - 1;
  // slot v + b (w_lo <= v <= w_hi) holds a partial when v's range is not
  // empty, which every range is when the split has at least one page (real
  // or pad) per workgroup; ranges between w_lo and w_hi lie within b's pages
  const bool all_hold = ptot >= nwg;
  auto holds = [&](int v) {
    return all_hold || (long long)v * ptot / nwg < (long long)(v + 1) * ptot / nwg;
  };

  const int D4 = a.v_dim / 4;
  const int G = VEC ? (D4 >= kMergeThreads ? 1 : kMergeThreads / D4) : 1;
  const int grp = VEC ? tid / (D4 >= kMergeThreads ? kMergeThreads : D4) : 0;
  const int d4 = VEC ? (D4 >= kMergeThreads ? tid : tid % D4) : tid;
  // K4: 4-column blocks per thread (VEC: ceil(v_dim / 4 / threads));
  // K1: columns per thread otherwise
  constexpr int K1 = VEC ? 1 : (kMaxD + kMergeThreads - 1) / kMergeThreads;
  f32x4 o4[K4];
  float o1[K1];
#pragma unroll
  for (int k = 0; k < K4; ++k) o4[k] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < K1; ++k) o1[k] = 0.f;
  float mg = -INFINITY, lg = 0.f;
  {
    for (int v0 = w_lo + grp; grp < G && v0 <= w_hi; v0 += G * kMergeBatch) {
      float mv[kMergeBatch], lv[kMergeBatch];
      u32x2 raw4[kMergeBatch][K4];
      uint16_t raw1[kMergeBatch][K1];
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {
        const int v = v0 + i * G, vc = v <= w_hi ? v : w_hi;  // in range
        const long long sp = ((long long)vc + b) * a.hq + head;
        mv[i] = a.ws_ml[sp * 2];
        lv[i] = a.ws_ml[sp * 2 + 1];
        const uint16_t* src = a.ws_oh + sp * a.v_dim;  // o / l in fp16
        if (VEC) {
#pragma unroll
          for (int k = 0; k < K4; ++k) {
            const int c = d4 + k * kMergeThreads;
            raw4[i][k] = *reinterpret_cast<const u32x2*>(src + 4 * (c < D4 ? c : D4 - 1));
          }
        } else {
#pragma unroll
          for (int k = 0; k < K1; ++k) {
            const int c = tid + k * kMergeThreads;
            raw1[i][k] = src[c < a.v_dim ? c : a.v_dim - 1];
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {
        const int v = v0 + i * G;
        if (v > w_hi || !holds(v) || mv[i] == -INFINITY) continue;  // no partial here
        const float mn = fmaxf(mg, mv[i]);
        // slot weight exp2(m_i - mn) l_i: the stored output is o_i / l_i
        const float so = exp2f(mg - mn), sn = exp2f(mv[i] - mn) * lv[i];  // exp2(-inf) = 0
        lg = lg * so + sn;
        if (VEC) {
#pragma unroll
          for (int k = 0; k < K4; ++k) {
            const int c = d4 + k * kMergeThreads;
            const f32x4 x = c < D4 ? unpack_f16x4(raw4[i][k]) : (f32x4){0.f, 0.f, 0.f, 0.f};
            o4[k] = o4[k] * so + x * sn;
          }
        } else {
#pragma unroll
          for (int k = 0; k < K1; ++k) {
            const int c = tid + k * kMergeThreads;
            const float x = c < a.v_dim ? f16_value(raw1[i][k]) : 0.f;
            o1[k] = o1[k] * so + x * sn;
          }
        }
        mg = mn;
      }
    }
  }
  float M = mg, Lsum = lg;
  if (VEC && G > 1) {
    // combine the G groups (here D4 < threads, so one column block: k = 0)
    if (d4 == 0 && grp < G) {
      s_m[grp] = mg;
      s_l[grp] = lg;
    }
    s_acc[tid] = o4[0];
    __syncthreads();
    M = -INFINITY;
    for (int gg = 0; gg < G; ++gg) M = fmaxf(M, s_m[gg]);
    Lsum = 0.f;
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
    for (int gg = 0; gg < G; ++gg) {
      if (s_m[gg] == -INFINITY) continue;
      const float wgt = exp2f(s_m[gg] - M);
      Lsum += s_l[gg] * wgt;
      if (tid < D4) t += s_acc[gg * D4 + tid] * wgt;
    }
    o4[0] = t;
  }
  const float inv = (Lsum > 0.f) ? a.gs_v / Lsum : 0.f;
  if (VEC) {
#pragma unroll
    for (int k = 0; k < K4; ++k) {
      const int c = d4 + k * kMergeThreads;
      if (grp == 0 && c < D4) {
        const f32x4 o = o4[k] * inv;
        u32x2 w2;
        w2.x = bf16_rne_bits(o.x) | (bf16_rne_bits(o.y) << 16);
        w2.y = bf16_rne_bits(o.z) | (bf16_rne_bits(o.w) << 16);
        *reinterpret_cast<u32x2*>(a.out + row * a.v_dim + 4 * c) = w2;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < K1; ++k) {
      const int c = tid + k * kMergeThreads;
      if (c < a.v_dim) a.out[row * a.v_dim + c] = (uint16_t)bf16_rne_bits(o1[k] * inv);
    }
  }
  if (tid == 0 && a.lse) {
    float v = (Lsum > 0.f) ? (M + log2f(Lsum)) * 0.6931471805599453f : -INFINITY;
    a.lse[row] = v;
  }
}

}  // namespace

DecodePlan plan_decode(const Geom& g, int batch, int hq, int v_dim, int max_seq_len_hint,
                       int num_cus) {
  DecodePlan p{};
  int hint = max_seq_len_hint > 0 ? max_seq_len_hint : 1;
  int pages_max = (hint + g.T - 1) / g.T;
  const int cus = num_cus > 0 ? num_cus : 256;
  if (batch <= 0) {
    p.splits = 1;
    p.pages_per_split = pages_max;
    p.nwg = 1;
    p.workspace_bytes = 0;
    return p;
  }
  if (mla_supported(g, hq, v_dim) || gqa_mfma_supported(g, hq, v_dim) ||
      gqa_supported(g, hq, v_dim)) {
    // balanced kernels: one workgroup per CU (or per page when fewer)
    p.kernel = mla_supported(g, hq, v_dim) ? 2 : gqa_mfma_supported(g, hq, v_dim) ? 3 : 1;
    long long target = cus;
    long long pages_ub = (long long)batch * pages_max;
    long long nwg = target < pages_ub ? target : pages_ub;
    p.nwg = (int)(nwg > 0 ? nwg : 1);
    // a segment pad is about 128 tokens of pages (a second segment's start
    // and stream merge cost about as long as streaming that many); none for
    // batches over 64 sequences or pages of more than 256 tokens
    p.seg_pad = batch <= 64 ? (128 + g.T / 2) / g.T : 0;
    p.splits = 0;
    p.pages_per_split = 0;
    // partial outputs (fp16), their (max, sum) (fp32), then the merge's
    // index ([batch][2] + the length of the split, padded)
    p.workspace_bytes =
        (size_t)(p.nwg + batch) * hq * ((size_t)v_dim * sizeof(uint16_t) + 2 * sizeof(float)) +
        (((size_t)2 * batch + 1) * sizeof(int32_t) + 15) / 16 * 16;
    return p;
  }
  p.kernel = 0;
  int G = hq / g.H;
  long long items = (long long)batch * g.H * ((G + kGenHeads - 1) / kGenHeads);
  long long want = 8LL * cus;  // the split loop is latency-bound: many workgroups per CU
  long long s = (want + items - 1) / items;
  if (s < 1) s = 1;
  if (s > pages_max) s = pages_max;
  p.pages_per_split = (int)((pages_max + s - 1) / s);
  p.splits = (pages_max + p.pages_per_split - 1) / p.pages_per_split;
  p.nwg = 0;
  p.workspace_bytes = (size_t)batch * hq * p.splits * (size_t)(v_dim + 2) * sizeof(float);
  return p;
}

hipError_t launch_decode(const DecodePlan& plan, const DecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  hipError_t e;
  if (plan.kernel == 3) {
    e = launch_decode_gqa_mfma(a, stream);
  } else if (plan.kernel == 2) {
    e = launch_decode_mla(a, stream);
  } else if (plan.kernel == 1) {
    e = launch_decode_gqa(a, stream);
  } else {
    int G = a.hq / a.g.H;
    int nqc = (G + kGenHeads - 1) / kGenHeads;
    const dim3 grid(a.splits, a.g.H * nqc, a.batch);
    const int dmax = a.g.D > a.v_dim ? a.g.D : a.v_dim;
    if (dmax <= 64)
      hipLaunchKernelGGL(decode_generic_kernel<64>, grid, dim3(kGenThreads), 0, stream, a);
    else if (dmax <= 128)
      hipLaunchKernelGGL(decode_generic_kernel<128>, grid, dim3(kGenThreads), 0, stream, a);
    else if (dmax <= 256)
      hipLaunchKernelGGL(decode_generic_kernel<256>, grid, dim3(kGenThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(decode_generic_kernel<kMaxD>, grid, dim3(kGenThreads), 0, stream, a);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  if (plan.kernel == 0) {
    hipLaunchKernelGGL(merge_kernel, dim3(a.hq, a.batch), dim3(kMergeThreads), 0, stream, a);
  } else {
    const bool vec = a.v_dim % 4 == 0 && ((uintptr_t)a.ws_oh & 15) == 0 &&
                     ((uintptr_t)a.out & 7) == 0;
    auto launch = [&](auto threads_c, auto k4_c, auto cols_c) {
      constexpr int kT = decltype(threads_c)::value, kK4 = decltype(k4_c)::value,
                    kC = decltype(cols_c)::value;
      auto kernel = vec ? merge_balanced_kernel<true, kK4, kT, kC>
                        : merge_balanced_kernel<false, 1, kT, kC>;
      hipLaunchKernelGGL(kernel, dim3(a.hq, a.batch), dim3(kT), 0, stream, a);
    };
    // the balanced kernels have v_dim <= 512.  Up to 128 columns: one
    // 4-column block a thread, and G = threads / (v_dim / 4) groups of
    // slots, kMergeBatch slots a group a round; with equal lengths a
    // sequence has about nwg / batch + 1 holders, so 128 threads (32 slots a
    // round for v_dim 128) when those fit, else 256 (64 a round; 128
    // threads measured 4.3 against 5.1 us on 32 sequences of 8 holders,
    // and 5.2 against 4.5 us on 8 sequences of about 32).  Wider
    // rows (MLA): one wave of 64 threads with two blocks each, one wave per
    // (head, sequence), which keeps the whole grid resident at once.
    if (a.v_dim <= 128) {
      if (a.nwg / a.batch + 2 <= (kBalMergeNarrowFew / 32) * kMergeBatch)
        launch(std::integral_constant<int, kBalMergeNarrowFew>{}, std::integral_constant<int, 1>{},
               std::integral_constant<int, 128>{});
      else
        launch(std::integral_constant<int, kBalMergeNarrow>{}, std::integral_constant<int, 1>{},
               std::integral_constant<int, 128>{});
    } else {
      launch(std::integral_constant<int, kBalMergeWide>{}, std::integral_constant<int, 2>{},
             std::integral_constant<int, 512>{});
    }
  }
  return hipGetLastError();
}

// Shapes without a specialised kernel run on the generic one.

}  // namespace kvfp4
