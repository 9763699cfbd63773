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

// Dequantized value c * sb of element d of a packed row (exact in fp32).
__device__ inline float packed_elem(const uint8_t* data_row, const uint8_t* scale_row, int d) {
  uint32_t byte = data_row[d >> 1];
  uint32_t nib = (d & 1) ? (byte >> 4) : (byte & 0xF);
  float v = e2m1_mag_to_float(nib & 7) * e4m3_to_float(scale_row[d >> 4]);
  return (nib & 8) ? -v : v;
}

// Generic decode: one workgroup per (split, kv head x 16-query-head chunk,
// sequence).  Thread (qh = tid / 16, r = tid % 16) keeps query head qh's
// elements r, r+16, ... in registers and the matching accumulator slice.
// Correct for every supported geometry (D <= 576); the shape-specialised
// kernels are the fast paths.
__global__ __launch_bounds__(kGenThreads) void decode_generic_kernel(DecodeArgs a) {
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

  __shared__ float ks[kGenTile][kMaxD + 1];
  __shared__ float vs[kGenTile][kMaxD + 1];

  const int D = g.D, Dv = a.v_dim;
  const int nd = (D + 15) / 16, nv = (Dv + 15) / 16;
  float qreg[kMaxD / 16];
  float acc[kMaxD / 16];
  const float qscale = a.softmax_scale * a.gs_k * kLog2e;
#pragma unroll
  for (int i = 0; i < kMaxD / 16; ++i) {
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
  if (t_end > L) t_end = L;

  const long long page_bytes = g.packed_bytes();
  const long long row_data = D / 2, row_scale = D / 16;
  for (int t0 = t_begin; t0 < t_end; t0 += kGenTile) {
    // dequantize the tile: K (tensor 0) and V (tensor 1, or the latent prefix)
    __syncthreads();
    for (int e = tid; e < kGenTile * D; e += kGenThreads) {
      int tt = e / D, d = e - tt * D;
      int tok = t0 + tt;
      float kv = 0.f, vv = 0.f;
      if (tok < t_end) {
        int slot = a.block_table[(long long)b * a.max_pages + tok / g.T];
        if (slot >= 0 && slot < a.pool_pages) {
          int row = tok % g.T;
          const uint8_t* page = a.pool + (long long)slot * page_bytes;
          long long r0 = (long long)row * g.H + h;  // row index within tensor 0
          kv = packed_elem(page + r0 * row_data, page + g.data_bytes() + r0 * row_scale, d);
          if (g.nt == 2) {
            long long r1 = (long long)(g.T + row) * g.H + h;  // tensor 1
            if (d < Dv)
              vv = packed_elem(page + r1 * row_data, page + g.data_bytes() + r1 * row_scale, d);
          } else {
            vv = kv;
          }
        }
      }
      ks[tt][d] = kv;
      vs[tt][d] = vv;
    }
    __syncthreads();
    float s[kGenTile];
#pragma unroll
    for (int tt = 0; tt < kGenTile; ++tt) {
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < kMaxD / 16; ++i)
        if (i < nd && r + 16 * i < D) p += qreg[i] * ks[tt][r + 16 * i];
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) p += __shfl_xor(p, off, 16);
      s[tt] = (t0 + tt < t_end) ? p : -INFINITY;
    }
    float mt = m;
#pragma unroll
    for (int tt = 0; tt < kGenTile; ++tt) mt = fmaxf(mt, s[tt]);
    float alpha = (m == -INFINITY) ? 0.f : exp2f(m - mt);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < kMaxD / 16; ++i) acc[i] *= alpha;
#pragma unroll
    for (int tt = 0; tt < kGenTile; ++tt) {
      float p = (s[tt] == -INFINITY) ? 0.f : exp2f(s[tt] - mt);
      l += p;
#pragma unroll
      for (int i = 0; i < kMaxD / 16; ++i)
        if (i < nv && r + 16 * i < Dv) acc[i] += p * vs[tt][r + 16 * i];
    }
    m = mt;
  }
  if (!active) return;
  long long base = (((long long)b * a.hq + head) * a.splits + split);
#pragma unroll
  for (int i = 0; i < kMaxD / 16; ++i) {
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

__device__ inline long long wave_sum_ll(long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ inline uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ inline float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / 64; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

__device__ inline float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int w = 0; w < kMergeThreads / 64; ++w) r += red[w];
  __syncthreads();
  return r;
}

constexpr int kMergeChunk = 512;  // partial weights staged in LDS per pass

// Merge for the balanced kernels: sequence b's partials sit in slots
// w + b for every workgroup w whose page range overlaps b's pages.  One
// workgroup per (head, sequence).  The page prefix over the batch, the
// running maximum and the weight sum are workgroup-wide reductions over
// the slots; the weights of up to kMergeChunk slots at a time sit in LDS.
// Output: with VEC (v_dim % 4 == 0, 16-byte aligned partials, 8-byte
// aligned out) a thread owns 4 columns of one group of slots (slot index
// mod G, G = threads / (v_dim / 4) groups when v_dim is small), the groups
// are summed through LDS; otherwise one column per thread.
template <bool VEC>
__global__ __launch_bounds__(kMergeThreads) void merge_balanced_kernel(DecodeArgs a) {
  const int head = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  __shared__ long long s_red[2][kMergeThreads / 64];
  __shared__ float s_f[kMergeThreads / 64];
  __shared__ float s_wt[kMergeChunk];
  __shared__ f32x4 s_acc[kMergeThreads];
  long long tot = 0, start = 0;
  for (int i = tid; i < a.batch; i += kMergeThreads) {
    const long long np = pages_of(a, i);
    tot += np;
    if (i < b) start += np;
  }
  tot = wave_sum_ll(tot);
  start = wave_sum_ll(start);
  if ((tid & 63) == 0) {
    s_red[0][tid >> 6] = tot;
    s_red[1][tid >> 6] = start;
  }
  __syncthreads();
  long long ptot = 0, first = 0;
#pragma unroll
  for (int w = 0; w < kMergeThreads / 64; ++w) {
    ptot += s_red[0][w];
    first += s_red[1][w];
  }
  const long long last = first + pages_of(a, b);
  const int nwg = a.nwg;
  int w_lo = 0, w_hi = -1;
  if (last > first) {
    // first workgroup whose range ends after `first`, last one starting before `last`
    int w = (int)(first * nwg / ptot);
    while (w > 0 && range_begin(ptot, w, nwg) > first) --w;
    while (range_begin(ptot, w + 1, nwg) <= first) ++w;
    w_lo = w;
    int hi = (int)(last * nwg / ptot);
    if (hi < w_lo) hi = w_lo;
    if (hi > nwg - 1) hi = nwg - 1;
    while (hi > w_lo && range_begin(ptot, hi, nwg) >= last) --hi;
    while (hi + 1 < nwg && range_begin(ptot, hi + 1, nwg) < last) ++hi;
    w_hi = hi;
  }
  const long long row = (long long)b * a.hq + head;
  // a slot holds a partial only if its workgroup's range is not empty
  auto ms_of = [&](int v) -> float {
    if (range_begin(ptot, v, nwg) >= range_begin(ptot, v + 1, nwg)) return -INFINITY;
    return a.ws_ml[(((long long)v + b) * a.hq + head) * 2];
  };
  float M = -INFINITY;
  for (int v = w_lo + tid; v <= w_hi; v += kMergeThreads) M = fmaxf(M, ms_of(v));
  M = block_max(M, s_f);

  const int D4 = a.v_dim / 4;
  const int G = VEC ? (D4 >= kMergeThreads ? 1 : kMergeThreads / D4) : 1;
  const int grp = VEC ? tid / (D4 >= kMergeThreads ? kMergeThreads : D4) : 0;
  const int d4 = VEC ? (D4 >= kMergeThreads ? tid : tid % D4) : tid;
  f32x4 o4[(kMaxD / 4 + kMergeThreads - 1) / kMergeThreads];  // VEC: columns d4 + k*threads
  float o1[(kMaxD + kMergeThreads - 1) / kMergeThreads];      // scalar: columns tid + k*threads
#pragma unroll
  for (int k = 0; k < (int)(sizeof(o4) / sizeof(o4[0])); ++k) o4[k] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < (int)(sizeof(o1) / sizeof(o1[0])); ++k) o1[k] = 0.f;
  float Lpart = 0.f;
  for (int c0 = w_lo; c0 <= w_hi; c0 += kMergeChunk) {
    const int cn = (w_hi - c0 + 1) < kMergeChunk ? (w_hi - c0 + 1) : kMergeChunk;
    for (int i = tid; i < cn; i += kMergeThreads) {
      const float ms = ms_of(c0 + i);
      float wt = 0.f;
      if (ms != -INFINITY) {
        wt = exp2f(ms - M);
        Lpart += wt * a.ws_ml[(((long long)c0 + i + b) * a.hq + head) * 2 + 1];
      }
      s_wt[i] = wt;
    }
    __syncthreads();
    if (VEC) {
      if (grp < G) {
        for (int i = grp; i < cn; i += G) {
          const float wt = s_wt[i];
          if (wt == 0.f) continue;
          const float* src = a.ws_o + (((long long)c0 + i + b) * a.hq + head) * a.v_dim;
#pragma unroll
          for (int k = 0; k < (int)(sizeof(o4) / sizeof(o4[0])); ++k) {
            const int c = d4 + k * kMergeThreads;
            if (c < D4) o4[k] += *reinterpret_cast<const f32x4*>(src + 4 * c) * wt;
          }
        }
      }
    } else {
      for (int i = 0; i < cn; ++i) {
        const float wt = s_wt[i];
        if (wt == 0.f) continue;
        const float* src = a.ws_o + (((long long)c0 + i + b) * a.hq + head) * a.v_dim;
#pragma unroll
        for (int k = 0; k < (int)(sizeof(o1) / sizeof(o1[0])); ++k) {
          const int c = tid + k * kMergeThreads;
          if (c < a.v_dim) o1[k] += src[c] * wt;
        }
      }
    }
    __syncthreads();  // s_wt is rewritten by the next chunk
  }
  const float Lsum = block_sum(Lpart, s_f);
  const float inv = (Lsum > 0.f) ? a.gs_v / Lsum : 0.f;
  if (VEC) {
    if (G > 1) {
      // sum the G slot groups of each column block (D4 < threads: one k)
      s_acc[tid] = o4[0];
      __syncthreads();
      if (tid < D4) {
        f32x4 t = s_acc[tid];
        for (int gg = 1; gg < G; ++gg) t += s_acc[gg * D4 + tid];
        o4[0] = t;
      }
    }
#pragma unroll
    for (int k = 0; k < (int)(sizeof(o4) / sizeof(o4[0])); ++k) {
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
    for (int k = 0; k < (int)(sizeof(o1) / sizeof(o1[0])); ++k) {
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
    p.splits = 0;
    p.pages_per_split = 0;
    p.workspace_bytes = (size_t)(p.nwg + batch) * hq * (size_t)(v_dim + 2) * sizeof(float);
    return p;
  }
  p.kernel = 0;
  int G = hq / g.H;
  long long items = (long long)batch * g.H * ((G + kGenHeads - 1) / kGenHeads);
  long long want = 2LL * cus;
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
    hipLaunchKernelGGL(decode_generic_kernel, dim3(a.splits, a.g.H * nqc, a.batch),
                       dim3(kGenThreads), 0, stream, a);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  if (plan.kernel == 0) {
    hipLaunchKernelGGL(merge_kernel, dim3(a.hq, a.batch), dim3(kMergeThreads), 0, stream, a);
  } else {
    const bool vec = a.v_dim % 4 == 0 && ((uintptr_t)a.ws_o & 15) == 0 &&
                     ((uintptr_t)a.out & 7) == 0;
    if (vec)
      hipLaunchKernelGGL(merge_balanced_kernel<true>, dim3(a.hq, a.batch), dim3(kMergeThreads),
                         0, stream, a);
    else
      hipLaunchKernelGGL(merge_balanced_kernel<false>, dim3(a.hq, a.batch), dim3(kMergeThreads),
                         0, stream, a);
  }
  return hipGetLastError();
}

// Shapes without a specialised kernel run on the generic one.

}  // namespace kvfp4
