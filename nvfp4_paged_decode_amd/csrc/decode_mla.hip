// Paged NVFP4 decode attention, MLA path on MFMA: one 576-value latent per
// token (512 + 64 rope, all NVFP4), values = the first 512 dims of the same
// latent, 16 to 128 query heads, pages of 32 or 64 tokens.
//
// "Accelerating Long-Context and Agentic Inference with NVFP4 KV Cache",
// NVFP4 KV Decode Attention Kernel Implementation / Figure 3: packed tiles
// and their E4M3 scales are staged, unpacked and scaled, and both attention
// products run in bf16 with the tensor scale applied as a scalar.  With 128
// query heads over one latent the products are real dense contractions
// (about 860 flop per cache byte), so here they run on MFMA
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//
// Per workgroup (up to 4 waves, two workgroups per CU): a contiguous page
// range of the batch (the balanced split of decode_plan.hpp) and a group of
// up to 64 query heads (blockIdx.y); wave w owns 16 heads of the group.
// For each 32-token tile:
//  1. every thread dequantizes part of the tile once: E2M1 codes decoded
//     exactly by the converter (scale 1.0) to fp32, times the E4M3 block
//     scale (exact: at most 6 significant bits), packed to bf16 (exact),
//     written to LDS twice: natural [token][576] for the scores and
//     transposed [512][token] for P.V;
//  2. scores as S^T = K Q^T (A = latent rows from LDS, B = the wave's
//     queries, held in registers for the whole kernel), so that each lane
//     ends up holding, for its head column, exactly the 8 tokens it feeds
//     to the P.V MFMA as A operand: no transpose of P;
//  3. online softmax per head (running max, lazy rescale of the output
//     accumulators only when a maximum grows);
//  4. O += P V with V from the transposed LDS copy.
// The wave's unnormalized partial (O, max, sum) goes to workspace slot
// (workgroup + sequence); merge_balanced_kernel combines them.
#include "common.hpp"
#include "decode_plan.hpp"

namespace kvfp4 {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kD = 576;       // latent dims per token (keys)
constexpr int kDv = 512;      // value dims (latent prefix)
constexpr int kTile = 32;     // tokens per tile
constexpr int kKs = kD / 32;  // k-steps of the score MFMA
constexpr int kVt = kDv / 16; // 16-column tiles of the output
constexpr int kKnPitch = kD + 8;   // bf16 per natural row (292 dwords: conflict-free reads)
constexpr int kVtPitch = 40;       // bf16 per transposed row (20 dwords)
constexpr float kNoMax = -1e30f;

struct MlaLds {
  __bf16 kn[kTile][kKnPitch];  // natural latent rows
  __bf16 vt[kDv][kVtPitch];    // transposed value rows, tokens in k-group order
};

// Position of token t (0..31) in a transposed row: k-group g of the P.V
// MFMA holds tokens 4g..4g+3 and 16+4g..16+4g+3 (the tokens that lane group
// g holds in the score output), contiguously at [8g, 8g+8).
__device__ inline int vt_pos(int t) { return ((t & 15) >> 2) * 8 + (t >> 4) * 4 + (t & 3); }

__device__ inline bf16x8 lds_read8(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Two workgroups per CU (2 x 78 KB of LDS, 256 registers per lane) so that
// one workgroup's dequantization overlaps the other's MFMA work.
#ifndef KVFP4_MLA_OCC
#define KVFP4_MLA_OCC __attribute__((amdgpu_waves_per_eu(2)))
#endif

template <int NW, int NHT>
__global__ __launch_bounds__(64 * NW) KVFP4_MLA_OCC void decode_mla_kernel(DecodeArgs a) {
  constexpr int HG = 16 * NHT * NW;  // query heads of this workgroup
  constexpr int NT = 64 * NW;
  const int HQ = a.hq, hg0 = blockIdx.y * HG;
  extern __shared__ __align__(16) unsigned char smem[];
  MlaLds& s = *reinterpret_cast<MlaLds*>(smem);
  const Geom g = a.g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int w = blockIdx.x, nwg = gridDim.x;
  const float qscale = a.softmax_scale * a.gs_k * kLog2e;
  const int row_data = kD / 2, row_scale = kD / 16;  // bytes per token row (H = 1)

  BalancedRange rng;
  balanced_range(a, w, nwg, rng);
  long long seq_start = rng.start_first;
  for (int b = rng.b_first; b < a.batch && seq_start < rng.p_end; ++b) {
    const int L = uniform(clamped_len(a, b));
    const int npages = (L + g.T - 1) / g.T;
    const long long first = seq_start;
    seq_start += npages;
    const long long p_lo = rng.p_begin > first ? rng.p_begin - first : 0;
    const long long p_hi = rng.p_end - first < npages ? rng.p_end - first : npages;
    if (p_lo >= p_hi) continue;

    // queries of this wave as the B operand of S^T = K Q^T: lane (head
    // column lr, k-group lg) holds q[head][32 ks + 8 lg .. + 8]
    bf16x8 qb[NHT][kKs];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int head = hg0 + (wave * NHT + ht) * 16 + lr;
      const uint16_t* qrow = a.q + ((long long)b * a.hq + head) * kD;
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks)
        qb[ht][ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks + 8 * lg);
    }
    f32x4 acc[NHT][kVt];
    float m[NHT], l[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      m[ht] = kNoMax;
      l[ht] = 0.f;
#pragma unroll
      for (int vt = 0; vt < kVt; ++vt) acc[ht][vt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }

    const int tiles_per_page = g.T / kTile;
    const long long tile_lo = p_lo * tiles_per_page, tile_hi = p_hi * tiles_per_page;
    for (long long tile = tile_lo; tile < tile_hi; ++tile) {
      const long long pg = tile / tiles_per_page;
      const int row0 = (int)(tile % tiles_per_page) * kTile;  // first row in the page
      const int slot = __builtin_amdgcn_readfirstlane(a.block_table[(long long)b * a.max_pages + pg]);
      int n_valid = L - (int)(pg * g.T) - row0;  // valid tokens of this tile
      if (n_valid > kTile) n_valid = kTile;
      if (slot < 0 || slot >= a.pool_pages) n_valid = 0;
      n_valid = uniform(n_valid);
      const uint8_t* page = a.pool + (long long)(slot < 0 ? 0 : slot) * g.packed_bytes();
      const uint8_t* tdat = page + (long long)row0 * row_data;
      const uint8_t* tsc = page + g.data_bytes() + (long long)row0 * row_scale;

      // 1. dequantize the tile into LDS: chunk = 8 values of one token
      __syncthreads();  // the previous tile's readers are done
      for (int c = tid; c < kTile * (kD / 8); c += NT) {
        const int t = c & (kTile - 1), d8 = c >> 5;  // 32 tokens per d8 column
        f32x2 v[4];
        if (t < n_valid) {
          const uint32_t wd = *reinterpret_cast<const uint32_t*>(tdat + t * row_data + d8 * 4);
          const float sb = __builtin_amdgcn_cvt_f32_fp8((int)tsc[t * row_scale + (d8 >> 1)], 0);
          v[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, 1.0f, 0);
          v[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, 1.0f, 1);
          v[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, 1.0f, 2);
          v[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(wd, 1.0f, 3);
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] *= sb;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (f32x2){0.f, 0.f};
        }
        bf16x8 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[2 * i] = (__bf16)v[i].x;
          o[2 * i + 1] = (__bf16)v[i].y;
        }
        *reinterpret_cast<bf16x8*>(&s.kn[t][d8 * 8]) = o;
        if (d8 < kDv / 8) {
          const int pos = vt_pos(t);
#pragma unroll
          for (int e = 0; e < 8; ++e) s.vt[d8 * 8 + e][pos] = o[e];
        }
      }
      __syncthreads();

      // 2. scores S^T[token][head]: lane (head lr, k-group lg) gets tokens
      //    16 tt + 4 lg + r
      f32x4 sc[NHT][2];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) sc[ht][0] = sc[ht][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) {
          const bf16x8 ka = lds_read8(&s.kn[16 * tt + lr][32 * ks + 8 * lg]);
#pragma unroll
          for (int ht = 0; ht < NHT; ++ht)
            sc[ht][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[ht][ks], sc[ht][tt], 0, 0, 0);
        }
      }

      // 3. online softmax per head column (log2 units)
      bf16x8 pa[NHT];
      bool grew = false;
      float mnew[NHT];
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        float mx = kNoMax;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tok = 16 * tt + 4 * lg + r;
            float v = sc[ht][tt][r] * qscale;
            v = tok < n_valid ? v : -INFINITY;
            sc[ht][tt][r] = v;
            mx = fmaxf(mx, v);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        mnew[ht] = fmaxf(m[ht], mx);
        grew |= mnew[ht] > m[ht];
      }
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(grew) != 0, 0)) {
        // output rows are heads 4 lg + r of the tile: fetch their factors
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
          const float alpha = __builtin_amdgcn_exp2f(m[ht] - mnew[ht]);
          l[ht] *= alpha;
          float ar[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * lg + r);
#pragma unroll
          for (int vt = 0; vt < kVt; ++vt)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[ht][vt][r] *= ar[r];
          m[ht] = mnew[ht];
        }
      }
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        float sum = 0.f;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = __builtin_amdgcn_exp2f(sc[ht][tt][r] - m[ht]);
            sum += p;
            pa[ht][4 * tt + r] = (__bf16)p;
          }
        sum += __shfl_xor(sum, 16);
        sum += __shfl_xor(sum, 32);
        l[ht] += sum;
      }

      // 4. O[head][v] += P[head][token] V[token][v]
#pragma unroll
      for (int vt = 0; vt < kVt; ++vt) {
        const bf16x8 vb = lds_read8(&s.vt[16 * vt + lr][8 * lg]);
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht)
          acc[ht][vt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[ht], vb, acc[ht][vt], 0, 0, 0);
      }
    }

    // partial for slot (workgroup + sequence): lane holds heads 4 lg + r of
    // each tile, value column 16 vt + lr
    const long long slotp = (long long)w + b;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int hbase = hg0 + (wave * NHT + ht) * 16;
#pragma unroll
      for (int vt = 0; vt < kVt; ++vt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          a.ws_o[(slotp * HQ + hbase + 4 * lg + r) * kDv + 16 * vt + lr] = acc[ht][vt][r];
      if (lg == 0) {
        a.ws_ml[(slotp * HQ + hbase + lr) * 2] = m[ht];
        a.ws_ml[(slotp * HQ + hbase + lr) * 2 + 1] = l[ht];
      }
    }
  }
}

template <int NW, int NHT>
hipError_t launch_nw(const DecodeArgs& a, hipStream_t stream) {
  const size_t lds = sizeof(MlaLds);  // above the 64 KiB default: opt in
  hipError_t e = hipFuncSetAttribute((const void*)decode_mla_kernel<NW, NHT>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int groups = a.hq / (16 * NHT * NW);
  hipLaunchKernelGGL((decode_mla_kernel<NW, NHT>), dim3(a.nwg, groups), dim3(64 * NW), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

bool mla_supported(const Geom& g, int hq, int v_dim) {
  if (g.nt != 1 || g.H != 1 || g.D != kD || v_dim != kDv) return false;
  if (g.T % kTile != 0 || g.T > 256) return false;
  return hq == 16 || hq == 32 || hq == 64 || hq == 128;
}

hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t stream) {
  switch (a.hq) {
    case 128: return launch_nw<4, 1>(a, stream);
    case 64: return launch_nw<4, 1>(a, stream);
    case 32: return launch_nw<2, 1>(a, stream);
    case 16: return launch_nw<1, 1>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvfp4
