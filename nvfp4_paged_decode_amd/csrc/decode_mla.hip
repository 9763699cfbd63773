// Paged NVFP4 decode attention, MLA path on MFMA: one 576-value latent per
// token (512 + 64 rope, all NVFP4), values = the first 512 dims of the same
// latent, up to 128 query heads, pages a multiple of 32 tokens.
//
// "Accelerating Long-Context and Agentic Inference with NVFP4 KV Cache",
// NVFP4 KV Decode Attention Kernel Implementation / Figure 3: packed tiles
// and their E4M3 scales are staged, unpacked and scaled, and both attention
// products run as 16-bit matrix products with the tensor scale applied as a
// scalar.  With up to 128 query heads over one latent the products are real
// dense contractions (about 820 flop per cache byte at 128 heads), so they
// run on v_mfma_f32_16x16x32_f16 with fp32 accumulation.
//
// 16-bit format: E2M1 x E4M3 has at most 6 significant bits in [2^-10,
// 2688], exact in fp16; the converter decodes E2M1 codes exactly (scale
// 1.0) and one v_pk_mul_f16 applies the block scale to two values.  Queries
// are scaled per head by a power of two that puts their largest magnitude
// in [2^14, 2^15) before the fp16 conversion (bf16 significands fit fp16's),
// and the power of two is undone on the fp32 scores.  Probabilities are
// rounded to fp16 for P.V, and the sums add those rounded values.
//
// Workgroup: one CU, all query heads of a page range (the balanced split of
// decode_plan.hpp).  Above 64 heads a wave owns 32 heads (two head blocks of
// 16): its 32 heads x 512 dims of fp32 accumulators take the whole
// accumulation register file, so the workgroup is 4 waves, one per SIMD;
// every K and V^T fragment a wave reads from LDS then feeds both head
// blocks, which halves the LDS reads per flop (the bound at 16 heads a
// wave).  Up to 64 heads a wave owns 16.
// Per 32-token tile:
//  1. the workgroup dequantizes the tile once into LDS in its natural
//     [token][576] layout (16-byte chunks XOR-swizzled by token bit 2,
//     which keeps the row reads, the transposed reads and the staging
//     writes free of bank conflicts); tiles are double-buffered, packed
//     bytes are requested two tiles ahead, and the staging work is spread
//     between the score products;
//  2. scores S^T = K Q^T per 16 tokens: A = latent rows read from LDS (16
//     bytes per lane), B = the wave's queries (the first head block's in
//     registers, the second's in LDS); lane (column c, group g) receives
//     rows 4g..4g+3 of head c.  These products use ordinary VGPRs (issued
//     through inline asm), since the accumulators fill the accumulation
//     registers;
//  3. softmax without rescaling: a column's maximum is fixed by its first
//     tile and later probabilities 2^(s - m) are used as they are (fp16
//     holds them up to 65504); if any column's sum ends a segment
//     non-finite, the workgroup votes for a second pass that finds every
//     column's maximum and a third that repeats the first with it;
//  4. O^T += V^T P^T over all 32 tokens at once: the B operand is exactly
//     the lane's own 8 probabilities (rows 4g..4g+3 of both 16-token
//     halves), and the A operand (V^T) comes from the same natural tile
//     through ds_read_b64_tr_b16 (4 tokens of one dim per lane), so no
//     transposed copy is made.
// The wave's unnormalized partial (O, max, sum) goes to workspace slot
// (workgroup + sequence); merge_balanced_kernel combines them.
#include <type_traits>

#include "common.hpp"
#include "decode_plan.hpp"

namespace kvfp4 {

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 576;            // latent dims per token (keys)
constexpr int kDv = 512;           // value dims (latent prefix)
constexpr int kTile = 32;          // tokens per tile
constexpr int kKs = kD / 32;       // 18 k-steps of the score product
constexpr int kDt = kDv / 16;      // 32 value-dim tiles of the output
constexpr int kBlocks = kD / 16;   // NVFP4 blocks per latent row
constexpr int kPitch = 592;        // fp16 per staged row (296 dwords = 8 mod 32 banks)
constexpr int kRowData = kD / 2, kRowScale = kD / 16;  // packed bytes per row
constexpr float kNoMax = -1e30f;
constexpr float kLog2e = 1.4426950408889634f;
#ifndef KVFP4_MLA_KA
#define KVFP4_MLA_KA 2
#endif
#ifndef KVFP4_MLA_VA
#define KVFP4_MLA_VA 3
#endif
#ifndef KVFP4_MLA_PVSB  // 1: a scheduling barrier after each P.V dim tile
#define KVFP4_MLA_PVSB 1
#endif
#ifndef KVFP4_MLA_PVSPLIT  // 1: P.V of head block 0, then of head block 1
#define KVFP4_MLA_PVSPLIT 0
#endif
constexpr int kKAhead = KVFP4_MLA_KA;  // k-steps of K fragments read ahead of the products
constexpr int kVAhead = KVFP4_MLA_VA;  // dim tiles of V^T fragments read ahead

struct MlaLds {
  _Float16 k[2][kTile][kPitch];  // double-buffered natural latent tiles
  int vote[8];                   // per wave: a head of its segment needs a second pass
};
// With 32 heads a wave the second head block's query fragments sit in LDS
// (each wave reads only its own): registers hold the first block's queries
// and the accumulators.
struct MlaLds2 {
  MlaLds t;
  f16x8 q1[4][kKs][64];  // [wave][k-step][lane]
};

// Partial-output staging (after a segment's passes, in the tile buffers):
// each wave 16 rows of kCh fp32 dims at a time, pitch kCh + 4 (the widest
// power-of-two chunk whose NW waves' rows fit).
template <int NW>
struct OutStage {
  static constexpr int kBuf = (int)sizeof(_Float16) * 2 * kTile * kPitch;
  static constexpr int fits(int ch) { return NW * 16 * (ch + 4) * 4 <= kBuf; }
  static constexpr int kCh = fits(512) ? 512 : fits(256) ? 256 : 128;
  static_assert(fits(kCh), "staging rows fit the tile buffers");
};

// Swizzle of staged row `row`: 16-byte chunk c sits at chunk c ^ swz(row).
// LDS has 32 banks of 4 bytes; with the pitch at 8 banks mod 32, rows r
// and r + 4 would collide for 16-byte accesses of 8 lanes, which the flip
// of chunk bit 0 on rows 4..7 (mod 8) separates.
__device__ inline int swz(int row) { return (row >> 2) & 1; }

// Physical fp16 index of chunk `chunk` (8 fp16) of staged row `row`.
__device__ inline int chunk_at(int row, int chunk) {
  return row * kPitch + ((chunk ^ swz(row)) << 3);
}

__device__ inline f16x2 fp4x2(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  }
}

// 8 values of dword w times their block scale (exact in fp16).
__device__ inline f16x8 dequant8(uint32_t w, _Float16 sb) {
  const f16x2 s2 = {sb, sb};
  const f16x2 a = fp4x2(w, 0) * s2, b = fp4x2(w, 1) * s2;
  const f16x2 c = fp4x2(w, 2) * s2, d = fp4x2(w, 3) * s2;
  return (f16x8){a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Score products of the 32-heads-a-wave layout.  The compiler selects one
// register form for every MFMA of a kernel; with the 256 output accumulators
// holding the whole accumulation register file, the score chains must use
// ordinary VGPRs, so they are issued here with VGPR operands.  A chain's
// first product takes a zero accumulator; the products of one chain are
// always four MFMAs apart (four chains interleaved), and mfma_settle pads
// the last product's result before any other instruction reads it (19 wait
// states cover the VALU-read latency of an 8-pass XDL product).
__device__ inline f32x4 mfma_v0(const f16x8& a, const f16x8& b) {
  f32x4 d;
  asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ inline void mfma_v(f32x4& c, const f16x8& a, const f16x8& b) {
  asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ inline void mfma_settle(f32x4& a, f32x4& b, f32x4& c, f32x4& d) {
  asm("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

__device__ inline f16x4 lds_read_tr(const _Float16* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(f16x4, r);
}

// A tile holds kTile x 2 kBlocks = 2304 half-blocks (4 data bytes and the
// block's scale byte each); thread tid stages half-blocks tid, tid + NT,
// ...  Half-block i is chunk i % 72 of token row i / 72: its data bytes sit
// at 4 i in the tile's data rows and its scale byte at i / 2, so a wave's
// loads cover contiguous bytes, and the 8 lanes of each 16-byte LDS store
// write 8 consecutive chunks of one row (distinct banks).
constexpr int kHalf = kTile * 2 * kBlocks;  // half-blocks per tile
template <int NW>
struct Prefetch {
  // half-blocks per thread (an equal share for 1, 2, 3, 4 and 6 waves;
  // otherwise the last round is partial)
  static constexpr int kPer = (kHalf + 64 * NW - 1) / (64 * NW);
  static constexpr bool kEven = kHalf % (64 * NW) == 0;
  uint32_t d[kPer];
  uint32_t s[kPer];
};

// HB head blocks of 16 per wave.  With HB = 2 (more than 64 heads) every K
// and V^T fragment a wave reads from LDS feeds two products, which halves
// the LDS traffic per flop -- the kernel's bound at 16 heads a wave -- and
// the wave's 32 heads x 512 dims of fp32 accumulators (256 registers) take
// the whole accumulation register file, so the kernel runs one wave per
// SIMD (4 waves, 512 registers each).
template <int NW, int HB>
__global__ __launch_bounds__(64 * NW) void decode_mla_kernel(DecodeArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int kPer = Prefetch<NW>::kPer;
  constexpr int HW = 16 * HB;  // heads per wave
  extern __shared__ __align__(16) unsigned char smem[];
  MlaLds& st = *reinterpret_cast<MlaLds*>(smem);
  const Geom g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;  // head column (or token row), k-group
  const int nwg = gridDim.x, w = split_index(blockIdx.x, nwg);  // position in the split
  const float base_scale = a.softmax_scale * a.gs_k * kLog2e;
  const long long page_bytes = g.packed_bytes(), data_bytes = g.data_bytes();
  const int tiles_per_page = g.T / kTile;

  // score A operand of token half tt: lane (row = token 16 tt + col,
  // k-group grp) reads chunk 4 ks + grp of its row (ks adds 32 fp16)
  int nat_off[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int row = 16 * tt + col;
    nat_off[tt] = row * kPitch + 8 * (grp ^ swz(row));
  }
  // transposed reads: in 16-lane subgroup grp, source lane 4q + j reads row
  // 16 h + 4 grp + q, dims 16 dt + 4 j (the row swizzle is constant within
  // the subgroup and only swaps the two chunks of a dim tile)
  const int q4 = (lane & 15) >> 2, j4 = lane & 3;
  const int sw = swz(4 * grp);
  int tr_off[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 16 * h + 4 * grp + q4;
    tr_off[h] = row * kPitch + 8 * ((j4 >> 1) ^ sw) + 4 * (j4 & 1);
  }
  // LDS element offset of each of this thread's staging rounds (see
  // stage_piece below)
  int st_off[Prefetch<NW>::kPer];
#pragma unroll
  for (int u = 0; u < Prefetch<NW>::kPer; ++u) {
    const unsigned hi = tid + NT * u, t = hi / (2 * kBlocks);
    st_off[u] = chunk_at((int)t, (int)(hi - t * (2 * kBlocks)));
  }

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
    // tile indices within the sequence (32-bit: a sequence holds at most
    // 2^31 tokens); tile t is tile t % tiles_per_page of page t / tiles_per_page
    const int t_lo = (int)p_lo * tiles_per_page;
    int t_hi = (int)p_hi * tiles_per_page;
    const int t_end = (L + kTile - 1) / kTile;
    if (t_hi > t_end) t_hi = t_end;

    // Page-table entries are read with scalar loads (a uniform address in
    // the constant address space): their wait is then on the scalar/LDS
    // counter, not on the vector-memory counter that also tracks the tile
    // loads, so reading an entry never waits for tiles in flight.  A page's
    // entry is requested one request ahead of its use.
    typedef __attribute__((address_space(4))) const int32_t* ConstI32;
    const ConstI32 bt_row = (ConstI32)(a.block_table + (long long)b * a.max_pages);
    auto slot_load = [&](int pg) -> int {  // -1 past the segment
      const int e = bt_row[pg < (int)p_hi ? pg : (int)p_hi - 1];
      return pg < (int)p_hi ? e : -1;
    };
    auto rows_of = [&](int slot, int ti) -> int {
      int n = L - ti * kTile;
      n = n > kTile ? kTile : n;
      if (slot < 0 || slot >= a.pool_pages) n = 0;
      return n < 0 ? 0 : n;
    };

    // Packed bytes of tile t are requested two tiles ahead, into one of two
    // register sets, and staged into LDS (dequantized) while tile t - 1 is
    // being scored; rows past the sequence end (or a whole tile of a bad
    // page) read as zero through the buffer resources' bounds.
    Prefetch<NW> pre[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int u = 0; u < kPer; ++u) pre[i].d[u] = pre[i].s[u] = 0u;
    // the next tile to request, as (page, tile within the page), and the
    // page's slot; tiles past the segment get slot -1 (no rows: the loads
    // read zero and fetch nothing), so the request is made every tile
    int nx_pg = (int)p_lo, nx_tip = 0, nx_slot = -1;
    auto issue = [&](Prefetch<NW>& pf, int ti) -> int {
      const int slot = nx_slot;
      const int n = rows_of(slot, ti);
      const int row0 = nx_tip * kTile;
      if (++nx_tip == tiles_per_page) {
        nx_tip = 0;
        ++nx_pg;
        nx_slot = slot_load(nx_pg);
      }
      const uint8_t* page = a.pool + (long long)(n > 0 ? slot : 0) * page_bytes;
      auto rd = __builtin_amdgcn_make_buffer_rsrc((void*)(page + (long long)row0 * kRowData),
                                                  (short)0, n * kRowData, 0x00020000);
      auto rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(page + data_bytes + (long long)row0 * kRowScale), (short)0, n * kRowScale,
          0x00020000);
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        // the round's constant part goes in the scalar offset; a half-block
        // past the tile (partial last round) reads past the buffer's range:
        // zero, nothing fetched
        const int hi = tid + NT * u;
        const bool in = Prefetch<NW>::kEven || hi < kHalf;
        pf.d[u] = __builtin_amdgcn_raw_buffer_load_b32(rd, in ? 4 * tid : 1 << 28, 4 * NT * u, 0);
        pf.s[u] = __builtin_amdgcn_raw_buffer_load_b8(rs, in ? tid >> 1 : 1 << 28, NT * u / 2, 0);
      }
      return n;
    };
    // Staging of half-block round u of the tile held in pf into LDS buffer
    // buf.  Round u of this thread is chunk c of row t with (t, c) =
    // divmod(tid + NT u, 72): its LDS offset is computed once per
    // workgroup (st_off).  The work of one round is split into pieces 0..5
    // so that the score loop can spread it between its MFMAs: 0 the block
    // scale, 1..4 a pair of codes each, 5 the 16-byte store.
    struct Stager {
      _Float16 sb;
      f16x8 v;
    };
    auto stager_start = [&]() -> Stager { return Stager{}; };
    auto stage_piece = [&](const Prefetch<NW>& pf, int u, int piece, int buf, Stager& g) {
      if (!Prefetch<NW>::kEven && tid + NT * u >= kHalf) return;
      if (piece == 0) {
        const f16x2 sp = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(pf.s[u], 1.0f, false);
        g.sb = sp[0];
      } else if (piece <= 4) {
        const f16x2 s2 = {g.sb, g.sb};
        const f16x2 h = fp4x2(pf.d[u], piece - 1) * s2;
        g.v[2 * (piece - 1)] = h.x;
        g.v[2 * (piece - 1) + 1] = h.y;
      } else {
        *reinterpret_cast<f16x8*>(&st.k[buf][0][0] + st_off[u]) = g.v;
      }
    };
    auto stage_one = [&](const Prefetch<NW>& pf, int u, int buf, Stager& g) {
#pragma unroll
      for (int piece = 0; piece < 6; ++piece) stage_piece(pf, u, piece, buf, g);
    };

    // queries of this wave's heads (B operand of the scores): for head block
    // hb, lane (column c, group g) holds dims 32 ks + 8 g .. +8 of head
    // HW wave + 16 hb + c
    f16x8 qb[kKs];  // head block 0 (head block 1: LDS)
    float qs[HB];
    MlaLds2& st2 = *reinterpret_cast<MlaLds2*>(smem);
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int head = HW * wave + 16 * hb + col;
      const bool head_ok = head < a.hq;
      const uint16_t* qrow = a.q + ((long long)b * a.hq + (head_ok ? head : 0)) * kD + 8 * grp;
      u32x4 raw[kKs];
      uint32_t mb = 0;
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) raw[ks] = *reinterpret_cast<const u32x4*>(qrow + 32 * ks);
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mb = max(mb, raw[ks][e] & 0x7FFFu);
          mb = max(mb, (raw[ks][e] >> 16) & 0x7FFFu);
        }
      mb = max(mb, (uint32_t)__shfl_xor((int)mb, 16));
      mb = max(mb, (uint32_t)__shfl_xor((int)mb, 32));
      int sh = 0;
      if (mb != 0) {
        int e;
        frexpf(__uint_as_float(mb << 16), &e);  // amax < 2^e
        sh = 15 - e;
      }
      const int shq = head_ok ? sh : -200;  // padding columns: exactly 0
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) {
        f16x8 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = (_Float16)ldexpf(__uint_as_float(raw[ks][e] << 16), shq);
          v[2 * e + 1] = (_Float16)ldexpf(__uint_as_float(raw[ks][e] & 0xFFFF0000u), shq);
        }
        if (hb == 0)
          qb[ks] = v;
        else
          st2.q1[wave][ks][lane] = v;
      }
      qs[hb] = ldexpf(base_scale, -sh);
    }

    // Softmax without rescaling the accumulators.  Pass 0: a column's
    // maximum m is fixed by its first tile with a valid token, and the
    // probabilities 2^(s - m) of later tiles are used as they are; fp16
    // holds them up to 65504, and a larger one becomes inf, which makes the
    // column's sum l non-finite.  If any column of the workgroup ends the
    // pass so, pass 1 computes only the scores and the maximum of every
    // column over the segment, and pass 2 repeats pass 0 with that maximum,
    // where no probability exceeds 1.  The accumulators are therefore only
    // ever zeroed or written by MFMA.
    f32x4 acc[HB][kDt];
    float m[HB], l[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) m[hb] = kNoMax;
    for (int mode = 0;;) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
      for (int dt = 0; dt < kDt; ++dt) acc[hb][dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
      l[hb] = 0.f;
      if (mode == 1) m[hb] = kNoMax;
    }
    nx_pg = (int)p_lo;
    nx_tip = 0;
    nx_slot = slot_load(nx_pg);
    int n_cur = issue(pre[0], t_lo);
    int n_nxt = issue(pre[1], t_lo + 1);
    {
      Stager g = stager_start();
#pragma unroll
      for (int u = 0; u < kPer; ++u) stage_one(pre[0], u, 0, g);
    }
    __syncthreads();

    // One tile: `nextp` holds the next tile's bytes (staged into the other
    // buffer during the score products), `freep` receives the tile after it.
    auto tile = [&](int ti, Prefetch<NW>& nextp, Prefetch<NW>& freep, auto buf_c) {
      constexpr int buf = decltype(buf_c)::value;  // LDS buffer of this tile
      const int n_nn = issue(freep, ti + 2);
      const _Float16* kb = &st.k[buf][0][0];
      Stager g = stager_start();

      // scores S^T[token][head] per 16-token half and head block; each K
      // fragment read from LDS feeds every head block.  Reads run kKAhead
      // k-steps ahead of the products through a small ring; the next tile's
      // staging is spread over the k-steps (a round of half-blocks every
      // k-step or two), so its VALU work runs while the MFMAs do; the
      // scheduling barriers keep that interleave and stop the compiler from
      // hoisting all 36 reads, which spills.
      f32x4 sc[HB][2];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) sc[hb][0] = sc[hb][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
      {
        // fragment ring: [0..1] K of the two token halves, [2] head block
        // 1's queries
        f16x8 kf[kKAhead + 1][HB + 1];
        auto kread = [&](int ks, f16x8 (&dst)[HB + 1]) {
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
            dst[tt] = *reinterpret_cast<const f16x8*>(kb + nat_off[tt] + 32 * ks);
          if (HB == 2) dst[HB] = st2.q1[wave][ks][lane];
        };
#pragma unroll
        for (int ks = 0; ks < kKAhead; ++ks) kread(ks, kf[ks]);
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) {
          if (ks + kKAhead < kKs) kread(ks + kKAhead, kf[(ks + kKAhead) % (kKAhead + 1)]);
          const int r = ks % (kKAhead + 1);
          if constexpr (HB == 2 && kPer * 2 == kKs) {
            // one staging round every two k-steps, its six pieces placed
            // after the first six of the eight products, each MFMA and its
            // piece in a scheduling group of their own (the VALU piece then
            // issues while the MFMA runs)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int tt = i >> 1, hb = i & 1;
              const f16x8& qf = hb == 0 ? qb[ks] : kf[r][HB];
              if (ks == 0)
                sc[hb][tt] = mfma_v0(kf[r][tt], qf);
              else
                mfma_v(sc[hb][tt], kf[r][tt], qf);
              const int piece = 4 * (ks & 1) + i;
              if (piece < 6) stage_piece(nextp, ks >> 1, piece, buf ^ 1, g);
              __builtin_amdgcn_sched_barrier(0);
            }
          } else {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
              for (int hb = 0; hb < HB; ++hb) {
                const f16x8& qf = hb == 0 ? qb[ks] : kf[r][HB];
                if (HB == 1)
                  sc[hb][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[r][tt], qf, sc[hb][tt],
                                                                      0, 0, 0);
                else if (ks == 0)
                  sc[hb][tt] = mfma_v0(kf[r][tt], qf);
                else
                  mfma_v(sc[hb][tt], kf[r][tt], qf);
              }
            // rounds [ks kPer / kKs, (ks + 1) kPer / kKs) of the next tile
#pragma unroll
            for (int u = ks * kPer / kKs; u < (ks + 1) * kPer / kKs; ++u)
              stage_one(nextp, u, buf ^ 1, g);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        if (HB == 2) mfma_settle(sc[0][0], sc[0][1], sc[HB - 1][0], sc[HB - 1][1]);
      }

      // softmax of each head column over rows 16 tt + 4 grp + r.  A column
      // maximum is needed on every tile of pass 1, and in passes 0 and 2 on
      // the tiles until a column has seen a valid token (rare: first).
      const bool full = n_cur >= kTile;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        if (mode == 1 || __builtin_amdgcn_ballot_w64(m[hb] == kNoMax) != 0) {
          float mx = kNoMax;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int tok = 16 * (e >> 2) + 4 * grp + (e & 3);
            if (tok < n_cur) mx = fmaxf(mx, sc[hb][e >> 2][e & 3] * qs[hb]);
          }
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          m[hb] = (mode == 1 || m[hb] == kNoMax) ? fmaxf(m[hb], mx) : m[hb];
        }
      }

      // P.V: O^T[dim][head] += V^T P^T over the 32 tokens, head block 0 then
      // head block 1 (each V^T fragment is read once per head block; LDS has
      // the bandwidth), so that head block 1's probabilities are computed
      // between head block 0's products, beside its MFMAs.  Fragments are
      // read kVAhead dim tiles ahead.
      if (mode != 1) {
        f16x8 pb[HB];
        const f16x2 one2 = {(_Float16)1.f, (_Float16)1.f};
        // probabilities e, e + 1 of head block hb: 2^(s - m) rounded to fp16
        auto probs = [&](int hb, int e, bool partial) {
          float x0 = fmaf(sc[hb][e >> 2][e & 3], qs[hb], -m[hb]);
          float x1 = fmaf(sc[hb][e >> 2][(e & 3) + 1], qs[hb], -m[hb]);
          if (partial) {
            const int tok = 16 * (e >> 2) + 4 * grp + (e & 3);
            x0 = tok < n_cur ? x0 : -INFINITY;
            x1 = tok + 1 < n_cur ? x1 : -INFINITY;
          }
          const f16x2 p2 = {(_Float16)__builtin_amdgcn_exp2f(x0),
                            (_Float16)__builtin_amdgcn_exp2f(x1)};
          pb[hb][e] = p2.x;
          pb[hb][e + 1] = p2.y;
          // the denominator sums the fp16-rounded values P.V multiplies
          l[hb] = __builtin_amdgcn_fdot2(p2, one2, l[hb], false);
        };
        // (a uniform branch: the masking of rows past the sequence end only
        // on the sequence's last tile)
        if (full) {
#pragma unroll
          for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int e = 0; e < 8; e += 2) probs(hb, e, false);
        } else {
#pragma unroll
          for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int e = 0; e < 8; e += 2) probs(hb, e, true);
        }
        f16x8 vf[kVAhead + 1];
        auto vread = [&](int dt) -> f16x8 {
          const f16x4 lo = lds_read_tr(kb + tr_off[0] + 16 * dt);
          const f16x4 hi = lds_read_tr(kb + tr_off[1] + 16 * dt);
          return (f16x8){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        };
        if (KVFP4_MLA_PVSPLIT) {
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
            for (int dt = 0; dt < kVAhead; ++dt) vf[dt] = vread(dt);
#pragma unroll
            for (int dt = 0; dt < kDt; ++dt) {
              if (dt + kVAhead < kDt) vf[(dt + kVAhead) % (kVAhead + 1)] = vread(dt + kVAhead);
              acc[hb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  vf[dt % (kVAhead + 1)], pb[hb], acc[hb][dt], 0, 0, 0);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        } else {
#pragma unroll
          for (int dt = 0; dt < kVAhead; ++dt) vf[dt] = vread(dt);
#pragma unroll
          for (int dt = 0; dt < kDt; ++dt) {
            if (dt + kVAhead < kDt) vf[(dt + kVAhead) % (kVAhead + 1)] = vread(dt + kVAhead);
#pragma unroll
            for (int hb = 0; hb < HB; ++hb)
              acc[hb][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  vf[dt % (kVAhead + 1)], pb[hb], acc[hb][dt], 0, 0, 0);
            if (KVFP4_MLA_PVSB) __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      // every wave is done with this tile's buffer, and the next tile is
      // staged in the other
      __syncthreads();
      n_cur = n_nxt;
      n_nxt = n_nn;
    };
    for (int ti = t_lo; ti < t_hi; ti += 2) {
      tile(ti, pre[1], pre[0], std::integral_constant<int, 0>{});
      if (ti + 1 < t_hi) tile(ti + 1, pre[0], pre[1], std::integral_constant<int, 1>{});
    }
    if (mode == 1) {
      mode = 2;
      continue;
    }
    if (mode == 2) break;
    // pass 0 done: a workgroup-wide vote on whether any column overflowed
    // (every wave takes the same branch; the next pass starts after this
    // barrier, when every wave is done with both tile buffers)
    bool bad = false;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) bad = bad || !(fabsf(l[hb]) <= 3.0e38f);
    const bool wave_bad = __builtin_amdgcn_ballot_w64(bad) != 0;  // all lanes vote
    if (lane == 0) st.vote[wave] = wave_bad;
    __syncthreads();
    bool again = false;
#pragma unroll
    for (int i = 0; i < NW; ++i) again = again || st.vote[i] != 0;
    if (!again) break;
    mode = 1;
    }

    // Partial for slot (workgroup + sequence), divided by its sum, in fp16.
    // Lane (col, grp) holds head `col` of each head block, dims 16 dt +
    // 4 grp + 0..3 in acc[hb][dt].  The accumulators go through LDS (each
    // wave its own rows of the free tile buffers, kOutCh dims of 16 heads at
    // a time) so that every global store writes 16 bytes of one head row and
    // whole lines, and so that the accumulators are only stored, never
    // operands of vector ALU work, which keeps them in the accumulation
    // registers through the tile loop.
    constexpr int kOutCh = OutStage<NW>::kCh, kOutPitch = kOutCh + 4;
    __syncthreads();  // every wave is done with the tile buffers
    float* const ob = reinterpret_cast<float*>(smem) + wave * (16 * kOutPitch);
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      float lt = l[hb];
      lt += __shfl_xor(lt, 16);
      lt += __shfl_xor(lt, 32);
      const float il = lt > 0.f ? 1.f / lt : 0.f;  // lane col: head col's
      const int head0 = HW * wave + 16 * hb;
      if (grp == 0 && head0 + col < a.hq) {
        const long long slotp = ((long long)w + b) * a.hq + head0 + col;
        a.ws_ml[slotp * 2] = m[hb];
        a.ws_ml[slotp * 2 + 1] = lt;
      }
#pragma unroll
      for (int ch = 0; ch < kDv / kOutCh; ++ch) {
#pragma unroll
        for (int dt = 0; dt < kOutCh / 16; ++dt)
          *reinterpret_cast<f32x4*>(ob + col * kOutPitch + 16 * dt + 4 * grp) =
              acc[hb][ch * (kOutCh / 16) + dt];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // lane: 8 dims of row (16 heads x kOutCh dims, kOutCh / 8 lanes a row)
        constexpr int kLanesRow = kOutCh / 8, kRowsIt = 64 / kLanesRow;
#pragma unroll
        for (int r0 = 0; r0 < 16; r0 += kRowsIt) {
          const int r = r0 + lane / kLanesRow, c8 = 8 * (lane % kLanesRow);
          const float ilr = __shfl(il, r);
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(ob + r * kOutPitch + c8);
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(ob + r * kOutPitch + c8 + 4);
          if (head0 + r < a.hq) {
            const long long slotp = ((long long)w + b) * a.hq + head0 + r;
            const u32x2 h0 = pack_f16x4(x0 * ilr), h1 = pack_f16x4(x1 * ilr);
            *reinterpret_cast<u32x4*>(a.ws_oh + slotp * kDv + ch * kOutCh + c8) =
                (u32x4){h0.x, h0.y, h1.x, h1.y};
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
    __syncthreads();  // the tile buffers hold the next segment's tiles again
  }
}

template <int NW, int HB>
hipError_t launch_nw(const DecodeArgs& a, hipStream_t stream) {
  const size_t lds = HB == 2 ? sizeof(MlaLds2) : sizeof(MlaLds);  // above 64 KiB: opt in
  static std::atomic<unsigned long long> lds_set{0};
  hipError_t e = allow_lds_once(lds_set, (const void*)decode_mla_kernel<NW, HB>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_mla_kernel<NW, HB>), dim3(a.nwg), dim3(64 * NW), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

bool mla_supported(const Geom& g, int hq, int v_dim) {
  if (g.nt != 1 || g.H != 1 || g.D != kD || v_dim != kDv) return false;
  if (g.T % kTile != 0 || g.T > 4096) return false;
  return hq >= 1 && hq <= 128;
}

hipError_t launch_decode_mla(const DecodeArgs& a, hipStream_t stream) {
  if (!mla_supported(a.g, a.hq, a.v_dim) || a.nwg <= 0) return hipErrorInvalidValue;
  if (((uintptr_t)a.ws_oh & 15) != 0 || ((uintptr_t)a.q & 15) != 0) return hipErrorInvalidValue;
  // up to 64 heads: 16 a wave (one to four waves); more: 32 a wave (four;
  // eight waves of 16 heads, whose fragments then feed one head block each,
  // spill and took 875 against 285 us on 128 heads)
  if (a.hq > 64) return launch_nw<4, 2>(a, stream);
  switch ((a.hq + 15) / 16) {
    case 1: return launch_nw<1, 1>(a, stream);
    case 2: return launch_nw<2, 1>(a, stream);
    case 3: return launch_nw<3, 1>(a, stream);
    default: return launch_nw<4, 1>(a, stream);
  }
}

}  // namespace kvfp4
