// Paged NVFP4 decode attention on MFMA for 1 to 16 query heads per KV head
// (padded to 4, 8 or 16 query columns: the padding columns hold zero
// queries and are never written) and 1 to 32 KV heads (padded to a multiple
// of 4: the padding slots load zeros and fetch nothing), head_dim 64 or
// 128, pages a multiple of 16 tokens.
//
// "Accelerating Long-Context and Agentic Inference with NVFP4 KV Cache",
// NVFP4 KV Decode Attention Kernel Implementation / Figure 3: packed K/V
// tiles and their E4M3 block scales are read from the cache, unpacked and
// scaled in registers, both attention products run as 16-bit matrix
// products with fp32 accumulation, and the tensor scales act as scalars.
// Decode is memory-read-bound (same page, Path 3: Decode): the kernel is
// built so that its per-value instruction count stays well under what
// streaming the cache at full HBM rate leaves.
//
// Why MFMA with 4 query heads.  On VALU every cached value costs one FMA
// per query head (4 per value) on top of its dequantization, which keeps
// the VALU busy for longer than HBM takes to deliver the bytes.  Here a
// wave takes 4 KV heads at once: one v_mfma_f32_16x16x32_f16 multiplies 16
// (token, KV head) rows of K by the 16 query columns of those 4 KV heads,
// and each lane keeps the quarter of the products whose row and column
// share a KV head (the MFMA has compute to spare; the other three quarters
// are discarded).
//
// Load layout.  A tile's K (and V) rows of the wave's 4 KV heads are read in
// 4 rounds of 4 tokens; in round j, lane (4a + b) + 16p takes quarter p of
// the row of token 4j + a, KV-head slot b, which is exactly its A operand
// (row 4a + b, k-group p).  Each load instruction therefore covers 4 whole
// token rows of the 4 KV heads, i.e. whole 128-byte lines, so the loads are
// non-temporal (streaming) without any line being fetched twice; a row-per-
// lane layout spreads each line over 4 instructions and streams about 30 %
// slower.
//
// 16-bit format.  E2M1 x E4M3 has at most 6 significant bits and lies in
// [2^-10, 2688]: exact in fp16 (normal range), so the dequantized values
// are exact; gfx950 converts E2M1 codes exactly to fp16 pairs
// (v_cvt_scalef32_pk_f16_fp4 with scale 1.0; its scale operand applies
// only a power of two, so it cannot take the E4M3 scale) and one
// v_pk_mul_f16 applies the block scale to two values.  Queries (bf16) are
// scaled per head by a power of two so that their largest magnitude sits
// just under 2^15, then converted to fp16: bf16's 8-bit significands fit
// fp16's 11, so the only loss is for elements 2^-39 of the head's largest
// or smaller.  The power of two is undone on the fp32 scores.
// Probabilities are rounded to fp16 (11 significant bits) for the P.V
// product.
//
// Per 16-token tile of a wave (4 KV heads):
//   scores   round j: A = K rows (token 4j + r/4, KV-head slot r%4), B = the
//            dense query operand (lane (column c, k-group p) holds quarter p
//            of column c's query row, kept in registers per sequence).
//            Lane (c, x) keeps row block c/4 of its column: the score of
//            token 4j + x, for j = 0..3.
//   softmax  online per column, running max shared by the column's 4
//            lanes; the accumulators are rescaled only when a tile's
//            maximum exceeds the running one by more than 2^8.
//   P.V      O^T = V^T P^T.  V rows are dequantized by the lanes that load
//            them and staged in LDS per KV head, token 4j + a at row 4a + j
//            (so that lane (c, x) holds the probabilities of rows
//            4x..4x+3); ds_read_b64_tr_b16 reads them transposed (4 rows
//            of one dim per lane).  Two products per 16 dims: the k-group
//            of KV head g takes rows 4x..4x+3 and 4y..4y+3 (x, y = g + 2m,
//            g + 2m + 1, mod 4, m = 0, 1), whose probabilities sit in lanes
//            (c, x), (c, y) and are fetched with ds_bpermute.
//
// Workgroup: 8 waves = NGT wave groups (groups of 4 KV-head slots x query
// subgroups of 4) x NS = 8 / NGT token streams; stream s takes tiles s,
// s + NS, ... of each sequence segment.
// The balanced split of decode_plan.hpp gives each workgroup a contiguous
// range of the batch's pages; at the end of each sequence segment the
// streams are merged through LDS and the partial goes to workspace slot
// (workgroup + sequence) for merge_balanced_kernel.
#include "common.hpp"
#include "decode_plan.hpp"

namespace kvfp4 {

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 16;     // tokens per tile
constexpr int kWaves = 8;     // waves per workgroup
// fp16 per staged V row for head dim KD: KD/2 + 8 dwords, which is 8 banks
// mod 32 for KD = 64 and 128, so the 16 lanes of a transposed read hit
// distinct banks
template <int KD>
constexpr int pitch_of() { return KD + 16; }
constexpr float kNoMax = -1e30f;
constexpr uint32_t kPastRange = 0x40000000u;  // buffer offset past every tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSlack = 8.f;  // the running max is raised only when a tile's
                               // maximum exceeds it by more than this (log2
                               // units): rescales stay rare, p stays < 2^8

// Tuning knobs (defaults are the measured best): XOR swizzle of staged V
// chunks, two independent accumulation chains for the scores, rotated tile
// order per KV-head group.
#ifndef KVFP4_GQA_ROT
#define KVFP4_GQA_ROT 1
#endif
#ifndef KVFP4_GQA_SWZ
#define KVFP4_GQA_SWZ 1
#endif
#ifndef KVFP4_GQA_SPLIT
#define KVFP4_GQA_SPLIT 1
#endif
#ifndef KVFP4_GQA_BALANCE  // priority to the SIMD's lagging wave
#define KVFP4_GQA_BALANCE 1
#endif
#ifndef KVFP4_GQA_SETS  // register sets of tiles (2: one in flight, 3: two)
#define KVFP4_GQA_SETS 2
#endif
#ifndef KVFP4_GQA_AUX  // cache-policy bits of the K/V data loads: non-temporal
#define KVFP4_GQA_AUX 2
#endif

// fp16 between the staged rows of consecutive KV heads: 16 rows plus 16 fp16
// (8 banks), so the 8 lanes of a 16-byte write that differ in KV head only
// hit distinct banks
template <int KD>
constexpr int head_stride_of() { return kTile * pitch_of<KD>() + 16; }
template <int KD>
struct StageLds {
  _Float16 v[kWaves][4 * head_stride_of<KD>()];  // per wave: 4 KV heads x 16 tokens
};
// floats per merge row: rows 4 banks apart, so the 8 lanes of a 16-byte
// access hit distinct banks
template <int KD>
constexpr int merge_pitch_of() { return KD + 4; }
template <int KD>
struct MergeLds {
  float o[kWaves][16][merge_pitch_of<KD>()];  // per wave: 16 query heads x KD dims
  float ml[kWaves][16][2];   // running max and sum per query head
};
// Staging or merge area, then one progress counter per wave.
template <int KD>
constexpr size_t area_bytes() {
  return sizeof(StageLds<KD>) > sizeof(MergeLds<KD>) ? sizeof(StageLds<KD>)
                                                     : sizeof(MergeLds<KD>);
}
template <int KD>
constexpr size_t lds_bytes() {
  return area_bytes<KD>() + kWaves * sizeof(int);
}

// One lane's packed share of a tile: in each of the 4 load rounds j (tokens
// 4j..4j+3), a quarter of one K row and of one V row (KD/8 bytes each) and
// the scale bytes of that quarter (KD/64 each).
template <int KD>
struct ChunkOf;
template <>
struct ChunkOf<128> {
  typedef u32x4 type;
  typedef uint16_t scale;
};
template <>
struct ChunkOf<64> {
  typedef u32x2 type;
  typedef uint8_t scale;
};
// The scale bytes are kept at their loaded width: widened to 32 bits in the
// register set, the widening (an AND after the load) was placed right after
// the first tile's request and waited for it before the next was requested.
template <int KD>
struct Packed {
  typename ChunkOf<KD>::type k[4], v[4];
  typename ChunkOf<KD>::scale ks[4], vs[4];
};

__device__ inline f16x2 fp4x2(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  }
}

// 8 values of dword w (8 consecutive dims of a row) times their block scale.
__device__ inline f16x8 dequant8(uint32_t w, _Float16 sb) {
  const f16x2 s2 = {sb, sb};
  const f16x2 a = fp4x2(w, 0) * s2, b = fp4x2(w, 1) * s2;
  const f16x2 c = fp4x2(w, 2) * s2, d = fp4x2(w, 3) * s2;
  return (f16x8){a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

__device__ inline _Float16 sp0(f16x2 s) { return s[0]; }
__device__ inline _Float16 sp1(f16x2 s) { return s[1]; }

__device__ inline uint32_t bperm(uint32_t v, int src_lane) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane << 2, (int)v);
}

__device__ inline uint32_t pack_f16(float a, float b) {
  const f16x2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

__device__ inline f16x4 lds_read_tr(const _Float16* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(f16x4, r);
}

// 8 bf16 of a query row (rows are 16-byte aligned: checked at launch).
__device__ inline u32x4 load_q8(const uint16_t* row, int i) {
  return *reinterpret_cast<const u32x4*>(row + 8 * i);
}

// Issues the loads of one lane's share of a tile of a sequence; rows past
// the sequence end (or a whole tile of a bad page, or a request past the
// stream's last tile) come back as zero from the buffer resources' bounds,
// and are never fetched.
struct TileGeom {
  const uint8_t* pool;
  long long page_bytes;
  int pool_pages, T, H, L, tiles_per_page;
  uint32_t off_data, off_scale;  // this lane's offsets in a tile, round 0
  uint32_t js_data, js_scale;    // advance per load round (4 token rows)
};

__device__ inline int tile_rows(const TileGeom& tg, int slot, int ti) {
  int n = tg.L - ti * kTile;
  n = n > kTile ? kTile : n;
  if (slot < 0 || slot >= tg.pool_pages) n = 0;
  return __builtin_amdgcn_readfirstlane(n < 0 ? 0 : n);
}

template <int KD>
__device__ inline void load_tile(Packed<KD>& p, const TileGeom& tg, int slot, int tip, int n) {
  const int row0 = tip * kTile;  // tip: the tile's index within its page
  const int rowb = tg.H * (KD / 2), rows = tg.H * (KD / 16);
  const uint8_t* page = tg.pool + (long long)(n > 0 ? slot : 0) * tg.page_bytes;
  const uint8_t* kd = page + (long long)row0 * rowb;
  const uint8_t* vd = page + (long long)tg.T * rowb + (long long)row0 * rowb;
  const uint8_t* kss = page + 2LL * tg.T * rowb + (long long)row0 * rows;
  const uint8_t* vss = kss + (long long)tg.T * rows;
  auto rk = __builtin_amdgcn_make_buffer_rsrc((void*)kd, (short)0, n * rowb, 0x00020000);
  auto rv = __builtin_amdgcn_make_buffer_rsrc((void*)vd, (short)0, n * rowb, 0x00020000);
  auto rks = __builtin_amdgcn_make_buffer_rsrc((void*)kss, (short)0, n * rows, 0x00020000);
  auto rvs = __builtin_amdgcn_make_buffer_rsrc((void*)vss, (short)0, n * rows, 0x00020000);
  // round j: every load instruction covers 4 whole token rows of the wave
  // group's KV heads (whole cache lines), so the data loads can be
  // non-temporal without a line being fetched twice
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (KD == 128) {
      p.k[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rk, tg.off_data, j * tg.js_data, KVFP4_GQA_AUX));
      p.v[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rv, tg.off_data, j * tg.js_data, KVFP4_GQA_AUX));
      p.ks[j] = __builtin_amdgcn_raw_buffer_load_b16(rks, tg.off_scale, j * tg.js_scale, 0);
      p.vs[j] = __builtin_amdgcn_raw_buffer_load_b16(rvs, tg.off_scale, j * tg.js_scale, 0);
    } else {
      p.k[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                             rk, tg.off_data, j * tg.js_data, KVFP4_GQA_AUX));
      p.v[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                             rv, tg.off_data, j * tg.js_data, KVFP4_GQA_AUX));
      p.ks[j] = __builtin_amdgcn_raw_buffer_load_b8(rks, tg.off_scale, j * tg.js_scale, 0);
      p.vs[j] = __builtin_amdgcn_raw_buffer_load_b8(rvs, tg.off_scale, j * tg.js_scale, 0);
    }
  }
}

// NKG groups of 4 KV heads (H = 4 NKG) and SUB subgroups of 4 query heads
// per KV head (G = 4 SUB query heads per KV head): wave group gt = (kg, sub)
// takes KV heads 4 kg .. 4 kg + 3 and, of each, query heads 4 sub .. +3.
// The SUB groups of one kg read the same K/V rows; their tile walks are
// staggered, so the later ones find the rows in L2.
template <int KD, int NKG, int SUB>
__global__ __launch_bounds__(64 * kWaves) void decode_gqa_mfma_kernel(DecodeArgs a) {
  static_assert(KD == 64 || KD == 128, "head dim 64 or 128");
  using Packed = ::kvfp4::Packed<KD>;
  constexpr int NGT = NKG * SUB;    // wave groups
  constexpr int NS = kWaves / NGT;  // token streams per wave group
  // query heads per KV head: up to 4 SUB; columns past it are padding
  // (zero queries, nothing written)
  const int G = a.hq / a.g.H;
  constexpr int kPitch = pitch_of<KD>();
  extern __shared__ __align__(16) unsigned char smem[];
  StageLds<KD>& st = *reinterpret_cast<StageLds<KD>*>(smem);
  MergeLds<KD>& mg = *reinterpret_cast<MergeLds<KD>*>(smem);
  int* progress = reinterpret_cast<int*>(smem + area_bytes<KD>());  // [kWaves]
  const Geom g = a.g;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int gt = wave / NS, s = wave % NS;
  const int kg = gt % NKG, sub = gt / NKG;
  const int lr = lane & 15, lg = lane >> 4;   // MFMA row/column, k-group
  const bool diag = (lr >> 2) == lg;          // column lr's KV head is group lg
  // load rounds: lane (4 la + lb) + 16 lg takes quarter lg of the K/V rows of
  // token 4j + la, KV-head slot lb
  const int la = lr >> 2, lb = lr & 3;
  const int nwg = gridDim.x, w = split_index(blockIdx.x, nwg);  // position in the split
  const float base_scale = a.softmax_scale * a.gs_k * kLog2e;

  // The 8 waves sit two to a SIMD (waves w and w ^ 4), and a SIMD issues
  // for its older ready wave first, which leaves the younger one about a
  // quarter slower; with a fixed split of the tiles the workgroup then
  // waits for it.  So each wave publishes its count of finished tiles and
  // runs at raised priority while it trails its SIMD partner: both finish
  // together and the tile split (and the result) stays fixed.  The counter
  // is a hint: a stale or unset value only costs balance.
  int tiles_done = 0;
  if (KVFP4_GQA_BALANCE && lane == 0) progress[wave] = 0;
  auto balance = [&]() {
    ++tiles_done;
    if (lane == 0)
      __hip_atomic_store(&progress[wave], tiles_done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const int other = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(&progress[wave ^ 4], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    if (tiles_done < other)
      __builtin_amdgcn_s_setprio(1);
    else
      __builtin_amdgcn_s_setprio(0);
  };

  TileGeom tg;
  tg.pool = a.pool;
  tg.page_bytes = g.packed_bytes();
  tg.pool_pages = a.pool_pages;
  tg.T = g.T;
  tg.H = g.H;
  tg.tiles_per_page = g.T / kTile;
  // KV-head slots past H (H not a multiple of 4 here) read past the
  // buffer's range: their rows load as zeros and fetch nothing
  const bool kv_ok = 4 * kg + lb < g.H;
  tg.off_data = kv_ok ? (uint32_t)((la * g.H + 4 * kg + lb) * (KD / 2) + lg * (KD / 8)) : kPastRange;
  tg.off_scale = kv_ok ? (uint32_t)((la * g.H + 4 * kg + lb) * (KD / 16) + lg * (KD / 64)) : kPastRange;
  tg.js_data = (uint32_t)(4 * g.H * (KD / 2));
  tg.js_scale = (uint32_t)(4 * g.H * (KD / 16));

  // transposed-read addresses: lane (q = (lane&15)>>2, j = lane&3) of
  // k-group lg points at row 4x + q, dims 4j.. of KV head lg
  constexpr int kHead = head_stride_of<KD>();
  _Float16* vw = &st.v[wave][lg * kHead];
  const int q4 = (lr >> 2), j4 = lr & 3;
  const _Float16* tr_base[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int x = (lg + 2 * m) & 3, y = (lg + 2 * m + 1) & 3;
    tr_base[m][0] = vw + (4 * x + q4) * kPitch;
    tr_base[m][1] = vw + (4 * y + q4) * kPitch;
  }
  // The 16-byte chunk c of staged row r sits at chunk c ^ ((r >> 2) & 1):
  // LDS has 32 banks of 4 bytes and the pitch is 8 banks mod 32, so rows r
  // and r + 4 would collide for the 16-byte writes of 8 lanes.  A
  // transposed read of dims 16dt + 4j.. of rows 4x..4x+3 (chunk 2dt + j/2)
  // therefore starts at fp16 16dt + 8((j/2) ^ (x & 1)) + 4(j%2).
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int x = (lg + 2 * m) & 3, y = (lg + 2 * m + 1) & 3;
    const int sx = KVFP4_GQA_SWZ ? x & 1 : 0, sy = KVFP4_GQA_SWZ ? y & 1 : 0;
    tr_base[m][0] += 8 * ((j4 >> 1) ^ sx) + 4 * (j4 & 1);
    tr_base[m][1] += 8 * ((j4 >> 1) ^ sy) + 4 * (j4 & 1);
  }
  const int src_x1 = lr + 16 * ((lg + 1) & 3);
  const int src_x2 = lr + 16 * ((lg + 2) & 3);
  const int src_x3 = lr + 16 * ((lg + 3) & 3);

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
    tg.L = L;
    // tile indices within the sequence (32-bit: a sequence holds at most
    // 2^31 tokens)
    const int t_lo = (int)p_lo * tg.tiles_per_page;
    int t_hi = (int)p_hi * tg.tiles_per_page;
    const int t_end = (L + kTile - 1) / kTile;
    if (t_hi > t_end) t_hi = t_end;

    // column lr: KV head 4 kg + lr / 4, its query head 4 sub + lr % 4
    const int q_of_kv = 4 * sub + (lr & 3);
    const int kv_of_col = 4 * kg + (lr >> 2);
    const bool col_ok = q_of_kv < G && kv_of_col < g.H;
    const int head = col_ok ? kv_of_col * G + q_of_kv : 0;
    f16x8 qb[KD / 32];  // queries: filled once the first tile is requested
    float qs = 0.f;

    f32x4 acc[KD / 16];
#pragma unroll
    for (int dt = 0; dt < KD / 16; ++dt) acc[dt] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m = kNoMax, l = 0.f;

    // Page-table entries are read with scalar loads (a uniform address in
    // the constant address space): their wait is on the scalar/LDS
    // counter, so reading an entry never waits for the vector-memory loads
    // of tiles in flight.  Each tile's entry is requested a tile ahead.
    typedef __attribute__((address_space(4))) const int32_t* ConstI32;
    const ConstI32 bt_row = (ConstI32)(a.block_table + (long long)b * a.max_pages);
    const int tpp = tg.tiles_per_page;
    const bool tpp_pow2 = (tpp & (tpp - 1)) == 0;
    const int tpp_sh = __builtin_ctz((unsigned)tpp);
    auto page_of = [&](int t) -> int { return tpp_pow2 ? t >> tpp_sh : t / tpp; };
    auto slot_load = [&](int pg) -> int {  // -1 past the segment
      const int e = bt_row[pg < (int)p_hi ? pg : (int)p_hi - 1];
      return pg < (int)p_hi ? e : -1;
    };

    // One tile of the stream, in two phases: (a) V rows to LDS and the
    // scores -- after which the tile's registers are free -- and (b)
    // softmax and P.V from LDS.
    auto phase_a = [&](const Packed& cur) -> f32x4 {
      // V rows -> LDS: round j's token 4j + la goes to row 4 la + j of KV
      // head lb (16-byte chunks swizzled by row bit 2, which is la & 1), so
      // that lane (column, x) holds the probabilities of rows 4x..4x+3
      {
        const int sw = KVFP4_GQA_SWZ ? la & 1 : 0;
        _Float16* vh = &st.v[wave][lb * kHead];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f16x2 vsc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cur.vs[j], 1.0f, false);
          _Float16* dst = vh + (4 * la + j) * kPitch;
#pragma unroll
          for (int e = 0; e < KD / 32; ++e)
            *reinterpret_cast<f16x8*>(dst + 8 * (((KD / 32) * lg + e) ^ sw)) =
                dequant8(cur.v[j][e], (KD == 128 && e >= 2) ? sp1(vsc) : sp0(vsc));
        }
      }

      // scores: round j's product has rows (token 4j + row/4, KV-head slot
      // row%4) and columns (query heads); a lane keeps the one entry of its
      // column whose row has the column's KV head, row block lr / 4 (a dense
      // query operand: the products of other KV heads are discarded)
      f32x4 d[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) d[j] = (f32x4){0.f, 0.f, 0.f, 0.f};
      f16x2 ksc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ksc[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cur.ks[j], 1.0f, false);
#pragma unroll
      for (int ks = 0; ks < KD / 32; ++ks)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f16x8 ka = dequant8(cur.k[j][ks], (KD == 128 && ks >= 2) ? sp1(ksc[j]) : sp0(ksc[j]));
          d[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb[ks], d[j], 0, 0, 0);
        }
      f32x4 sc;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sc[j] = la == 0 ? d[j].x : la == 1 ? d[j].y : la == 2 ? d[j].z : d[j].w;
      return sc;
    };
    auto phase_b = [&](const f32x4 sc, int n_cur) {
      // online softmax of column lr over rows 4 lg + r
      float sv[4];
      float mx = kNoMax;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[r] = (4 * r + lg < n_cur) ? sc[r] * qs : -INFINITY;  // token 4r + lg
        mx = fmaxf(mx, sv[r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(mx > m + kSlack) != 0, 0)) {
        const float mn = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < KD / 16; ++dt) acc[dt] *= alpha;
        m = mn;
      }
      // P.V multiplies the fp16-rounded probabilities, so the denominator
      // sums those same values
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = (float)(_Float16)__builtin_amdgcn_exp2f(sv[r] - m);
        l += p[r];
      }
      const uint32_t pw0 = pack_f16(p[0], p[1]), pw1 = pack_f16(p[2], p[3]);

      // P^T operands: m = 0 takes groups (lg, lg+1), m = 1 (lg+2, lg+3)
      const uint32_t a1 = bperm(pw0, src_x1), b1 = bperm(pw1, src_x1);
      const uint32_t a2 = bperm(pw0, src_x2), b2 = bperm(pw1, src_x2);
      const uint32_t a3 = bperm(pw0, src_x3), b3 = bperm(pw1, src_x3);
      const u32x4 pb0 = diag ? (u32x4){pw0, pw1, a1, b1} : (u32x4){0u, 0u, 0u, 0u};
      const u32x4 pb1 = diag ? (u32x4){a2, b2, a3, b3} : (u32x4){0u, 0u, 0u, 0u};
      const f16x8 pbm[2] = {__builtin_bit_cast(f16x8, pb0), __builtin_bit_cast(f16x8, pb1)};

      // the V rows written above are read back by other lanes of this wave
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      // O^T[dim][column] += V^T P^T
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int dt = 0; dt < KD / 16; ++dt) {
          const f16x4 lo = lds_read_tr(tr_base[mm][0] + 16 * dt);
          const f16x4 hi = lds_read_tr(tr_base[mm][1] + 16 * dt);
          const f16x8 va = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pbm[mm], acc[dt], 0, 0, 0);
        }
      // the next tile's V rows overwrite these only after every lane's reads
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    // the loads of tile t of the sequence from slot sl (-1: no tile; the
    // loads then read zero and fetch nothing, so a request needs no branch)
    auto issue = [&](Packed& p, int& n, int t, int sl) {
      n = tile_rows(tg, sl, t);
      load_tile(p, tg, sl, t - page_of(t) * tpp, n);
    };
    // queries of this wave's 16 columns as the dense B operand: lane
    // (column lr, k-group lg) holds quarter lg of its column's query row,
    // 8 values per product.  The column's largest magnitude (from the bf16
    // bit patterns, over its 4 lanes) sets a power of two that puts it in
    // [2^14, 2^15).  The loads are requested before the first tile's and
    // are unconditional (a padding column reads head 0's row and zeroes
    // it), so that waiting for them leaves the tile's loads in flight.
    u32x4 qraw[KD / 32];
    auto request_queries = [&]() {
      const uint16_t* qrow = a.q + ((long long)b * a.hq + head) * KD + lg * (KD / 4);
#pragma unroll
      for (int i = 0; i < KD / 32; ++i) qraw[i] = load_q8(qrow, i);
    };
    auto load_queries = [&]() {
      u32x4 raw[KD / 32];
#pragma unroll
      for (int i = 0; i < KD / 32; ++i) raw[i] = col_ok ? qraw[i] : (u32x4){0u, 0u, 0u, 0u};
      uint32_t mb = 0;
#pragma unroll
      for (int i = 0; i < KD / 32; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mb = max(mb, raw[i][e] & 0x7FFFu);
          mb = max(mb, (raw[i][e] >> 16) & 0x7FFFu);
        }
      mb = max(mb, (uint32_t)__shfl_xor((int)mb, 16));
      mb = max(mb, (uint32_t)__shfl_xor((int)mb, 32));
      int sh = 0;
      if (mb != 0) {
        int e;
        frexpf(__uint_as_float(mb << 16), &e);  // amax < 2^e
        sh = 15 - e;
      }
#pragma unroll
      for (int i = 0; i < KD / 32; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qb[i][2 * e] = (_Float16)ldexpf(__uint_as_float(raw[i][e] << 16), sh);
          qb[i][2 * e + 1] = (_Float16)ldexpf(__uint_as_float(raw[i][e] & 0xFFFF0000u), sh);
        }
      qs = ldexpf(base_scale, -sh);
    };

    // The KV-head groups walk the stream's tiles in rotated orders (group kg
    // starts kg tiles later and wraps round), so the block-scale lines the
    // groups share are fetched by one group and found in L2 by the next,
    // instead of being missed by all of them at once.
    const int first_t = t_lo + s;
    const int nk = first_t < t_hi ? (t_hi - first_t + NS - 1) / NS : 0;
    const int rot = (KVFP4_GQA_ROT && nk > 0) ? gt % nk : 0;
    auto tile_at = [&](int k) -> int {  // k-th tile of the walk (k < nk)
      int kk = k + rot;
      if (kk >= nk) kk -= nk;
      return first_t + kk * NS;
    };
    // slot of the k-th tile of the walk, -1 past its end (the entry read is
    // always in bounds)
    auto slot_for = [&](int k) -> int {
      const int sl = slot_load(page_of(tile_at(k < nk ? k : 0)));
      return k < nk ? sl : -1;
    };
    // register sets in static roles, the loop unrolled by their number:
    // tile k + kSets - 1 is requested into the set whose tile was computed
    // last, then tile k is computed.  The odd last tiles run after the loop,
    // so that round it every set is requested on every path and each wait
    // leaves the later tiles' loads in flight.
    constexpr int kSets = KVFP4_GQA_SETS;
    static_assert(kSets == 2 || kSets == 3, "2 or 3 register sets");
    Packed pk0, pk1, pk2;
    int n0 = 0, n1 = 0, n2 = 0;
    // Start of the segment, three rounds of requests: the queries and the
    // first two page-table entries, then the first tile, whose loads are
    // issued before the queries are waited for.  The empty asm statements
    // pin that order (the compiler would otherwise use each entry before
    // requesting the next, and convert the queries before the tile's loads).
    request_queries();
    const int pg0 = page_of(tile_at(0)), pg1 = page_of(tile_at(1 < nk ? 1 : 0));
    int e0 = bt_row[pg0 < (int)p_hi ? pg0 : (int)p_hi - 1];
    int e1 = bt_row[pg1 < (int)p_hi ? pg1 : (int)p_hi - 1];
    asm volatile("" : "+s"(e0), "+s"(e1));
    int sl_next = (0 < nk && pg0 < (int)p_hi) ? e0 : -1;
    const int sl_after = (1 < nk && pg1 < (int)p_hi) ? e1 : -1;
    issue(pk0, n0, tile_at(0), sl_next);
#pragma unroll
    for (int i = 0; i < KD / 32; ++i) asm volatile("" : "+v"(qraw[i]) : : "memory");
    sl_next = sl_after;
    if constexpr (kSets == 3) {
      issue(pk1, n1, tile_at(1 < nk ? 1 : 0), sl_next);
      sl_next = slot_for(2);
    }
    load_queries();
    auto step = [&](int k, Packed& cur, int& n_cur, Packed& nxt, int& n_nxt) {
      const int kn = k + kSets - 1;
      issue(nxt, n_nxt, tile_at(kn < nk ? kn : 0), sl_next);
      sl_next = slot_for(kn + 1);
      phase_b(phase_a(cur), n_cur);
      if constexpr (KVFP4_GQA_BALANCE) balance();
    };
    if constexpr (kSets == 3) {
      int k = 0;
      for (; k + 3 <= nk; k += 3) {
        step(k, pk0, n0, pk2, n2);
        step(k + 1, pk1, n1, pk0, n0);
        step(k + 2, pk2, n2, pk1, n1);
      }
      if (k < nk) step(k, pk0, n0, pk2, n2);
      if (k + 1 < nk) step(k + 1, pk1, n1, pk0, n0);
    } else {
      for (int k = 0; k < nk; k += 2) {
        step(k, pk0, n0, pk1, n1);
        if (k + 1 < nk) step(k + 1, pk1, n1, pk0, n0);
      }
    }

    // merge the NS streams of each KV-head group, then write the partial
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    __syncthreads();  // every wave is done with its staged V rows
#pragma unroll
    for (int dt = 0; dt < KD / 16; ++dt)
      *reinterpret_cast<f32x4*>(&mg.o[wave][lr][16 * dt + 4 * lg]) = acc[dt];
    if (lg == 0) {
      mg.ml[wave][lr][0] = m;
      mg.ml[wave][lr][1] = l;
    }
    __syncthreads();
    {
      // wave (kg, s) finishes dims [s * KD/NS, (s+1) * KD/NS) of its group
      constexpr int DW = KD / NS, DL = DW / 4;  // dims per wave, per lane
      float M = kNoMax;
#pragma unroll
      for (int u = 0; u < NS; ++u) M = fmaxf(M, mg.ml[gt * NS + u][lr][0]);
      float wt[NS], Ls = 0.f;
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        wt[u] = __builtin_amdgcn_exp2f(mg.ml[gt * NS + u][lr][0] - M);
        Ls += wt[u] * mg.ml[gt * NS + u][lr][1];
      }
      const long long slotp = ((long long)w + b) * a.hq + head;
      const int d0 = s * DW + lg * DL;
      // the partial output divided by its sum, in fp16
      const float il = Ls > 0.f ? 1.f / Ls : 0.f;
      if (col_ok) {
        if constexpr (DL % 4 == 0) {
#pragma unroll
          for (int i = 0; i < DL; i += 4) {
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < NS; ++u)
              o += *reinterpret_cast<const f32x4*>(&mg.o[gt * NS + u][lr][d0 + i]) * wt[u];
            *reinterpret_cast<u32x2*>(a.ws_oh + slotp * KD + d0 + i) = pack_f16x4(o * il);
          }
        } else {
#pragma unroll
          for (int i = 0; i < DL; ++i) {
            float o = 0.f;
#pragma unroll
            for (int u = 0; u < NS; ++u) o += mg.o[gt * NS + u][lr][d0 + i] * wt[u];
            a.ws_oh[slotp * KD + d0 + i] = f16_bits(o * il);
          }
        }
        if (s == 0 && lg == 0) {
          a.ws_ml[slotp * 2] = M;
          a.ws_ml[slotp * 2 + 1] = Ls;
        }
      }
    }
    __syncthreads();  // the merge area is staged V rows again next segment
  }
}

template <int KD, int NKG, int SUB>
hipError_t launch_nkg(const DecodeArgs& a, hipStream_t stream) {
  static std::atomic<unsigned long long> lds_set{0};
  constexpr size_t bytes = lds_bytes<KD>();
  hipError_t e = allow_lds_once(lds_set, (const void*)decode_gqa_mfma_kernel<KD, NKG, SUB>, bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_gqa_mfma_kernel<KD, NKG, SUB>), dim3(a.nwg), dim3(64 * kWaves), bytes,
                     stream, a);
  return hipGetLastError();
}

// Query subgroups of 4 per KV head for G query heads per KV head (G <= 16),
// and groups of 4 KV heads for H KV heads (H <= 32; slots past H are
// padding): the wave groups of a workgroup are their product, 1, 2, 4 or 8.
int gqa_subgroups(int G) { return G <= 4 ? 1 : G <= 8 ? 2 : 4; }
int gqa_kv_groups(int H) { return H <= 4 ? 1 : H <= 8 ? 2 : H <= 16 ? 4 : 8; }

template <int KD>
hipError_t launch_kd(const DecodeArgs& a, hipStream_t stream) {
  const int nkg = gqa_kv_groups(a.g.H), sub = gqa_subgroups(a.hq / a.g.H);
  switch (nkg * 16 + sub) {
    case 1 * 16 + 1: return launch_nkg<KD, 1, 1>(a, stream);
    case 2 * 16 + 1: return launch_nkg<KD, 2, 1>(a, stream);
    case 4 * 16 + 1: return launch_nkg<KD, 4, 1>(a, stream);
    case 8 * 16 + 1: return launch_nkg<KD, 8, 1>(a, stream);
    case 1 * 16 + 2: return launch_nkg<KD, 1, 2>(a, stream);
    case 2 * 16 + 2: return launch_nkg<KD, 2, 2>(a, stream);
    case 4 * 16 + 2: return launch_nkg<KD, 4, 2>(a, stream);
    case 1 * 16 + 4: return launch_nkg<KD, 1, 4>(a, stream);
    case 2 * 16 + 4: return launch_nkg<KD, 2, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool gqa_supported(const Geom& g, int hq, int v_dim);

bool gqa_mfma_supported(const Geom& g, int hq, int v_dim) {
  if (g.nt != 2 || !(g.D == 64 || g.D == 128) || v_dim != g.D) return false;
  if (g.T % kTile != 0 || g.T > 4096) return false;
  if (g.H < 1 || g.H > 32) return false;
  if (hq % g.H != 0) return false;
  const int G = hq / g.H;
  if (G < 1 || G > 16) return false;
  // fewer than 4 KV heads: the shapes the VALU kernel takes stay there
  if (g.H < 4 && gqa_supported(g, hq, v_dim)) return false;
  // one wave group per (KV-head group, query subgroup)
  return gqa_kv_groups(g.H) * gqa_subgroups(G) <= kWaves;
}

hipError_t launch_decode_gqa_mfma(const DecodeArgs& a, hipStream_t stream) {
  if (!gqa_mfma_supported(a.g, a.hq, a.v_dim) || a.nwg <= 0) return hipErrorInvalidValue;
  if (((uintptr_t)a.ws_oh & 15) != 0 || ((uintptr_t)a.q & 15) != 0) return hipErrorInvalidValue;
  return a.g.D == 64 ? launch_kd<64>(a, stream) : launch_kd<128>(a, stream);
}

}  // namespace kvfp4
