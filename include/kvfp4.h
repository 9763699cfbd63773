/*
 * kvfp4.h -- NVFP4 paged KV cache for AMD MI355X (gfx950): page codec and
 * single-token decode attention that dequantizes NVFP4 K/V in-kernel.
 *
 * Format ("Accelerating Long-Context and Agentic Inference with NVFP4 KV
 * Cache", introduction and Figure 1; NVFP4 KV Decode Attention Kernel
 * Implementation): E2M1 4-bit values, one E4M3 (OCP E4M3FN) scale per
 * block of 16 values, one FP32 scale per tensor.  A block is 8 bytes of
 * packed codes plus 1 scale byte.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Plain C ABI; pointers are device pointers unless marked HOST.
 * - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *   default stream), never synchronizes, never allocates, and keeps no
 *   state between calls beyond two per-device caches (the CU count, and
 *   whether a decode kernel's dynamic-LDS limit has been raised), so calls
 *   are thread-safe and re-entrant, and after the first call on a device
 *   they can be captured into a HIP graph.  The caller owns every buffer;
 *   they must stay valid until the stream work has completed.  Input and
 *   output buffers must not overlap.
 * - All arguments are validated on the host BEFORE anything is launched;
 *   on error nothing is launched and a negative status is returned, with
 *   a thread-local message in kvfp4_last_error_message().
 * - Device-side data (slot ids, page table entries, sequence lengths) is
 *   bounds-checked by the kernels: an out-of-range slot id makes that
 *   page (or that page of the sequence) contribute nothing / be skipped.
 *   NaN or Inf bf16 inputs are outside the contract (unspecified output).
 *
 * Page layout (one fixed-size block per page, "KV Cache Compression in
 * TensorRT LLM", NVFP4 Cold-Page Compression / How It Works, Figure 6;
 * the KV cache manager addresses a page as base + slot * size):
 * - hot page slot (bf16):   [n_t][T][H][D] row-major, 2*E bytes,
 *   E = n_t * T * H * D elements, n_t = num_kv_tensors (K then V).
 * - packed page slot:       E/2 data bytes [n_t][T][H][D/2] followed by
 *   E/16 scale bytes [n_t][T][H][D/16]: 9*E/16 bytes.  Byte k of a block
 *   holds element 2k in bits 3:0 and element 2k+1 in bits 7:4; a nibble is
 *   sign<<3 | E2M1 magnitude code.  A block is 16 consecutive elements
 *   along D of one (tensor, token, head) row.
 *
 * Arithmetic (the readings the pages leave open):
 * - global_scale[t] is the decode multiplier of tensor t:
 *   x ~= e2m1 * e4m3 * global_scale[t].
 * - block scale = E4M3(amax / (6 * gs)), element code = E2M1(|x| / (sb*gs)),
 *   each rounded once from the exact quotient, to nearest, ties to the
 *   even code, saturating (448, 6); a block whose scale rounds to 0 stores
 *   magnitude 0 everywhere; every nibble keeps its input's sign bit.
 * - dequantized value = bf16_RNE(+-e2m1 * e4m3 * gs), one rounding.
 */
#ifndef KVFP4_H_
#define KVFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define KVFP4_OK 0
#define KVFP4_ERR_INVALID_ARG (-1) /* bad pointer, size, scale or shape      */
#define KVFP4_ERR_UNSUPPORTED (-2) /* valid geometry with no compiled kernel  */
#define KVFP4_ERR_WORKSPACE (-3)   /* workspace smaller than required         */
#define KVFP4_ERR_HIP (-4)         /* a HIP launch or runtime call failed     */

/* Page geometry.  num_kv_tensors: 2 = separate K and V (MHA/GQA), 1 = one
 * shared latent (MLA: the key is the whole row, the value its first v_dim
 * elements).  head_dim must be a positive multiple of 16, and a page holds
 * at most 2^28 values. */
typedef struct kvfp4_geometry {
  int32_t num_kv_tensors;
  int32_t page_size;    /* tokens per page T          */
  int32_t num_kv_heads; /* H                          */
  int32_t head_dim;     /* D (576 = 512 + 64 for MLA) */
} kvfp4_geometry;

/* Bytes of one bf16 hot page slot (2*E) and one packed slot (9*E/16); 0 for
 * an invalid geometry.  Storage: 0.5625 bytes per value ("KV Cache
 * Compression in TensorRT LLM", Evaluation / Performance, Figure 10). */
size_t kvfp4_hot_page_bytes(const kvfp4_geometry* g);
size_t kvfp4_packed_page_bytes(const kvfp4_geometry* g);

/* Encode bf16 hot pages into packed NVFP4 pages ("KV Cache Compression in
 * TensorRT LLM", How It Works: quantize on offload, one block per page).
 *   hot_pool    bf16 slots [hot_pool_pages][2*E bytes]           (read)
 *   src_slots   int32 [num_pages] hot slot of page i; NULL = i
 *   packed_pool packed slots [packed_pool_pages][9*E/16 bytes]  (written)
 *               device memory, or pinned host memory from hipHostMalloc
 *               (mapped into the GPU's address space): then the encoder's
 *               stores cross the host link directly and the compression
 *               rides the offload copy (same page, NVFP4 Cold-Page
 *               Compression: compress while the page leaves the GPU).
 *   dst_slots   int32 [num_pages] packed slot of page i; NULL = i
 *   global_scale HOST float [num_kv_tensors]: finite, > 0, and
 *               2688 * gs <= FLT_MAX.
 * Pages whose src or dst slot is out of range are skipped.  With NULL slot
 * arrays num_pages must not exceed the pool.  num_pages == 0 is a no-op.
 * Duplicate dst slots race (unspecified winner). */
int32_t kvfp4_quantize_pages(const kvfp4_geometry* g, const void* hot_pool,
                             int32_t hot_pool_pages, const int32_t* src_slots,
                             void* packed_pool, int32_t packed_pool_pages,
                             const int32_t* dst_slots, int32_t num_pages,
                             const float* global_scale, void* stream);

/* Decode packed pages back into bf16 hot slots (onboard), bit-exact per the
 * arithmetic above.  Same argument rules as kvfp4_quantize_pages with the
 * roles of the pools swapped; packed_pool may likewise be pinned host
 * memory, read across the host link by the decoder. */
int32_t kvfp4_dequantize_pages(const kvfp4_geometry* g, const void* packed_pool,
                               int32_t packed_pool_pages, const int32_t* src_slots,
                               void* hot_pool, int32_t hot_pool_pages,
                               const int32_t* dst_slots, int32_t num_pages,
                               const float* global_scale, void* stream);

/* Sort a page list for the codec calls above by slot.  The offload and
 * onboard of "KV Cache Compression in TensorRT LLM" (How It Works) move
 * lists of blocks; these calls take their pages in list order, and the
 * memory system streams faster when the workgroups running at once touch
 * neighbouring slots.  On MI355X, 4096 Llama-3-8B-shaped pages listed in a
 * random slot order took about 3.5% longer to encode and 11% longer to
 * decode than the same pages sorted.  The results of the codec calls do not
 * depend on the order (duplicate destination slots aside, which race either
 * way).
 *   key        int32 [num_pages] sort key, normally the hot-pool slots (the
 *              src_slots of kvfp4_quantize_pages, the dst_slots of
 *              kvfp4_dequantize_pages)                                 (read)
 *   other      int32 [num_pages] the paired slots, moved with their keys,
 *              or NULL (then other_out must be NULL too)               (read)
 *   key_out, other_out  int32 [num_pages]                           (written)
 * Pairs come out in ascending order of key taken as an unsigned 32-bit value
 * (negative keys, which the codec calls skip, last), equal keys in their
 * input order; the result is the same on every call.  Lists of up to 16384
 * pages are sorted whole, longer lists in consecutive runs of 16384.  The
 * outputs must not overlap the inputs.  Device memory; num_pages == 0 is a
 * no-op. */
int32_t kvfp4_sort_page_list(const int32_t* key, const int32_t* other, int32_t num_pages,
                             int32_t* key_out, int32_t* other_out, void* stream);

/* Element types of the token rows kvfp4_append_quantize reads and
 * kvfp4_gather_dequantize writes. */
#define KVFP4_ROWS_BF16 0     /* bf16, 2 bytes a value                          */
#define KVFP4_ROWS_FP8_E4M3 1 /* OCP E4M3FN, 1 byte a value (NaN codes: unspecified) */

/* Quantize newly computed tokens straight into packed pages ("Accelerating
 * Long-Context and Agentic Inference with NVFP4 KV Cache", Path 1: Initial
 * prefill, Path 2: the current chunk, Path 3: Decode -- the new K/V, bf16
 * or FP8, are quantized into the NVFP4 cache as they are written).
 *   rows        [num_tokens][n_t][H][D] of rows_dtype, 16-byte aligned (read)
 *               (token i's K rows of every head, then its V rows).  An FP8
 *               value is widened exactly (every finite E4M3 value is a bf16
 *               value) and encoded as that bf16 value.
 *   token_slots int32 [num_tokens] packed slot of token i
 *   token_rows  int32 [num_tokens] row (token position) within that page
 *   packed_pool packed slots [packed_pool_pages][9*E/16 bytes]  (written)
 *   global_scale HOST float [num_kv_tensors], as for kvfp4_quantize_pages.
 * Row r of tensor t of the slot gets exactly the data and scale bytes that
 * kvfp4_quantize_pages writes for that row; every other byte of the pool is
 * left untouched.  Tokens whose slot is outside [0, packed_pool_pages) or
 * whose row is outside [0, T) are skipped.  Two tokens naming the same
 * (slot, row) race (unspecified winner).  num_tokens == 0 is a no-op;
 * num_tokens * n_t * H * D must stay below 2^34. */
int32_t kvfp4_append_quantize(const kvfp4_geometry* g, const void* rows, int32_t rows_dtype,
                              int32_t num_tokens, const int32_t* token_slots,
                              const int32_t* token_rows, void* packed_pool,
                              int32_t packed_pool_pages, const float* global_scale,
                              void* stream);

/* Gather rows of packed pages into a contiguous workspace, dequantized
 * ("Accelerating Long-Context and Agentic Inference with NVFP4 KV Cache",
 * Path 2: Chunked prefill / Extend -- the cached prefix's NVFP4 entries are
 * gathered, dequantized and written to a workspace, FP8 there, that the
 * chunk's attention reads together with the chunk's own K/V).
 *   packed_pool  packed slots [packed_pool_pages][9*E/16 bytes]       (read)
 *   token_slots  int32 [num_tokens] packed slot of output row i
 *   token_rows   int32 [num_tokens] row (token position) in that page
 *   out          [num_tokens][n_t][H][D] of out_dtype (KVFP4_ROWS_BF16:
 *                16-byte aligned; KVFP4_ROWS_FP8_E4M3: 8-byte aligned)
 *   global_scale HOST float [num_kv_tensors], as for the other calls.
 * Each value is the exact +-e2m1 * e4m3 * gs rounded once: to bf16 exactly
 * as kvfp4_dequantize_pages does, or to OCP E4M3FN, nearest with ties to
 * the even code and saturating at +-448 (never NaN); the sign bit is the
 * nibble's.  A token whose slot is outside [0, packed_pool_pages) or whose
 * row is outside [0, T) gives an all-zero output row.  num_tokens == 0 is a
 * no-op; num_tokens * n_t * H * D must stay below 2^34. */
int32_t kvfp4_gather_dequantize(const kvfp4_geometry* g, const void* packed_pool,
                                int32_t packed_pool_pages, const int32_t* token_slots,
                                const int32_t* token_rows, int32_t num_tokens, void* out,
                                int32_t out_dtype, const float* global_scale, void* stream);

/* RoPE-part storage of the cold-page codec ("KV Cache Compression in
 * TensorRT LLM", How It Works / The RoPE part of K).  The RoPE part is the
 * last rope_dims dims of every head row of tensor 0 (K; for MLA the latent,
 * whose last 64 of 576 dims carry the rotary embedding).
 *   KVFP4_ROPE_NVFP4  quantized like the rest (the plain layout)
 *   KVFP4_ROPE_BF16   kept at its original bf16 precision
 *   KVFP4_ROPE_2FP4   two NVFP4 layers: the second encodes the exact
 *                     residual x - D1 of the first with the same rules and
 *                     tensor scale; decoding gives bf16_RNE(D1 + D2), one
 *                     rounding of the exact sum.  A zero residual keeps the
 *                     sign of x.
 * A packed slot keeps the plain layout (every value NVFP4-encoded) and
 * appends an extension region [T][H][rope_dims]: bf16 values (mode BF16),
 * or the second layer's data [T][H][rope_dims/2] then its scales
 * [T][H][rope_dims/16] (mode 2FP4).  The decoder returns the RoPE dims from
 * the extension.  Pages in these layouts are for the cold-page path (they
 * are decoded before attention reads them); the decode-attention call reads
 * the plain layout only. */
#define KVFP4_ROPE_NVFP4 0
#define KVFP4_ROPE_BF16 1
#define KVFP4_ROPE_2FP4 2
typedef struct kvfp4_rope_layout {
  int32_t rope_dims; /* multiple of 16, 0 < rope_dims <= head_dim */
  int32_t mode;      /* KVFP4_ROPE_*                              */
} kvfp4_rope_layout;

/* Bytes of one packed slot in this layout (0 when invalid). */
size_t kvfp4_packed_page_bytes_rope(const kvfp4_geometry* g, const kvfp4_rope_layout* rope);

/* kvfp4_quantize_pages / kvfp4_dequantize_pages for slots in a RoPE layout;
 * same arguments plus `rope`, slots of kvfp4_packed_page_bytes_rope bytes.
 * KVFP4_ERR_UNSUPPORTED unless the plain slot size and the extension size
 * are both multiples of 16 bytes (true for page sizes of 16 or more). */
int32_t kvfp4_quantize_pages_rope(const kvfp4_geometry* g, const kvfp4_rope_layout* rope,
                                  const void* hot_pool, int32_t hot_pool_pages,
                                  const int32_t* src_slots, void* packed_pool,
                                  int32_t packed_pool_pages, const int32_t* dst_slots,
                                  int32_t num_pages, const float* global_scale, void* stream);
int32_t kvfp4_dequantize_pages_rope(const kvfp4_geometry* g, const kvfp4_rope_layout* rope,
                                    const void* packed_pool, int32_t packed_pool_pages,
                                    const int32_t* src_slots, void* hot_pool,
                                    int32_t hot_pool_pages, const int32_t* dst_slots,
                                    int32_t num_pages, const float* global_scale, void* stream);

/* Workspace bytes kvfp4_paged_decode_attention needs for these sizes on the
 * current device (0 is a valid answer); 0 also for sizes that call would
 * reject.  The workspace holds the split-K partials (o, max, sum) of the
 * decode kernels before they are merged: "Accelerating Long-Context and
 * Agentic Inference with NVFP4 KV Cache", Path 3: Decode describes decode
 * as a memory-read-bound pass over the whole cached context, which only
 * fills the GPU when a sequence's context is split over many workgroups. */
size_t kvfp4_decode_workspace_bytes(const kvfp4_geometry* g, int32_t batch,
                                    int32_t num_q_heads, int32_t v_dim,
                                    int32_t max_seq_len_hint);

/* Single-token decode attention over the packed cache ("Accelerating
 * Long-Context and Agentic Inference with NVFP4 KV Cache", Path 3: Decode
 * and NVFP4 KV Decode Attention Kernel Implementation / Figure 3): NVFP4
 * K/V are dequantized in registers, the per-tensor scales enter as scalar
 * multipliers of the two products.  For sequence b and query head h (KV
 * head h / (num_q_heads / num_kv_heads)):
 *   s_j = softmax_scale * q . k_j,  out = sum_j softmax(s)_j v_j,
 *   lse = log sum_j exp(s_j),   over the seq_lens[b] cached tokens,
 * token j living in slot block_table[b][j / T], row j % T.
 *   packed_pool   [packed_pool_pages][9*E/16 bytes]
 *   global_scale  HOST float [num_kv_tensors] (K, V; MLA: one)
 *   q             bf16 [batch][num_q_heads][head_dim], 16-byte aligned
 *   v_dim         == head_dim when num_kv_tensors == 2; <= head_dim for MLA
 *   block_table   int32 [batch][max_pages_per_seq]
 *   seq_lens      int32 [batch]; values above max_pages_per_seq * T are
 *                 clamped to it, negative values to 0
 *   max_seq_len_hint HOST estimate of the longest seq_lens entry; it only
 *                 sizes the split-K plan (a longer sequence is still
 *                 attended in full, a wrong hint only costs speed)
 *   out           bf16 [batch][num_q_heads][v_dim]
 *   lse           float [batch][num_q_heads] natural-log LSE, or NULL;
 *                 seq_lens[b] == 0 gives out = 0 and lse = -inf.
 *   workspace     >= kvfp4_decode_workspace_bytes(...) bytes, 16-byte
 *                 aligned (may be NULL when that is 0); its contents need no
 *                 initialization and are scratch after the call.
 * num_q_heads must be a multiple of num_kv_heads. */
int32_t kvfp4_paged_decode_attention(
    const kvfp4_geometry* g, const void* packed_pool, int32_t packed_pool_pages,
    const float* global_scale, const void* q, int32_t batch, int32_t num_q_heads,
    int32_t v_dim, const int32_t* block_table, int32_t max_pages_per_seq,
    const int32_t* seq_lens, int32_t max_seq_len_hint, float softmax_scale,
    void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* kvfp4_paged_decode_attention without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments, layouts
 * and results otherwise (the same kernels and split-K plan, bit-identical
 * outputs).  The split-K partials go to a scratch array of 96 MiB that the
 * library holds on every device it runs on (allocated with its code
 * object, kept until the process ends); this call allocates nothing.
 * Sizes whose kvfp4_decode_workspace_bytes() exceeds 96 MiB are rejected
 * with KVFP4_ERR_WORKSPACE before anything is launched (the MLA shape of
 * batch 64 x 128 heads needs about 41 MiB; Llama- and Qwen-shaped batches
 * of 32 need under 3 MiB).  Every call on a device shares that device's scratch:
 * calls that overlap in time on one device (concurrent streams, or threads
 * without ordering) race on it and must not be issued; calls ordered on one
 * stream are fine.  The scratch needs no clearing between calls. */
int32_t kvfp4_paged_decode_attention_noalloc(
    const kvfp4_geometry* g, const void* packed_pool, int32_t packed_pool_pages,
    const float* global_scale, const void* q, int32_t batch, int32_t num_q_heads,
    int32_t v_dim, const int32_t* block_table, int32_t max_pages_per_seq,
    const int32_t* seq_lens, int32_t max_seq_len_hint, float softmax_scale,
    void* out, float* lse, void* stream);

/* Static text for a status code.  "KV Cache Compression in TensorRT LLM",
 * Configuration and Setup of KV Cache Compression: an unsupported
 * combination is turned away with a clear message, not run. */
const char* kvfp4_status_string(int32_t status);

/* Detail of the last failure on the calling thread ("" if none): which
 * argument was rejected and why (same passage as kvfp4_status_string).
 * The pointer stays valid until the thread's next call into the library. */
const char* kvfp4_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* KVFP4_H_ */
