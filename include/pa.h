/*
 * pa.h -- paged KV-cache attention for one mixed continuous batch, on AMD
 * Instinct MI355X (gfx950).  C ABI of libpa.so.
 *
 * The four calls follow the per-step data flow that "Tour: One forward pass"
 * (explainvllm) walks through and that "vLLM MHA Code Path: From QKV to Paged
 * KV Cache" summarises in its worked decode trace:
 *
 *   once per step   pa_metadata_build  -> query_start_loc, seq_lens,
 *                                          positions, slot_mapping
 *   per layer       pa_cache_write     -> scatter new K/V into the paged cache
 *                   (or pa_rope_cache_write: rotate Q and K by position, then
 *                    the same scatter, in one launch)
 *                   pa_decode          -> attention of 1-token requests
 *                   pa_prefill_varlen  -> causal attention of (chunked) prefills
 *   per step, when the scheduler asks for it
 *                   pa_copy_blocks     -> swap blocks out to / in from host
 *                                         memory, copy shared blocks
 *
 * Conventions shared by every call
 * --------------------------------
 * - Ownership: the caller allocates every buffer (device memory unless stated
 *   otherwise) and keeps it alive until the work on `stream` has finished.
 *   The library allocates nothing, frees nothing and keeps no state between
 *   calls, except the fixed device array of pa_decode_noalloc (held per GPU
 *   for the process's lifetime).  Calls are thread-safe and reentrant
 *   (pa_decode_noalloc: see there).
 * - Ordering: every call only enqueues kernels on `stream` (a hipStream_t;
 *   NULL means the default stream) and returns without waiting.  It never
 *   copies device data to the host.  The write of a layer's new K/V must be
 *   enqueued before that layer's attention on the same stream: attention reads
 *   the current tokens' keys and values from the cache, not from the K/V
 *   inputs (the write-before-read order of the tour's stop 10 and of step 8 of
 *   the MHA trace).
 * - Errors: all argument checks run on the host before any launch.  A failed
 *   check returns PA_ERR_INVALID_ARG or PA_ERR_UNSUPPORTED and enqueues
 *   nothing.  A launch failure returns PA_ERR_HIP.  Faults inside a kernel
 *   surface at the caller's next synchronisation, as for any HIP call.
 * - Cache layout: one key cache and one value cache per layer, each
 *   [num_blocks, block_size, num_kv_heads, head_dim] row-major (the global
 *   pool of "vLLM 推理全流程深度解析", reshape_and_cache description).  The pool
 *   is shared by all requests; several requests may list the same block.
 * - Index types: query_start_loc, seq_lens, num_computed_tokens, query_lens
 *   and block tables are int32; positions and slot_mapping are int64 (the
 *   dtypes printed in stops 3 and 4 of the tour).
 * - Block tables: int32 [num_reqs, max_blocks_per_req] row-major, in batch
 *   order (row r belongs to request r of the call's numbering).  Entry j of a
 *   row is the physical block holding logical tokens j*block_size ..
 *   j*block_size+block_size-1.  Entries at or past ceil(seq_len/block_size)
 *   are never read.  An entry outside [0, num_blocks) is never dereferenced;
 *   its tokens are treated as absent.
 * - Rows: query/output rows are [num_tokens, num_q_heads, head_dim] with a
 *   row stride (in elements) that may exceed num_q_heads*head_dim, so views
 *   into a fused QKV buffer work.  Strides and base pointers must be 16-byte
 *   aligned.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,        /* null pointer, bad size, misaligned pointer/stride */
  PA_ERR_UNSUPPORTED = 2,        /* valid request outside the built kernel set */
  PA_ERR_WORKSPACE_TOO_SMALL = 3,
  PA_ERR_HIP = 4                 /* a HIP launch reported an error */
} pa_status;

typedef enum pa_dtype {
  PA_F16 = 0,       /* IEEE binary16 */
  PA_BF16 = 1,      /* bfloat16 */
  PA_FP8_E4M3 = 2,  /* OCP e4m3fn (max 448, no inf); cache only */
  PA_INT8 = 3       /* symmetric signed int8 codes -127..127; cache only */
} pa_dtype;

/*
 * Per-layer attention geometry (immutable for the layer).
 *
 * num_q_heads % num_kv_heads == 0: query head h reads K/V head h / G with
 * G = num_q_heads / num_kv_heads, which covers MHA (G = 1), GQA and MQA
 * (num_kv_heads = 1) with one path ("vLLM MHA Code Path", "One Path Covers
 * MHA, GQA, and MQA").  Supported: head_dim 64 or 128; block_size 16;
 * act_dtype F16 or BF16; cache_dtype equal to act_dtype, FP8_E4M3 or INT8;
 * G <= 32 for decode.
 *
 * softmax_scale multiplies q.k (1/sqrt(head_dim) is the usual value); it must
 * be finite and > 0 (PA_ERR_INVALID_ARG otherwise: masked scores are -inf
 * before the scale, and a zero or negative scale would make them NaN / +inf).
 * k_scale / v_scale apply to a quantized (fp8 or int8) cache only: a stored
 * code c means the value c * scale, one scale per tensor.  The write path
 * encodes y = float32(x) * (1.0f / scale) (one float32 multiply, the
 * reciprocal rounded once on the host) with round-to-nearest-even: fp8
 * saturates to +-448 and keeps NaN; int8 saturates to +-127 (the code -128 is
 * never written) and stores 0 for NaN.  KV-cache int8 is the quantization the
 * "vLLM 推理全流程深度解析" PagedAttention section names as a throughput lever.
 *
 * k_scales / v_scales (optional, quantized caches only; PA_ERR_INVALID_ARG
 * with a 16-bit cache or a pointer not 4-byte aligned): device float32
 * [num_kv_heads], one scale per K/V head in place of k_scale / v_scale (either
 * may be set alone).  A code of head h means c * scales[h]; the write paths
 * encode head h with the IEEE float32 reciprocal 1.0f / scales[h], computed on
 * the device (correctly rounded, so the same value the host would compute).
 * Each value must be finite and > 0; the library reads them on the device and
 * does not check them.  The arrays stay owned by the caller and must live
 * until the calls that use this descriptor have finished.
 *
 * decode_workers: number of waves pa_decode divides its key stream among
 * (see pa_decode); 0 lets the library choose (per compute unit of the
 * current device: four for 16-bit caches, eight for 8-bit ones).  Otherwise
 * 1 .. 2^20; the result does not depend on it beyond float32 rounding.
 *
 * Mask variants of pa_decode and pa_prefill_varlen (the alibi_slopes and
 * window_size arguments of the attention call in stop 10 of "Tour: One
 * forward pass"; the causal/window rules of step 10 of the worked trace in
 * "vLLM MHA Code Path"):
 * - sliding_window W > 0: the query at position p attends only keys j with
 *   p - W < j <= p (its W most recent positions, itself included); blocks
 *   wholly before the window are not read.  0 = plain causal attention.
 *   A window of 2^30 keys or more sees every key (positions are below 2^30:
 *   the attention calls reject max_seq_len > 2^30) and runs as such.
 * - alibi_slopes: when not NULL, query head h adds slope[h] * (j - p) to the
 *   scaled score softmax_scale * q.k of key j (fp8 / int8: the
 *   scale-corrected score) before the softmax.  The array stays owned by the caller and must
 *   live until the calls that use this descriptor have finished; 4-byte
 *   aligned.
 * Both use the query position p = seq_len - query_len + i for row i of a
 * request (the decode row: p = seq_len - 1).
 */
typedef struct pa_attn_desc {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t act_dtype;      /* pa_dtype */
  int32_t cache_dtype;    /* pa_dtype */
  float softmax_scale;
  float k_scale;
  float v_scale;
  int32_t decode_workers;
  int32_t sliding_window;     /* 0: none; W > 0: see below */
  const float* alibi_slopes;  /* NULL: none; else device float32 [num_q_heads] */
  const float* k_scales;      /* NULL: k_scale; else device float32 [num_kv_heads] */
  const float* v_scales;      /* NULL: v_scale; else device float32 [num_kv_heads] */
} pa_attn_desc;

/* Human-readable name of a status code (static storage). */
const char* pa_status_string(pa_status status);

/*
 * pa_metadata_build -- per-step batch metadata ("Tour: One forward pass",
 * stops 3 and 4).  One kernel launch.
 *
 * In (device):  num_computed_tokens int32 [num_reqs], query_lens int32
 *               [num_reqs], block_tables int32 [num_reqs, max_blocks_per_req].
 * Out (device): query_start_loc int32 [qsl_len] with qsl_len >= num_reqs + 1:
 *                 qsl[0] = 0, qsl[r+1] = qsl[r] + query_lens[r], and every
 *                 entry past num_reqs equals the token total T (so the buffer
 *                 never decreases);
 *               seq_lens int32 [num_reqs] = num_computed_tokens + query_lens;
 *               positions int64 [num_tokens_padded]: token t of request r at
 *                 batch row qsl[r] + i gets num_computed_tokens[r] + i; rows
 *                 >= T are not written;
 *               slot_mapping int64 [num_tokens_padded]:
 *                 block_tables[r][pos / block_size] * block_size
 *                 + pos % block_size, or -1 (PAD_SLOT_ID) for rows >= T and
 *                 for positions whose block index is >= max_blocks_per_req.
 * Requires T <= num_tokens_padded; rows past num_tokens_padded are not
 * written.  Empty requests (query_len 0) are allowed.
 */
pa_status pa_metadata_build(int32_t num_reqs, int32_t block_size, int32_t max_blocks_per_req,
                            int32_t num_tokens_padded, int32_t qsl_len,
                            const int32_t* num_computed_tokens, const int32_t* query_lens,
                            const int32_t* block_tables,
                            int32_t* query_start_loc, int32_t* seq_lens,
                            int64_t* positions, int64_t* slot_mapping,
                            void* stream);

/*
 * pa_cache_write -- scatter the step's new K/V rows into the paged cache
 * (reshape_and_cache in "vLLM 推理全流程深度解析"; reshape_and_cache_flash in
 * stop 10 of the tour).  One kernel launch.
 *
 * key, value: act_dtype [num_tokens, num_kv_heads, head_dim] with row strides
 *   key_row_stride / value_row_stride in elements.
 * slot_mapping: int64 [num_tokens].  Token t with slot s >= 0 and
 *   s < num_blocks*block_size goes to cache[s / block_size][s % block_size];
 *   other tokens (the -1 padding) are skipped.  Two tokens with one slot race.
 * key_cache, value_cache: cache_dtype [num_blocks, block_size, num_kv_heads,
 *   head_dim]; only the addressed slots are written, bit-exact copies (or
 *   fp8 / int8 encodings, see pa_attn_desc) of the inputs.
 */
pa_status pa_cache_write(const pa_attn_desc* desc, int64_t num_tokens,
                         const void* key, int64_t key_row_stride,
                         const void* value, int64_t value_row_stride,
                         const int64_t* slot_mapping,
                         void* key_cache, void* value_cache, int64_t num_blocks,
                         void* stream);

/*
 * pa_rope_cache_write -- rotary position embedding of Q and K fused with the
 * cache write ("Tour: One forward pass", stop 9: RoPE turns q and k by each
 * token's position from stop 3, using that position's cosines and sines from
 * cos_sin_cache on every head's pairs; then stop 10's cache write).  One
 * kernel launch.
 *
 * positions: int64 [num_tokens] (as built by pa_metadata_build).
 * cos_sin_cache: float32 [max_position, rotary_dim], 16-byte aligned: row p
 *   holds rotary_dim/2 cosines c_j then rotary_dim/2 sines s_j for position p
 *   (the caller builds it, e.g. angle p * base^(-2j/rotary_dim)).
 * rotary_dim: rotated leading dimensions of every head; a multiple of 16,
 *   16 .. head_dim.  Dimensions from rotary_dim on are left unchanged.
 * is_neox: 1 rotates the pairs (j, j + rotary_dim/2) (half-split layout),
 *   0 the pairs (2j, 2j+1) (interleaved).
 * query: act_dtype [num_tokens, num_q_heads, head_dim], row stride in
 *   elements; rotated in place.
 * key, value: act_dtype [num_tokens, num_kv_heads, head_dim] (not modified).
 * For token t at position p in [0, max_position), each pair (a, b) of every
 * query and key head becomes a*c - b*s, b*c + a*s, computed in float32 with
 * every product and sum rounded once (no fused multiply-add), rounded to
 * act_dtype (nearest even).  The rotated key and the value then go to the
 * slot exactly as pa_cache_write would store them (fp8 / int8 caches: the
 * rotated key rounded to act_dtype is encoded).  A token with a slot that is negative
 * or past the pool has its query rotated and writes nothing; a token whose
 * position is outside [0, max_position) is left entirely alone.
 */
pa_status pa_rope_cache_write(const pa_attn_desc* desc, int64_t num_tokens,
                              const int64_t* positions, const float* cos_sin_cache,
                              int64_t max_position, int32_t rotary_dim, int32_t is_neox,
                              void* query, int64_t query_row_stride,
                              const void* key, int64_t key_row_stride,
                              const void* value, int64_t value_row_stride,
                              const int64_t* slot_mapping,
                              void* key_cache, void* value_cache, int64_t num_blocks,
                              void* stream);

/*
 * pa_copy_blocks -- copy whole cache blocks (K and V) from one block pool to
 * another by a list of (source block, destination block) pairs.  Serves the
 * three pair lists of the scheduler output in "vLLM 推理全流程深度解析":
 * blocks_to_swap_out (device pool -> host pool, when GPU memory runs short),
 * blocks_to_swap_in (host pool -> device pool) and blocks_to_copy (inside one
 * device pool: the private copy of a block that sequences share, e.g. beam
 * candidates sharing the prompt's blocks).  One kernel launch for all pairs.
 *
 * src_key_cache, src_value_cache: the source pool, [src_num_blocks,
 *   block_size, num_kv_heads, head_dim] of cache_dtype each.
 * dst_key_cache, dst_value_cache: the destination pool, [dst_num_blocks, ...]
 *   of the same element type and block shape (the same pointers as the source
 *   for a copy inside one pool).
 * block_pairs: int64 [num_pairs][2], (source block, destination block).
 * Memory: each of the five buffers may be device memory or pinned host memory
 *   (hipHostMalloc, torch's pin_memory) that the device can map; the kernel
 *   moves the bytes itself.  Pageable or managed memory is rejected with
 *   PA_ERR_INVALID_ARG (checked by a pointer-attribute query before launch).
 *   Host buffers must stay pinned and untouched by the host until the work on
 *   `stream` has finished.
 * Result: destination block d of both caches holds the bytes of source block
 *   s, for every pair with 0 <= s < src_num_blocks and 0 <= d < dst_num_blocks;
 *   other pairs are skipped; no other byte of the destination is written.
 *   Destinations must be distinct and, inside one pool, must not be sources
 *   of other pairs (such pairs race; the result is then undefined).
 * Alignment: cache pointers 16-byte aligned, block_pairs 8-byte aligned.
 * Errors: PA_ERR_INVALID_ARG for a negative count or size, a null or
 *   misaligned pointer, memory the device cannot reach; PA_ERR_UNSUPPORTED for
 *   more than 2^30 - 1 pairs.  num_pairs == 0 returns PA_OK, enqueues nothing.
 */
pa_status pa_copy_blocks(const pa_attn_desc* desc,
                         const void* src_key_cache, const void* src_value_cache,
                         int64_t src_num_blocks,
                         void* dst_key_cache, void* dst_value_cache, int64_t dst_num_blocks,
                         const int64_t* block_pairs, int64_t num_pairs, void* stream);

/*
 * pa_decode -- attention of decode requests through their block tables
 * (PagedAttention decode in "vLLM 推理全流程深度解析"; the decode rows of the
 * varlen call in stop 10 of the tour).
 *
 * Requests req_begin .. req_end-1 (indices into query_start_loc / seq_lens /
 * block_tables).  Each must have query_len == 1; a request with another
 * query length is skipped and its output rows are not written.  The query
 * row of request r is q[qsl[r]]; it attends keys 0 .. seq_lens[r]-1 (the
 * token written this step included):
 *   out[qsl[r], h] = softmax_j(softmax_scale * q.k_j) v_j, k_j/v_j of K/V head
 *   h / G.
 * max_seq_len (host scalar) must be >= every seq_len of the range; keys past
 * it are ignored; above 2^30 the call returns PA_ERR_UNSUPPORTED.  Accumulation is float32; out is act_dtype, rounded to
 * nearest even.  The (request, K/V head, 16-token block) stream of the range
 * is cut into desc->decode_workers equal contiguous shares, one per wave,
 * and consecutive waves form workgroups; a K/V head cut between waves leaves
 * float32 partial results (running max, sum, weighted sum) that the
 * workgroup merges, and a head cut between workgroups leaves one partial
 * per workgroup in `workspace` that a second kernel merges (fixed orders:
 * the output is deterministic for a given worker count).
 *
 * Workspace: 16-byte aligned device memory of at least
 * pa_decode_workspace_size() bytes for the same desc and request count (else
 * PA_ERR_WORKSPACE_TOO_SMALL), required whenever the range is not empty.
 * Its contents need no initialisation and are scratch after the call; two
 * calls in flight at once need two workspaces.
 * PA_ERR_UNSUPPORTED (besides the descriptor's own limits) when a block of
 * one K/V cache spans 2^32 bytes or more (16 * num_kv_heads * head_dim *
 * element size), or when (req_end - req_begin) * num_kv_heads *
 * max_blocks_per_req exceeds the worker count times 2^31 - 1.
 */
pa_status pa_decode(const pa_attn_desc* desc, int32_t req_begin, int32_t req_end,
                    const void* q, int64_t q_row_stride,
                    const int32_t* query_start_loc, const int32_t* seq_lens,
                    const int32_t* block_tables, int32_t max_blocks_per_req,
                    const void* key_cache, const void* value_cache, int64_t num_blocks,
                    int32_t max_seq_len,
                    void* workspace, size_t workspace_bytes,
                    void* out, int64_t out_row_stride, void* stream);

/*
 * pa_decode_noalloc -- pa_decode without a caller's workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments, result
 * and checks as pa_decode, minus the workspace pair.
 *
 * It uses a device array that the library holds, one per GPU, of
 * PA_DECODE_NOALLOC_SCRATCH_BYTES bytes (64 MiB: enough for head_dim <= 128
 * and G <= 32 at the default worker count of a 256-compute-unit device),
 * which lives until the process ends; its address is looked up on the first
 * call on each device.  The call allocates and frees nothing.  A call that would need more workspace than
 * the array holds (pa_decode_workspace_size larger than
 * PA_DECODE_NOALLOC_SCRATCH_BYTES) returns PA_ERR_WORKSPACE_TOO_SMALL and
 * enqueues nothing.  Every call on one GPU shares that GPU's array: calls
 * whose work may overlap on one GPU (other streams, other host threads)
 * race and give undefined results; serialise them.  PA_ERR_HIP if the
 * array's address cannot be obtained on the current device.
 */
#define PA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

pa_status pa_decode_noalloc(const pa_attn_desc* desc, int32_t req_begin, int32_t req_end,
                            const void* q, int64_t q_row_stride,
                            const int32_t* query_start_loc, const int32_t* seq_lens,
                            const int32_t* block_tables, int32_t max_blocks_per_req,
                            const void* key_cache, const void* value_cache, int64_t num_blocks,
                            int32_t max_seq_len, void* out, int64_t out_row_stride,
                            void* stream);

/*
 * pa_decode_workspace_size -- bytes of workspace pa_decode needs for
 * num_reqs = req_end - req_begin requests of this desc (a prefix sum over the
 * requests, two partial slots per workgroup of G float32 running maxima, sums
 * and head_dim weighted sums, and one slot per worker of G * head_dim
 * weighted sums).  max_seq_len and
 * max_blocks_per_req are validated but do not change the size.  0 when
 * num_reqs is 0.  Host only; launches nothing (it may query the current
 * device's compute-unit count).
 */
pa_status pa_decode_workspace_size(const pa_attn_desc* desc, int32_t num_reqs,
                                   int32_t max_seq_len, int32_t max_blocks_per_req,
                                   size_t* bytes);

/*
 * pa_prefill_varlen -- causal attention of prefill / chunked-prefill requests
 * over the paged cache (flash_attn_varlen_func with cu_seqlens_q =
 * query_start_loc, seqused_k = seq_lens and a block table, stop 10 of the
 * tour).
 *
 * Requests req_begin .. req_end-1, any query_len >= 0.  Request r has
 * n = qsl[r+1] - qsl[r] new tokens and c = seq_lens[r] - n cached ones; its
 * query i (row qsl[r] + i) attends keys 0 .. c + i (bottom-right causal: the
 * new token sees the whole cached prefix and itself, never a later token).
 * max_query_len and max_seq_len (host scalars, as the tour's metadata keeps
 * them on the CPU) must bound every n and seq_len of the range: max_query_len
 * sizes the launch (the kernel takes each request's length from
 * query_start_loc; max_query_len 0 computes nothing) and max_seq_len caps the
 * keys read; max_seq_len above 2^30 returns PA_ERR_UNSUPPORTED.  Output rows
 * of other requests and padding rows are never written.  Accumulation
 * float32; out act_dtype.  Results do not depend on the order in which the
 * work is spread over the device (each output row is computed by one wave
 * along one fixed key order).
 */
pa_status pa_prefill_varlen(const pa_attn_desc* desc, int32_t req_begin, int32_t req_end,
                            const void* q, int64_t q_row_stride,
                            const int32_t* query_start_loc, const int32_t* seq_lens,
                            const int32_t* block_tables, int32_t max_blocks_per_req,
                            const void* key_cache, const void* value_cache, int64_t num_blocks,
                            int32_t max_query_len, int32_t max_seq_len,
                            void* out, int64_t out_row_stride, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
