// Launch parameters and launchers of the paged-attention kernels (internal to
// libpa.so; the C ABI in include/pa.h validates arguments and calls these).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum DType : int { kF16 = 0, kBF16 = 1, kFP8 = 2, kINT8 = 3 };

struct MetadataParams {
  int32_t num_reqs, block_size, max_blocks_per_req, num_tokens_padded, qsl_len;
  const int32_t* num_computed;
  const int32_t* query_lens;
  const int32_t* block_tables;
  int32_t* qsl;
  int32_t* seq_lens;
  int64_t* positions;
  int64_t* slot_mapping;
};

struct CacheWriteParams {
  int64_t num_tokens;
  int32_t row_elems;       // num_kv_heads * head_dim
  int32_t block_size;
  const void* key;
  const void* value;
  int64_t key_row_stride;  // elements
  int64_t value_row_stride;
  const int64_t* slot_mapping;
  void* key_cache;
  void* value_cache;
  int64_t num_slots;       // num_blocks * block_size
  float k_inv_scale, v_inv_scale;  // 8-bit caches only
  // per K/V head scales (8-bit caches; null: the inverse scales above): head
  // h is encoded with 1.0f / scales[h]
  const float* k_scales;
  const float* v_scales;
  int32_t head_dim;
};

struct RopeParams {
  int64_t num_tokens;
  int32_t num_q_heads, num_kv_heads, head_dim, rotary_dim, is_neox;
  const int64_t* positions;
  const float* cos_sin;    // [max_position, rotary_dim]: cos half, then sin half
  int64_t max_position;
  void* query;             // [T, Hq, D] rotated in place
  int64_t query_row_stride;  // elements
  const void* key;
  int64_t key_row_stride;
  const void* value;
  int64_t value_row_stride;
  const int64_t* slot_mapping;
  void* key_cache;
  void* value_cache;
  int64_t num_slots;
  float k_inv_scale, v_inv_scale;  // 8-bit caches only
  const float* k_scales;           // per K/V head scales, as in CacheWriteParams
  const float* v_scales;
};

struct CopyBlocksParams {
  const void* src_key;     // device-visible addresses of the two pools
  const void* src_value;
  int64_t src_blocks;
  void* dst_key;
  void* dst_value;
  int64_t dst_blocks;
  const int64_t* pairs;    // [num_pairs][2]: (source block, destination block)
  int64_t num_pairs;
  int64_t block_bytes;     // block_size * num_kv_heads * head_dim * element bytes, a multiple of 16
};

constexpr int32_t kNoWindow = 1 << 30;

struct AttnParams {
  // geometry
  int32_t num_q_heads, num_kv_heads, group, head_dim;
  // requests
  int32_t req_begin, num_reqs;
  const int32_t* qsl;
  const int32_t* seq_lens;
  const int32_t* block_tables;
  int32_t max_blocks_per_req;
  // tensors
  const void* q;
  int64_t q_row_stride;
  const void* key_cache;
  const void* value_cache;
  int64_t num_blocks;
  void* out;
  int64_t out_row_stride;
  // scalars
  float scale_log2;   // softmax_scale * k_scale * log2(e) (without k_scale when k_scales is set)
  float v_scale;      // 1 unless the cache is quantized
  // per K/V head scales of a quantized cache (null: k_scale / v_scale): the
  // kernels multiply scale_log2 by k_scales[kv head] and use v_scales[kv head]
  // in place of v_scale
  const float* k_scales;
  const float* v_scales;
  // mask variants: keys j < p - window_left are masked for the query at
  // position p (kNoWindow when there is no window); alibi (may be null):
  // per query head slope of the bias slope * (j - p) on the scaled score
  int32_t window_left;
  const float* alibi;
  bool masked;        // window or ALiBi present: the kernels' masked variants run
  int32_t max_seq_len;
  int32_t max_query_len;
  // prefill: query heads (of one K/V head) per workgroup
  int32_t heads_per_wg;
  // decode: the flattened (request, K/V head, block) key stream is cut into
  // num_workers equal contiguous ranges, one per wave; wg_waves consecutive
  // workers form one workgroup, whose range is the union of theirs
  int32_t num_workers;
  int32_t wg_waves;
  int64_t* ws_cum;    // [num_reqs + 1] first stream unit of each request; [num_reqs] = total
  // per workgroup, two partials of K/V heads the workgroup shares with its
  // neighbours (slot 0: the head holding the workgroup's first unit, slot 1:
  // its last head): weighted sums [num_wg, 2, G, D], running max (log2
  // units) and sum [num_wg, 2, G, 2]
  float* ws_acc;
  float* ws_ml;
  // per worker, the weighted sums of its first head when that head began
  // before its range and ended inside it (merged inside the workgroup)
  float* ws_facc;     // [num_workers, G, D]
};

// Decode waves per workgroup (= per compute unit: one resident workgroup of
// independent waves).  8-bit caches (fp8, int8) stream half the bytes per
// block for the same per-block math and use eight; 16-bit caches four.
constexpr int decode_waves_per_cu(int cache_dtype) {
  return (cache_dtype == kFP8 || cache_dtype == kINT8) ? 8 : 4;
}

// Most decode workers a call may use.
constexpr int kMaxDecodeWorkers = 1 << 20;

hipError_t launch_metadata(const MetadataParams& p, hipStream_t stream);
hipError_t launch_cache_write(const CacheWriteParams& p, int act_dtype, int cache_dtype,
                              hipStream_t stream);
hipError_t launch_rope_cache_write(const RopeParams& p, int act_dtype, int cache_dtype,
                                   hipStream_t stream);
// Workgroups per (pair, K or V) of the block copy: grid y of launch_copy_blocks.
int64_t copy_blocks_slices(int64_t block_bytes);
hipError_t launch_copy_blocks(const CopyBlocksParams& p, hipStream_t stream);
// Returns hipErrorInvalidValue for a combination no kernel is built for.
hipError_t launch_decode(const AttnParams& p, int act_dtype, int cache_dtype, hipStream_t stream);
hipError_t launch_prefill(const AttnParams& p, int act_dtype, int cache_dtype, hipStream_t stream);

// A validated pa_decode call: its kernel parameters (workspace pointers not
// yet set), where each workspace part sits, and the bytes the call needs.
struct DecodeCall {
  AttnParams p;
  size_t cum_off, acc_off, ml_off, facc_off, ws_bytes;
  int act_dtype, cache_dtype;
  bool empty;   // no requests: nothing to launch
};

}  // namespace pa
