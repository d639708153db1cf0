// C ABI of libpa.so (declared in include/pa.h): host-side argument checks,
// split-K planning and kernel launches.  Every check runs before any launch
// (the only HIP calls before it are queries), so a rejected call enqueues
// nothing.
#include "pa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "pa_decode_call.h"
#include "pa_kernels.h"

namespace {

constexpr int kBlockSize = 16;
constexpr int kMaxGridYZ = 65535;
// longest sequence the attention calls take: positions stay below 2^30, so a
// sliding window of 2^30 keys or more leaves every key visible and is
// clamped to that length (the kernels then never form position - window
// below -2^31)
constexpr int32_t kMaxSeqLen = 1 << 30;
constexpr float kLog2e = 1.4426950408889634f;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// 8-bit codes with a per-tensor scale (fp8 e4m3fn or int8)
bool quantized(int dt) { return dt == PA_FP8_E4M3 || dt == PA_INT8; }

int elem_bytes(int dt) { return quantized(dt) ? 1 : 2; }

pa_status check_desc(const pa_attn_desc* d) {
  if (d == nullptr) return PA_ERR_INVALID_ARG;
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0) return PA_ERR_INVALID_ARG;
  if (d->num_q_heads % d->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (d->head_dim <= 0 || d->block_size <= 0) return PA_ERR_INVALID_ARG;
  if (d->act_dtype != PA_F16 && d->act_dtype != PA_BF16) {
    return quantized(d->act_dtype) ? PA_ERR_UNSUPPORTED : PA_ERR_INVALID_ARG;
  }
  if (d->cache_dtype != d->act_dtype && !quantized(d->cache_dtype)) {
    return (d->cache_dtype == PA_F16 || d->cache_dtype == PA_BF16) ? PA_ERR_UNSUPPORTED
                                                                  : PA_ERR_INVALID_ARG;
  }
  if (d->head_dim != 64 && d->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (d->block_size != kBlockSize) return PA_ERR_UNSUPPORTED;
  // masked scores are -inf before the scale multiplies them: a zero or
  // negative scale would turn them into NaN or +inf
  if (!std::isfinite(d->softmax_scale) || !(d->softmax_scale > 0.f)) return PA_ERR_INVALID_ARG;
  if (quantized(d->cache_dtype)) {
    if (!(d->k_scale > 0.f) || !(d->v_scale > 0.f) || !std::isfinite(d->k_scale) ||
        !std::isfinite(d->v_scale)) {
      return PA_ERR_INVALID_ARG;
    }
  }
  if (d->decode_workers < 0 || d->decode_workers > pa::kMaxDecodeWorkers) return PA_ERR_INVALID_ARG;
  if (d->sliding_window < 0) return PA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(d->alibi_slopes) & 3u) != 0) return PA_ERR_INVALID_ARG;
  // per-head scales: quantized caches only, float32-aligned
  if ((d->k_scales != nullptr || d->v_scales != nullptr) && !quantized(d->cache_dtype)) {
    return PA_ERR_INVALID_ARG;
  }
  if (((reinterpret_cast<uintptr_t>(d->k_scales) | reinterpret_cast<uintptr_t>(d->v_scales)) & 3u) != 0) {
    return PA_ERR_INVALID_ARG;
  }
  return PA_OK;
}

// the kernels' cache-format code of a pa_dtype
int cache_kind(int cache_dtype) {
  return cache_dtype == PA_FP8_E4M3 ? pa::kFP8 : cache_dtype == PA_INT8 ? pa::kINT8 : pa::kF16;
}

// Decode workers: waves that each stream one contiguous share of the
// (request, K/V head, block) stream.  decode_waves_per_cu() per compute unit
// of the current device (one workgroup of independent waves per CU, all
// resident for the whole launch) unless the descriptor fixes the count.
int decode_workers(const pa_attn_desc* d) {
  if (d->decode_workers > 0) return d->decode_workers;
  const int per_cu = pa::decode_waves_per_cu(cache_kind(d->cache_dtype));
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    cus = 256;
  }
  return per_cu * cus;
}

struct DecodePlan {
  int workers, wg_waves;
  size_t cum_off, acc_off, ml_off, facc_off, ws_bytes;
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace: the stream prefix (int64, num_reqs + 1); two float32 partial
// slots per workgroup of G * (head_dim + 2) values (weighted sums, then
// running maxima and sums) and one per worker of G * head_dim weighted sums.
DecodePlan plan_decode(const pa_attn_desc* d, int num_reqs) {
  DecodePlan pl{};
  pl.workers = decode_workers(d);
  pl.wg_waves = pa::decode_waves_per_cu(cache_kind(d->cache_dtype));
  const size_t G = (size_t)(d->num_q_heads / d->num_kv_heads);
  const size_t wg_slots = (size_t)((pl.workers + pl.wg_waves - 1) / pl.wg_waves) * 2;
  const size_t w_slots = (size_t)pl.workers;
  pl.cum_off = 0;
  pl.acc_off = round_up((size_t)(num_reqs + 1) * sizeof(int64_t), 256);
  pl.ml_off = pl.acc_off + round_up(wg_slots * G * d->head_dim * sizeof(float), 256);
  pl.facc_off = pl.ml_off + round_up(wg_slots * G * 2 * sizeof(float), 256);
  pl.ws_bytes = pl.facc_off + round_up(w_slots * G * d->head_dim * sizeof(float), 256);
  return pl;
}

pa_status from_hip(hipError_t e) {
  if (e == hipSuccess) return PA_OK;
  if (e == hipErrorInvalidValue) return PA_ERR_UNSUPPORTED;
  return PA_ERR_HIP;
}

// The address at which the device reaches `ptr`: device memory as it is,
// pinned host memory (hipHostMalloc) through the device mapping the runtime
// reports for it.  False for anything else (pageable host memory, managed
// memory, unknown pointers).  Queries only.
bool device_address(const void* ptr, const void** out) {
  hipPointerAttribute_t a{};
  if (hipPointerGetAttributes(&a, ptr) != hipSuccess) {
    (void)hipGetLastError();   // clear the query's error so no later call reports it
    return false;
  }
  if (a.type == hipMemoryTypeDevice && !a.isManaged) {
    *out = ptr;
    return true;
  }
  if (a.type == hipMemoryTypeHost && !a.isManaged) {
    // succeeds only for pinned host memory the runtime has mapped for the device
    void* dev = nullptr;
    if (hipHostGetDevicePointer(&dev, const_cast<void*>(ptr), 0) != hipSuccess || dev == nullptr) {
      (void)hipGetLastError();
      return false;
    }
    *out = dev;
    return true;
  }
  return false;
}

// The score scale in log2 units; with per-head K scales the kernels multiply
// it by the head's scale.
float scale_log2(const pa_attn_desc* d) {
  const float ks = (quantized(d->cache_dtype) && d->k_scales == nullptr) ? d->k_scale : 1.0f;
  return d->softmax_scale * ks * kLog2e;
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "PA_ERR_WORKSPACE_TOO_SMALL";
    case PA_ERR_HIP: return "PA_ERR_HIP";
  }
  return "PA_ERR_UNKNOWN";
}

pa_status pa_metadata_build(int32_t num_reqs, int32_t block_size, int32_t max_blocks_per_req,
                            int32_t num_tokens_padded, int32_t qsl_len,
                            const int32_t* num_computed_tokens, const int32_t* query_lens,
                            const int32_t* block_tables, int32_t* query_start_loc,
                            int32_t* seq_lens, int64_t* positions, int64_t* slot_mapping,
                            void* stream) {
  if (num_reqs < 0 || block_size <= 0 || max_blocks_per_req < 0 || num_tokens_padded < 0) {
    return PA_ERR_INVALID_ARG;
  }
  if (qsl_len < num_reqs + 1) return PA_ERR_INVALID_ARG;
  if (query_start_loc == nullptr) return PA_ERR_INVALID_ARG;
  if (num_reqs > 0 && (num_computed_tokens == nullptr || query_lens == nullptr ||
                       seq_lens == nullptr)) {
    return PA_ERR_INVALID_ARG;
  }
  if (num_reqs > 0 && max_blocks_per_req > 0 && block_tables == nullptr) return PA_ERR_INVALID_ARG;
  if (num_tokens_padded > 0 && (positions == nullptr || slot_mapping == nullptr)) {
    return PA_ERR_INVALID_ARG;
  }
  pa::MetadataParams p{};
  p.num_reqs = num_reqs;
  p.block_size = block_size;
  p.max_blocks_per_req = max_blocks_per_req;
  p.num_tokens_padded = num_tokens_padded;
  p.qsl_len = qsl_len;
  p.num_computed = num_computed_tokens;
  p.query_lens = query_lens;
  p.block_tables = block_tables;
  p.qsl = query_start_loc;
  p.seq_lens = seq_lens;
  p.positions = positions;
  p.slot_mapping = slot_mapping;
  return from_hip(pa::launch_metadata(p, static_cast<hipStream_t>(stream)));
}

pa_status pa_cache_write(const pa_attn_desc* desc, int64_t num_tokens, const void* key,
                         int64_t key_row_stride, const void* value, int64_t value_row_stride,
                         const int64_t* slot_mapping, void* key_cache, void* value_cache,
                         int64_t num_blocks, void* stream) {
  pa_status st = check_desc(desc);
  if (st != PA_OK) return st;
  if (num_tokens < 0 || num_blocks < 0) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !slot_mapping || !key_cache || !value_cache) return PA_ERR_INVALID_ARG;
  const int64_t row = (int64_t)desc->num_kv_heads * desc->head_dim;
  if (key_row_stride < row || value_row_stride < row) return PA_ERR_INVALID_ARG;
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache)) {
    return PA_ERR_INVALID_ARG;
  }
  if ((key_row_stride * 2) % 16 != 0 || (value_row_stride * 2) % 16 != 0) return PA_ERR_INVALID_ARG;
  if (num_tokens * (row / 8) > (int64_t)0x7FFFFFFF * 256) return PA_ERR_UNSUPPORTED;
  pa::CacheWriteParams p{};
  p.num_tokens = num_tokens;
  p.row_elems = (int32_t)row;
  p.block_size = desc->block_size;
  p.key = key;
  p.value = value;
  p.key_row_stride = key_row_stride;
  p.value_row_stride = value_row_stride;
  p.slot_mapping = slot_mapping;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.num_slots = num_blocks * desc->block_size;
  p.k_inv_scale = quantized(desc->cache_dtype) ? 1.0f / desc->k_scale : 1.0f;
  p.v_inv_scale = quantized(desc->cache_dtype) ? 1.0f / desc->v_scale : 1.0f;
  p.k_scales = desc->k_scales;
  p.v_scales = desc->v_scales;
  p.head_dim = desc->head_dim;
  return from_hip(pa::launch_cache_write(p, desc->act_dtype, desc->cache_dtype,
                                         static_cast<hipStream_t>(stream)));
}

pa_status pa_rope_cache_write(const pa_attn_desc* desc, int64_t num_tokens,
                              const int64_t* positions, const float* cos_sin_cache,
                              int64_t max_position, int32_t rotary_dim, int32_t is_neox,
                              void* query, int64_t query_row_stride, const void* key,
                              int64_t key_row_stride, const void* value, int64_t value_row_stride,
                              const int64_t* slot_mapping, void* key_cache, void* value_cache,
                              int64_t num_blocks, void* stream) {
  pa_status st = check_desc(desc);
  if (st != PA_OK) return st;
  if (num_tokens < 0 || num_blocks < 0 || max_position <= 0) return PA_ERR_INVALID_ARG;
  if (rotary_dim < 2 || rotary_dim % 2 != 0 || rotary_dim > desc->head_dim) return PA_ERR_INVALID_ARG;
  if (is_neox != 0 && is_neox != 1) return PA_ERR_INVALID_ARG;
  if (rotary_dim % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!positions || !cos_sin_cache || !query || !key || !value || !slot_mapping || !key_cache ||
      !value_cache) {
    return PA_ERR_INVALID_ARG;
  }
  const int64_t qrow = (int64_t)desc->num_q_heads * desc->head_dim;
  const int64_t kvrow = (int64_t)desc->num_kv_heads * desc->head_dim;
  if (query_row_stride < qrow || key_row_stride < kvrow || value_row_stride < kvrow) {
    return PA_ERR_INVALID_ARG;
  }
  if (!aligned16(query) || !aligned16(key) || !aligned16(value) || !aligned16(key_cache) ||
      !aligned16(value_cache) || !aligned16(cos_sin_cache)) {
    return PA_ERR_INVALID_ARG;
  }
  if ((query_row_stride * 2) % 16 != 0 || (key_row_stride * 2) % 16 != 0 ||
      (value_row_stride * 2) % 16 != 0) {
    return PA_ERR_INVALID_ARG;
  }
  const int64_t per_token = (int64_t)desc->num_q_heads * (rotary_dim / 16) +
                            (int64_t)desc->num_kv_heads *
                                (rotary_dim / 16 + (desc->head_dim - rotary_dim) / 8 + desc->head_dim / 8);
  if (num_tokens * per_token > (int64_t)0x7FFFFFFF * 256) return PA_ERR_UNSUPPORTED;
  pa::RopeParams p{};
  p.num_tokens = num_tokens;
  p.num_q_heads = desc->num_q_heads;
  p.num_kv_heads = desc->num_kv_heads;
  p.head_dim = desc->head_dim;
  p.rotary_dim = rotary_dim;
  p.is_neox = is_neox;
  p.positions = positions;
  p.cos_sin = cos_sin_cache;
  p.max_position = max_position;
  p.query = query;
  p.query_row_stride = query_row_stride;
  p.key = key;
  p.key_row_stride = key_row_stride;
  p.value = value;
  p.value_row_stride = value_row_stride;
  p.slot_mapping = slot_mapping;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.num_slots = num_blocks * desc->block_size;
  p.k_inv_scale = quantized(desc->cache_dtype) ? 1.0f / desc->k_scale : 1.0f;
  p.v_inv_scale = quantized(desc->cache_dtype) ? 1.0f / desc->v_scale : 1.0f;
  p.k_scales = desc->k_scales;
  p.v_scales = desc->v_scales;
  return from_hip(pa::launch_rope_cache_write(p, desc->act_dtype, desc->cache_dtype,
                                              static_cast<hipStream_t>(stream)));
}

pa_status pa_copy_blocks(const pa_attn_desc* desc, const void* src_key_cache,
                         const void* src_value_cache, int64_t src_num_blocks, void* dst_key_cache,
                         void* dst_value_cache, int64_t dst_num_blocks, const int64_t* block_pairs,
                         int64_t num_pairs, void* stream) {
  pa_status st = check_desc(desc);
  if (st != PA_OK) return st;
  if (src_num_blocks < 0 || dst_num_blocks < 0 || num_pairs < 0) return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!src_key_cache || !src_value_cache || !dst_key_cache || !dst_value_cache || !block_pairs) {
    return PA_ERR_INVALID_ARG;
  }
  if (!aligned16(src_key_cache) || !aligned16(src_value_cache) || !aligned16(dst_key_cache) ||
      !aligned16(dst_value_cache) || (reinterpret_cast<uintptr_t>(block_pairs) & 7u) != 0) {
    return PA_ERR_INVALID_ARG;
  }
  if (num_pairs > 0x3FFFFFFF) return PA_ERR_UNSUPPORTED;   // grid x = 2 * num_pairs
  const int64_t block_bytes = (int64_t)desc->block_size * desc->num_kv_heads * desc->head_dim *
                              elem_bytes(desc->cache_dtype);
  if (pa::copy_blocks_slices(block_bytes) > kMaxGridYZ) return PA_ERR_UNSUPPORTED;
  pa::CopyBlocksParams p{};
  const void* dev[5];
  const void* host[5] = {src_key_cache, src_value_cache, dst_key_cache, dst_value_cache, block_pairs};
  for (int i = 0; i < 5; ++i) {
    if (!device_address(host[i], &dev[i])) return PA_ERR_INVALID_ARG;
  }
  p.src_key = dev[0];
  p.src_value = dev[1];
  p.src_blocks = src_num_blocks;
  p.dst_key = const_cast<void*>(dev[2]);
  p.dst_value = const_cast<void*>(dev[3]);
  p.dst_blocks = dst_num_blocks;
  p.pairs = static_cast<const int64_t*>(dev[4]);
  p.num_pairs = num_pairs;
  p.block_bytes = block_bytes;
  return from_hip(pa::launch_copy_blocks(p, static_cast<hipStream_t>(stream)));
}

static pa_status check_attn_common(const pa_attn_desc* desc, int32_t req_begin, int32_t req_end,
                                   const void* q, int64_t q_row_stride,
                                   const int32_t* query_start_loc, const int32_t* seq_lens,
                                   const int32_t* block_tables, int32_t max_blocks_per_req,
                                   const void* key_cache, const void* value_cache,
                                   int64_t num_blocks, const void* out, int64_t out_row_stride) {
  pa_status st = check_desc(desc);
  if (st != PA_OK) return st;
  if (req_begin < 0 || req_end < req_begin) return PA_ERR_INVALID_ARG;
  if (req_end - req_begin > kMaxGridYZ) return PA_ERR_UNSUPPORTED;
  if (req_end == req_begin) return PA_OK;
  if (!q || !query_start_loc || !seq_lens || !block_tables || !key_cache || !value_cache || !out) {
    return PA_ERR_INVALID_ARG;
  }
  if (max_blocks_per_req <= 0 || num_blocks <= 0) return PA_ERR_INVALID_ARG;
  const int64_t row = (int64_t)desc->num_q_heads * desc->head_dim;
  if (q_row_stride < row || out_row_stride < row) return PA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out) || !aligned16(key_cache) || !aligned16(value_cache)) {
    return PA_ERR_INVALID_ARG;
  }
  if ((q_row_stride * 2) % 16 != 0 || (out_row_stride * 2) % 16 != 0) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

static pa::AttnParams make_params(const pa_attn_desc* desc, int32_t req_begin, int32_t req_end,
                                  const void* q, int64_t q_row_stride,
                                  const int32_t* query_start_loc, const int32_t* seq_lens,
                                  const int32_t* block_tables, int32_t max_blocks_per_req,
                                  const void* key_cache, const void* value_cache,
                                  int64_t num_blocks, void* out, int64_t out_row_stride) {
  pa::AttnParams p{};
  p.num_q_heads = desc->num_q_heads;
  p.num_kv_heads = desc->num_kv_heads;
  p.group = desc->num_q_heads / desc->num_kv_heads;
  p.head_dim = desc->head_dim;
  p.req_begin = req_begin;
  p.num_reqs = req_end - req_begin;
  p.qsl = query_start_loc;
  p.seq_lens = seq_lens;
  p.block_tables = block_tables;
  p.max_blocks_per_req = max_blocks_per_req;
  p.q = q;
  p.q_row_stride = q_row_stride;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.num_blocks = num_blocks;
  p.out = out;
  p.out_row_stride = out_row_stride;
  p.scale_log2 = scale_log2(desc);
  p.v_scale = quantized(desc->cache_dtype) ? desc->v_scale : 1.0f;
  p.k_scales = desc->k_scales;
  p.v_scales = desc->v_scales;
  p.window_left = (desc->sliding_window > 0 && desc->sliding_window - 1 < pa::kNoWindow)
                      ? desc->sliding_window - 1
                      : pa::kNoWindow;
  p.alibi = desc->alibi_slopes;
  p.masked = desc->sliding_window > 0 || desc->alibi_slopes != nullptr;
  return p;
}

pa_status pa_decode_workspace_size(const pa_attn_desc* desc, int32_t num_reqs,
                                   int32_t max_seq_len, int32_t max_blocks_per_req,
                                   size_t* bytes) {
  pa_status st = check_desc(desc);
  if (st != PA_OK) return st;
  if (bytes == nullptr || num_reqs < 0 || max_seq_len < 0 || max_blocks_per_req < 0) {
    return PA_ERR_INVALID_ARG;
  }
  if (desc->num_q_heads / desc->num_kv_heads > 32) return PA_ERR_UNSUPPORTED;
  *bytes = num_reqs == 0 ? 0 : plan_decode(desc, num_reqs).ws_bytes;
  return PA_OK;
}

pa_status pa_decode(const pa_attn_desc* desc, int32_t req_begin, int32_t req_end, const void* q,
                    int64_t q_row_stride, const int32_t* query_start_loc, const int32_t* seq_lens,
                    const int32_t* block_tables, int32_t max_blocks_per_req,
                    const void* key_cache, const void* value_cache, int64_t num_blocks,
                    int32_t max_seq_len, void* workspace, size_t workspace_bytes, void* out,
                    int64_t out_row_stride, void* stream) {
  pa::DecodeCall call{};
  pa_status st = pa::decode_prepare(desc, req_begin, req_end, q, q_row_stride, query_start_loc,
                                    seq_lens, block_tables, max_blocks_per_req, key_cache,
                                    value_cache, num_blocks, max_seq_len, out, out_row_stride,
                                    &call);
  if (st != PA_OK || call.empty) return st;
  if (workspace == nullptr || workspace_bytes < call.ws_bytes) return PA_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(workspace)) return PA_ERR_INVALID_ARG;
  return pa::decode_launch(call, workspace, stream);
}

pa_status pa_prefill_varlen(const pa_attn_desc* desc, int32_t req_begin, int32_t req_end,
                            const void* q, int64_t q_row_stride, const int32_t* query_start_loc,
                            const int32_t* seq_lens, const int32_t* block_tables,
                            int32_t max_blocks_per_req, const void* key_cache,
                            const void* value_cache, int64_t num_blocks, int32_t max_query_len,
                            int32_t max_seq_len, void* out, int64_t out_row_stride,
                            void* stream) {
  pa_status st = check_attn_common(desc, req_begin, req_end, q, q_row_stride, query_start_loc,
                                   seq_lens, block_tables, max_blocks_per_req, key_cache,
                                   value_cache, num_blocks, out, out_row_stride);
  if (st != PA_OK) return st;
  if (max_query_len < 0 || max_seq_len < 0) return PA_ERR_INVALID_ARG;
  if (max_seq_len > kMaxSeqLen) return PA_ERR_UNSUPPORTED;
  if (req_end == req_begin || max_query_len == 0) return PA_OK;
  pa::AttnParams p = make_params(desc, req_begin, req_end, q, q_row_stride, query_start_loc,
                                 seq_lens, block_tables, max_blocks_per_req, key_cache,
                                 value_cache, num_blocks, out, out_row_stride);
  p.max_seq_len = max_seq_len;
  p.max_query_len = max_query_len;
  return from_hip(pa::launch_prefill(p, desc->act_dtype, desc->cache_dtype,
                                     static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace pa {

pa_status decode_prepare(const pa_attn_desc* desc, int32_t req_begin, int32_t req_end,
                         const void* q, int64_t q_row_stride, const int32_t* query_start_loc,
                         const int32_t* seq_lens, const int32_t* block_tables,
                         int32_t max_blocks_per_req, const void* key_cache,
                         const void* value_cache, int64_t num_blocks, int32_t max_seq_len,
                         void* out, int64_t out_row_stride, DecodeCall* call) {
  pa_status st = check_attn_common(desc, req_begin, req_end, q, q_row_stride, query_start_loc,
                                   seq_lens, block_tables, max_blocks_per_req, key_cache,
                                   value_cache, num_blocks, out, out_row_stride);
  if (st != PA_OK) return st;
  if (max_seq_len < 0) return PA_ERR_INVALID_ARG;
  if (max_seq_len > kMaxSeqLen) return PA_ERR_UNSUPPORTED;
  if (desc->num_q_heads / desc->num_kv_heads > 32) return PA_ERR_UNSUPPORTED;
  const int num_reqs = req_end - req_begin;
  call->empty = num_reqs == 0;
  if (call->empty) return PA_OK;
  const DecodePlan pl = plan_decode(desc, num_reqs);
  // the kernel keeps a block's byte offset in 32 bits and each worker's share
  // of the (request, K/V head, block) stream below 2^31 units
  if ((int64_t)16 * desc->num_kv_heads * desc->head_dim * elem_bytes(desc->cache_dtype) > 0xFFFFFFFFll) {
    return PA_ERR_UNSUPPORTED;
  }
  if ((double)num_reqs * desc->num_kv_heads * max_blocks_per_req >
      (double)pl.workers * 2147483647.0) {
    return PA_ERR_UNSUPPORTED;
  }
  call->p = make_params(desc, req_begin, req_end, q, q_row_stride, query_start_loc, seq_lens,
                        block_tables, max_blocks_per_req, key_cache, value_cache, num_blocks, out,
                        out_row_stride);
  call->p.max_seq_len = max_seq_len;
  call->p.num_workers = pl.workers;
  call->p.wg_waves = pl.wg_waves;
  call->cum_off = pl.cum_off;
  call->acc_off = pl.acc_off;
  call->ml_off = pl.ml_off;
  call->facc_off = pl.facc_off;
  call->ws_bytes = pl.ws_bytes;
  call->act_dtype = desc->act_dtype;
  call->cache_dtype = desc->cache_dtype;
  return PA_OK;
}

pa_status decode_launch(const DecodeCall& call, void* workspace, void* stream) {
  AttnParams p = call.p;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  p.ws_cum = reinterpret_cast<int64_t*>(ws + call.cum_off);
  p.ws_acc = reinterpret_cast<float*>(ws + call.acc_off);
  p.ws_ml = reinterpret_cast<float*>(ws + call.ml_off);
  p.ws_facc = reinterpret_cast<float*>(ws + call.facc_off);
  return from_hip(launch_decode(p, call.act_dtype, call.cache_dtype,
                                static_cast<hipStream_t>(stream)));
}

}  // namespace pa
