// The two halves of a pa_decode call, shared by the entry points that take a
// caller's workspace (pa_decode) and the one that uses the library's own
// device scratch array (pa_decode_noalloc).  Internal to libpa.so.
#pragma once

#include "pa.h"
#include "pa_kernels.h"

namespace pa {

// Every host-side check of pa_decode except the workspace's; fills `call`
// (call->empty when the range holds no request).  Launches nothing; the only
// runtime calls are device queries (the compute-unit count).
pa_status decode_prepare(const pa_attn_desc* desc, int32_t req_begin, int32_t req_end,
                         const void* q, int64_t q_row_stride, const int32_t* query_start_loc,
                         const int32_t* seq_lens, const int32_t* block_tables,
                         int32_t max_blocks_per_req, const void* key_cache,
                         const void* value_cache, int64_t num_blocks, int32_t max_seq_len,
                         void* out, int64_t out_row_stride, DecodeCall* call);

// Enqueue the decode kernels of a prepared call on `stream` with `workspace`
// (device memory of at least call.ws_bytes, 16-byte aligned).
pa_status decode_launch(const DecodeCall& call, void* workspace, void* stream);

}  // namespace pa
