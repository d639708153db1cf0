// pa_decode_noalloc: pa_decode on a device scratch array that belongs to the
// library, for callers that cannot allocate (code under graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The array lives for the whole process, one copy per GPU (each device's
// copy of a __device__ variable sits at its own address).  Host code never
// passes the array's name to a kernel or a memory call: in host code that
// name is a host-side stand-in, not a device address.  Instead the device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) on the entry point's first call there, and kept.
//
// The decode kernels need no zeroed workspace (every partial they read was
// written in the same call), so nothing is cleared here; the array keeps the
// last call's contents.  Every call on one GPU shares its array: two calls
// whose work overlaps on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa.h"
#include "pa_decode_call.h"

namespace {

constexpr size_t kScratchBytes = PA_DECODE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::once_flag g_once[kMaxDevices];
void* g_addr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// Device address of this device's scratch array (looked up once per device).
pa_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return PA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  std::call_once(g_once[dev], [dev]() {
    void* ptr = nullptr;
    g_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_addr[dev] = g_err[dev] == hipSuccess ? ptr : nullptr;
    if (g_err[dev] != hipSuccess) (void)hipGetLastError();
  });
  if (g_err[dev] != hipSuccess || g_addr[dev] == nullptr) return PA_ERR_HIP;
  *out = g_addr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_decode_noalloc(const pa_attn_desc* desc, int32_t req_begin, int32_t req_end,
                            const void* q, int64_t q_row_stride, const int32_t* query_start_loc,
                            const int32_t* seq_lens, const int32_t* block_tables,
                            int32_t max_blocks_per_req, const void* key_cache,
                            const void* value_cache, int64_t num_blocks, int32_t max_seq_len,
                            void* out, int64_t out_row_stride, void* stream) {
  pa::DecodeCall call{};
  pa_status st = pa::decode_prepare(desc, req_begin, req_end, q, q_row_stride, query_start_loc,
                                    seq_lens, block_tables, max_blocks_per_req, key_cache,
                                    value_cache, num_blocks, max_seq_len, out, out_row_stride,
                                    &call);
  if (st != PA_OK || call.empty) return st;
  // a call that needs more than the fixed array is refused before any device work
  if (call.ws_bytes > kScratchBytes) return PA_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != PA_OK) return st;
  return pa::decode_launch(call, ws, stream);
}

}  // extern "C"
