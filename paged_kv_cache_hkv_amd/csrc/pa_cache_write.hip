// pa_cache_write kernel: the slot_mapping scatter (reshape_and_cache in
// "vLLM 推理全流程深度解析"; reshape_and_cache_flash in stop 10 of "Tour: One
// forward pass").
//
// A token's [num_kv_heads, head_dim] row is contiguous both in the input
// (modulo the row stride) and in the cache (a slot is one row of the
// [num_blocks, block_size, Hkv, D] pool), so the scatter is a row copy.  Each
// thread moves 8 elements: one 16-byte load and one 16-byte store (8-byte
// store for fp8).  The flat thread index runs over (token, 8-element chunk)
// pairs so consecutive lanes touch consecutive bytes of one row; blockIdx.y
// picks key or value.  Negative slots (padding) and slots past the pool are
// skipped, so no address outside the pool is formed.
//
// fp8 encode (OCP e4m3fn) is integer code of our own: y = float32(x) * inv_scale
// in one float32 multiply, then round-to-nearest-even on the float32 bit
// pattern with saturation to +-448 and NaN kept.  int8 encode: the same y,
// rounded to the nearest even integer with saturation to +-127, NaN -> 0.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ inline float elem_to_float(unsigned short b) { return Mfma<T>::to_float(b); }

// eight elements -> eight 8-bit codes (ENC 1: fp8 e4m3fn, 2: int8)
template <typename T, int ENC>
__device__ inline u32x2 encode8(const u32x4& v, float inv) {
  unsigned out[2] = {0u, 0u};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const unsigned w = v[k >> 1];
    const unsigned short h = (unsigned short)((k & 1) ? (w >> 16) : (w & 0xFFFFu));
    const float y = elem_to_float<T>(h) * inv;
    const unsigned code = ENC == 2 ? encode_int8(y) : encode_e4m3fn(y);
    out[k >> 2] |= code << (8 * (k & 3));
  }
  return u32x2{out[0], out[1]};
}

// ENC: 0 copy (cache in the activation dtype), 1 fp8 e4m3fn, 2 int8
template <typename T, int ENC>
__global__ __launch_bounds__(kThreads) void cache_write_kernel(CacheWriteParams p) {
  const bool is_v = blockIdx.y != 0;
  const int vec_per_row = p.row_elems >> 3;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t total = p.num_tokens * vec_per_row;
  if (idx >= total) return;
  const int64_t t = idx / vec_per_row;
  const int c = (int)(idx - t * vec_per_row);
  const int64_t slot = p.slot_mapping[t];
  if (slot < 0 || slot >= p.num_slots) return;
  const unsigned short* src = static_cast<const unsigned short*>(is_v ? p.value : p.key);
  const int64_t stride = is_v ? p.value_row_stride : p.key_row_stride;
  const u32x4 v = ld16(src + t * stride + (int64_t)c * 8);
  // cache row of the slot: [block, offset] flattened = slot
  const int64_t dst_elem = slot * p.row_elems + (int64_t)c * 8;
  if constexpr (ENC != 0) {
    unsigned char* dst = static_cast<unsigned char*>(is_v ? p.value_cache : p.key_cache);
    float inv = is_v ? p.v_inv_scale : p.k_inv_scale;
    const float* hs = is_v ? p.v_scales : p.k_scales;
    if (hs != nullptr) inv = 1.0f / hs[(c * 8) / p.head_dim];   // IEEE division: the host's reciprocal
    st8(dst + dst_elem, encode8<T, ENC>(v, inv));
  } else {
    unsigned short* dst = static_cast<unsigned short*>(is_v ? p.value_cache : p.key_cache);
    st16(dst + dst_elem, v);
  }
}

template <typename T, int ENC>
hipError_t launch_typed(const CacheWriteParams& p, hipStream_t stream) {
  const int64_t total = p.num_tokens * (p.row_elems >> 3);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((cache_write_kernel<T, ENC>), dim3((unsigned)blocks, 2), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteParams& p, int act_dtype, int cache_dtype,
                              hipStream_t stream) {
  if (act_dtype == kF16 && cache_dtype == kF16) return launch_typed<_Float16, 0>(p, stream);
  if (act_dtype == kBF16 && cache_dtype == kBF16) return launch_typed<__bf16, 0>(p, stream);
  if (act_dtype == kF16 && cache_dtype == kFP8) return launch_typed<_Float16, 1>(p, stream);
  if (act_dtype == kBF16 && cache_dtype == kFP8) return launch_typed<__bf16, 1>(p, stream);
  if (act_dtype == kF16 && cache_dtype == kINT8) return launch_typed<_Float16, 2>(p, stream);
  if (act_dtype == kBF16 && cache_dtype == kINT8) return launch_typed<__bf16, 2>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
