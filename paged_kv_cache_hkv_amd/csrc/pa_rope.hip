// pa_rope_cache_write kernel: rotary position embedding of Q and K fused with
// the slot_mapping scatter of K and V.
//
// What is computed ("Tour: One forward pass", stop 9: RoPE turns q and k by
// each token's position from stop 3, with the per-position cosines and sines
// of cos_sin_cache applied to every head's pairs; stop 10: the cache write of
// K and V; the same order in the LlamaAttention listing of "vLLM 推理全流程深度解析"):
// for token t at position p with cos_sin_cache[p] = (c_0..c_{R/2-1},
// s_0..s_{R/2-1}), R = rotary_dim, every head of q and k has its pairs
// (j, j + R/2) (half-split layout) or (2j, 2j+1) (interleaved) rotated:
//     a' = a*c_j - b*s_j,   b' = b*c_j + a*s_j
// in float32 with every product and every sum rounded once (no fused
// multiply-add, so the result is the same on any IEEE float32 machine), then
// rounded to the activation dtype.  Dimensions from R on are unchanged.  q is
// rotated in place; the rotated k (already rounded to the activation dtype)
// and v are written to the cache exactly as pa_cache_write writes them, so the
// fusion changes nothing stored -- it saves the round trip of the rotated K
// through HBM before the scatter.
//
// Work decomposition: one thread per 16-byte unit of work of a token: a
// rotation unit covers 8 pairs (two 16-byte chunks of one head: the chunk and
// its partner R/2 elements on for the half-split layout, two adjacent chunks
// for the interleaved one) plus their 8 cos and 8 sin; a copy unit is one
// 16-byte chunk of K past R, or of V.  Per token: Hq*R/16 query rotations,
// Hkv*R/16 key rotations, Hkv*(D-R)/8 key copies, Hkv*D/8 value copies.
// Tokens whose position is outside the table are left alone; tokens whose
// slot is negative or past the pool have their query rotated and nothing
// written.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kThreads = 256;

// float32 rotation of 8 pairs held as two 8-element 16-bit vectors
template <typename T>
__device__ inline void rotate8(const u32x4& xa, const u32x4& xb, const float* c, const float* s,
                               bool neox, u32x4& ya, u32x4& yb) {
  using M = Mfma<T>;
  float a[8], b[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (neox) {
      // pair k: element k of the first chunk and element k of its partner
      a[k] = M::to_float((unsigned short)(xa[k >> 1] >> (16 * (k & 1))));
      b[k] = M::to_float((unsigned short)(xb[k >> 1] >> (16 * (k & 1))));
    } else {
      // pair k: elements 2k, 2k+1 of the 16-element run xa|xb
      const u32x4& x = (k < 4) ? xa : xb;
      const unsigned w = x[k & 3];
      a[k] = M::to_float((unsigned short)(w & 0xFFFFu));
      b[k] = M::to_float((unsigned short)(w >> 16));
    }
  }
  float ra[8], rb[8];
  {
    // each product and each sum rounded on its own: no contraction to fma
#pragma clang fp contract(off)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float ac = a[k] * c[k], bs = b[k] * s[k];
      const float bc = b[k] * c[k], as = a[k] * s[k];
      ra[k] = ac - bs;
      rb[k] = bc + as;
    }
  }
  if (neox) {
    ya = u32x4{pack2<T>(ra[0], ra[1]), pack2<T>(ra[2], ra[3]), pack2<T>(ra[4], ra[5]), pack2<T>(ra[6], ra[7])};
    yb = u32x4{pack2<T>(rb[0], rb[1]), pack2<T>(rb[2], rb[3]), pack2<T>(rb[4], rb[5]), pack2<T>(rb[6], rb[7])};
  } else {
    ya = u32x4{pack2<T>(ra[0], rb[0]), pack2<T>(ra[1], rb[1]), pack2<T>(ra[2], rb[2]), pack2<T>(ra[3], rb[3])};
    yb = u32x4{pack2<T>(ra[4], rb[4]), pack2<T>(ra[5], rb[5]), pack2<T>(ra[6], rb[6]), pack2<T>(ra[7], rb[7])};
  }
}

// 8 activation-dtype elements -> 8 codes of value * inv (ENC 1: e4m3fn,
// 2: int8, as the cache write encodes them)
template <typename T, int ENC>
__device__ inline u32x2 encode8(const u32x4& v, float inv) {
  unsigned out[2] = {0u, 0u};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const unsigned short h = (unsigned short)(v[k >> 1] >> (16 * (k & 1)));
    const float y = Mfma<T>::to_float(h) * inv;
    out[k >> 2] |= (ENC == 2 ? encode_int8(y) : encode_e4m3fn(y)) << (8 * (k & 3));
  }
  return u32x2{out[0], out[1]};
}

// The inverse scale K/V head h is encoded with: the tensor's, or with
// per-head scales the IEEE float32 reciprocal of the head's (the value the
// host computes for a tensor scale)
template <int ENC>
__device__ inline float head_inv(const float* scales, int h, float tensor_inv) {
  if constexpr (ENC == 0) return tensor_inv;
  return scales != nullptr ? 1.0f / scales[h] : tensor_inv;
}

// ENC: 0 copy (cache in the activation dtype), 1 fp8 e4m3fn, 2 int8
template <typename T, int ENC>
__device__ inline void store_chunk(void* cache, int64_t elem, const u32x4& v, float inv) {
  if constexpr (ENC != 0) {
    st8(static_cast<unsigned char*>(cache) + elem, encode8<T, ENC>(v, inv));
  } else {
    st16(static_cast<unsigned short*>(cache) + elem, v);
  }
}

template <typename T, int ENC>
__global__ __launch_bounds__(kThreads) void rope_cache_write_kernel(RopeParams p) {
  const int D = p.head_dim, R = p.rotary_dim;
  const int R16 = R >> 4, P8 = (D - R) >> 3, D8 = D >> 3;
  const int Hq = p.num_q_heads, Hkv = p.num_kv_heads;
  const int uq = Hq * R16, uk = Hkv * R16, ukp = Hkv * P8, uv = Hkv * D8;
  const int per_token = uq + uk + ukp + uv;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= p.num_tokens * per_token) return;
  const int64_t t = idx / per_token;
  int u = (int)(idx - t * per_token);
  const int64_t pos = p.positions[t];
  if (pos < 0 || pos >= p.max_position) return;
  const int64_t slot = p.slot_mapping[t];
  const bool write = slot >= 0 && slot < p.num_slots;
  const int64_t row = (int64_t)Hkv * D;   // cache elements per slot

  if (u < uq + uk) {
    // ---- rotation unit: head h, pairs 8c .. 8c+7 ----
    const bool is_q = u < uq;
    if (!is_q) u -= uq;
    const int h = u / R16, c = u % R16;
    if (!is_q && !write) return;
    const bool neox = p.is_neox != 0;
    const int ea = neox ? 8 * c : 16 * c;            // first chunk
    const int eb = neox ? R / 2 + 8 * c : 16 * c + 8; // second chunk
    const float* cs = p.cos_sin + pos * R;
    float cv[8], sv[8];
    {
      // whole-vector casts: clang's bit cast of a single vector element
      // reads element 0
      const f32x4 c0 = __builtin_bit_cast(f32x4, ld16(cs + 8 * c));
      const f32x4 c1 = __builtin_bit_cast(f32x4, ld16(cs + 8 * c + 4));
      const f32x4 s0 = __builtin_bit_cast(f32x4, ld16(cs + R / 2 + 8 * c));
      const f32x4 s1 = __builtin_bit_cast(f32x4, ld16(cs + R / 2 + 8 * c + 4));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        cv[k] = c0[k];
        cv[4 + k] = c1[k];
        sv[k] = s0[k];
        sv[4 + k] = s1[k];
      }
    }
    unsigned short* base;
    if (is_q) {
      base = static_cast<unsigned short*>(p.query) + t * p.query_row_stride + (int64_t)h * D;
    } else {
      base = const_cast<unsigned short*>(static_cast<const unsigned short*>(p.key)) +
             t * p.key_row_stride + (int64_t)h * D;
    }
    const u32x4 xa = ld16(base + ea), xb = ld16(base + eb);
    u32x4 ya, yb;
    rotate8<T>(xa, xb, cv, sv, neox, ya, yb);
    if (is_q) {
      st16(base + ea, ya);
      st16(base + eb, yb);
    } else {
      const int64_t dst = slot * row + (int64_t)h * D;
      const float inv = head_inv<ENC>(p.k_scales, h, p.k_inv_scale);
      store_chunk<T, ENC>(p.key_cache, dst + ea, ya, inv);
      store_chunk<T, ENC>(p.key_cache, dst + eb, yb, inv);
    }
    return;
  }
  if (!write) return;
  u -= uq + uk;
  if (u < ukp) {
    // ---- key chunk past the rotated dimensions: copied ----
    const int h = u / P8, e = R + 8 * (u % P8);
    const unsigned short* src = static_cast<const unsigned short*>(p.key) + t * p.key_row_stride +
                                (int64_t)h * D + e;
    store_chunk<T, ENC>(p.key_cache, slot * row + (int64_t)h * D + e, ld16(src),
                        head_inv<ENC>(p.k_scales, h, p.k_inv_scale));
    return;
  }
  u -= ukp;
  {
    // ---- value chunk: copied ----
    const int h = u / D8, e = 8 * (u % D8);
    const unsigned short* src = static_cast<const unsigned short*>(p.value) + t * p.value_row_stride +
                                (int64_t)h * D + e;
    store_chunk<T, ENC>(p.value_cache, slot * row + (int64_t)h * D + e, ld16(src),
                        head_inv<ENC>(p.v_scales, h, p.v_inv_scale));
  }
}

template <typename T, int ENC>
hipError_t launch_typed(const RopeParams& p, hipStream_t stream) {
  const int R16 = p.rotary_dim >> 4, P8 = (p.head_dim - p.rotary_dim) >> 3, D8 = p.head_dim >> 3;
  const int64_t per_token = (int64_t)p.num_q_heads * R16 + (int64_t)p.num_kv_heads * (R16 + P8 + D8);
  const int64_t total = p.num_tokens * per_token;
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((rope_cache_write_kernel<T, ENC>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_cache_write(const RopeParams& p, int act_dtype, int cache_dtype,
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
