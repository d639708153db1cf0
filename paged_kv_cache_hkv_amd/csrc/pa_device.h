// Device-side building blocks shared by the paged-attention kernels (gfx950).
//
// Wave64 everywhere.  MFMA operand layouts used below (CDNA3/CDNA4 matrix
// cores, lane l of a wave):
//   v_mfma_f32_16x16x32_{bf16,f16}: A[i][k] in lane (i + 16*(k/8)), element k%8;
//     B[k][j] in lane (j + 16*(k/8)), element k%8; D[i][j] in lane (j + 16*(i/4)),
//     register i%4.
//   v_mfma_f32_32x32x16_{bf16,f16}: A[i][k] in lane (i + 32*(k/8)), element k%8;
//     B[k][j] in lane (j + 32*(k/8)), element k%8; D[i][j] in lane (j + 32*((i/4)%2)),
//     register 4*(i/8) + i%4.
// Only the D layout matters for correctness of a product whose K ordering is a
// permutation both operands share; every kernel here builds A and B with the
// same K permutation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// ---- compute-type traits: bf16 or fp16 MFMA --------------------------------
template <typename T> struct Mfma;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

template <> struct Mfma<__bf16> {
  typedef bf16x8 vec8;
  __device__ static inline f32x4 mma16(const vec8& a, const vec8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // v_mfma_f32_16x16x16_bf16: A[i][k] in lane (i + 16*(k/4)), element k%4
  // (two packed dwords); B likewise; D as for 16x16x32.
  __device__ static inline f32x4 mma16k16(u32x2 a, u32x2 b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  }
  __device__ static inline f32x16 mma32(const vec8& a, const vec8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // two fp8 (e4m3fn) codes from 16-bit word `word` of `src` -> two exact values
  __device__ static inline unsigned from_fp8x2(unsigned src, bool hi_word) {
    bf16x2 v = hi_word ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, 1.0f, true)
                       : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, 1.0f, false);
    return __builtin_bit_cast(unsigned, v);
  }
  __device__ static inline unsigned short from_float(float f) {
    return __builtin_bit_cast(unsigned short, (__bf16)f);
  }
  // acc + lo + hi of a dword holding two bf16 values (v_dot2c_f32_bf16 by ones)
  __device__ static inline float sum2(unsigned pk, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), one, acc, false);
  }
  __device__ static inline float to_float(unsigned short b) {
    return __builtin_bit_cast(float, ((unsigned)b) << 16);
  }
};

template <> struct Mfma<_Float16> {
  typedef f16x8 vec8;
  __device__ static inline f32x4 mma16(const vec8& a, const vec8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static inline f32x4 mma16k16(u32x2 a, u32x2 b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  __device__ static inline f32x16 mma32(const vec8& a, const vec8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static inline unsigned from_fp8x2(unsigned src, bool hi_word) {
    f16x2 v = hi_word ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src, 1.0f, true)
                      : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src, 1.0f, false);
    return __builtin_bit_cast(unsigned, v);
  }
  __device__ static inline unsigned short from_float(float f) {
    return __builtin_bit_cast(unsigned short, (_Float16)f);
  }
  __device__ static inline float sum2(unsigned pk, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk), one, acc, false);
  }
  __device__ static inline float to_float(unsigned short b) {
    return (float)__builtin_bit_cast(_Float16, b);
  }
};

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Pack two floats into one dword of two 16-bit compute-type values (lo, hi),
// round to nearest even: one v_cvt_pk_{bf16,f16}_f32.
template <typename T>
__device__ inline unsigned pack2(float lo, float hi) {
  typedef T t2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{lo, hi}, t2));
}

// Two 8-bit cache codes -- bytes 2*hi and 2*hi+1 of src -- widened exactly to
// two 16-bit values of T (one dword, low value first): OCP e4m3fn codes with
// the packed gfx950 convert, or symmetric int8 codes (every integer in
// -127..127 is exact in bf16 and fp16).  The cache scale is applied elsewhere.
template <typename T, bool I8>
__device__ inline unsigned widen8x2(unsigned src, bool hi_word) {
  if constexpr (I8) {
    const int sh = hi_word ? 16 : 0;
    const float a = (float)(int)(signed char)(src >> sh);
    const float b = (float)(int)(signed char)(src >> (sh + 8));
    return pack2<T>(a, b);
  } else {
    return Mfma<T>::from_fp8x2(src, hi_word);
  }
}

// float32 -> symmetric int8 code (two's complement byte): round to nearest
// even, saturating to +-127 (-128 is never produced); NaN gives 0.  Clamping
// first and rounding second equals rounding first and saturating second
// because +-127 are integers.
__device__ inline unsigned encode_int8(float y) {
  if (!(y == y)) return 0u;
  const float r = __builtin_rintf(fminf(fmaxf(y, -127.f), 127.f));
  return (unsigned)(int)r & 0xFFu;
}

// 2^x with the hardware v_exp_f32 (results below 2^-126 flush to zero, which
// only ever affects softmax weights that are negligible against the max).
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Byte permute: result byte k = byte sel.k of the 8-byte value {hi:lo}.
__device__ inline unsigned perm(unsigned hi, unsigned lo, unsigned sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Wave-wide shuffles (ds_bpermute based).
__device__ inline float shfl(float v, int src_lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src_lane << 2, __builtin_bit_cast(int, v)));
}
__device__ inline float shfl_xor(float v, int mask) {
  int lane = __lane_id();
  return shfl(v, lane ^ mask);
}

// max / sum of a value over lanes l and l ^ 32.
__device__ inline float pair32_max(float v) { return fmaxf(v, shfl_xor(v, 32)); }
__device__ inline float pair32_sum(float v) { return v + shfl_xor(v, 32); }
// The same with v_permlane32_swap (gfx950): no LDS round trip.  With both
// operands equal, the two results hold the low and the high half of the wave
// broadcast over both halves, so combining them gives every lane the value of
// its pair, bit-identical in both lanes.
// max of three floats in one instruction.  Written out because the builtin
// fmaxf first quiets each operand the compiler cannot prove canonical (one
// extra v_max_f32 x, x per MFMA result); v_max3_f32 follows the same maxNum
// rule for quiet NaNs and -inf.
__device__ inline float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ inline float pair32_max_swap(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ inline float pair32_sum_swap(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

__device__ inline int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Read a wave-uniform element of a table the kernel never writes (block
// tables, query_start_loc, seq_lens) through the constant address space: a
// scalar load, counted by lgkmcnt, so waiting for it never waits for vector
// loads or LDS transfers still in flight.
__device__ inline int32_t load_uniform(const int32_t* table, int64_t idx) {
  typedef __attribute__((address_space(4))) const int32_t const_i32;
  const const_i32* p = (const const_i32*)(table);
  return p[idx];
}

// Per-K/V-head scale h of a quantized cache (a scalar load of a wave-uniform
// entry, so it never waits for vector loads or LDS transfers in flight).
__device__ inline float head_scale(const float* scales, int h) {
  return __builtin_bit_cast(float, load_uniform(reinterpret_cast<const int32_t*>(scales),
                                                __builtin_amdgcn_readfirstlane(h)));
}

// Byte offset of an LDS location (the M0 / ds address of a __shared__ pointer).
__device__ inline unsigned lds_offset(const void* p) {
  typedef __attribute__((address_space(3))) const void lds_cvoid;
  return (unsigned)(uintptr_t)(lds_cvoid*)p;
}

// Asynchronous global -> LDS copy of 16 bytes per lane: lane l's bytes at
// base + voff (voff per lane, base wave-uniform) land at LDS byte
// m0 + 16 * l (m0 wave-uniform).  Issued from inline assembly so that the
// compiler does not track it: it would otherwise make every LDS read wait for
// every transfer in flight, as it cannot tell ring stages apart.  The caller
// orders the transfers itself: a transfer into a buffer is issued only after
// the reads of the buffer's previous contents have returned (the leading
// lgkmcnt wait covers those still in flight), and the buffer is read only
// after wait_vmcnt has retired the transfer.  The compiler's own vector loads
// stay safe: transfers it does not count only make its counted waits stricter.
// NT: non-temporal (data read once, e.g. a K/V stream): measurably higher
// HBM throughput for streams that are not re-read.
// WAIT_LDS = false drops the leading lgkmcnt wait, for callers whose own
// barriers already order the copy after every read of the buffer's previous
// contents (scalar loads in flight are then not waited for either).
template <bool NT = false, bool WAIT_LDS = true>
__device__ inline void lds_dma16(const void* base, unsigned voff, unsigned m0) {
  if constexpr (!WAIT_LDS && NT) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1 nt"
        :
        : "v"(voff), "s"(base), "s"(m0)
        : "memory");
  } else if constexpr (!WAIT_LDS) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(base), "s"(m0)
        : "memory");
  } else if constexpr (NT) {
    asm volatile(
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1 nt"
        :
        : "v"(voff), "s"(base), "s"(m0)
        : "memory");
  } else {
    asm volatile(
        "s_waitcnt lgkmcnt(0)\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(base), "s"(m0)
        : "memory");
  }
}

// Wait until at most N vector-memory operations of this wave are in flight
// (asynchronous LDS copies included); a compiler barrier for memory as well.
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// float32 -> OCP e4m3fn code, round to nearest even, saturating to +-448,
// NaN kept (integer code on the float32 bit pattern).
__device__ inline unsigned encode_e4m3fn(float y) {
  const unsigned bits = __builtin_bit_cast(unsigned, y);
  const unsigned sign = (bits >> 24) & 0x80u;
  const unsigned abits = bits & 0x7FFFFFFFu;
  if (abits > 0x7F800000u) return sign | 0x7Fu;           // NaN
  if (abits >= 0x43E00000u) return sign | 0x7Eu;          // |y| >= 448 (and inf): saturate
  if (abits < 0x3C800000u) {                              // |y| < 2^-6: subnormal grid 2^-9
    const float a = __builtin_bit_cast(float, abits);
    const float q = __builtin_rintf(a * 512.0f);          // exact scaling, RNE
    return sign | (unsigned)q;                            // q in 0..8; 8 is 2^-6 (code 0x08)
  }
  // normal: keep 3 mantissa bits, round to nearest even on the dropped 20 bits
  const unsigned lsb = (abits >> 20) & 1u;
  const unsigned r = (abits + 0x7FFFFu + lsb) & ~0xFFFFFu;
  const int e = (int)(r >> 23) - 127;                     // -6 .. 8
  const unsigned m = (r >> 20) & 7u;
  return sign | ((unsigned)(e + 7) << 3) | m;
}

// 16-byte and 8-byte global loads / stores.
__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ inline unsigned ld4(const void* p) { return *reinterpret_cast<const unsigned*>(p); }
__device__ inline void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ inline void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

}  // namespace pa
