// pa_prefill_varlen kernel: causal attention of prefill / chunked-prefill
// requests over the paged cache.
//
// What is computed (flash_attn_varlen_func in stop 10 of "Tour: One forward
// pass", driven by cu_seqlens_q = query_start_loc, seqused_k = seq_lens and
// the block table): request r has n new tokens at batch rows qsl[r] .. and
// c = seq_lens[r] - n cached ones; its query i (position c + i) attends keys
// 0 .. c + i through block_table[r].  Query head h reads K/V head h / G.
// The scores never leave the chip: softmax and both products are done tile by
// tile in registers and LDS ("vLLM 推理全流程深度解析", FlashAttention keeps
// softmax and matmul in on-chip memory and never writes the score matrix out).
//
// Work decomposition.  A workgroup of 4 waves owns (request, K/V head, group
// of `hpw` query heads of that K/V head, tile of 128/hpw queries); wave w
// takes query head w % hpw and 32 queries.  All 4 waves share each 64-key
// K/V tile, staged through LDS:
//   * Ks[key][d] row-major (row padded by 16 bytes, conflict-free 16-byte
//     reads of 32 different rows);
//   * Vt[d][key'] transposed, key' = key with bits 2 and 3 swapped, so the 8
//     keys one lane feeds into one MFMA step are adjacent (one 16-byte read).
// Per tile a wave computes S^T = K . Q^T (v_mfma_f32_32x32x16, keys x queries)
// so each lane holds 32 scores of ONE query: the row max needs one exchange
// with the lane 32 apart and the rescale of the O^T accumulator is
// lane-local.  The scores, as bf16/fp16, are directly the B operand of
// O^T = V^T . P^T.  The next tile's global loads are issued before the
// current tile's math, into registers, and written to LDS after it.
// fp8 caches are widened to bf16/fp16 when the tile is written to LDS.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlock = 16;
constexpr int kTileK = 64;   // keys per LDS tile

__device__ inline int swap_bits23(int k) {
  return (k & ~0xC) | ((k & 0x4) << 1) | ((k & 0x8) >> 1);
}

template <int D, typename CT, int KVB>
struct TileRegs {
  // 16-byte chunks of K and V this thread moves per tile
  static constexpr int kElemsPerChunk = 16 / KVB;                 // 8 (2-byte) or 16 (fp8)
  static constexpr int kChunksPerRow = D / kElemsPerChunk;
  static constexpr int kChunks = kTileK * kChunksPerRow / kThreads;
  u32x4 k[kChunks];
  u32x4 v[kChunks];
};

template <int D, typename CT, int KVB>
__device__ inline void load_tile(TileRegs<D, CT, KVB>& regs, const AttnParams& p,
                                 const int32_t* bt_row, int nblk, int s_eff, int kt, int kvh) {
  using R = TileRegs<D, CT, KVB>;
  const unsigned char* kc = static_cast<const unsigned char*>(p.key_cache);
  const unsigned char* vc = static_cast<const unsigned char*>(p.value_cache);
  const int64_t tok_stride = (int64_t)p.num_kv_heads * D * KVB;
  const int64_t blk_stride = tok_stride * kBlock;
#pragma unroll
  for (int c = 0; c < R::kChunks; ++c) {
    const int idx = threadIdx.x + kThreads * c;
    const int key = idx / R::kChunksPerRow;
    const int dc = idx % R::kChunksPerRow;
    const int bi = kt * (kTileK / kBlock) + key / kBlock;
    int b = -1;
    if (bi < nblk) b = bt_row[bi];
    // keys past the sequence may hold anything (the tail of the last block):
    // load zeros so that 0-probability keys cannot turn P.V into NaN
    if (b >= 0 && (int64_t)b < p.num_blocks && kt * kTileK + key < s_eff) {
      const int64_t off = (int64_t)b * blk_stride + (int64_t)(key % kBlock) * tok_stride +
                          (int64_t)kvh * D * KVB + (int64_t)dc * 16;
      regs.k[c] = ld16(kc + off);
      regs.v[c] = ld16(vc + off);
    } else {
      regs.k[c] = u32x4{0u, 0u, 0u, 0u};   // absent block: zeros, and masked
      regs.v[c] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <int D, typename CT, int KVB>
__device__ inline void store_tile(const TileRegs<D, CT, KVB>& regs, unsigned short* Ks,
                                  unsigned short* Vt) {
  using R = TileRegs<D, CT, KVB>;
  using M = Mfma<CT>;
  constexpr int KROW = D + 8;        // Ks row stride (elements)
  constexpr int VROW = kTileK + 8;   // Vt row stride (elements)
#pragma unroll
  for (int c = 0; c < R::kChunks; ++c) {
    const int idx = threadIdx.x + kThreads * c;
    const int key = idx / R::kChunksPerRow;
    const int dc = idx % R::kChunksPerRow;
    const int d0 = dc * R::kElemsPerChunk;
    const int kp = swap_bits23(key);
    if constexpr (KVB == 2) {
      *reinterpret_cast<u32x4*>(Ks + key * KROW + d0) = regs.k[c];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const unsigned w = regs.v[c][e >> 1];
        Vt[(d0 + e) * VROW + kp] = (unsigned short)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
      }
    } else {
      u32x4 lo, hi;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const unsigned w0 = regs.k[c][2 * h], w1 = regs.k[c][2 * h + 1];
        u32x4 o{M::from_fp8x2(w0, false), M::from_fp8x2(w0, true),
                M::from_fp8x2(w1, false), M::from_fp8x2(w1, true)};
        if (h == 0) lo = o; else hi = o;
      }
      *reinterpret_cast<u32x4*>(Ks + key * KROW + d0) = lo;
      *reinterpret_cast<u32x4*>(Ks + key * KROW + d0 + 8) = hi;
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) {
        const unsigned pr = M::from_fp8x2(regs.v[c][e2 >> 1], (e2 & 1) != 0);
        Vt[(d0 + 2 * e2) * VROW + kp] = (unsigned short)(pr & 0xFFFFu);
        Vt[(d0 + 2 * e2 + 1) * VROW + kp] = (unsigned short)(pr >> 16);
      }
    }
  }
}

template <int D, typename CT, int KVB>
__global__ __launch_bounds__(kThreads) void prefill_kernel(AttnParams p, int hpw) {
  using M = Mfma<CT>;
  using vec8 = typename M::vec8;
  constexpr int QS = D / 16;      // QK MFMA steps (16 d each)
  constexpr int DT = D / 32;      // 32-row d tiles of O^T
  constexpr int KROW = D + 8;
  constexpr int VROW = kTileK + 8;

  __shared__ __attribute__((aligned(16))) unsigned short Ks[kTileK * KROW];
  __shared__ __attribute__((aligned(16))) unsigned short Vt[D * VROW];

  const int rr = blockIdx.z;
  const int r = p.req_begin + rr;
  const int q_first = p.qsl[r];
  const int n = p.qsl[r + 1] - q_first;
  const int QB = 128 / hpw;
  const int qtile = blockIdx.x;
  if (qtile * QB >= n) return;
  const int G = p.group;
  const int s_all = p.seq_lens[r];
  const int c = s_all - n;
  int s_eff = min(s_all, p.max_seq_len);
  s_eff = min(s_eff, p.max_blocks_per_req * kBlock);
  const int nblk = (s_eff + kBlock - 1) / kBlock;
  const int q_hi = min((qtile + 1) * QB, n);           // exclusive
  const int k_end = min(c + q_hi, s_eff);              // keys any query of the tile may see
  const int ntiles = (k_end + kTileK - 1) / kTileK;

  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int qh = blockIdx.y * hpw + (wave % hpw);
  const int kvh = qh / G;
  const int wq0 = qtile * QB + (wave / hpw) * 32;       // first query of the wave
  const int qi = wq0 + l32;                             // this lane's query
  const bool q_ok = qi < n;
  const int qpos = c + qi;                              // its position

  // Q as the B operand of S^T = K . Q^T: B[k = 8*half + e][col = l32] = Q[qi][16 s + 8 half + e]
  vec8 qop[QS];
  {
    const CT* qrow = static_cast<const CT*>(p.q) + (int64_t)(q_first + qi) * p.q_row_stride +
                     (int64_t)qh * D;
#pragma unroll
    for (int s = 0; s < QS; ++s) {
      qop[s] = q_ok ? __builtin_bit_cast(vec8, ld16(qrow + 16 * s + 8 * half))
                    : __builtin_bit_cast(vec8, u32x4{0u, 0u, 0u, 0u});
    }
  }

  const int32_t* bt_row = p.block_tables + (int64_t)r * p.max_blocks_per_req;
  f32x16 acc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) acc[t] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  TileRegs<D, CT, KVB> regs;
  if (ntiles > 0) load_tile<D, CT, KVB>(regs, p, bt_row, nblk, s_eff, 0, kvh);
  const int wave_last_pos = c + min(wq0 + 31, n - 1);  // largest position in the wave
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();                 // previous tile fully consumed
    store_tile<D, CT, KVB>(regs, Ks, Vt);
    __syncthreads();
    if (kt + 1 < ntiles) load_tile<D, CT, KVB>(regs, p, bt_row, nblk, s_eff, kt + 1, kvh);
    const int k0 = kt * kTileK;
    if (k0 > wave_last_pos) continue;   // whole tile is in the future of every query of the wave

    // ---- S^T (keys x queries), two 32-key subtiles ----
    f32x16 sc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x16 a = f32x16{};
      const unsigned short* krow = Ks + (32 * u + l32) * KROW + 8 * half;
#pragma unroll
      for (int s = 0; s < QS; ++s) {
        const vec8 kop = __builtin_bit_cast(vec8, *reinterpret_cast<const u32x4*>(krow + 16 * s));
        a = M::mma32(kop, qop[s], a);
      }
      sc[u] = a;
    }

    // ---- scale, causal / length / absent-block mask ----
    bool blk_ok[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int bi = kt * 4 + b;
      bool ok = bi < nblk;
      if (ok) {
        const int id = bt_row[bi];
        ok = id >= 0 && (int64_t)id < p.num_blocks;
      }
      blk_ok[b] = ok;
    }
    const bool need_mask = (k0 + kTileK - 1 > c + wq0) || (k0 + kTileK > s_eff) ||
                           !blk_ok[0] || !blk_ok[1] || !blk_ok[2] || !blk_ok[3];
    float x[2][16];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        float v = sc[u][g] * p.scale_log2;
        if (need_mask) {
          const int key = k0 + 32 * u + 8 * (g / 4) + 4 * half + (g % 4);
          const bool ok = key <= qpos && key < s_eff && blk_ok[(32 * u + 8 * (g / 4)) / kBlock];
          v = ok ? v : -INFINITY;
        }
        x[u][g] = v;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int g = 0; g < 16; ++g) mx = fmaxf(mx, x[u][g]);
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_safe = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_safe);
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        x[u][g] = exp2f(x[u][g] - m_safe);
        psum += x[u][g];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[t] *= alpha;

    // ---- O^T += V^T . P^T, four 16-key steps ----
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const u32x4 pw{pack2<CT>(x[u][8 * v + 0], x[u][8 * v + 1]),
                       pack2<CT>(x[u][8 * v + 2], x[u][8 * v + 3]),
                       pack2<CT>(x[u][8 * v + 4], x[u][8 * v + 5]),
                       pack2<CT>(x[u][8 * v + 6], x[u][8 * v + 7])};
        const vec8 pop = __builtin_bit_cast(vec8, pw);
        const int col = 32 * u + 16 * v + 8 * half;   // Vt column of this lane's 8 keys
#pragma unroll
        for (int t = 0; t < DT; ++t) {
          const vec8 vop = __builtin_bit_cast(
              vec8, *reinterpret_cast<const u32x4*>(Vt + (32 * t + l32) * VROW + col));
          acc[t] = M::mma32(vop, pop, acc[t]);
        }
      }
    }
  }

  // ---- normalise and store: lane holds O[qi][32 t + 8 j + 4 half + i] ----
  float lt = l_run + shfl_xor(l_run, 32);
  if (!q_ok) return;
  const float inv = (lt > 0.f) ? p.v_scale / lt : 0.f;
  unsigned short* orow = static_cast<unsigned short*>(p.out) +
                         (int64_t)(q_first + qi) * p.out_row_stride + (int64_t)qh * D;
#pragma unroll
  for (int t = 0; t < DT; ++t) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d = 32 * t + 8 * j + 4 * half;
      u32x2 w{pack2<CT>(acc[t][4 * j] * inv, acc[t][4 * j + 1] * inv),
              pack2<CT>(acc[t][4 * j + 2] * inv, acc[t][4 * j + 3] * inv)};
      st8(orow + d, w);
    }
  }
}

int heads_per_wg(int G) {
  if (G % 4 == 0) return 4;
  if (G % 2 == 0) return 2;
  return 1;
}

template <int D, typename CT, int KVB>
hipError_t launch_typed(const AttnParams& p, hipStream_t stream) {
  const int hpw = heads_per_wg(p.group);
  const int QB = 128 / hpw;
  const int qtiles = (p.max_query_len + QB - 1) / QB;
  if (qtiles == 0) return hipSuccess;
  dim3 grid((unsigned)qtiles, (unsigned)(p.num_q_heads / hpw), (unsigned)p.num_reqs);
  hipLaunchKernelGGL((prefill_kernel<D, CT, KVB>), grid, dim3(kThreads), 0, stream, p, hpw);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dim(const AttnParams& p, int act, int cache, hipStream_t stream) {
  if (act == kF16 && cache == kF16) return launch_typed<D, _Float16, 2>(p, stream);
  if (act == kBF16 && cache == kBF16) return launch_typed<D, __bf16, 2>(p, stream);
  if (act == kF16 && cache == kFP8) return launch_typed<D, _Float16, 1>(p, stream);
  if (act == kBF16 && cache == kFP8) return launch_typed<D, __bf16, 1>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const AttnParams& p, int act_dtype, int cache_dtype, hipStream_t stream) {
  if (p.num_reqs == 0) return hipSuccess;
  if (p.head_dim == 128) return launch_dim<128>(p, act_dtype, cache_dtype, stream);
  if (p.head_dim == 64) return launch_dim<64>(p, act_dtype, cache_dtype, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
