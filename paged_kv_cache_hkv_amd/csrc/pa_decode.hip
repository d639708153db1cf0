// pa_decode kernels: attention of one-token (decode) requests through their
// block tables, with split-K over long contexts.
//
// What is computed (PagedAttention decode in "vLLM 推理全流程深度解析"; the
// decode rows of stop 10 in "Tour: One forward pass"): for request r with
// s keys and query row q, query head h (K/V head h/G, "vLLM MHA Code Path",
// "One Path Covers MHA, GQA, and MQA"):
//     out[h] = sum_j softmax_j(scale * q[h].k_j) v_j,  j = 0 .. s-1.
// Decode is bound by reading the K/V history once ("vLLM 推理全流程深度解析":
// decode is memory-bound; PagedAttention reads the cache block by block with
// coalesced bursts), so the design goal is to stream every K/V byte of a
// request exactly once, for all G query heads that share it.
//
// Work decomposition.  A workgroup of 4 waves owns one (request, K/V head,
// partition of part_tokens keys).  Its waves take the partition's 32-key
// chunks (two 16-token cache blocks) round-robin.  For one chunk a wave:
//   * loads the chunk's K rows straight into MFMA A-operand registers: lane
//     (token t = lane%16 of a block, quarter q4 = lane/16) reads 16 contiguous
//     bytes per step, so one load instruction covers 16 rows x 64 bytes;
//   * computes S^T[token][head] = K . Q^T on v_mfma_f32_16x16x32 with the
//     G <= 16 query heads of the group as the 16 columns (zero-padded; G = 32
//     uses two column tiles sharing the same K/V registers);
//   * keeps an online softmax per head in float32 (max shared by the 4 lanes
//     that hold a head's scores, exp2 with the scale folded into log2 units);
//   * loads V rows as 8 tokens x (D/16) contiguous elements per lane (a load
//     instruction covers 4 whole rows) and re-pairs them in registers with
//     byte permutes into the B operand of O = P . V, so the PV product is also
//     an MFMA and no LDS transpose is needed.
// At the end the 4 waves merge their (max, sum, weighted sum) in LDS.  A
// request that fits one partition writes its output row directly; otherwise
// each partition writes float32 partials to the workspace and the reduce
// kernel merges them in partition order (deterministic, no atomics).
//
// fp8 (OCP e4m3fn) caches are widened to bf16/fp16 exactly in registers with
// the gfx950 packed converts; the K scale is folded into the score scale and
// the V scale into the final division.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlock = 16;   // tokens per cache block
constexpr int kChunk = 32;   // tokens per wave iteration

template <int D, typename CT, int KVB, int HT>
__global__ __launch_bounds__(kThreads) void decode_kernel(AttnParams p) {
  using M = Mfma<CT>;
  using vec8 = typename M::vec8;
  constexpr int KS = D / 32;               // QK MFMA steps (32 d each)
  constexpr int NM = D / 16;               // PV MFMAs (16 output columns each)
  constexpr int VE = D / 16;               // V elements per lane per token
  constexpr int VW = (VE * KVB + 3) / 4;   // dwords per lane per V token
  constexpr int KP = (KVB == 2) ? KS : KS / 2;  // 16-byte K loads per lane per block

  __shared__ float red_acc[kWaves][16][D];
  __shared__ float red_m[kWaves][16];
  __shared__ float red_l[kWaves][16];

  const int rr = blockIdx.z;
  const int r = p.req_begin + rr;
  const int kvh = blockIdx.y;
  const int part = blockIdx.x;
  const int q_row = p.qsl[r];
  if (p.qsl[r + 1] - q_row != 1) return;
  int s_eff = min(p.seq_lens[r], p.max_seq_len);
  s_eff = min(s_eff, p.max_blocks_per_req * kBlock);
  const int P = p.part_tokens;
  const int tok_begin = part * P;
  if (tok_begin >= s_eff) return;
  const int tok_end = min(tok_begin + P, s_eff);
  const int nparts = (s_eff + P - 1) / P;
  const int nblk = (s_eff + kBlock - 1) / kBlock;
  const int G = p.group;
  const int Hkv = p.num_kv_heads;

  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int q4 = lane >> 4;
  const int c16 = lane & 15;

  // ---- Q as the B operand of S^T = K.Q^T: lane holds head (ht*16 + c16) ----
  vec8 qop[HT][KS];
  const CT* qbase = static_cast<const CT*>(p.q) + (int64_t)q_row * p.q_row_stride;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int hig = ht * 16 + c16;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int d0 = (KVB == 2) ? (32 * s + 8 * q4) : (64 * (s / 2) + 16 * q4 + 8 * (s % 2));
      if (hig < G) {
        qop[ht][s] = __builtin_bit_cast(vec8, ld16(qbase + (int64_t)(kvh * G + hig) * D + d0));
      } else {
        qop[ht][s] = __builtin_bit_cast(vec8, u32x4{0u, 0u, 0u, 0u});
      }
    }
  }

  const int32_t* bt_row = p.block_tables + (int64_t)r * p.max_blocks_per_req;
  const unsigned char* kc = static_cast<const unsigned char*>(p.key_cache);
  const unsigned char* vc = static_cast<const unsigned char*>(p.value_cache);
  const int64_t tok_stride = (int64_t)Hkv * D * KVB;     // bytes between slots
  const int64_t blk_stride = tok_stride * kBlock;        // bytes between blocks
  const int64_t head_off = (int64_t)kvh * D * KVB;

  float m_run[HT], l_run[HT];
  f32x4 acc[HT][NM];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    m_run[ht] = -INFINITY;
    l_run[ht] = 0.f;
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[ht][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int first_chunk = tok_begin / kChunk;
  const int end_chunk = (tok_end + kChunk - 1) / kChunk;
  for (int ch = first_chunk + wave; ch < end_chunk; ch += kWaves) {
    const int j0 = ch * kChunk;
    // physical blocks of the chunk's two 16-token halves
    int64_t boff[2];
    bool bvalid[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int bi = j0 / kBlock + t;
      int b = 0;
      bool ok = bi < nblk;
      if (ok) {
        b = bt_row[bi];
        ok = (b >= 0) && ((int64_t)b < p.num_blocks);
      }
      bvalid[t] = ok;
      boff[t] = ok ? (int64_t)b * blk_stride : 0;   // absent blocks read block 0, then masked
    }
    const bool need_mask = (j0 + kChunk > tok_end) || !bvalid[0] || !bvalid[1];

    // ---- issue K and V loads ----
    u32x4 kraw[2][KP];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const unsigned char* row = kc + boff[t] + (int64_t)c16 * tok_stride + head_off;
#pragma unroll
      for (int s = 0; s < KP; ++s) {
        const int d0 = (KVB == 2) ? (32 * s + 8 * q4) : (64 * s + 16 * q4);
        kraw[t][s] = ld16(row + d0 * KVB);
      }
    }
    unsigned vraw[8][VW];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = i / 4;
      const int off = 4 * q4 + (i % 4);
      const unsigned char* row = vc + boff[t] + (int64_t)off * tok_stride + head_off +
                                 (int64_t)(VE * c16) * KVB;
      if constexpr (VW == 4) {
        u32x4 v = ld16(row);
        vraw[i][0] = v[0]; vraw[i][1] = v[1]; vraw[i][2] = v[2]; vraw[i][3] = v[3];
      } else if constexpr (VW == 2) {
        u32x2 v = ld8(row);
        vraw[i][0] = v[0]; vraw[i][1] = v[1];
      } else {
        vraw[i][0] = ld4(row);
      }
    }

    // ---- K operands ----
    vec8 kop[2][KS];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        if constexpr (KVB == 2) {
          kop[t][s] = __builtin_bit_cast(vec8, kraw[t][s]);
        } else {
          const u32x4& w = kraw[t][s / 2];
          const unsigned d0 = w[2 * (s % 2)], d1 = w[2 * (s % 2) + 1];
          u32x4 o{M::from_fp8x2(d0, false), M::from_fp8x2(d0, true),
                  M::from_fp8x2(d1, false), M::from_fp8x2(d1, true)};
          kop[t][s] = __builtin_bit_cast(vec8, o);
        }
      }
    }

    // ---- S^T = K . Q^T ----
    f32x4 sc[HT][2];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) a = M::mma16(kop[t][s], qop[ht][s], a);
        sc[ht][t] = a;
      }
    }

    // ---- masking of absent tokens (last chunk, absent blocks) ----
    if (need_mask) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = i / 4;
        const int tok = j0 + 16 * t + 4 * q4 + (i % 4);
        // selects, not a branch per token: every register is written on
        // every path (0 * NaN would poison P.V, so absent V rows become 0)
        const bool bad = !bvalid[t] || tok >= tok_end;
#pragma unroll
        for (int w = 0; w < VW; ++w) vraw[i][w] = bad ? 0u : vraw[i][w];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) sc[ht][t][i % 4] = bad ? -INFINITY : sc[ht][t][i % 4];
      }
    }

    // ---- V operands: B[k = 8*q4 + i][n = c16] = V[token(i)][VE*c16 + m] ----
    vec8 vop[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      unsigned w4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned* a = vraw[2 * j];
        const unsigned* b = vraw[2 * j + 1];
        if constexpr (KVB == 2) {
          w4[j] = (m & 1) ? perm(b[m / 2], a[m / 2], 0x07060302u)
                          : perm(b[m / 2], a[m / 2], 0x05040100u);
        } else {
          const unsigned aw = a[m / 4], bw = b[m / 4];
          const unsigned x = (m & 2) ? perm(bw, aw, 0x07030602u) : perm(bw, aw, 0x05010400u);
          w4[j] = M::from_fp8x2(x, (m & 1) != 0);
        }
      }
      vop[m] = __builtin_bit_cast(vec8, u32x4{w4[0], w4[1], w4[2], w4[3]});
    }

    // ---- online softmax and P.V per head tile ----
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = sc[ht][i / 4][i % 4] * p.scale_log2;
      float mx = x[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[ht], mx);
      const float m_safe = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[ht] - m_safe);
      float pr[8];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pr[i] = fast_exp2(x[i] - m_safe);
        psum += pr[i];
      }
      l_run[ht] = l_run[ht] * alpha + psum;
      m_run[ht] = m_new;
      // accumulator rows are heads 4*q4 + i: fetch their rescale factors
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a_i = shfl(alpha, 4 * q4 + i);
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[ht][m][i] *= a_i;
      }
      const u32x4 pw{pack2<CT>(pr[0], pr[1]), pack2<CT>(pr[2], pr[3]),
                     pack2<CT>(pr[4], pr[5]), pack2<CT>(pr[6], pr[7])};
      const vec8 pop = __builtin_bit_cast(vec8, pw);
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[ht][m] = M::mma16(pop, vop[m], acc[ht][m]);
    }
  }

  // ---- merge the 4 waves, then write the output or the partition partials ----
  const int Hq = p.num_q_heads;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    float lt = l_run[ht];
    lt += shfl_xor(lt, 16);
    lt += shfl_xor(lt, 32);
    if (ht > 0) __syncthreads();
#pragma unroll
    for (int m = 0; m < NM; ++m) {
#pragma unroll
      for (int i = 0; i < 4; ++i) red_acc[wave][4 * q4 + i][VE * c16 + m] = acc[ht][m][i];
    }
    if (q4 == 0) {
      red_m[wave][c16] = m_run[ht];
      red_l[wave][c16] = lt;
    }
    __syncthreads();
    constexpr int EPT = D / 16;   // outputs per thread: 16 heads x D over 256 threads
    const int hh = threadIdx.x / 16;
    const int d0 = (threadIdx.x % 16) * EPT;
    const int hig = ht * 16 + hh;
    if (hig < G) {
      float mw[kWaves];
      float mmax = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        mw[w] = red_m[w][hh];
        mmax = fmaxf(mmax, mw[w]);
      }
      const float msafe = (mmax == -INFINITY) ? 0.f : mmax;
      float L = 0.f;
      float wgt[kWaves];
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        wgt[w] = fast_exp2(mw[w] - msafe);
        L += wgt[w] * red_l[w][hh];
      }
      float o[EPT];
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) v += wgt[w] * red_acc[w][hh][d0 + e];
        o[e] = v;
      }
      const int qh = kvh * G + hig;
      if (nparts == 1) {
        const float inv = (L > 0.f) ? p.v_scale / L : 0.f;
        unsigned short* orow = static_cast<unsigned short*>(p.out) +
                               (int64_t)q_row * p.out_row_stride + (int64_t)qh * D + d0;
        unsigned pk[EPT / 2];
#pragma unroll
        for (int e = 0; e < EPT / 2; ++e) pk[e] = pack2<CT>(o[2 * e] * inv, o[2 * e + 1] * inv);
        if constexpr (EPT == 8) {
          st16(orow, u32x4{pk[0], pk[1], pk[2], pk[3]});
        } else {
          st8(orow, u32x2{pk[0], pk[1]});
        }
      } else {
        const int64_t slot = ((int64_t)rr * Hq + qh) * p.max_parts + part;
        float* wa = p.ws_acc + slot * D + d0;
#pragma unroll
        for (int e = 0; e < EPT; ++e) wa[e] = o[e];
        if ((threadIdx.x % 16) == 0) {
          p.ws_ml[slot * 2] = mmax;
          p.ws_ml[slot * 2 + 1] = L;
        }
      }
    }
  }
}

// Merge of the partition partials of one (request, query head): one wave.
// Lanes take partitions (64 at a time) for the global max and the weighted
// sum of the row sums; then each lane accumulates its D/64 output columns
// over the partitions in increasing order with the weights broadcast from
// the lane that owns them.  Fixed order, no atomics: deterministic.
template <int D, typename CT>
__global__ __launch_bounds__(64) void decode_reduce_kernel(AttnParams p) {
  constexpr int DPL = D / 64;   // output columns per lane
  const int rr = blockIdx.y;
  const int r = p.req_begin + rr;
  const int qh = blockIdx.x;
  const int lane = threadIdx.x;
  const int q_row = p.qsl[r];
  if (p.qsl[r + 1] - q_row != 1) return;
  int s_eff = min(p.seq_lens[r], p.max_seq_len);
  s_eff = min(s_eff, p.max_blocks_per_req * kBlock);
  if (s_eff <= 0) return;
  const int P = p.part_tokens;
  int nparts = (s_eff + P - 1) / P;
  if (nparts <= 1) return;
  nparts = min(nparts, p.max_parts);
  const int64_t base = ((int64_t)rr * p.num_q_heads + qh) * p.max_parts;
  const float* ml = p.ws_ml + base * 2;
  const float* acc = p.ws_acc + base * D;

  float mloc = -INFINITY;
  for (int i = lane; i < nparts; i += 64) mloc = fmaxf(mloc, ml[2 * i]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mloc = fmaxf(mloc, shfl_xor(mloc, off));
  const float msafe = (mloc == -INFINITY) ? 0.f : mloc;

  float lsum = 0.f;
  float o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  for (int g = 0; g < nparts; g += 64) {
    const int i = g + lane;
    const float w = (i < nparts) ? fast_exp2(ml[2 * min(i, nparts - 1)] - msafe) : 0.f;
    const float lw = (i < nparts) ? w * ml[2 * min(i, nparts - 1) + 1] : 0.f;
    float t = lw;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) t += shfl_xor(t, off);
    lsum += t;
    const int cnt = min(64, nparts - g);
    for (int j = 0; j < cnt; ++j) {
      const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
      const float* a = acc + (int64_t)(g + j) * D + lane;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] += wj * a[64 * e];
    }
  }
  const float inv = (lsum > 0.f) ? p.v_scale / lsum : 0.f;
  unsigned short* orow = static_cast<unsigned short*>(p.out) + (int64_t)q_row * p.out_row_stride +
                         (int64_t)qh * D;
#pragma unroll
  for (int e = 0; e < DPL; ++e) orow[lane + 64 * e] = Mfma<CT>::from_float(o[e] * inv);
}

template <int D, typename CT, int KVB, int HT>
hipError_t launch_typed(const AttnParams& p, hipStream_t stream) {
  dim3 grid((unsigned)p.max_parts, (unsigned)p.num_kv_heads, (unsigned)p.num_reqs);
  hipLaunchKernelGGL((decode_kernel<D, CT, KVB, HT>), grid, dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.max_parts <= 1) return e;
  dim3 rgrid((unsigned)p.num_q_heads, (unsigned)p.num_reqs);
  hipLaunchKernelGGL((decode_reduce_kernel<D, CT>), rgrid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

template <int D, typename CT, int KVB>
hipError_t launch_heads(const AttnParams& p, hipStream_t stream) {
  if (p.group <= 16) return launch_typed<D, CT, KVB, 1>(p, stream);
  if (p.group <= 32) return launch_typed<D, CT, KVB, 2>(p, stream);
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_dim(const AttnParams& p, int act, int cache, hipStream_t stream) {
  if (act == kF16 && cache == kF16) return launch_heads<D, _Float16, 2>(p, stream);
  if (act == kBF16 && cache == kBF16) return launch_heads<D, __bf16, 2>(p, stream);
  if (act == kF16 && cache == kFP8) return launch_heads<D, _Float16, 1>(p, stream);
  if (act == kBF16 && cache == kFP8) return launch_heads<D, __bf16, 1>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const AttnParams& p, int act_dtype, int cache_dtype, hipStream_t stream) {
  if (p.num_reqs == 0 || p.max_parts == 0) return hipSuccess;
  if (p.head_dim == 128) return launch_dim<128>(p, act_dtype, cache_dtype, stream);
  if (p.head_dim == 64) return launch_dim<64>(p, act_dtype, cache_dtype, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
