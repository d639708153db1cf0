// pa_decode kernels: attention of one-token (decode) requests through their
// block tables.
//
// What is computed (PagedAttention decode in "vLLM 推理全流程深度解析"; the
// decode rows of stop 10 in "Tour: One forward pass"): for request r with
// s keys and query row q, query head h (K/V head h/G, "vLLM MHA Code Path",
// "One Path Covers MHA, GQA, and MQA"):
//     out[h] = sum_j softmax_j(scale * q[h].k_j) v_j,  j = 0 .. s-1.
// Decode is bound by reading the K/V history once ("vLLM 推理全流程深度解析":
// decode is memory-bound; PagedAttention reads the cache block by block with
// coalesced bursts), so the design goal is to stream every K/V byte of a
// request exactly once, for all G query heads that share it, at the rate
// HBM delivers.
//
// Work decomposition (persistent, stream-split).  Flatten the batch into one
// stream of work units: for each decode request, for each K/V head, its
// 16-token cache blocks in order.  The stream of T units is cut into W equal
// contiguous ranges, one per wave ("worker"); W is a few waves per compute
// unit and every worker is resident for the whole launch, so each wave
// streams ~T/W blocks back to back with no start-up or tail bubbles and no
// dependence on how the contexts' lengths are distributed.  A worker's range
// covers a few (request, K/V head) segments.  A segment that is a whole
// (request, K/V head) is finished in place and its output rows written
// directly; a segment cut by a range boundary leaves a float32 partial
// (running max, sum, weighted sum).  Consecutive workers form a workgroup
// (one per compute unit), which merges in LDS, in worker order, every head
// cut only between its own workers; a head cut between workgroups leaves one
// partial per workgroup, merged in workgroup order by the reduce kernel
// (deterministic, no atomics).
//
// Streaming.  Each wave owns a ring of S LDS stages, one block (K and V rows
// of one head) each, and a query area for one segment's G query rows, copied
// when the segment's first block is issued (the issue side holds back while a
// copied query is still unread).  Asynchronous global -> LDS copies are
// issued S-1 blocks ahead, so the bytes in flight cost no registers.  A copy
// instruction moves 1 KB: whole 16-byte chunks of 16/8/4 consecutive token
// rows, each row's chunks scattered by an XOR of the token so the MFMA
// operand reads below hit distinct LDS banks.  Per block a wave:
//   * computes S^T[token][head] = K . Q^T on v_mfma_f32_16x16x32 with the
//     G <= 16 query heads of the group as the 16 columns (zero-padded; G = 32
//     uses two column tiles sharing the same K/V operands); K rows are read
//     from LDS as 16-byte A-operand pieces;
//   * keeps an online softmax per head in float32: the max is shared by the 4
//     lanes that hold a head's scores, exp2 with the scale folded in, and the
//     accumulator is only rescaled when a head's max grows by more than 2^8
//     (exact up to rounding: the reference max of a softmax is arbitrary as
//     long as nothing overflows);
//   * accumulates O^T[d][head] = V^T . P^T on v_mfma_f32_16x16x16: the scores
//     are already the B operand (one head per lane column, 4 tokens per lane)
//     and V^T comes from LDS with the transposing ds_read_b64_tr_b16 (16-bit
//     caches) or row reads re-paired by byte permutes (fp8), so a lane's
//     accumulators all belong to one head and every rescale is lane-local.
//
// 8-bit caches -- fp8 (OCP e4m3fn) or int8 codes -- are widened to bf16/fp16
// exactly in registers (fp8 with the gfx950 packed converts, int8 by way of
// float32: every code -127..127 is exact); the K scale is folded into the
// score scale and the V scale into the final division.
//
// Mask variants (the alibi_slopes and window_size arguments of the attention
// call in stop 10 of "Tour: One forward pass"): with a sliding window of W
// keys a request streams only the blocks from its window's first key on (the
// stream, the worker ranges and the reduce all count those blocks), and keys
// before the window inside the first block are masked; ALiBi adds
// slope[h] * (key - query position) to each score in log2 units.  Both live in
// a separate instantiation (MASK), so the plain kernel carries neither.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kBlock = 16;                // tokens per cache block
constexpr float kRescaleLog2 = 8.f;       // lazy rescale threshold (log2 units)
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kLdsBudget = 160 * 1024;    // LDS of one compute unit
#ifndef PA_DECODE_STAGES
#define PA_DECODE_STAGES 3
#endif
constexpr int kStages = PA_DECODE_STAGES; // LDS ring depth per wave (where it fits)
constexpr int kStages8 = 4;               // the same for 8-bit caches (half-size blocks)

// Token of MFMA row i (0..15) of a block.  Any permutation works as long as
// scores and V use the same one; this one makes the four lane groups that
// read one V token slot at a time (fp8 path) land on different LDS bank
// halves.
__device__ inline int row_token(int i) { return i ^ ((i >> 2) & 3); }

// Geometry of one block of one head in a ring stage.
template <int D, int KVB>
struct Ring {
  static constexpr int kRowBytes = D * KVB;             // one token row
  static constexpr int kCPR = kRowBytes / 16;           // 16-byte chunks per row: 16, 8 or 4
  static constexpr int kBlkBytes = kBlock * kRowBytes;  // K (or V) bytes of a block
  static constexpr int kIPT = kBlkBytes / 1024;         // copy instructions per tensor
  static constexpr int kIPB = 2 * kIPT;                 // per block (K and V)
  static constexpr int kSh = kCPR == 16 ? 0 : (kCPR == 8 ? 1 : 2);   // log2(16 / kCPR)
  // chunk c of token t sits at slot c ^ swk(t) (K) / c ^ swv(t) (V) of its row
  __device__ static inline int swk(int t) { return (t >> kSh) & (kCPR - 1); }
  __device__ static inline int swv(int t) {
    return KVB == 2 ? 2 * ((t >> kSh) & (kCPR / 2 - 1)) : 0;
  }
};

// Wait until at most n (wave-uniform, clamped to N) blocks' copies are in
// flight.
// Copies of query rows are issued before the block they belong to, so they
// only make the count conservative.
template <int IPB, int N>
__device__ inline void wait_blocks(int n) {
  if constexpr (N == 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= N) {
      wait_vmcnt<N * IPB>();
    } else {
      wait_blocks<IPB, N - 1>(n);
    }
  }
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// ds_read_b64_tr_b16: in each 16-lane group, lane i supplies the address of
// an 8-byte row R_i of four 16-bit values; lane j receives R_{4k + j/4}[j%4]
// for k = 0..3.
__device__ inline u32x2 lds_read_tr16(const unsigned char* p) {
  lds_bf16x4* lp = (lds_bf16x4*)(const_cast<unsigned char*>(p));
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lp));
}

// First key a decode row of s keys may see (its position is s - 1), and the
// first block holding one: 0 without a sliding window.
// The kernel's parameter block in the kernarg segment, read through a pointer
// the compiler cannot see through: a field used only where a segment starts
// or ends is loaded there instead of being held in scalar registers through
// the stream.
typedef __attribute__((address_space(4))) const AttnParams CAttnParams;
__device__ inline const CAttnParams* kernarg_params() {
  const CAttnParams* q = (const CAttnParams*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(q));
  return q;
}

// V scale of K/V head kvh: the tensor's, or the head's own (per-head scales
// exist for 8-bit caches only)
template <int KVB>
__device__ inline float v_scale_of(const AttnParams& p, int kvh) {
  if constexpr (KVB == 1) {
    const CAttnParams* kp = kernarg_params();
    return kp->v_scales != nullptr ? head_scale(kp->v_scales, kvh) : kp->v_scale;
  } else {
    return p.v_scale;
  }
}

__device__ inline int first_key(const AttnParams& p, int s) { return max(0, s - 1 - p.window_left); }
__device__ inline int first_block(const AttnParams& p, int s) { return first_key(p, s) / kBlock; }

// Cache blocks a request streams, from its query_start_loc entries q0, q1 and
// its seq_len s: 0 for a request that is not a decode (query length != 1)
// or has no keys; with a sliding window only the blocks from the window's
// first key on.
__device__ inline int blocks_of(const AttnParams& p, int q0, int q1, int s) {
  if (q1 - q0 != 1) return 0;
  s = min(min(s, p.max_seq_len), p.max_blocks_per_req * kBlock);
  return s > 0 ? (s + kBlock - 1) / kBlock - first_block(p, s) : 0;
}

// The same for request rr (index within the call), the same in every lane
// (scalar loads, all three issued together).
__device__ inline int stream_blocks(const AttnParams& p, int rr) {
  const int r = p.req_begin + rr;
  const int q0 = load_uniform(p.qsl, r);
  const int q1 = load_uniform(p.qsl, r + 1);
  const int s = load_uniform(p.seq_lens, r);
  return blocks_of(p, q0, q1, s);
}

__device__ inline int64_t readlane64(int64_t v, int l) {
  const int lo = __builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const int hi = __builtin_amdgcn_readlane((int)(v >> 32), l);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Inclusive prefix sum over the 64 lanes: shifts within each 16-lane row,
// then the row totals carried into the rows above (DPP row broadcasts of
// lanes 15 and 31); lanes a shift leaves without a source add 0.
template <int CTRL, int ROWS>
__device__ inline int64_t dpp_shift64(int64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROWS, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(v >> 32), CTRL, ROWS, 0xF, false);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ inline int64_t wave_scan(int64_t v) {
  v += dpp_shift64<0x111, 0xF>(v);   // row_shr:1
  v += dpp_shift64<0x112, 0xF>(v);   // row_shr:2
  v += dpp_shift64<0x114, 0xF>(v);   // row_shr:4
  v += dpp_shift64<0x118, 0xF>(v);   // row_shr:8
  v += dpp_shift64<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_shift64<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

// floor(x / y) for x >= 0, y > 0.  Below 2^53 both convert to double exactly
// and the double quotient is off by at most one, which the integer check
// corrects; the generic 64-bit division is a long instruction sequence.
__device__ inline int64_t div_floor(int64_t x, int64_t y) {
  if (x < (int64_t(1) << 53)) {
    int64_t q = (int64_t)((double)x / (double)y);
    q -= (q * y > x) ? 1 : 0;
    q += ((q + 1) * y <= x) ? 1 : 0;
    return q;
  }
  return x / y;
}

// First stream unit of worker w (W workers over T units).
__device__ inline int64_t range_begin(int64_t w, int64_t T, int64_t W) { return div_floor(w * T, W); }

// Position in the stream: request (index within the call), K/V head, block
// of that head counted from b0 (the first block the request streams: 0, or
// the window's first block); and the request's streamed block count, key
// count, first visible key and query row.
struct Cursor {
  int rr, kvh, b, nb;
  int s_eff, q_row;
  int b0, lo;
  const int32_t* row;   // the request's block-table entries from block b0 on
};

// Fill the request fields of c for request c.rr from its query_start_loc
// entries q0, q1 and its seq_len s_raw.
__device__ inline void set_request(const AttnParams& p, Cursor& c, int q0, int q1, int s_raw) {
  const int r = p.req_begin + c.rr;
  const int s = min(min(s_raw, p.max_seq_len), p.max_blocks_per_req * kBlock);
  c.q_row = q0;
  c.s_eff = s;
  c.lo = first_key(p, s);
  c.b0 = c.lo / kBlock;
  c.nb = (q1 - q0 == 1 && s > 0) ? (s + kBlock - 1) / kBlock - c.b0 : 0;
  c.row = p.block_tables + (int64_t)r * p.max_blocks_per_req + c.b0;
}

// The same from wave-uniform loads.
__device__ inline void load_request(const AttnParams& p, Cursor& c) {
  const int r = p.req_begin + c.rr;
  const int q0 = load_uniform(p.qsl, r);
  const int q1 = load_uniform(p.qsl, r + 1);
  const int s = load_uniform(p.seq_lens, r);
  set_request(p, c, q0, q1, s);
}

// Advance by one unit (wave-uniform); skips requests that stream nothing.
__device__ inline void advance(const AttnParams& p, Cursor& c) {
  if (++c.b < c.nb) return;
  c.b = 0;
  if (++c.kvh < p.num_kv_heads) return;
  c.kvh = 0;
  do {
    if (++c.rr >= p.num_reqs) {   // past the stream: never used
      c.nb = 1;
      return;
    }
    load_request(p, c);
  } while (c.nb == 0);
}

template <int D, typename CT, int KVB, bool I8, int HT, int S, int WV, bool MASK>
__global__ __launch_bounds__(64 * WV) void decode_kernel(AttnParams p) {
  using M = Mfma<CT>;
  using vec8 = typename M::vec8;
  using R = Ring<D, KVB>;
  constexpr int KS = D / 32;               // QK MFMA steps (32 d each)
  constexpr int NM = D / 16;               // PV MFMAs per block (16 rows of O^T each)
  constexpr int VE = D / 16;               // fp8 path: V bytes per lane per token
  constexpr int kStage = 2 * R::kBlkBytes; // K | V of one block
  constexpr int kQCap = HT * 16 * D * 2;   // query rows of one segment (<= 16*HT heads)
  constexpr int kWaveBytes = S * kStage + kQCap;
  static_assert(S >= 2 && S <= 8, "ring depth");
  static_assert(WV * kWaveBytes <= kLdsBudget, "rings exceed LDS");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[WV * kWaveBytes];

  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int q4 = lane >> 4;
  const int c16 = lane & 15;
  const int W = p.num_workers;
  const int worker = blockIdx.x * WV + wave;
  // waves past the worker count (a last workgroup of fewer workers) and
  // workers with empty ranges stream nothing but still take part in the
  // workgroup's merge of partials below, so no wave leaves early
  const bool in_range = worker < W;
  const int Rn = p.num_reqs;
  const int G = p.group;
  const int Hkv = p.num_kv_heads;

  // ---- the stream: total units T, this worker's range, its first unit.
  // Lanes take 64 requests at a time (their three fields loaded together);
  // with at most 64 requests in the call the first pass's values serve the
  // search too. ----
  int64_t T = 0;
  int f_q0 = 0, f_q1 = 0, f_s = 0;   // lane's request of the first 64
  int64_t f_v = 0, f_incl = 0;
  for (int c = 0; c < Rn; c += 64) {
    int q0 = 0, q1 = 0, s = 0;
    if (c + lane < Rn) {
      const int r = p.req_begin + c + lane;
      q0 = p.qsl[r];
      q1 = p.qsl[r + 1];
      s = p.seq_lens[r];
    }
    const int64_t v = (c + lane < Rn) ? (int64_t)Hkv * blocks_of(p, q0, q1, s) : 0;
    const int64_t incl = wave_scan(v);
    if (c == 0) {
      f_q0 = q0;
      f_q1 = q1;
      f_s = s;
      f_v = v;
      f_incl = incl;
    }
    T += readlane64(incl, 63);
  }
  const int64_t g0 = in_range ? range_begin(worker, T, W) : T;
  // units of this worker: the host keeps every share below 2^31
  const int n = in_range ? (int)(range_begin(worker + 1, T, W) - g0) : 0;
  Cursor cur{0, 0, 0, 0, 0, 0, 0, 0, nullptr};
  bool found = false;
  if (in_range && Rn <= 64) {
    if (worker == 0 && lane < Rn) p.ws_cum[lane] = f_incl - f_v;
    const int64_t excl = f_incl - f_v;
    const uint64_t hit = __builtin_amdgcn_ballot_w64(f_v > 0 && excl <= g0 && g0 < f_incl);
    if (hit != 0) {
      const int l = __builtin_ctzll(hit);
      cur.rr = l;
      const int64_t within = g0 - readlane64(excl, l);
      set_request(p, cur, __builtin_amdgcn_readlane(f_q0, l), __builtin_amdgcn_readlane(f_q1, l),
                  __builtin_amdgcn_readlane(f_s, l));
      cur.kvh = (int)(within / cur.nb);
      cur.b = (int)(within % cur.nb);
      found = true;
    }
  } else if (in_range) {
    // worker 0 also publishes the exclusive prefix for the reduce kernel
    int64_t run = 0;
    for (int c = 0; c < Rn; c += 64) {
      int q0 = 0, q1 = 0, s = 0;
      if (c + lane < Rn) {
        const int r = p.req_begin + c + lane;
        q0 = p.qsl[r];
        q1 = p.qsl[r + 1];
        s = p.seq_lens[r];
      }
      const int64_t v = (c + lane < Rn) ? (int64_t)Hkv * blocks_of(p, q0, q1, s) : 0;
      const int64_t incl = wave_scan(v);
      const int64_t excl = run + incl - v;
      if (worker == 0 && c + lane < Rn) p.ws_cum[c + lane] = excl;
      const uint64_t hit = __builtin_amdgcn_ballot_w64(v > 0 && excl <= g0 && g0 < excl + v);
      if (!found && hit != 0) {
        const int l = __builtin_ctzll(hit);
        cur.rr = c + l;
        const int64_t within = g0 - readlane64(excl, l);
        set_request(p, cur, __builtin_amdgcn_readlane(q0, l), __builtin_amdgcn_readlane(q1, l),
                    __builtin_amdgcn_readlane(s, l));
        cur.kvh = (int)(within / cur.nb);
        cur.b = (int)(within % cur.nb);
        found = true;
        if (worker != 0) break;
      }
      run += readlane64(incl, 63);
    }
  }
  if (in_range && worker == 0 && lane == 0) p.ws_cum[Rn] = T;
  const bool active = found && n > 0;

  // partial state of the worker's last head when a range boundary cuts it
  // (kept for the workgroup merge), and whether its first head left one
  bool has_l = false, has_f = false;
  int64_t l_first = 0, l_end = 0, f_first = 0, f_end = 0;   // stream units of those heads
  int l_kvh = 0, l_qrow = 0, f_kvh = 0, f_qrow = 0;
  float m_used[HT], l_run[HT];
  f32x4 acc[HT][NM];
  float f_m[HT], f_l[HT];   // the first head's running max and sum, when it left a partial
  // a partial -- weighted sums [G][D], then running max and sum [G][2] --
  // from the lanes' accumulator layout
  auto store_partial = [&](float* pacc, float* pml, const f32x4 (&a)[HT][NM], const float (&mu)[HT],
                           const float (&lr)[HT]) __attribute__((always_inline)) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float lt = lr[ht];
      lt += shfl_xor(lt, 16);
      lt += shfl_xor(lt, 32);
      const int hig = ht * 16 + c16;
      if (hig < G) {
        float* wa = pacc + hig * D;
        if constexpr (KVB == 2) {
#pragma unroll
          for (int m = 0; m < NM; ++m) *reinterpret_cast<f32x4*>(wa + 16 * m + 4 * q4) = a[ht][m];
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int m = 0; m < NM; m += 4)
              *reinterpret_cast<f32x4*>(wa + VE * (4 * q4 + k) + m) =
                  f32x4{a[ht][m][k], a[ht][m + 1][k], a[ht][m + 2][k], a[ht][m + 3][k]};
        }
        if (q4 == 0 && pml != nullptr) {
          pml[2 * hig] = mu[ht];
          pml[2 * hig + 1] = lt;
        }
      }
    }
  };
  if (active) {

  const int64_t tok_stride = (int64_t)Hkv * D * KVB;     // bytes between slots
  // bytes between blocks (below 2^32, checked on the host)
  const uint32_t blk_stride = (uint32_t)(tok_stride * kBlock);
  // a table entry is a pool block when (unsigned) id < nblk
  const uint32_t nblk = p.num_blocks > 0x7FFFFFFF ? 0x80000000u : (uint32_t)p.num_blocks;

  // per-lane source offsets of the copy instructions of one block
  int koff[R::kIPT], voff[R::kIPT];
#pragma unroll
  for (int j = 0; j < R::kIPT; ++j) {
    const int pidx = 64 * j + lane;
    const int t = pidx / R::kCPR;
    const int pos = pidx % R::kCPR;
    koff[j] = (int)(t * tok_stride) + 16 * (pos ^ R::swk(t));
    voff[j] = (int)(t * tok_stride) + 16 * (pos ^ R::swv(t));
  }
  unsigned char* ring = lds + wave * kWaveBytes;
  const unsigned char* qarea = ring + S * kStage;
  const unsigned ring_m0 = lds_offset(ring);
  const unsigned q_m0 = ring_m0 + S * kStage;
  const int qbytes = G * D * 2;

  // ---- issue side.  Unit j goes to stage j % S; the first unit of a
  // segment first copies the segment's query rows into the wave's query
  // area.  That area holds one segment's rows, so the issue side waits
  // (issues nothing) while rows it copied are not yet read. ----
  Cursor ic = cur;
  int jn = 0;                // units issued
  int ist = 0;               // stage of unit jn (jn mod S)
  bool q_pending = false;    // query rows copied but not yet read
  unsigned okbits = 0;       // bit st: the unit in stage st has its block
  auto can_issue = [&](int lim) { return jn < n && jn < lim && !(q_pending && ic.b == 0); };
  auto issue_one = [&]() __attribute__((always_inline)) {
    const int st = ist;
    const unsigned dst = ring_m0 + st * kStage;
    if (ic.b == 0 || jn == 0) {
      const unsigned char* qb = static_cast<const unsigned char*>(p.q) +
                                ((int64_t)ic.q_row * p.q_row_stride + (int64_t)ic.kvh * G * D) * 2;
      for (int k = 0; k < qbytes; k += 1024)
        if (k + 16 * lane < qbytes) lds_dma16(qb, (unsigned)(k + 16 * lane), q_m0 + k);
      q_pending = true;
    }
    const int32_t id = load_uniform(ic.row, ic.b);
    const bool ok = (uint32_t)id < nblk;
    okbits = (okbits & ~(1u << st)) | ((ok ? 1u : 0u) << st);
    const uint64_t boff = (uint64_t)(ok ? (uint32_t)id : 0u) * blk_stride + (uint32_t)(ic.kvh * (D * KVB));
    const unsigned char* kb = static_cast<const unsigned char*>(p.key_cache) + boff;
    const unsigned char* vb = static_cast<const unsigned char*>(p.value_cache) + boff;
    // one LDS wait for the block's copies (they overwrite the stage read
    // S - 1 units ago)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < R::kIPT; ++i) {
      lds_dma16<true, false>(kb, (unsigned)koff[i], dst + 1024 * i);
      lds_dma16<true, false>(vb, (unsigned)voff[i], dst + R::kBlkBytes + 1024 * i);
    }
    advance(p, ic);
    ++jn;
    ist = (ist == S - 1) ? 0 : ist + 1;
  };

  // ---- per-lane LDS read offsets within a stage ----
  const int tk = row_token(c16);                  // token of this lane's K row
  int kread[KVB == 2 ? KS : KS / 2];
#pragma unroll
  for (int s = 0; s < (KVB == 2 ? KS : KS / 2); ++s) {
    const int chunk = 4 * s + q4;
    kread[s] = 16 * (tk * R::kCPR + (chunk ^ R::swk(tk)));
  }
  int vread[KVB == 2 ? NM : 4];
  if constexpr (KVB == 2) {
    // V^T rows: lane supplies token row_token(4*q4 + c16/4), d = 16m + 4*(c16%4)
    const int tv = row_token(4 * q4 + c16 / 4);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int chunk = 2 * m + (c16 % 4) / 2;
      vread[m] = R::kBlkBytes + 16 * (tv * R::kCPR + (chunk ^ R::swv(tv))) + 8 * (c16 & 1);
    }
  } else {
    // fp8 rows: tokens row_token(4*q4 + k), bytes VE*c16 .. VE*c16 + VE-1
#pragma unroll
    for (int k = 0; k < 4; ++k) vread[k] = R::kBlkBytes + row_token(4 * q4 + k) * R::kRowBytes + VE * c16;
  }

  while (can_issue(S - 1)) issue_one();

  float c2 = p.scale_log2;   // per segment with per-head K scales
  vec8 qop[HT][KS];
  float slope2[HT];     // ALiBi slope of this lane's head, in log2 units
  int seg = 0;          // segments this worker has finished
  int seg_b0 = 0;       // first block of the current segment

  int st_i = 0;         // stage of unit i
  for (int i = 0; i < n; ++i) {
    while (can_issue(i + S)) issue_one();
    wait_blocks<R::kIPB, S - 1>(jn - 1 - i);    // unit i landed (jn > i always holds here)
    const unsigned char* st = ring + st_i * kStage;

    // ---- segment start: query operands, fresh softmax state ----
    if (cur.b == 0 || i == 0) {
      seg_b0 = cur.b;
      if constexpr (KVB == 1) {
        const CAttnParams* kp = kernarg_params();
        if (kp->k_scales != nullptr) c2 = kp->scale_log2 * head_scale(kp->k_scales, cur.kvh);
      }
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        const int hig = ht * 16 + c16;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const int d0 = (KVB == 2) ? (32 * s + 8 * q4) : (64 * (s / 2) + 16 * q4 + 8 * (s % 2));
          const u32x4 v = *reinterpret_cast<const u32x4*>(qarea + (hig * D + d0) * 2);
          qop[ht][s] = __builtin_bit_cast(vec8, hig < G ? v : u32x4{0u, 0u, 0u, 0u});
        }
        m_used[ht] = -INFINITY;
        l_run[ht] = 0.f;
        if constexpr (MASK) {
          // the group's slopes by scalar loads (a vector load here would be
          // counted with the ring's copies), each lane keeping its head's
          slope2[ht] = 0.f;
          if (p.alibi != nullptr) {
            const int32_t* sl = reinterpret_cast<const int32_t*>(p.alibi) + cur.kvh * G;
            for (int h = ht * 16; h < min(G, ht * 16 + 16); ++h) {
              const float v = __builtin_bit_cast(float, load_uniform(sl, h));
              slope2[ht] = (hig == h) ? v * kLog2e : slope2[ht];
            }
          }
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[ht][m] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      q_pending = false;   // the next copy waits for these reads (lgkmcnt) before it lands
    }

    // ---- S^T = K . Q^T ----
    f32x4 sc[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) sc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      vec8 kop;
      if constexpr (KVB == 2) {
        kop = __builtin_bit_cast(vec8, *reinterpret_cast<const u32x4*>(st + kread[s]));
      } else {
        const u32x4 w = *reinterpret_cast<const u32x4*>(st + kread[s / 2]);
        const unsigned d0 = w[2 * (s % 2)], d1 = w[2 * (s % 2) + 1];
        kop = __builtin_bit_cast(vec8, u32x4{widen8x2<CT, I8>(d0, false), widen8x2<CT, I8>(d0, true),
                                             widen8x2<CT, I8>(d1, false), widen8x2<CT, I8>(d1, true)});
      }
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) sc[ht] = M::mma16(kop, qop[ht][s], sc[ht]);
    }

    // ---- masks: tokens past the sequence or before the window, absent
    // blocks (selects only) ----
    const int tok0 = (cur.b0 + cur.b) * kBlock;
    const bool blk_ok = (okbits >> st_i) & 1u;
    unsigned vm0 = 0xFFFFFFFFu, vm1 = 0xFFFFFFFFu;
    if (!blk_ok || tok0 + kBlock > cur.s_eff || (MASK && tok0 < cur.lo)) {
      bool bad[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int tok = tok0 + row_token(4 * q4 + k);
        bad[k] = !blk_ok || tok >= cur.s_eff || (MASK && tok < cur.lo);
      }
      vm0 = (bad[0] ? 0u : 0x0000FFFFu) | (bad[1] ? 0u : 0xFFFF0000u);
      vm1 = (bad[2] ? 0u : 0x0000FFFFu) | (bad[3] ? 0u : 0xFFFF0000u);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int k = 0; k < 4; ++k) sc[ht][k] = bad[k] ? -INFINITY : sc[ht][k];
    }

    // ---- online softmax (lazy rescale), P^T as the B operand ----
    u32x2 pop[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float x[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) x[k] = sc[ht][k] * c2;
      if constexpr (MASK) {
        // ALiBi: slope * (key - query position), the query at position s - 1
#pragma unroll
        for (int k = 0; k < 4; ++k)
          x[k] += slope2[ht] * (float)(tok0 + row_token(4 * q4 + k) - (cur.s_eff - 1));
      }
      // A head's reference max only moves when one of its scores exceeds it
      // by 2^8; each lane tests its own 4 scores, and only when some lane
      // does (rare after a segment's first block) is the head max formed
      // across the head's 4 lanes and the accumulator rescaled.
      const float lm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      if (__builtin_amdgcn_ballot_w64(lm > m_used[ht] + kRescaleLog2)) {
        float mx = fmaxf(lm, shfl_xor(lm, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const bool grow = mx > m_used[ht] + kRescaleLog2;
        const float m_new = grow ? mx : m_used[ht];
        const float alpha = grow ? fast_exp2(m_used[ht] - m_new) : 1.f;
        l_run[ht] *= alpha;
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[ht][m] *= alpha;
        m_used[ht] = m_new;
      }
      const float msub = (m_used[ht] == -INFINITY) ? 0.f : m_used[ht];
      float pr[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) pr[k] = fast_exp2(x[k] - msub);
      pop[ht] = u32x2{pack2<CT>(pr[0], pr[1]), pack2<CT>(pr[2], pr[3])};
      // the row sum adds the rounded probabilities the PV product multiplies
      l_run[ht] = M::sum2(pop[ht][1], M::sum2(pop[ht][0], l_run[ht]));
    }

    // ---- O^T += V^T . P^T ----
    if constexpr (KVB == 2) {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        u32x2 a = lds_read_tr16(st + vread[m]);
        a = u32x2{a[0] & vm0, a[1] & vm1};
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc[ht][m] = M::mma16k16(a, pop[ht], acc[ht][m]);
      }
    } else {
      unsigned w[4][(VE + 3) / 4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (VE == 8) {
          const u32x2 v = *reinterpret_cast<const u32x2*>(st + vread[k]);
          w[k][0] = v[0];
          w[k][1] = v[1];
        } else {
          w[k][0] = *reinterpret_cast<const unsigned*>(st + vread[k]);
        }
      }
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const unsigned sel = (m & 2) ? 0x07030602u : 0x05010400u;
        const unsigned x01 = perm(w[1][m / 4], w[0][m / 4], sel);
        const unsigned x23 = perm(w[3][m / 4], w[2][m / 4], sel);
        u32x2 a{widen8x2<CT, I8>(x01, (m & 1) != 0), widen8x2<CT, I8>(x23, (m & 1) != 0)};
        a = u32x2{a[0] & vm0, a[1] & vm1};
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc[ht][m] = M::mma16k16(a, pop[ht], acc[ht][m]);
      }
    }

    // ---- segment end: output rows of a whole head; a head cut at the
    // range's start that ends inside it leaves its partial in the worker's
    // slot; a head cut at the range's end keeps its state in registers for
    // the workgroup merge ----
    if (cur.b == cur.nb - 1 || i == n - 1) {
      const bool whole = seg_b0 == 0 && cur.b == cur.nb - 1;
      if (whole) {
        const float vsc = v_scale_of<KVB>(p, cur.kvh);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          float lt = l_run[ht];
          lt += shfl_xor(lt, 16);
          lt += shfl_xor(lt, 32);
          const int hig = ht * 16 + c16;
          if (hig < G) {
            const float inv = (lt > 0.f) ? vsc / lt : 0.f;
            unsigned short* orow = static_cast<unsigned short*>(p.out) +
                                   (int64_t)cur.q_row * p.out_row_stride +
                                   (int64_t)(cur.kvh * G + hig) * D;
            if constexpr (KVB == 2) {
#pragma unroll
              for (int m = 0; m < NM; ++m) {
                // rows 4*q4 .. 4*q4+3 of tile m: d = 16m + 4*q4 + k, contiguous
                st8(orow + 16 * m + 4 * q4,
                    u32x2{pack2<CT>(acc[ht][m][0] * inv, acc[ht][m][1] * inv),
                          pack2<CT>(acc[ht][m][2] * inv, acc[ht][m][3] * inv)});
              }
            } else {
              // 8-bit rows: d = VE*(4*q4 + k) + m, so m = 0..NM-1 is contiguous
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                unsigned w[NM / 2];
#pragma unroll
                for (int m = 0; m < NM; m += 2)
                  w[m / 2] = pack2<CT>(acc[ht][m][k] * inv, acc[ht][m + 1][k] * inv);
                unsigned short* dst = orow + VE * (4 * q4 + k);
                if constexpr (NM == 8) {
                  st16(dst, u32x4{w[0], w[1], w[2], w[3]});
                } else {
                  st8(dst, u32x2{w[0], w[1]});
                }
              }
            }
          }
        }
      } else if (i < n - 1) {
        // the worker's first head, begun before its range: its weighted
        // sums wait in the worker's slot for the workgroup merge, its
        // running max and sum in registers
        store_partial(p.ws_facc + (int64_t)worker * G * D, nullptr, acc, m_used, l_run);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
          float lt = l_run[ht];
          lt += shfl_xor(lt, 16);
          lt += shfl_xor(lt, 32);
          f_m[ht] = m_used[ht];
          f_l[ht] = lt;
        }
        has_f = true;
        f_first = g0 + i - cur.b;
        f_end = g0 + i + 1;
        f_kvh = cur.kvh;
        f_qrow = cur.q_row;
      } else {
        has_l = true;
        l_first = g0 + i - cur.b;
        l_end = l_first + cur.nb;
        l_kvh = cur.kvh;
        l_qrow = cur.q_row;
      }
      ++seg;
    }
    advance(p, cur);
    st_i = (st_i == S - 1) ? 0 : st_i + 1;
  }
  }   // active

  // ---- workgroup merge.  The workgroup's range is the union of its
  // workers' ranges.  Each worker with a cut last head stages that partial in
  // its own LDS region (its ring has drained), and the running max and sum of
  // a first head it left in its slot.  After a barrier the whole workgroup
  // merges every head cut between its workers, in worker order: a head that
  // begins and ends inside the workgroup's range is finished here, and the at
  // most two heads it shares with neighbouring workgroups (the one holding
  // its first unit -> slot 0, the one holding its last -> slot 1) leave one
  // partial each for the reduce kernel.  All global loads of the merge (the
  // first-head weighted sums) are issued before any of its stores, so no wait
  // for them covers a store. ----
  // a wave's region: the last-head partial ([G][D] sums, [G][2] max and
  // sum), the first head's [G][2] max and sum, and a record of its heads
  struct MergeInfo {
    int64_t l_first, l_end, f_first, f_end;
    int flags, l_kvh, l_qrow, f_kvh, f_qrow;
  };
  constexpr int kFmlOff = 16 * HT * (D + 2) * 4;
  constexpr int kInfoOff = kWaveBytes - 64;
  static_assert(sizeof(MergeInfo) <= 64, "merge record");
  static_assert(kFmlOff + 16 * HT * 2 * 4 <= kInfoOff, "partials must fit a wave's LDS region");
  constexpr int kL = 1, kF = 2, kBusy = 4;
  auto info = [&](int w) __attribute__((always_inline)) {
    return reinterpret_cast<MergeInfo*>(lds + w * kWaveBytes + kInfoOff);
  };
  auto lacc = [&](int w) __attribute__((always_inline)) {
    return reinterpret_cast<float*>(lds + w * kWaveBytes);
  };
  auto lml = [&](int w) __attribute__((always_inline)) { return lacc(w) + G * D; };
  auto fml = [&](int w) __attribute__((always_inline)) {
    return reinterpret_cast<float*>(lds + w * kWaveBytes + kFmlOff);
  };
  if (has_l) store_partial(lacc(wave), lml(wave), acc, m_used, l_run);
  if (has_f) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int hig = ht * 16 + c16;
      if (hig < G && q4 == 0) {
        fml(wave)[2 * hig] = f_m[ht];
        fml(wave)[2 * hig + 1] = f_l[ht];
      }
    }
  }
  if (lane == 0) {
    MergeInfo* mi = info(wave);
    mi->flags = (active ? kBusy : 0) | (has_l ? kL : 0) | (has_f ? kF : 0);
    mi->l_first = l_first;
    mi->l_end = l_end;
    mi->f_first = f_first;
    mi->f_end = f_end;
    mi->l_kvh = l_kvh;
    mi->l_qrow = l_qrow;
    mi->f_kvh = f_kvh;
    mi->f_qrow = f_qrow;
  }
  // the workgroup's range (formed while the other waves finish)
  const int64_t wg0 = (int64_t)blockIdx.x * WV;
  const int64_t wg_begin = range_begin(wg0, T, W);
  const int64_t wg_end = range_begin(min(wg0 + WV, (int64_t)W), T, W);
  wait_vmcnt<0>();   // the first-head sums (and this worker's output rows) are stored
  __syncthreads();
  const int tid = threadIdx.x;
  constexpr int NT = 64 * WV;
  // each thread takes groups of 4 consecutive elements (one head each)
  constexpr int kGPT = (16 * HT * D / 4 + NT - 1) / NT;   // element groups per thread, at most
  // the workers' records, lane v of every wave holding worker v's
  const MergeInfo* mi_l = info(lane < WV ? lane : 0);
  const int r_flags = lane < WV ? mi_l->flags : 0;
  const int64_t r_lfirst = mi_l->l_first, r_lend = mi_l->l_end, r_ffirst = mi_l->f_first;
  const int r_lkvh = mi_l->l_kvh, r_lqrow = mi_l->l_qrow, r_fkvh = mi_l->f_kvh, r_fqrow = mi_l->f_qrow;
  const unsigned fmask = (unsigned)__builtin_amdgcn_ballot_w64((r_flags & kF) != 0);
  // every first-head partial's sums of this thread's groups, loaded first
  f32x4 fa[WV][kGPT];
#pragma unroll
  for (int v = 0; v < WV; ++v) {
    const bool fv = (fmask >> v) & 1u;
    const float* src = p.ws_facc + (wg0 + v) * G * D;
#pragma unroll
    for (int q = 0; q < kGPT; ++q) {
      const int e = 4 * (tid + q * NT);
      fa[v][q] = (fv && e < G * D) ? *reinterpret_cast<const f32x4*>(src + e) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  float* const slot_acc = p.ws_acc + (int64_t)blockIdx.x * 2 * G * D;
  float* const slot_ml = p.ws_ml + (int64_t)blockIdx.x * 2 * G * 2;
  // one run: the last-head partials of `lmask` and the first-head partial
  // of worker fw (or none), merged in worker order
  // Every wave's region is read whatever the mask says (a region outside
  // the run may hold anything, so its terms are removed by selects, never by
  // a zero weight): reads behind a branch per wave would each wait out a
  // full LDS latency on their own.
  auto merge_run = [&](unsigned lmask, int fw, bool complete, int slot, int kvh, int q_row)
      __attribute__((always_inline)) {
    const int fsel = fw >= 0 ? fw : 0;
#pragma unroll
    for (int q = 0; q < kGPT; ++q) {
      const int e = 4 * (tid + q * NT);
      if (e >= G * D) break;
      const int h = e / D;
      f32x2 ml[WV];
      f32x4 av[WV];
#pragma unroll
      for (int v = 0; v < WV; ++v) {
        ml[v] = *reinterpret_cast<const f32x2*>(lml(v) + 2 * h);
        av[v] = *reinterpret_cast<const f32x4*>(lacc(v) + e);
      }
      const f32x2 fml_h = *reinterpret_cast<const f32x2*>(fml(fsel) + 2 * h);
      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < WV; ++v) mx = ((lmask >> v) & 1u) ? fmaxf(mx, ml[v][0]) : mx;
      if (fw >= 0) mx = fmaxf(mx, fml_h[0]);
      const float Ms = (mx == -INFINITY) ? 0.f : mx;
      float L = 0.f;
      f32x4 A{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < WV; ++v) {
        const bool in = (lmask >> v) & 1u;
        const float wgt = fast_exp2(ml[v][0] - Ms);
        L = in ? L + wgt * ml[v][1] : L;
        const f32x4 t = A + wgt * av[v];
        A = in ? t : A;
      }
      if (fw >= 0) {
        const float wgt = fast_exp2(fml_h[0] - Ms);
        L += wgt * fml_h[1];
        f32x4 fv{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int v = 0; v < WV; ++v) fv = (v == fw) ? fa[v][q] : fv;
        A += wgt * fv;
      }
      if (complete) {
        const float inv = (L > 0.f) ? v_scale_of<KVB>(p, kvh) / L : 0.f;
        unsigned short* orow = static_cast<unsigned short*>(p.out) + (int64_t)q_row * p.out_row_stride +
                               (int64_t)kvh * G * D + e;
        st8(orow, u32x2{pack2<CT>(A[0] * inv, A[1] * inv), pack2<CT>(A[2] * inv, A[3] * inv)});
      } else {
        *reinterpret_cast<f32x4*>(slot_acc + slot * G * D + e) = A;
        if (e % D == 0) {
          slot_ml[slot * G * 2 + 2 * h] = mx;
          slot_ml[slot * G * 2 + 2 * h + 1] = L;
        }
      }
    }
  };
  // The runs, found lane-parallel from the records (lane v = worker v):
  // worker v continues a run when it holds a cut last head equal to the one
  // of the previous worker that streamed anything; its first head ends that
  // worker's run when it equals that worker's last head.  A run starts at
  // each last head that continues nothing and ends before the first
  // streaming worker after it that does not continue it, whose first head
  // (if attached) closes it; a first head attached to nothing began before
  // the workgroup's range and is its only piece here (slot 0).
  const unsigned bmask = (unsigned)__builtin_amdgcn_ballot_w64((r_flags & kBusy) != 0);
  const unsigned lmask_all = (unsigned)__builtin_amdgcn_ballot_w64((r_flags & kL) != 0);
  const unsigned below = lane < WV ? bmask & ((1u << lane) - 1u) : 0u;
  const int prv = below != 0u ? 31 - __builtin_clz(below) : 0;
  const int p_flags = __builtin_amdgcn_ds_bpermute(prv << 2, r_flags);
  const int p_lo = __builtin_amdgcn_ds_bpermute(prv << 2, (int)(uint32_t)r_lfirst);
  const int p_hi = __builtin_amdgcn_ds_bpermute(prv << 2, (int)(r_lfirst >> 32));
  const int64_t p_lfirst = (int64_t)(((uint64_t)(uint32_t)p_hi << 32) | (uint32_t)p_lo);
  const bool prev_l = below != 0u && (p_flags & kL) != 0;
  const unsigned cmask =
      (unsigned)__builtin_amdgcn_ballot_w64((r_flags & kL) != 0 && prev_l && p_lfirst == r_lfirst);
  const unsigned amask =
      (unsigned)__builtin_amdgcn_ballot_w64((r_flags & kF) != 0 && prev_l && p_lfirst == r_ffirst);
  for (unsigned a = fmask & ~amask; a != 0u; a &= a - 1u) {   // uniform
    const int w = __builtin_ctz(a);
    merge_run(0u, w, false, 0, __builtin_amdgcn_readlane(r_fkvh, w), __builtin_amdgcn_readlane(r_fqrow, w));
  }
  for (unsigned st = lmask_all & ~cmask; st != 0u; st &= st - 1u) {   // uniform
    const int w = __builtin_ctz(st);
    const unsigned after = bmask & ~cmask & ~((2u << w) - 1u);
    const int e1 = after != 0u ? __builtin_ctz(after) : WV;
    const unsigned lmask = (cmask & ((1u << e1) - 1u) & ~((2u << w) - 1u)) | (1u << w);
    const int fw = (e1 < WV && ((amask >> e1) & 1u)) ? e1 : -1;
    const int64_t X = readlane64(r_lfirst, w);
    const int64_t Xend = readlane64(r_lend, w);
    merge_run(lmask, fw, X >= wg_begin && Xend <= wg_end, X <= wg_begin ? 0 : 1,
              __builtin_amdgcn_readlane(r_lkvh, w), __builtin_amdgcn_readlane(r_lqrow, w));
  }
}

// Merge of the partials of one (request, query head) whose K/V head was cut
// between workgroups g_a .. g_b (a head cut only between workers of one
// workgroup was finished by that workgroup): one wave.  Lanes take partials
// (64 at a time) for the global max and the weighted sum of the row sums;
// then each lane accumulates its D/64 output columns over the partials in
// workgroup order with the weights broadcast from the lane that owns them.
// Fixed order, no atomics: deterministic.
template <int D, typename CT>
__global__ __launch_bounds__(64) void decode_reduce_kernel(AttnParams p) {
  constexpr int DPL = D / 64;   // output columns per lane
  constexpr int RB = 16;        // partials whose loads are in flight together
  const int rr = blockIdx.y;
  const int qh = blockIdx.x;
  const int lane = threadIdx.x;
  // every value the partials' location depends on, loaded together
  const int r = p.req_begin + rr;
  const int rq0 = load_uniform(p.qsl, r);
  const int rq1 = load_uniform(p.qsl, r + 1);
  const int rs = load_uniform(p.seq_lens, r);
  const int64_t T = p.ws_cum[p.num_reqs];
  const int64_t cum = p.ws_cum[rr];
  const int nb = blocks_of(p, rq0, rq1, rs);
  if (nb == 0) return;
  const int G = p.group;
  const int kvh = qh / G;
  const int hig = qh % G;
  const int64_t W = p.num_workers;
  const int64_t WV = p.wg_waves;
  const int64_t a = cum + (int64_t)kvh * nb;
  const int64_t b = a + nb;
  // workgroups holding units a and b-1 (worker indices fit 32 bits)
  const int64_t ga = (int)div_floor((a + 1) * W - 1, T) / (int)WV;
  const int64_t gb = (int)div_floor(b * W - 1, T) / (int)WV;
  if (ga == gb) return;
  const int cnt = (int)(gb - ga + 1);
  // partial of the i-th workgroup of the cut: slot 1 for g_a if its range
  // began before this head (the head holds its last unit), else slot 0;
  // when T >= W every workgroup range holds units, otherwise a workgroup
  // whose range is empty holds none
  const int sl_a = range_begin(ga * WV, T, W) < a ? 1 : 0;
  auto part_index = [&](int i, bool& valid) -> int64_t {
    const int64_t g = ga + i;
    valid = T >= W || range_begin(g * WV, T, W) < range_begin(min(g * WV + WV, W), T, W);
    return (g * 2 + (i == 0 ? sl_a : 0)) * G + hig;
  };

  float lsum = 0.f;
  float o[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) o[e] = 0.f;
  bool ok0;
  const int64_t ix0 = part_index(0, ok0);   // workgroup g_a always holds a partial
  if (cnt <= RB) {
    // the common case: every partial's (max, sum) pair (one per lane) and
    // columns loaded at once, then the weights
    bool ok = false;
    int64_t ix = ix0;
    if (lane < cnt) {
      ix = part_index(lane, ok);
      ix = ok ? ix : ix0;   // a missing partial reads an existing one, weight 0
    }
    const f32x2 ml = *reinterpret_cast<const f32x2*>(p.ws_ml + ix * 2);
    float v[RB][DPL];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const float* ap = p.ws_acc + readlane64(ix, min(u, cnt - 1)) * D + lane;
#pragma unroll
      for (int e = 0; e < DPL; ++e) v[u][e] = ap[64 * e];
    }
    float mx = ok ? ml[0] : -INFINITY;
#pragma unroll
    for (int off = RB / 2; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor(mx, off));
    mx = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, mx)));
    const float msafe = (mx == -INFINITY) ? 0.f : mx;
    const float w = ok ? fast_exp2(ml[0] - msafe) : 0.f;
    float t = ok ? w * ml[1] : 0.f;
#pragma unroll
    for (int off = RB / 2; off >= 1; off >>= 1) t += shfl_xor(t, off);
    lsum = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, t)));
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), u));
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[e] += (u < cnt ? wu : 0.f) * v[u][e];
    }
  } else {
  float mloc = -INFINITY;
  for (int i = lane; i < cnt; i += 64) {
    bool ok;
    const int64_t ix = part_index(i, ok);
    if (ok) mloc = fmaxf(mloc, p.ws_ml[ix * 2]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mloc = fmaxf(mloc, shfl_xor(mloc, off));
  const float msafe = (mloc == -INFINITY) ? 0.f : mloc;
  for (int g = 0; g < cnt; g += 64) {
    const int i = g + lane;
    bool ok = false;
    int64_t ix = (i < cnt) ? part_index(i, ok) : 0;
    const float w = ok ? fast_exp2(p.ws_ml[ix * 2] - msafe) : 0.f;
    float t = ok ? w * p.ws_ml[ix * 2 + 1] : 0.f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) t += shfl_xor(t, off);
    lsum += t;
    // a missing partial reads an existing one with weight 0 (its memory may
    // hold anything, and 0 * NaN is NaN); batches of RB keep loads in flight
    ix = ok ? ix : ix0;
    const int m = min(64, cnt - g);
    for (int j0 = 0; j0 < m; j0 += RB) {
      float wj[RB], v[RB][DPL];
#pragma unroll
      for (int u = 0; u < RB; ++u) {
        const int j = min(j0 + u, m - 1);
        wj[u] = (j0 + u < m) ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j))
                             : 0.f;
        const float* ap = p.ws_acc + readlane64(ix, j) * D + lane;
#pragma unroll
        for (int e = 0; e < DPL; ++e) v[u][e] = ap[64 * e];
      }
#pragma unroll
      for (int u = 0; u < RB; ++u)
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] += wj[u] * v[u][e];
    }
  }
  }
  const float inv = (lsum > 0.f) ? v_scale_of<1>(p, kvh) / lsum : 0.f;
  unsigned short* orow = static_cast<unsigned short*>(p.out) + (int64_t)rq0 * p.out_row_stride +
                         (int64_t)qh * D;
#pragma unroll
  for (int e = 0; e < DPL; ++e) orow[lane + 64 * e] = Mfma<CT>::from_float(o[e] * inv);
}

// Waves per workgroup and ring depth for one instantiation: a block of an
// 8-bit cache carries half the bytes of a 16-bit one for the same per-block
// math, so eight waves per compute unit share the work (two waves per SIMD
// keep its issue slots busy); 16-bit caches use four.  The ring is as deep as
// the configured depth where it fits the LDS.
template <int D, int KVB, int HT>
constexpr int waves_per_wg() { return decode_waves_per_cu(KVB == 1 ? kFP8 : kF16); }

template <int D, int KVB, int HT>
constexpr int ring_depth() {
  constexpr int wv = waves_per_wg<D, KVB, HT>();
  constexpr int stage = 2 * Ring<D, KVB>::kBlkBytes;
  constexpr int qcap = HT * 16 * D * 2;
  constexpr int fit = (kLdsBudget / wv - qcap) / stage;
  constexpr int want = KVB == 1 ? kStages8 : kStages;
  return want < fit ? want : fit;
}

template <int D, typename CT, int KVB, bool I8, int HT>
hipError_t launch_typed(const AttnParams& p, hipStream_t stream) {
  constexpr int WV = waves_per_wg<D, KVB, HT>();
  constexpr int S = ring_depth<D, KVB, HT>();
  dim3 grid((unsigned)((p.num_workers + WV - 1) / WV));
  if (p.masked) {
    hipLaunchKernelGGL((decode_kernel<D, CT, KVB, I8, HT, S, WV, true>), grid, dim3(64 * WV), 0, stream, p);
  } else {
    hipLaunchKernelGGL((decode_kernel<D, CT, KVB, I8, HT, S, WV, false>), grid, dim3(64 * WV), 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 rgrid((unsigned)p.num_q_heads, (unsigned)p.num_reqs);
  hipLaunchKernelGGL((decode_reduce_kernel<D, CT>), rgrid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

template <int D, typename CT, int KVB, bool I8>
hipError_t launch_heads(const AttnParams& p, hipStream_t stream) {
  if (p.group <= 16) return launch_typed<D, CT, KVB, I8, 1>(p, stream);
  if (p.group <= 32) return launch_typed<D, CT, KVB, I8, 2>(p, stream);
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_dim(const AttnParams& p, int act, int cache, hipStream_t stream) {
  if (act == kF16 && cache == kF16) return launch_heads<D, _Float16, 2, false>(p, stream);
  if (act == kBF16 && cache == kBF16) return launch_heads<D, __bf16, 2, false>(p, stream);
  if (act == kF16 && cache == kFP8) return launch_heads<D, _Float16, 1, false>(p, stream);
  if (act == kBF16 && cache == kFP8) return launch_heads<D, __bf16, 1, false>(p, stream);
  if (act == kF16 && cache == kINT8) return launch_heads<D, _Float16, 1, true>(p, stream);
  if (act == kBF16 && cache == kINT8) return launch_heads<D, __bf16, 1, true>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const AttnParams& p, int act_dtype, int cache_dtype, hipStream_t stream) {
  if (p.num_reqs == 0 || p.num_workers == 0) return hipSuccess;
  if (p.head_dim == 128) return launch_dim<128>(p, act_dtype, cache_dtype, stream);
  if (p.head_dim == 64) return launch_dim<64>(p, act_dtype, cache_dtype, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
