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
// Work decomposition.  An item is (request, group of `hpw` query heads
// sharing one K/V head, tile of queries); each wave of the workgroup working
// on it takes one query head and 32 queries, and all waves share each 64-key
// K/V tile in LDS.  The grid is one resident workgroup per compute unit, each
// working through its own list of items (see the kernel's schedule comment):
// no unit waits for the dispatcher between items.  Within a request, items
// run from the END of the request (the most keys) to its start.
// One kernel, prefill_pp_kernel: 8 waves, 256/hpw queries per item,
// K/V tiles copied global -> LDS by DMA into 4-stage rings, and two groups of
// 4 waves alternating between the MFMA phase and the softmax phase (see the
// kernel's own comment); 8-bit tiles (fp8, int8) land in a ring of their own
// and each wave widens the rows it copied into two bf16/fp16 operand stages.
// Per tile a wave computes S^T = K . Q^T (v_mfma_f32_32x32x16, keys x queries)
// so each lane holds 32 scores of ONE query: the row max needs one exchange
// with the lane 32 apart and every rescale is lane-local.  The probabilities,
// rounded to bf16/fp16, are directly the B operand of O^T = V^T . P^T.
// Softmax in exp2 form with the scale folded into one FMA; the accumulator is
// only rescaled when a row's running max grows by more than 2^8 (exact up to
// rounding: the reference max of a softmax is arbitrary as long as nothing
// overflows).
// Mask variants (MASK instantiations; the alibi_slopes and window_size
// arguments of the same call): a sliding window starts the key loop at the
// first tile any query of the workgroup may see and skips a wave's softmax
// on tiles wholly before its queries' windows (their MFMAs run with zero
// probabilities); ALiBi adds slope * (key - query
// position) to each score, applied together with the window mask when the
// scores are moved to log2 units (window_alibi).
#include <type_traits>

#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kBlock = 16;
constexpr int kTileK = 64;          // keys per LDS tile
constexpr float kRescaleLog2 = 8.f; // lazy rescale threshold (log2 units)
constexpr float kLog2e = 1.4426950408889634f;

// Mask variants (sliding window, ALiBi) of one score tile, in place: every
// score is moved to log2 units with its ALiBi bias, slope * (key - query
// position), and on tiles that reach before some row's window (`edge`) the
// keys before a row's window get -inf.  The caller's softmax then runs with a
// unit scale.  Lane layout as in the kernel: element g of subtile u is key
// k0 + 4*half + (32u + 8(g/4) + g%4) of the lane's query, so the bias is
// slope * (k0 + 4*half - qpos) plus slope times a compile-time offset.
__device__ inline void window_alibi(f32x16 (&sc)[2], int k0, int half, int qpos, int window_left,
                                    float scale_log2, float slope2, bool edge) {
  const int base = k0 + 4 * half - qpos;
  const float sb = slope2 * (float)base;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      const int off = 32 * u + 8 * (g / 4) + (g % 4);
      sc[u][g] = __builtin_fmaf(sc[u][g], scale_log2, __builtin_fmaf(slope2, (float)off, sb));
    }
  if (edge) {
    // key < qpos - window_left  <=>  off < -window_left - base (clamped to
    // the offsets' range 0..63, in 64 bits so no window width can overflow)
    const int64_t lim64 = -(int64_t)window_left - base;
    int lim = (int)(lim64 < -1 ? -1 : (lim64 > 64 ? 64 : lim64));
    // compare in 32 bits below (left to itself the compiler folds the clamp
    // into 64-bit compares against constants held in scalar registers)
    asm volatile("" : "+v"(lim));
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int g = 0; g < 16; ++g)
        sc[u][g] = (32 * u + 8 * (g / 4) + (g % 4) < lim) ? -INFINITY : sc[u][g];
  }
}

// ---------------------------------------------------------------------------
// K/V tiles are moved global -> LDS by the DMA path (global_load_lds, 16
// bytes per lane, no registers) and V is read back transposed with
// ds_read_b64_tr_b16.
//
// LDS layout: per tile, K and V are each [64 keys][D/8 16-byte chunks] with
// the chunks of key k stored at position (chunk ^ sw(k)); one DMA wave
// instruction fills 64 consecutive positions, so each lane fetches the global
// chunk that belongs at its position.  The swizzles keep every read
// conflict-free: the S^T operand reads one chunk of 32 consecutive keys
// (sw_k spreads 16 consecutive keys over 16 bank groups); the transposing V
// read takes 4 consecutive keys x 32 bytes per 16 lanes (sw_v gives the 4
// keys disjoint 64-byte bank groups).
//
// ds_read_b64_tr_b16 (gfx950): within each 16-lane group lane i supplies the
// address of a row R_i of four 16-bit values and lane j receives
// R_{4k + j/4}[j % 4], k = 0..3.  With lane i = 4a + b pointing at
// V[key_a][d0 + 4b .. 4b+3], lane j receives V[key_0..3][d0 + j]: four keys of
// one d column, i.e. half of a v_mfma_f32_32x32x16 A operand of V^T.
// Keys the tile does not have (past the sequence, absent blocks) are loaded
// from a valid address and their V rows are overwritten with zeros once the
// DMA has landed, so 0-probability keys never meet a NaN.
template <int D>
struct LdsTile {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per key row
  static constexpr int kPos = kTileK * CPR;         // 16-byte positions per tile (K or V)
  static constexpr int kInst = kPos / 64;           // DMA wave instructions per tile (K or V)
  __device__ static inline int swk(int key) { return D == 128 ? (key & 15) : ((key >> 1) & 7); }
  __device__ static inline int swv(int key) { return D == 128 ? 4 * (key & 3) : 4 * ((key >> 1) & 1); }
};

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
// the kernel's parameter block in the kernarg segment (read-only, scalar loads)
typedef __attribute__((address_space(4))) const AttnParams CParams;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

__device__ inline u32x2 lds_read_tr16(const u32x4* base, int pos16, int byte_off) {
  const char* p = reinterpret_cast<const char*>(base + pos16) + byte_off;
  lds_bf16x4* lp = (lds_bf16x4*)(const_cast<char*>(p));
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lp));
}

// ---------------------------------------------------------------------------
// Eight waves in two groups of four (one wave of each group on every SIMD)
// that alternate between a matrix phase and a softmax phase, so the MFMAs of
// one group run while the other group computes its softmax.
//
// Per wave and 64-key tile j the work splits into
//   M(j): S_j = K_j . Q^T and O^T += V_{j-1}^T . P_{j-1}^T (MFMA, LDS reads)
//   V(j): the copies of K tile j+3 and V tile j+2 are issued first (the
//         address unit works through the group's copies while the softmax
//         runs, instead of holding up the barrier), then P_j from S_j (mask,
//         row max, lazy rescale, exp2, bf16/fp16 pack, row sum)
// and every wave runs M(j), barrier, V(j), barrier.  Group B passes one extra
// barrier before its loop (group A one after it), so between two consecutive
// barriers one group is in M and the other in V.
// K and V tiles live in two rings of four LDS stages (tile t in stage
// (t - first tile) % 4) with the LdsTile layout above, filled by global -> LDS
// copies issued from inline assembly (untracked by the compiler) and retired
// by explicit vmcnt waits: a copy issued in V(j) is waited for at the end of
// M(j+2), and the barrier after that wait publishes it.  Stage reuse: K tile
// t+4 is issued in V(t+1), after every wave has passed M(t), the last read of
// K tile t; V tile t+4 in V(t+2), after every M(t+1).  Each wave copies the
// rows of one block of every tile, so it needs one table entry per tile: a
// scalar load issued one V phase ahead of its use (no vector load the
// compiler would wait for behind the copies in flight).  The workgroup checks
// the table entries of an item once, when the item starts; only rows holding
// ids outside the pool test block presence per tile.
// 8-bit caches: the copies fill rings of 8-bit tiles in plain [key][chunk]
// order (one instruction per wave per tile: 1 KB at head_dim 128, 512 bytes
// from the lower 32 lanes at head_dim 64), and in M(j) each wave widens the
// rows it copied of K tile j+1 and V tile j into two operand stages (tile t
// in stage t % 2, LdsTile layout, V rows of absent keys zeroed); the barrier
// that ends M(j) publishes them.  Two operand stages suffice: K(j+1) and V(j)
// replace K(j-1) and V(j-2), whose last reads were in M(j-1), and the other
// group is in its softmax phase.  The widening (one 16-byte LDS read, 8
// converts, two 16-byte writes per lane and tensor) has to run in the MFMA
// phase: a wave can wait only for its own copies, and every row of K(j+1) and
// V(j) must be widened before the first group's M(j+1).  At head_dim 128 the
// copies are retired before the MFMAs, the 8-bit rows read ahead of them and
// converted among them, so only the two stores follow the last MFMA; at
// head_dim 64 (a phase half as long) the rows are read and widened after the
// MFMAs and the retiring wait.
constexpr int kPPWaves = 8;
constexpr int kPPThreads = 64 * kPPWaves;
constexpr int kPPStages = 4;

// Workgroup barrier that leaves the copies in flight: only this wave's LDS
// operations (and scalar loads) are waited for when `lds` is set.
template <bool LDS>
__device__ inline void barrier_nowait() {
  if constexpr (LDS) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Present blocks of key tile t as a 4-bit mask (block b present: inside the
// sequence's blocks and a pool id).  Only rows holding entries outside the
// pool take this path; all other tiles have every block present.
__device__ inline unsigned tile_okmask(const int32_t* bt_row, int nblk, int nb32, int t) {
  unsigned ok = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int id = load_uniform(bt_row, min(4 * t + b, nblk - 1));
    ok |= ((4 * t + b < nblk) & (id >= 0) & (id < nb32)) ? (1u << b) : 0u;
  }
  return ok;
}

template <int D, typename CT, int KVB, bool I8, bool MASK>
__global__ __launch_bounds__(kPPThreads) void prefill_pp_kernel(AttnParams p) {
  using M = Mfma<CT>;
  using vec8 = typename M::vec8;
  using L = LdsTile<D>;
  constexpr int QS = D / 16;                 // QK MFMA steps (16 d each)
  constexpr int DT = D / 32;                 // 32-row d tiles of O^T
  constexpr int NS = kPPStages;              // copy ring depth
  // operand stages (16-bit, LdsTile layout): the copy ring itself for 16-bit
  // caches; for 8-bit caches two stages that each wave fills by widening the
  // rows it copied into an 8-bit ring (tile t in 8-bit stage t % NS, operand
  // stage t % 2)
  constexpr int NO = KVB == 2 ? NS : 2;
  constexpr int CPR8 = D / 16;               // 16-byte chunks of an 8-bit key row
  constexpr int kPos8 = kTileK * CPR8;       // 16-byte positions of an 8-bit tile
  constexpr int kCopyPos = KVB == 2 ? L::kPos : kPos8;
  // lanes of a copy instruction: an 8-bit tile at head_dim 64 (4 KB) is too
  // small for eight full-wave instructions, so each wave copies 512 bytes
  // with its lower 32 lanes
  constexpr int LPI = kCopyPos >= 64 * kPPWaves ? 64 : kCopyPos / kPPWaves;
  constexpr int IPW = kCopyPos / LPI / kPPWaves;   // copy instructions per wave per tile (K and V each)
  constexpr int KPI = LPI / (KVB == 2 ? L::CPR : CPR8);   // keys per copy instruction
  constexpr int PPS = 4 * DT / QS;           // PV MFMAs per QK step
  static_assert(IPW * kPPWaves * LPI == kCopyPos && PPS * QS == 4 * DT, "tile shape");
  static_assert(2 * IPW * KPI == kBlock, "two waves copy each block of a tile");
  static_assert(KVB == 2 || IPW == 1, "8-bit tiles: one copy instruction per wave");
  constexpr unsigned kTileBytes = kCopyPos * 16;
  // 8-bit caches at head_dim 128 widen among the MFMAs of the phase (at
  // head_dim 64 the phase is too short to cover the earlier wait for the
  // copies: measured slower there)
  constexpr bool kWidenInM = KVB == 1 && D == 128;

  __shared__ u32x4 Kr[NO * L::kPos];
  __shared__ u32x4 Vr[NO * L::kPos];
  __shared__ u32x4 K8[KVB == 1 ? NS * kPos8 : 1];
  __shared__ u32x4 V8[KVB == 1 ? NS * kPos8 : 1];

  // ---- roles that hold for every item ----
  const int lane = threadIdx.x & 63;
  const int wave = wave_uniform(threadIdx.x >> 6);
  const int grp = wave >> 2;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  // The parameters are read afresh where an item starts and where it ends
  // (scalar loads through a pointer the compiler cannot see through), so the
  // values used only there are not held in scalar registers through the tile
  // loop: the loop needs nearly all of them, and over budget the compiler
  // stops running LDS reads ahead of the MFMAs.
  auto params = []() __attribute__((always_inline)) {
    const CParams* q = (const CParams*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(q));
    return q;
  };
  const int64_t tok_stride = (int64_t)p.num_kv_heads * D * KVB;

  // copy roles: instruction i of this wave fills positions inst*LPI ..
  // inst*LPI+LPI-1 of a tile, inst = wave*IPW + i: keys of block wave/2 of
  // the tile only, so a wave needs one block id per tile
  const int cb = wave >> 1;
  const bool copy_lane = LPI == 64 || lane < LPI;
  unsigned koff[IPW], voff[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int pidx = (wave * IPW + i) * LPI + (copy_lane ? lane : 0);
    if constexpr (KVB == 2) {
      const int key = pidx / L::CPR, pos = pidx % L::CPR;
      const unsigned row = (unsigned)((key % kBlock) * tok_stride);
      koff[i] = row + (unsigned)((pos ^ L::swk(key)) * 16);
      voff[i] = row + (unsigned)((pos ^ L::swv(key)) * 16);
    } else {
      // 8-bit ring: plain [key][chunk] order, each lane widens what it copied
      const int key = pidx / CPR8, pos = pidx % CPR8;
      koff[i] = voff[i] = (unsigned)((key % kBlock) * tok_stride) + (unsigned)(pos * 16);
    }
  }
  const unsigned kr0 = lds_offset(KVB == 2 ? Kr : K8), vr0 = lds_offset(KVB == 2 ? Vr : V8);

  // lane roles in the LDS reads
  const int kswz = L::swk(l32);                   // key 32u + l32 has the swizzle of l32
  const int g16 = lane >> 4;                      // 16-lane group
  const int ta = (lane & 15) >> 2, tb = lane & 3; // transposed-read row supplier (key a, d 4b)
  const int vswz = L::swv(ta);                    // keys ... + 4h + a share a's swizzle

  // ---- schedule ----
  // One resident workgroup per compute unit works through a list of items
  // (request, head group, QB-query tile); no workgroup waits for another, so
  // a unit goes from one item straight to its next.  With the grid a
  // multiple of the head-group count, workgroup w keeps head group w % nhg
  // (workgroups are spread over the 8 XCDs by number, so with 8 head groups
  // an XCD's L2 serves one K/V head) and takes that head group's items in
  // rounds of C = grid / nhg, in snake order (round k: position cw in even
  // rounds, C-1-cw in odd ones), so the longest and shortest items of
  // consecutive rounds pair up.  Items are ordered by request -- requests by
  // decreasing sequence length within each run of 64, ties by index -- and
  // within a request from its last tile (the most keys) to its first.
  // Request cursor over runs of 64 requests, lane l holding request 64*ch + l:
  // its first batch row, new tokens, sequence length, items, and the items
  // of the run ahead of it.  Each wave keeps its own copy in LDS (every wave
  // computes the same values), so none of it stays in registers while an
  // item runs.
  __shared__ int cur_lane[kPPWaves][5][64];
  __shared__ int cur_sc[kPPWaves][4];   // run, items before it, items in it, next item number
  cur_sc[wave][0] = -1;
  cur_sc[wave][1] = 0;
  cur_sc[wave][2] = 0;
  cur_sc[wave][3] = 0;

  // the first block-table entries of an item, read while the item before it
  // starts (tag = the item's number, then this wave's entries of its first
  // four tiles), so an item issues its first copies without a round trip
  __shared__ int pre_ids[kPPWaves][5];
  pre_ids[wave][0] = -1;

  struct ItemRec {
    int hg, r, bz, q_first, n, s_all;
  };
  // item number kk of this workgroup's list (false past its end); moves the
  // cursor forward only, so numbers must not decrease between calls
  auto lookup = [&](int kk, const CParams* pp, int QB, int nhg, ItemRec& it) __attribute__((always_inline)) {
    const int P = (int)gridDim.x;
    const bool pinned = P % nhg == 0;
    const int C = pinned ? P / nhg : P;
    const int cw = pinned ? (int)blockIdx.x / nhg : (int)blockIdx.x;
    const int pos = kk * C + ((kk & 1) ? C - 1 - cw : cw);
    it.hg = pinned ? (int)blockIdx.x % nhg : pos % nhg;
    const int tt = pinned ? pos : pos / nhg;
    int ch = wave_uniform(cur_sc[wave][0]);
    int ch_base = wave_uniform(cur_sc[wave][1]);
    int ch_total = wave_uniform(cur_sc[wave][2]);
    bool found = true;
    while (ch < 0 || tt >= ch_base + ch_total) {
      if (ch >= 0) ch_base += ch_total;
      ++ch;
      if (ch * 64 >= pp->num_reqs) {
        found = false;
        break;
      }
      const int rr = ch * 64 + lane;
      const bool v = rr < pp->num_reqs;
      const int ra = pp->req_begin + (v ? rr : 0);
      const int q0 = pp->qsl[ra];
      const int nn = v ? max(pp->qsl[ra + 1] - q0, 0) : 0;
      const int sl = pp->seq_lens[ra];
      const int cnt = (nn + QB - 1) / QB;
      const int key = v ? sl : -1;
      int rank = 0;
      for (int j = 0; j < 64; ++j) {
        const int kj = __builtin_amdgcn_readlane(key, j);
        rank += (kj > key) | ((kj == key) & (j < lane));
      }
      int pre = 0, tot = 0;
      for (int j = 0; j < 64; ++j) {
        const int rj = __builtin_amdgcn_readlane(rank, j), cj = __builtin_amdgcn_readlane(cnt, j);
        pre += rj < rank ? cj : 0;
        tot += cj;
      }
      cur_lane[wave][0][lane] = q0;
      cur_lane[wave][1][lane] = nn;
      cur_lane[wave][2][lane] = sl;
      cur_lane[wave][3][lane] = cnt;
      cur_lane[wave][4][lane] = pre;
      ch_total = tot;
    }
    if (!found) return false;
    cur_sc[wave][0] = ch;
    cur_sc[wave][1] = ch_base;
    cur_sc[wave][2] = ch_total;
    const int rel = tt - ch_base;
    const int c_cnt = cur_lane[wave][3][lane], c_pre = cur_lane[wave][4][lane];
    const bool mine = c_cnt > 0 && rel >= c_pre && rel < c_pre + c_cnt;
    const int sel = (int)__builtin_ctzll(__ballot(mine));
    it.r = pp->req_begin + ch * 64 + sel;
    it.bz = rel - wave_uniform(cur_lane[wave][4][sel]);   // tile, counted from the request's end
    it.q_first = wave_uniform(cur_lane[wave][0][sel]);
    it.n = wave_uniform(cur_lane[wave][1][sel]);
    it.s_all = wave_uniform(cur_lane[wave][2][sel]);
    return true;
  };

  for (;;) {
    const CParams* pp = params();
    const int hpw = pp->heads_per_wg;
    const int QB = (32 * kPPWaves) / hpw;   // queries per item
    const int nhg = pp->num_q_heads / hpw;  // head groups
    const int k = wave_uniform(cur_sc[wave][3]);
    ItemRec it;
    if (!lookup(k, pp, QB, nhg, it)) break;
    cur_sc[wave][3] = k + 1;
    const int hg = it.hg, r = it.r, bz = it.bz, q_first = it.q_first, n = it.n, s_all = it.s_all;

    const int q_hi = n - bz * QB;      // the item covers queries [q_hi - QB, q_hi)
    const int c = s_all - n;
    int s_eff = min(s_all, pp->max_seq_len);
    s_eff = min(s_eff, pp->max_blocks_per_req * kBlock);
    const int k_end = min(c + q_hi, s_eff);
    const int ntiles = (k_end + kTileK - 1) / kTileK;
    const int window_left = pp->window_left;
    const int kt0 = MASK ? max(0, c + max(q_hi - QB, 0) - window_left) / kTileK : 0;
    const int G = pp->group;
    const int nb32 = (int)min(pp->num_blocks, (int64_t)0x7FFFFFFF);
    const int64_t blk_stride = (int64_t)pp->num_kv_heads * D * KVB * kBlock;

    const int qh = hg * hpw + (wave % hpw);
    const int kvh = qh / G;
    const int wq0 = q_hi - QB + (wave / hpw) * 32;   // first query of the wave (may be < 0)
    const int qi = wq0 + l32;                        // this lane's query
    const bool q_ok = qi >= 0;
    const int qpos = c + qi;
    const int wave_first_pos = c + wq0;
    const int wave_last_pos = c + wq0 + 31;

    const int32_t* bt_row = pp->block_tables + (int64_t)r * pp->max_blocks_per_req;
    const int nblk = (s_eff + kBlock - 1) / kBlock;
    const unsigned char* kbase = static_cast<const unsigned char*>(pp->key_cache) + (int64_t)kvh * D * KVB;
    const unsigned char* vbase = static_cast<const unsigned char*>(pp->value_cache) + (int64_t)kvh * D * KVB;

    // this wave's table entry for tile t (index clamped into the sequence), and
    // the id its copies use (absent -> block 0: masked keys, zeroed V rows)
    auto raw_id = [&](int t) __attribute__((always_inline)) {
      return load_uniform(bt_row, min(4 * t + cb, nblk - 1));
    };
    auto copy_id = [&](int raw, int t) __attribute__((always_inline)) {
      return ((4 * t + cb < nblk) & (raw >= 0) & (raw < nb32)) ? raw : 0;
    };
    // The LDS destination is formed where the copy is issued: the add is
    // hidden from loop-invariant hoisting, which would otherwise hold one
    // scalar register per (stage, instruction) through the tile loop and push
    // the loop over the scalar register budget (the compiler then stops
    // running LDS reads ahead of the MFMAs).
    auto copy_tile = [&](const unsigned char* base, const unsigned (&off)[IPW], int id,
                         unsigned lds0) __attribute__((always_inline)) {
      const unsigned char* src = base + (int64_t)id * blk_stride;
      unsigned wdst = (unsigned)(wave * IPW * LPI * 16);
      asm volatile("" : "+s"(wdst));
      if (copy_lane) {
#pragma unroll
        for (int i = 0; i < IPW; ++i)
          lds_dma16<false, false>(src, off[i], lds0 + wdst + (unsigned)(i * LPI * 16));
      }
    };

    // The item's first copies (K tiles t0 .. t0+2, V tiles t0 .. t0+1) go out
    // before its Q rows and table check are loaded, so the three transfers
    // overlap; the loads' wait below covers the copies as well.
    int raw_n = 0, id_v = 0;
    if (ntiles > kt0) {
      const bool pre = wave_uniform(pre_ids[wave][0]) == k;
      const int raw0 = pre ? wave_uniform(pre_ids[wave][1]) : raw_id(kt0);
      const int raw1 = pre ? wave_uniform(pre_ids[wave][2]) : raw_id(kt0 + 1);
      const int raw2 = pre ? wave_uniform(pre_ids[wave][3]) : raw_id(kt0 + 2);
      raw_n = pre ? wave_uniform(pre_ids[wave][4]) : raw_id(kt0 + 3);   // tile j+3's entry, checked in V(j)
      const int id0 = copy_id(raw0, kt0);
      const int id1 = copy_id(raw1, kt0 + 1);
      const int id2 = copy_id(raw2, kt0 + 2);
      id_v = id2;                   // tile j+2's id (its V copy in V(j))
      copy_tile(kbase, koff, id0, kr0);
      copy_tile(vbase, voff, id0, vr0);
      if (kt0 + 1 < ntiles) {
        copy_tile(kbase, koff, id1, kr0 + kTileBytes);
        copy_tile(vbase, voff, id1, vr0 + kTileBytes);
      }
      if (kt0 + 2 < ntiles) copy_tile(kbase, koff, id2, kr0 + 2 * kTileBytes);
    }

    // the next item's first four block-table entries for this wave (scalar
    // loads, in flight with the Q loads below; stored once they are retired)
    int nraw[4] = {0, 0, 0, 0};
    bool nxt_ok = false;
    {
      ItemRec nx;
      if (lookup(k + 1, pp, QB, nhg, nx)) {
        const int q_hi2 = nx.n - nx.bz * QB;
        const int c2_ = nx.s_all - nx.n;
        const int s_eff2 = min(min(nx.s_all, pp->max_seq_len), pp->max_blocks_per_req * kBlock);
        const int nblk2 = (s_eff2 + kBlock - 1) / kBlock;
        const int kt02 = MASK ? max(0, c2_ + max(q_hi2 - QB, 0) - pp->window_left) / kTileK : 0;
        if (nblk2 > 0) {
          const int32_t* bt2 = pp->block_tables + (int64_t)nx.r * pp->max_blocks_per_req;
#pragma unroll
          for (int u = 0; u < 4; ++u) nraw[u] = load_uniform(bt2, min(4 * (kt02 + u) + cb, nblk2 - 1));
          nxt_ok = true;
        }
      }
    }

    // Q as the B operand of S^T = K . Q^T: B[k = 8*half + e][col = l32] = Q[qi][16 s + 8 half + e]
    vec8 qop[QS];
    {
      const CT* qrow = static_cast<const CT*>(pp->q) + (int64_t)(q_first + (q_ok ? qi : 0)) * pp->q_row_stride +
                       (int64_t)qh * D;
#pragma unroll
      for (int s = 0; s < QS; ++s)
        qop[s] = q_ok ? __builtin_bit_cast(vec8, ld16(qrow + 16 * s + 8 * half))
                      : __builtin_bit_cast(vec8, u32x4{0u, 0u, 0u, 0u});
    }
    // One pass over the table entries the item's tiles use: when all of them
    // are pool ids (the normal case) every block of every tile is present,
    // and keys past the sequence are handled by the length tests alone.
    bool my_ok = true;
    for (int b = 4 * kt0 + (int)threadIdx.x; b < nblk; b += kPPThreads) {
      const int id = bt_row[b];
      my_ok &= (id >= 0) & (id < nb32);
    }
    // consume Q here, so the compiler retires these loads (and with them the
    // copies above) before the loop: a wait it placed inside the loop would
    // also wait for every copy in flight
#pragma unroll
    for (int s = 0; s < QS; ++s) asm volatile("" : : "v"(__builtin_bit_cast(u32x4, qop[s])));
    if (nxt_ok) {
      pre_ids[wave][1] = nraw[0];
      pre_ids[wave][2] = nraw[1];
      pre_ids[wave][3] = nraw[2];
      pre_ids[wave][4] = nraw[3];
      pre_ids[wave][0] = k + 1;
    }
    const bool rowok = __syncthreads_and(my_ok);
    auto okmask = [&](int t) __attribute__((always_inline)) {
      return rowok ? 0xFu : tile_okmask(bt_row, nblk, nb32, t);
    };

    // after the copy of V tile t has landed: zero the rows of keys the tile
    // lacks (past the sequence, absent blocks), each lane exactly the positions
    // its own copies wrote
    auto fix_v = [&](int t, u32x4* Vs) __attribute__((always_inline)) {
      if (kTileK * t + kTileK <= s_eff && rowok) return;
      const unsigned ok = okmask(t);
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int pidx = (wave * IPW + i) * LPI + lane;
        const int key = pidx / L::CPR;
        if (kTileK * t + key >= s_eff || !((ok >> (key / kBlock)) & 1u)) Vs[pidx] = u32x4{0u, 0u, 0u, 0u};
      }
    };

    // 8-bit caches: after this wave's copies of tile t have landed, widen them
    // (16 bytes per lane) into the operand stage in the LdsTile layout; V rows
    // of keys the tile lacks become zeros (K rows need not: their scores are
    // masked by selects)
    auto widen = [&](const u32x4* src8, u32x4* dst, int t, bool is_v) __attribute__((always_inline)) {
      if (!copy_lane) return;
      const int pidx = wave * LPI + lane;
      const int key = pidx / CPR8, c8 = pidx % CPR8;
      const u32x4 w = src8[pidx];
      u32x4 lo{widen8x2<CT, I8>(w[0], false), widen8x2<CT, I8>(w[0], true),
               widen8x2<CT, I8>(w[1], false), widen8x2<CT, I8>(w[1], true)};
      u32x4 hi{widen8x2<CT, I8>(w[2], false), widen8x2<CT, I8>(w[2], true),
               widen8x2<CT, I8>(w[3], false), widen8x2<CT, I8>(w[3], true)};
      int sw = L::swk(key);
      if (is_v) {
        sw = L::swv(key);
        if (!(kTileK * t + kTileK <= s_eff && rowok)) {
          const unsigned ok = okmask(t);
          if (kTileK * t + key >= s_eff || !((ok >> (key / kBlock)) & 1u)) lo = hi = u32x4{0u, 0u, 0u, 0u};
        }
      }
      dst[key * L::CPR + ((2 * c8) ^ sw)] = lo;
      dst[key * L::CPR + ((2 * c8 + 1) ^ sw)] = hi;
    };

    // the same widening in two parts, for the MFMA phase: the 8-bit row is read
    // before the MFMAs, converted among them and stored after them
    auto widen_store = [&](const u32x4 w, u32x4* dst, bool is_v, bool vz) __attribute__((always_inline)) {
      const int pidx = wave * LPI + lane;
      const int key = pidx / CPR8, c8 = pidx % CPR8;
      u32x4 lo{widen8x2<CT, I8>(w[0], false), widen8x2<CT, I8>(w[0], true),
               widen8x2<CT, I8>(w[1], false), widen8x2<CT, I8>(w[1], true)};
      u32x4 hi{widen8x2<CT, I8>(w[2], false), widen8x2<CT, I8>(w[2], true),
               widen8x2<CT, I8>(w[3], false), widen8x2<CT, I8>(w[3], true)};
      const int sw = is_v ? L::swv(key) : L::swk(key);
      if (is_v) {
        const u32x4 z{0u, 0u, 0u, 0u};
        lo = vz ? z : lo;
        hi = vz ? z : hi;
      }
      if (copy_lane) {
        dst[key * L::CPR + ((2 * c8) ^ sw)] = lo;
        dst[key * L::CPR + ((2 * c8 + 1) ^ sw)] = hi;
      }
    };

    // per-head K scales exist for 8-bit caches only (the 16-bit kernels never read them)
    const float scale_log2 = (KVB == 1 && pp->k_scales != nullptr)
                                 ? pp->scale_log2 * head_scale(pp->k_scales, kvh)
                                 : pp->scale_log2;
    const float c2 = MASK ? 1.f : scale_log2;
    const float slope2 = (MASK && pp->alibi != nullptr)
                             ? __builtin_bit_cast(float, load_uniform(reinterpret_cast<const int32_t*>(pp->alibi), qh)) * kLog2e
                             : 0.f;
    f32x16 acc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[t] = f32x16{};
    float m_used = -INFINITY, l_run = 0.f;
    f32x16 sc[2];
    u32x4 pk[4];    // P of the previous tile, two 16-bit values per dword: pk[2u + v] feeds PV step (u, v)
#pragma unroll
    for (int i = 0; i < 4; ++i) pk[i] = u32x4{0u, 0u, 0u, 0u};
    auto active = [&](int t) __attribute__((always_inline)) {
      const int k0 = t * kTileK;
      return k0 <= wave_last_pos && (!MASK || k0 + kTileK - 1 >= wave_first_pos - window_left);
    };

    // M phase: S_j (QK) and O += V_{j-1} P_{j-1} (PV), the two MFMA chains interleaved
    auto mphase = [&](const u32x4* Kt, const u32x4* Vt) __attribute__((always_inline)) {
      sc[0] = f32x16{};
      sc[1] = f32x16{};
#pragma unroll
      for (int s = 0; s < QS; ++s) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const vec8 kop = __builtin_bit_cast(vec8, Kt[(32 * u + l32) * L::CPR + ((2 * s + half) ^ kswz)]);
          sc[u] = M::mma32(kop, qop[s], sc[u]);
        }
#pragma unroll
        for (int e = 0; e < PPS; ++e) {
          const int pv = s * PPS + e;
          const int uv = pv / DT, t = pv % DT;
          // keys of this step: 32u + 16v + 8r + 4h + a (h = lane/32), element e = 4r + a
          const int key_r0 = 32 * (uv >> 1) + 16 * (uv & 1) + 4 * half + ta;
          const int chunk = 4 * t + 2 * (g16 & 1) + (tb >> 1);
          const int byte_off = 8 * (tb & 1);
          const u32x2 lo = lds_read_tr16(Vt, key_r0 * L::CPR + (chunk ^ vswz), byte_off);
          const u32x2 hi = lds_read_tr16(Vt, (key_r0 + 8) * L::CPR + (chunk ^ vswz), byte_off);
          const vec8 vop = __builtin_bit_cast(vec8, u32x4{lo[0], lo[1], hi[0], hi[1]});
          acc[t] = M::mma32(vop, __builtin_bit_cast(vec8, pk[uv]), acc[t]);
        }
      }
      // issue order: LDS reads run ahead of the MFMAs that consume them
      constexpr int kReads = 2 * QS + 8 * DT;
      constexpr int kMfma = 2 * QS + 4 * DT;
      constexpr int kLead = 6;
      constexpr int W8V = 2 * 24;   // widening in the phase: 2 x (16 converts + 8 packs) per lane
      constexpr int kPer = (kReads - kLead + kMfma - 1) / kMfma;
      __builtin_amdgcn_sched_group_barrier(0x100, kLead, 0);
#pragma unroll
      for (int i = 0; i < kMfma; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, kPer, 0);
        if constexpr (kWidenInM) {
          if (i >= 2 && i < 2 + W8V / 2) __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
      }
    };

    // V phase softmax of tile j: scores in sc -> probabilities in pk, row sums in l_run
    auto softmax = [&](int j) __attribute__((always_inline)) {
      const int k0 = j * kTileK;
      if (k0 + kTileK - 1 > wave_first_pos || k0 + kTileK > s_eff) {
        // element g of subtile u is key k0 + 4 half + (32u + 8(g/4) + g%4):
        // masked past the query's position and past the sequence
        const int lim = min(qpos, s_eff - 1) - (k0 + 4 * half);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int g = 0; g < 16; ++g)
            sc[u][g] = (32 * u + 8 * (g / 4) + (g % 4) > lim) ? -INFINITY : sc[u][g];
      }
      if (!rowok) {
        const unsigned okj = okmask(j);
        // absent blocks: block b of the tile holds elements 8(b%2) .. 8(b%2)+7 of subtile b/2
#pragma unroll
        for (int b = 0; b < 4; ++b)
          if (!((okj >> b) & 1u)) {
#pragma unroll
            for (int g = 0; g < 8; ++g) sc[b >> 1][8 * (b & 1) + g] = -INFINITY;
          }
      }
      if constexpr (MASK)
        window_alibi(sc, k0, half, qpos, window_left, scale_log2, slope2, k0 < wave_last_pos - window_left);
      // row max of the lane's 32 scores as a tree of three-input maxima (16
      // instructions, short dependency chains)
      float m10[11];
#pragma unroll
      for (int k = 0; k < 10; ++k)
        m10[k] = max3f(sc[(3 * k) >> 4][(3 * k) & 15], sc[(3 * k + 1) >> 4][(3 * k + 1) & 15],
                       sc[(3 * k + 2) >> 4][(3 * k + 2) & 15]);
      m10[10] = fmaxf(sc[1][14], sc[1][15]);
      const float m3a = max3f(m10[0], m10[1], m10[2]), m3b = max3f(m10[3], m10[4], m10[5]);
      const float m3c = max3f(m10[6], m10[7], m10[8]);
      float mx = max3f(max3f(m3a, m3b, m3c), m10[9], m10[10]);
      mx = pair32_max_swap(mx);
      // lazy rescale: move the reference max only when it grew by more than 2^8
      const bool grow = (m_used == -INFINITY) ? (mx > -INFINITY) : ((mx - m_used) * c2 > kRescaleLog2);
      if (__ballot(grow)) {
        const float m_new = grow ? mx : m_used;
        const float alpha = (m_used == -INFINITY) ? 0.f : fast_exp2((m_used - m_new) * c2);
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t) acc[t] *= alpha;
        m_used = m_new;
      }
      const float mref = (m_used == -INFINITY) ? 0.f : m_used * c2;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int g = 0; g < 16; ++g) sc[u][g] = fast_exp2(__builtin_fmaf(sc[u][g], c2, -mref));
      // pack to the MFMA operand; row sums of the rounded probabilities the PV
      // product uses, in four independent chains
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          const u32x4 w{pack2<CT>(sc[u][8 * v + 0], sc[u][8 * v + 1]), pack2<CT>(sc[u][8 * v + 2], sc[u][8 * v + 3]),
                        pack2<CT>(sc[u][8 * v + 4], sc[u][8 * v + 5]), pack2<CT>(sc[u][8 * v + 6], sc[u][8 * v + 7])};
          pk[2 * u + v] = w;
#pragma unroll
          for (int k = 0; k < 4; ++k) ls[k] = M::sum2(w[k], ls[k]);
        }
      l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    };

    if (ntiles > kt0) {
      // the first M phase multiplies zero probabilities with V operand stage
      // NO-1: clear it, so stale LDS contents cannot turn 0 * V into NaN
      for (int i = threadIdx.x; i < L::kPos; i += kPPThreads)
        Vr[(NO - 1) * L::kPos + i] = u32x4{0u, 0u, 0u, 0u};
      wait_vmcnt<0>();
      if constexpr (KVB == 2) {
        fix_v(kt0, Vr);
        if (kt0 + 1 < ntiles) fix_v(kt0 + 1, Vr + L::kPos);
      } else {
        widen(K8, Kr, kt0, false);   // K(kt0); K(kt0 + 1) and V(kt0) in M(kt0)
      }
      barrier_nowait<true>();

      auto step = [&](auto st_c, int j) __attribute__((always_inline)) {
        constexpr int ST = decltype(st_c)::value;
        const u32x4* Kt = Kr + (ST % NO) * L::kPos;
        const u32x4* Vt = Vr + ((ST + NO - 1) % NO) * L::kPos;
        // ---- M(j) ----
        // one straight MFMA path (branches around MFMAs cost accumulator
        // copies): a tile the wave does not need still runs, with zero
        // probabilities (P of the first tile, of tiles past the wave's queries
        // or before its window); its scores are discarded
        if constexpr (!kWidenInM) {
          mphase(Kt, Vt);
          // retire the copies of V(j-2) (those of V(j-1) may stay in flight)
          if (j - 1 >= kt0 && j + 2 < ntiles) wait_vmcnt<2 * IPW>();
          else if (j - 1 >= kt0 && j + 1 < ntiles) wait_vmcnt<IPW>();
          else wait_vmcnt<0>();
          if constexpr (KVB == 2) {
            if (j >= kt0 + 2 && j < ntiles) fix_v(j, Vr + ST * L::kPos);
          } else {
            // operand stages of K(j+1) and V(j): their previous tiles, K(j-1) and
            // V(j-2), were last read in M(j-1), which every wave has finished
            if (j + 1 < ntiles) widen(K8 + ((ST + 1) % NS) * kPos8, Kr + ((ST + 1) % NO) * L::kPos, j + 1, false);
            if (j < ntiles) widen(V8 + ST * kPos8, Vr + (ST % NO) * L::kPos, j, true);
          }
        } else {
          // retire the copies of V(j-2) first (those of V(j-1) may stay in
          // flight): this wave's 8-bit rows of K(j+1) and V(j) are read before
          // the MFMAs and widened among them into the operand stages of K(j+1)
          // and V(j), whose previous tiles, K(j-1) and V(j-2), were last read
          // in M(j-1), which every wave has finished.  Past the last tile the
          // rows are stale and their widened copies are never read.
          if (j - 1 >= kt0 && j + 2 < ntiles) wait_vmcnt<2 * IPW>();
          else if (j - 1 >= kt0 && j + 1 < ntiles) wait_vmcnt<IPW>();
          else wait_vmcnt<0>();
          const int pidx = wave * LPI + (copy_lane ? lane : 0);
          const u32x4 wk = K8[((ST + 1) % NS) * kPos8 + pidx];
          const u32x4 wv = V8[ST * kPos8 + pidx];
          bool vz = false;
          if (!(kTileK * j + kTileK <= s_eff && rowok)) {
            const int key = pidx / CPR8;
            const unsigned ok = okmask(j);
            vz = kTileK * j + key >= s_eff || !((ok >> (key / kBlock)) & 1u);
          }
          mphase(Kt, Vt);
          widen_store(wk, Kr + ((ST + 1) % NO) * L::kPos, false, false);
          widen_store(wv, Vr + (ST % NO) * L::kPos, true, vz);
        }
        barrier_nowait<true>();
        // ---- V(j) ----
        const int id_k = copy_id(raw_n, j + 3);
        raw_n = raw_id(j + 4);
        if (j + 3 < ntiles) copy_tile(kbase, koff, id_k, kr0 + (unsigned)((ST + 3) % NS) * kTileBytes);
        if (j + 2 < ntiles) copy_tile(vbase, voff, id_v, vr0 + (unsigned)((ST + 2) % NS) * kTileBytes);
        if (j < ntiles && active(j)) {
          softmax(j);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) pk[i] = u32x4{0u, 0u, 0u, 0u};
        }
        id_v = id_k;
        barrier_nowait<false>();
      };

      if (grp == 1) barrier_nowait<false>();
      for (int j = kt0; j <= ntiles; j += NS) {
        step(std::integral_constant<int, 0>{}, j);
        if (j + 1 <= ntiles) step(std::integral_constant<int, 1>{}, j + 1);
        if (j + 2 <= ntiles) step(std::integral_constant<int, 2>{}, j + 2);
        if (j + 3 <= ntiles) step(std::integral_constant<int, 3>{}, j + 3);
      }
      if (grp == 0) barrier_nowait<false>();
    }

    // ---- normalise and store: lane holds O[qi][32 t + 8 j + 4 half + i] ----
    const float lt = pair32_sum_swap(l_run);
    if (q_ok) {
      const CParams* pe = params();
      // (the K/V head from the re-read parameters: no value of the item's
      // start stays live through the tile loop for this)
      const float vsc = (KVB == 1 && pe->v_scales != nullptr) ? head_scale(pe->v_scales, qh / pe->group)
                                                              : pe->v_scale;
      const float inv = (lt > 0.f) ? vsc / lt : 0.f;
      unsigned short* orow = static_cast<unsigned short*>(pe->out) +
                             (int64_t)(q_first + qi) * pe->out_row_stride + (int64_t)qh * D;
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
  }
}

// Compute units of the current device (256 on MI355X when the query fails).
int compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  return cus;
}

int heads_per_wg(int G) {
  if (G % 4 == 0) return 4;
  if (G % 2 == 0) return 2;
  return 1;
}

template <int D, typename CT, int KVB, bool I8 = false>
hipError_t launch_typed(const AttnParams& p, hipStream_t stream) {
  const int hpw = heads_per_wg(p.group);
  const int QB = 32 * kPPWaves / hpw;
  const int qtiles = (p.max_query_len + QB - 1) / QB;
  if (qtiles == 0) return hipSuccess;
  // one workgroup per compute unit (a multiple of the head-group count when
  // there are no more head groups than units), no more than there can be items
  const int nhg = p.num_q_heads / hpw;
  const int cus = compute_units();
  int wgs = nhg <= cus ? cus / nhg * nhg : cus;
  const int64_t max_items = (int64_t)nhg * p.num_reqs * qtiles;
  if (max_items < wgs) wgs = (int)max_items;
  dim3 grid((unsigned)wgs);
  AttnParams pk = p;
  pk.heads_per_wg = hpw;
  if (p.masked) {
    hipLaunchKernelGGL((prefill_pp_kernel<D, CT, KVB, I8, true>), grid, dim3(kPPThreads), 0, stream, pk);
  } else {
    hipLaunchKernelGGL((prefill_pp_kernel<D, CT, KVB, I8, false>), grid, dim3(kPPThreads), 0, stream, pk);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_dim(const AttnParams& p, int act, int cache, hipStream_t stream) {
  if (act == kF16 && cache == kF16) return launch_typed<D, _Float16, 2>(p, stream);
  if (act == kBF16 && cache == kBF16) return launch_typed<D, __bf16, 2>(p, stream);
  if (act == kF16 && cache == kFP8) return launch_typed<D, _Float16, 1>(p, stream);
  if (act == kBF16 && cache == kFP8) return launch_typed<D, __bf16, 1>(p, stream);
  if (act == kF16 && cache == kINT8) return launch_typed<D, _Float16, 1, true>(p, stream);
  if (act == kBF16 && cache == kINT8) return launch_typed<D, __bf16, 1, true>(p, stream);
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
