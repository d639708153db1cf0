// pa_metadata_build kernel: query_start_loc, seq_lens, positions, slot_mapping
// of one step ("Tour: One forward pass", stops 3 and 4).
//
// One workgroup of 1024 threads.  Pass 1 scans query_lens in 1024-entry
// chunks (wave prefix sums with shuffles, then the 16 wave totals) and writes
// query_start_loc and seq_lens.  Pass 2 gives every token row its request by a
// binary search over query_start_loc and writes its position and slot.  The
// metadata is built once per step and read by every layer, so one small launch
// is the whole cost; the work is integer only and bit-exact.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kThreads = 1024;

__global__ __launch_bounds__(kThreads) void metadata_kernel(MetadataParams p) {
  __shared__ int wave_sums[kThreads / 64];
  __shared__ int carry_s;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (tid == 0) carry_s = 0;
  if (tid == 0) p.qsl[0] = 0;
  __syncthreads();

  // ---- pass 1: inclusive scan of query_lens -> query_start_loc[1..R] -------
  for (int base = 0; base < p.num_reqs; base += kThreads) {
    const int r = base + tid;
    int n = 0;
    if (r < p.num_reqs) {
      n = p.query_lens[r];
      p.seq_lens[r] = p.num_computed[r] + n;
    }
    int x = n;  // inclusive prefix within the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) wave_sums[wave] = x;
    __syncthreads();
    int wave_prefix = 0;
    for (int w = 0; w < wave; ++w) wave_prefix += wave_sums[w];
    const int carry = carry_s;
    if (r < p.num_reqs) p.qsl[r + 1] = carry + wave_prefix + x;
    __syncthreads();
    if (tid == kThreads - 1) carry_s = carry + wave_prefix + x;
    __syncthreads();
  }
  const int total = carry_s;  // T, the number of real token rows
  for (int i = p.num_reqs + 1 + tid; i < p.qsl_len; i += kThreads) p.qsl[i] = total;
  __syncthreads();  // query_start_loc is complete and visible to the workgroup

  // ---- pass 2: per token row -----------------------------------------------
  for (int t = tid; t < p.num_tokens_padded; t += kThreads) {
    if (t >= total) {
      p.slot_mapping[t] = -1;  // PAD_SLOT_ID; positions of padding rows are left alone
      continue;
    }
    // request r: the largest r with qsl[r] <= t (empty requests share a start)
    int lo = 0, hi = p.num_reqs - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (p.qsl[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int r = lo;
    const int64_t pos = (int64_t)p.num_computed[r] + (t - p.qsl[r]);
    p.positions[t] = pos;
    const int64_t block_index = pos / p.block_size;
    const int64_t offset = pos % p.block_size;
    int64_t slot = -1;
    if (block_index < p.max_blocks_per_req) {
      const int64_t block = p.block_tables[(int64_t)r * p.max_blocks_per_req + block_index];
      slot = block * p.block_size + offset;
    }
    p.slot_mapping[t] = slot;
  }
}

}  // namespace

hipError_t launch_metadata(const MetadataParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(metadata_kernel, dim3(1), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
