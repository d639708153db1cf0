// pa_copy_blocks kernel: whole-block copies between two block pools.
//
// What is moved ("vLLM 推理全流程深度解析": the scheduler output's
// blocks_to_swap_in, blocks_to_swap_out and blocks_to_copy pair lists;
// swapping evicts a sequence's KV blocks to host memory when GPU memory runs
// short, and sequences that share a block through the global pool get a
// private copy before one of them changes it): for each pair (src, dst),
// block dst of the destination K and V caches receives the bytes of block src
// of the source K and V caches.  A block is block_size * num_kv_heads *
// head_dim cache elements, contiguous in the [num_blocks, block_size, Hkv, D]
// layout, so a pair is two contiguous copies whatever the cache dtype.
//
// One launch serves the three lists: the pools may be device memory or pinned
// host memory mapped into the device's address space (swap out: device ->
// host, swap in: host -> device, copy: one device pool), and the kernel moves
// the bytes with its own loads and stores -- no copy call per block.
//
// Work decomposition: workgroup (pair, K or V, slice of the block); each
// thread moves kChunks 16-byte chunks, issuing all of its loads before its
// stores so that kChunks requests per lane are in flight (a swap crosses the
// host link, whose latency is far above HBM's).  A pair whose source or
// destination is outside its pool is skipped.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int kThreads = 256;
constexpr int kChunks = 4;
constexpr int64_t kSliceBytes = (int64_t)kThreads * kChunks * 16;

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(CopyBlocksParams p) {
  const int64_t pair = blockIdx.x >> 1;
  const bool is_v = (blockIdx.x & 1) != 0;
  const int64_t s = p.pairs[2 * pair], d = p.pairs[2 * pair + 1];
  if (s < 0 || s >= p.src_blocks || d < 0 || d >= p.dst_blocks) return;
  const unsigned char* src = static_cast<const unsigned char*>(is_v ? p.src_value : p.src_key) +
                             s * p.block_bytes;
  unsigned char* dst = static_cast<unsigned char*>(is_v ? p.dst_value : p.dst_key) +
                       d * p.block_bytes;
  const int64_t first = (int64_t)blockIdx.y * kSliceBytes + 16 * (int64_t)threadIdx.x;
  u32x4 v[kChunks];
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    const int64_t off = first + (int64_t)k * kThreads * 16;
    if (off < p.block_bytes) v[k] = ld16(src + off);
  }
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    const int64_t off = first + (int64_t)k * kThreads * 16;
    if (off < p.block_bytes) st16(dst + off, v[k]);
  }
}

}  // namespace

int64_t copy_blocks_slices(int64_t block_bytes) { return (block_bytes + kSliceBytes - 1) / kSliceBytes; }

hipError_t launch_copy_blocks(const CopyBlocksParams& p, hipStream_t stream) {
  if (p.num_pairs == 0) return hipSuccess;
  const dim3 grid((unsigned)(2 * p.num_pairs), (unsigned)copy_blocks_slices(p.block_bytes));
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
