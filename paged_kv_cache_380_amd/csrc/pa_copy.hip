// copy_blocks for gfx950: the device half of copy-on-write. Before a sequence
// writes into a physical block it shares with other sequences, the block is
// copied to a block of its own ("vLLM 前世今生" §3.2). One (block, K and V)
// copy is Hkv * 16 * head_size elements of contiguous memory per cache, moved
// with 16-byte loads and stores: each workgroup copies one 4 KiB chunk of one
// pair in each cache, consecutive threads taking consecutive 16-byte pieces.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = kThreads * 16;  // bytes per workgroup and cache

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(char* k_cache, char* v_cache, const int32_t* src,
                                                               const int32_t* dst, int64_t block_bytes,
                                                               int64_t num_blocks) {
  const int pair = blockIdx.y;
  const int64_t s = src[pair];
  const int64_t d = dst[pair];
  if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks || s == d) return;  // outside the pool: nothing moves
  const int64_t off = (int64_t)blockIdx.x * kChunk + threadIdx.x * 16;
  if (off >= block_bytes) return;
  const uint4 kv = *reinterpret_cast<const uint4*>(k_cache + s * block_bytes + off);
  const uint4 vv = *reinterpret_cast<const uint4*>(v_cache + s * block_bytes + off);
  *reinterpret_cast<uint4*>(k_cache + d * block_bytes + off) = kv;
  *reinterpret_cast<uint4*>(v_cache + d * block_bytes + off) = vv;
}

}  // namespace

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst, int num_pairs,
                              int64_t block_bytes, int64_t num_blocks, hipStream_t stream) {
  const int64_t chunks = (block_bytes + kChunk - 1) / kChunk;
  if (num_pairs > 65535 || chunks > 0x7fffffff) return hipErrorInvalidConfiguration;
  copy_blocks_kernel<<<dim3((unsigned)chunks, (unsigned)num_pairs), dim3(kThreads), 0, stream>>>(
      static_cast<char*>(k_cache), static_cast<char*>(v_cache), src, dst, block_bytes, num_blocks);
  return hipGetLastError();
}

}  // namespace pa
