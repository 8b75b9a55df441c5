// reshape_and_cache for gfx950: scatter new tokens' K and V into their paged
// cache slots ("vLLM" note, section "PagedAttention": slot / block_size is the
// page, slot % block_size the row inside it), copying the bits or quantising
// to OCP E4M3 ("vLLM 前世今生", §5.2).
//
// One thread moves one 16-byte chunk of a (token, kv head) source row for both
// K and V; consecutive threads take consecutive chunks, so the reads of the
// source and the writes of each destination row are coalesced.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

// x / scale for scale > 0, computed as |x| / scale (one correctly rounded
// float32 division) with x's sign bit put back, so that a NaN keeps its sign.
template <int SRC, int CACHE>
__global__ __launch_bounds__(kThreads) void reshape_kernel(ReshapeArgs a) {
  constexpr int kSrcBytes = KindBytes<SRC>::value;
  constexpr int E = 16 / kSrcBytes;  // source elements per chunk
  // The launch holds fewer than 2^31 source chunks, so the index math runs in 32 bits.
  const uint32_t chunks_per_row = (uint32_t)(a.head_size / E);
  const uint32_t chunks_per_tok = (uint32_t)a.num_kv_heads * chunks_per_row;
  const uint32_t idx = blockIdx.x * kThreads + threadIdx.x;
  if ((int64_t)idx >= a.num_tokens * (int64_t)chunks_per_tok) return;
  const uint32_t t = idx / chunks_per_tok;
  const int rem = (int)(idx - t * chunks_per_tok);
  // The source chunk is in bounds whatever the slot: its loads go out together
  // with the slot's, so the kernel waits for memory once, not twice.
  const int64_t src_elem = (int64_t)idx * E;  // == t*Hkv*D + head*D + chunk*E
  const uint4 kv = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.key) + src_elem * kSrcBytes);
  const uint4 vv = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.value) + src_elem * kSrcBytes);
  const int64_t slot = a.slot_is_int64 ? static_cast<const int64_t*>(a.slots)[t]
                                       : (int64_t) static_cast<const int32_t*>(a.slots)[t];
  if (slot < 0 || slot >= a.num_blocks * 16) return;  // padding, or outside the pool
  const int head = rem / (int)chunks_per_row;
  const int chunk = rem - head * (int)chunks_per_row;
  const int64_t blk = slot >> 4;  // block_size is 16
  const int row = (int)(slot & 15);
  const int64_t dst_elem = ((blk * a.num_kv_heads + head) * 16 + row) * a.head_size + (int64_t)chunk * E;

  if constexpr (CACHE == SRC) {
    *reinterpret_cast<uint4*>(static_cast<char*>(a.k_cache) + dst_elem * kSrcBytes) = kv;
    *reinterpret_cast<uint4*>(static_cast<char*>(a.v_cache) + dst_elem * kSrcBytes) = vv;
  } else if constexpr (SRC == kF32) {
    *reinterpret_cast<uint32_t*>(static_cast<char*>(a.k_cache) + dst_elem) = e4m3_chunk32(kv, a.k_scale);
    *reinterpret_cast<uint32_t*>(static_cast<char*>(a.v_cache) + dst_elem) = e4m3_chunk32(vv, a.v_scale);
  } else {
    *reinterpret_cast<uint2*>(static_cast<char*>(a.k_cache) + dst_elem) = e4m3_chunk16<SRC>(kv, a.k_scale);
    *reinterpret_cast<uint2*>(static_cast<char*>(a.v_cache) + dst_elem) = e4m3_chunk16<SRC>(vv, a.v_scale);
  }
}

template <int SRC, int CACHE>
hipError_t launch(const ReshapeArgs& a, hipStream_t stream) {
  constexpr int E = 16 / KindBytes<SRC>::value;
  const int64_t total = a.num_tokens * a.num_kv_heads * (a.head_size / E);
  const int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks == 0) return hipSuccess;
  if (blocks * kThreads > 0x7fffffffLL) return hipErrorInvalidConfiguration;  // 32-bit index math in the kernel
  reshape_kernel<SRC, CACHE><<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reshape(const ReshapeArgs& a, int src_kind, int cache_kind, hipStream_t stream) {
  switch (src_kind * 4 + cache_kind) {
    case kF32 * 4 + kF32: return launch<kF32, kF32>(a, stream);
    case kF16 * 4 + kF16: return launch<kF16, kF16>(a, stream);
    case kBF16 * 4 + kBF16: return launch<kBF16, kBF16>(a, stream);
    case kF32 * 4 + kFP8: return launch<kF32, kFP8>(a, stream);
    case kF16 * 4 + kFP8: return launch<kF16, kFP8>(a, stream);
    case kBF16 * 4 + kFP8: return launch<kBF16, kFP8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
