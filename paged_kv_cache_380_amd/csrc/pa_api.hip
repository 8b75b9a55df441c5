// C ABI of libpa.so (declared and documented in include/pa.h): argument
// validation on the host, partition and workspace sizing, kernel dispatch.
// Nothing here reads device memory, allocates or synchronises.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "pa.h"
#include "pa_error.h"
#include "pa_internal.h"

namespace {

using pa::fail;
using pa::ok;

bool activation_kind(int k) { return k == PA_DTYPE_F32 || k == PA_DTYPE_F16 || k == PA_DTYPE_BF16; }

// Workgroups wanted before a context is split: one resident round on 256
// compute units at two workgroups each. Splitting further was measured to
// lose more to per-workgroup start-up, partial-result traffic and the merge
// than it gains in balance; a round of 512 long-running workgroups keeps
// every unit streaming until the end.
constexpr int64_t kTargetWorkgroups = 512;

// Groups of 32 and more query heads per KV head (a multiple of 32) decode on
// the prefill kernel with 16-bit queries: one workgroup per (sequence, KV head,
// 16 * waves heads, partition), every K/V tile loaded once into LDS for all
// its heads. Waves per workgroup: 8, 4 or 2 (the most that divides G / 16).
bool wide_group(int group) { return group >= 32 && group % 32 == 0; }
int wide_waves(int group) { return (group / 16) % 8 == 0 ? 8 : (group / 16) % 4 == 0 ? 4 : 2; }
// Workgroup shape of the wide decode: 128 heads go to 4 waves of two 16-head
// tiles each rather than 8 waves of one (each tile read from LDS once per 32
// heads; measured 0.261 against 0.267 ms on 64 x 32768 tokens at G = 128).
void wide_shape(int group, int& waves, int& wave_tiles) {
  waves = wide_waves(group);
  wave_tiles = 1;
  if (waves == 8) {
    waves = 4;
    wave_tiles = 2;
  }
}

// Workgroups the wide decode aims at before it splits contexts: two per
// compute unit, whatever the workgroup's waves (measured on 64 sequences of
// 32768 tokens over one KV head: 8-wave workgroups at two per unit 0.274 ms
// against 0.306 ms at one; 4-wave workgroups at G = 64 0.197 ms against 0.240
// at one per unit and 0.214 at four; 2-wave workgroups at G = 32 0.182 ms
// against 0.185 at four per unit and 0.214 at eight: more partitions leave
// more partial results to write and merge).
int64_t wide_target_workgroups(int) { return 512; }

int choose_partition_blocks(int num_seqs, int num_heads, int num_kv_heads, int max_blocks) {
  const int group = num_heads / num_kv_heads;
  if (wide_group(group)) {
    int waves, wave_tiles;
    wide_shape(group, waves, wave_tiles);
    const int64_t tiles = (int64_t)num_seqs * num_kv_heads * (group / (16 * waves * wave_tiles));
    const int64_t target = wide_target_workgroups(waves);
    int64_t parts = 1;
    if (tiles > 0 && tiles < target) parts = (target + tiles - 1) / tiles;
    int64_t pb = (max_blocks + parts - 1) / parts;
    pb = (pb + 3) / 4 * 4;
    if (pb < 4) pb = 4;
    if (pb > pa::kMaxPartitionBlocks) pb = pa::kMaxPartitionBlocks;
    return (int)pb;
  }
  // Head tiles per KV head as the default kernel for 16-bit queries launches
  // them (the sizing functions see no dtype; any tile count works, this one
  // only steers how far contexts are split).
  const int tile = pa::mfma_group_tile(group) ? pa::mfma_group_tile(group) : pa::group_tile_for(group);
  const int64_t tiles = (int64_t)num_seqs * num_kv_heads * (group / tile);
  int64_t parts = 1;
  if (tiles > 0 && tiles < kTargetWorkgroups) parts = (kTargetWorkgroups + tiles - 1) / tiles;
  int64_t pb = (max_blocks + parts - 1) / parts;
  pb = (pb + 3) / 4 * 4;
  if (pb < 4) pb = 4;
  if (pb > pa::kMaxPartitionBlocks) pb = pa::kMaxPartitionBlocks;
  return (int)pb;
}

// Decode kernel family: PA_DECODE_PATH=valu or =mfma forces one (mfma only
// where it applies); unset or anything else picks automatically. Read on every
// call (a getenv costs far less than a launch), so a process can switch.
enum class Path { kAuto, kValu, kMfma };
Path requested_path() {
  const char* e = std::getenv("PA_DECODE_PATH");
  if (e && !std::strcmp(e, "valu")) return Path::kValu;
  if (e && !std::strcmp(e, "mfma")) return Path::kMfma;
  return Path::kAuto;
}

// The matrix-core kernel serves 16-bit queries whose group of query heads per
// KV head is a multiple of 4: there one K/V tile feeds a [group x head_size]
// product. Below that (and for float32 data) the vector-ALU kernels run.
bool use_mfma(int q_dtype, int group) {
  const bool applies = (q_dtype == PA_DTYPE_F16 || q_dtype == PA_DTYPE_BF16) && pa::mfma_group_tile(group) != 0;
  return applies && requested_path() != Path::kValu;
}

// PA_DECODE_LOADS=cached makes the MHA vector kernel read K/V with ordinary
// cached loads instead of nontemporal ones (read on every call; comparison
// runs only: the default streaming loads measured faster).
bool cached_loads_requested() {
  const char* e = std::getenv("PA_DECODE_LOADS");
  return e && !std::strcmp(e, "cached");
}

bool shapes_ok(int num_seqs, int num_heads, int num_kv_heads, int head_size, int max_blocks, int block_size) {
  return num_seqs >= 0 && num_seqs <= 65535 && num_heads >= 1 && num_kv_heads >= 1 &&
         num_heads % num_kv_heads == 0 && (head_size == 64 || head_size == 128) && max_blocks >= 1 &&
         block_size == 16;
}

struct Layout {
  int partition_blocks;
  int num_parts;
  size_t out_bytes;    // partition outputs, at offset 0
  size_t ml_offset;    // partition max/sum pairs
  size_t pref_offset;  // balanced schedule: per-sequence block prefix
  size_t total;
};

// Balanced schedule of the matrix-core kernel: the blocks of all sequences
// are cut into R equal ranges, one per wave, R a multiple of 4 (a workgroup
// takes four ranges). R aims at kBalancedWaves16 waves in all for 16-bit
// caches, one 4-wave workgroup per CU (more, shorter waves measured slower:
// each pays the start of its stream), and at twice that for FP8 caches, whose
// tiles carry half the bytes for more vector work (widening), so that a
// second wave per SIMD hides one wave's arithmetic behind the other's loads.
constexpr int kBalancedWaves16 = 1024;
constexpr int kBalancedWavesFp8 = 2048;

// Query heads per wave in the balanced schedule: the matrix-core tile. The
// schedule serves groups below 32 and those that are not a multiple of 32
// (multiples of 32 take the wide decode).
int balanced_tile(int group) { return wide_group(group) ? 0 : pa::mfma_group_tile(group); }

bool balanced_fits(int num_seqs, int max_blocks) {
  return num_seqs <= pa::kBalancedMaxSeqs && (int64_t)num_seqs * max_blocks <= 0x7fffffffLL;
}

int64_t balanced_ranges(int num_heads, int group_tile, bool fp8_cache) {
  const int64_t columns = num_heads / group_tile;
  // A 32-head tile holds more than 256 registers: one wave per SIMD whatever the cache.
  const int64_t waves = fp8_cache && group_tile <= 16 ? kBalancedWavesFp8 : kBalancedWaves16;
  const int64_t r = (waves + columns - 1) / columns;
  return (r + 3) / 4 * 4;
}

Layout balanced_layout(int num_seqs, int num_heads, int head_size, int64_t ranges) {
  Layout L{};
  const size_t rows = (size_t)num_heads * ((size_t)num_seqs + ranges);
  L.out_bytes = rows * head_size * sizeof(float);
  L.ml_offset = (L.out_bytes + 255) / 256 * 256;
  L.pref_offset = (L.ml_offset + rows * 2 * sizeof(float) + 255) / 256 * 256;
  L.total = L.pref_offset + ((size_t)num_seqs + 1) * sizeof(int);
  return L;
}

// Shared-prefix pass: after the balanced schedule's workspace (at offset
// base), [S] ints of shared block counts, then [H, S, P1, D] and
// [H, S, P1, 2] floats of per-part partial results, each 256-byte aligned.
struct PrefixLayout {
  size_t shared_offset, out_offset, ml_offset, total;
};

PrefixLayout prefix_layout(size_t base, int num_seqs, int num_heads, int head_size, int parts) {
  PrefixLayout P{};
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  P.shared_offset = up(base);
  P.out_offset = up(P.shared_offset + (size_t)num_seqs * sizeof(int));
  const size_t rows = (size_t)num_heads * num_seqs * parts;
  P.ml_offset = up(P.out_offset + rows * head_size * sizeof(float));
  P.total = P.ml_offset + rows * 2 * sizeof(float);
  return P;
}

// Parts of the shortest length (the workspace bound).
int prefix_parts_for(int shared_blocks) {
  return (shared_blocks + pa::kPrefixPartBlocks - 1) / pa::kPrefixPartBlocks;
}

// Blocks per part of the shared-prefix pass for a call: the longest part
// that still gives 512 workgroups (two per CU), else the shortest. Longer
// parts leave fewer partial results to write and merge (a 4096-token prefix
// shared by 256 sequences, 8 KV heads, FP8: parts of 64 / 128 / 256 blocks
// 116.3 / 106.2 / 99.8 us per call; 32 and 16 blocks slower still).
int prefix_part_blocks_for(int64_t num_kv_heads, int64_t tiles, int shared_blocks) {
  for (int p = pa::kMaxPartitionBlocks; p > pa::kPrefixPartBlocks; p /= 2)
    if (num_kv_heads * tiles * ((shared_blocks + p - 1) / p) >= 512) return p;
  return pa::kPrefixPartBlocks;
}

Layout workspace_layout(int num_seqs, int num_heads, int head_size, int max_blocks, int pb) {
  Layout L{};
  L.partition_blocks = pb;
  L.num_parts = (max_blocks + pb - 1) / pb;
  if (L.num_parts <= 1 || num_seqs == 0) return L;
  const size_t rows = (size_t)num_seqs * num_heads * L.num_parts;
  L.out_bytes = rows * head_size * sizeof(float);
  L.ml_offset = (L.out_bytes + 255) / 256 * 256;
  L.total = L.ml_offset + rows * 2 * sizeof(float);
  return L;
}

// pa_reshape_and_cache's host checks (also run by pa_decode_append before it
// launches anything). num_tokens == 0 passes without looking at the pointers.
int reshape_check(const void* key, const void* value, const void* k_cache, const void* v_cache,
                  const void* slot_mapping, int64_t num_tokens, int num_kv_heads, int head_size, int64_t num_blocks,
                  int block_size, pa_dtype kv_dtype, pa_dtype cache_dtype, float k_scale, float v_scale) {
  if (num_tokens < 0 || num_kv_heads < 1 || num_blocks < 1)
    return fail(PA_ERR_SHAPE, "reshape_and_cache: bad sizes (num_tokens=%lld, num_kv_heads=%d, num_blocks=%lld)",
                (long long)num_tokens, num_kv_heads, (long long)num_blocks);
  if (block_size != 16)
    return fail(PA_ERR_UNSUPPORTED, "reshape_and_cache: block_size must be 16 (got %d)", block_size);
  if (head_size != 64 && head_size != 128)
    return fail(PA_ERR_UNSUPPORTED, "reshape_and_cache: head_size must be 64 or 128 (got %d)", head_size);
  if (!activation_kind(kv_dtype))
    return fail(PA_ERR_DTYPE, "reshape_and_cache: key/value dtype must be F32, F16 or BF16");
  if (cache_dtype != kv_dtype && cache_dtype != PA_DTYPE_FP8_E4M3)
    return fail(PA_ERR_DTYPE, "reshape_and_cache: cache dtype must equal the key dtype or be FP8_E4M3");
  if (cache_dtype == PA_DTYPE_FP8_E4M3 &&
      !(std::isfinite(k_scale) && std::isfinite(v_scale) && k_scale > 0.f && v_scale > 0.f))
    return fail(PA_ERR_SHAPE, "reshape_and_cache: FP8 scales must be finite and positive");
  if (num_tokens == 0) return ok();
  // The kernel indexes 16-byte source chunks in 32 bits (one thread each).
  const int64_t chunks = num_tokens * num_kv_heads * (int64_t)head_size *
                         (kv_dtype == PA_DTYPE_F32 ? 4 : 2) / 16;
  if (chunks + 255 > 0x7fffffffLL)
    return fail(PA_ERR_SHAPE, "reshape_and_cache: %lld tokens of %d KV heads are too many for one call",
                (long long)num_tokens, num_kv_heads);
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return fail(PA_ERR_NULL, "reshape_and_cache: NULL pointer argument");
  return ok();
}

int reshape_launch(const void* key, const void* value, void* k_cache, void* v_cache, const void* slot_mapping,
                   int slot_is_int64, int64_t num_tokens, int num_kv_heads, int head_size, int64_t num_blocks,
                   pa_dtype kv_dtype, pa_dtype cache_dtype, float k_scale, float v_scale, void* stream) {
  pa::ReshapeArgs a{key, value, k_cache, v_cache, slot_mapping, num_tokens, num_blocks, num_kv_heads, head_size,
                    slot_is_int64 ? 1 : 0, k_scale, v_scale};
  const hipError_t e = pa::launch_reshape(a, kv_dtype, cache_dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "reshape_and_cache: launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* pa_version(void) { return "0.1.0"; }

int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const void* slot_mapping, int slot_is_int64, int64_t num_tokens,
                         int num_kv_heads, int head_size, int64_t num_blocks, int block_size,
                         pa_dtype kv_dtype, pa_dtype cache_dtype, float k_scale, float v_scale,
                         void* stream) {
  const int rc = reshape_check(key, value, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads, head_size,
                               num_blocks, block_size, kv_dtype, cache_dtype, k_scale, v_scale);
  if (rc != PA_OK || num_tokens == 0) return rc;
  return reshape_launch(key, value, k_cache, v_cache, slot_mapping, slot_is_int64, num_tokens, num_kv_heads,
                        head_size, num_blocks, kv_dtype, cache_dtype, k_scale, v_scale, stream);
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_blocks, const int32_t* dst_blocks, int num_pairs,
                   int64_t num_blocks, int num_kv_heads, int head_size, int block_size, pa_dtype cache_dtype,
                   void* stream) {
  if (num_pairs < 0 || num_pairs > 65535 || num_kv_heads < 1 || num_blocks < 1)
    return fail(PA_ERR_SHAPE, "copy_blocks: bad sizes (num_pairs=%d in [0,65535], num_kv_heads=%d, num_blocks=%lld)",
                num_pairs, num_kv_heads, (long long)num_blocks);
  if (block_size != 16) return fail(PA_ERR_UNSUPPORTED, "copy_blocks: block_size must be 16 (got %d)", block_size);
  if (head_size != 64 && head_size != 128)
    return fail(PA_ERR_UNSUPPORTED, "copy_blocks: head_size must be 64 or 128 (got %d)", head_size);
  if (cache_dtype < PA_DTYPE_F32 || cache_dtype > PA_DTYPE_FP8_E4M3)
    return fail(PA_ERR_DTYPE, "copy_blocks: unknown cache dtype %d", (int)cache_dtype);
  if (num_pairs == 0) return ok();
  if (!k_cache || !v_cache || !src_blocks || !dst_blocks) return fail(PA_ERR_NULL, "copy_blocks: NULL pointer argument");
  static const int kBytes[] = {4, 2, 2, 1};
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_size * kBytes[cache_dtype];
  const hipError_t e = pa::launch_copy_blocks(k_cache, v_cache, src_blocks, dst_blocks, num_pairs, block_bytes,
                                              num_blocks, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "copy_blocks: launch failed: %s", hipGetErrorString(e));
  return ok();
}

int pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
               const int32_t* context_lens, const int32_t* query_start_loc, float scale, int num_kv_heads,
               int block_size, int num_seqs, int num_heads, int head_size, int max_blocks_per_seq,
               int64_t num_blocks, int max_query_len, pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype,
               float k_scale, float v_scale, void* stream) {
  if (block_size != 16) return fail(PA_ERR_UNSUPPORTED, "prefill: block_size must be 16 (got %d)", block_size);
  if (head_size != 64 && head_size != 128)
    return fail(PA_ERR_UNSUPPORTED, "prefill: head_size must be 64 or 128 (got %d)", head_size);
  if (num_seqs < 0 || num_seqs > 65535 || num_heads < 1 || num_kv_heads < 1 || max_blocks_per_seq < 1 ||
      num_blocks < 1 || max_query_len < 0)
    return fail(PA_ERR_SHAPE,
                "prefill: bad sizes (num_seqs=%d in [0,65535], num_heads=%d, num_kv_heads=%d, "
                "max_blocks_per_seq=%d, num_blocks=%lld, max_query_len=%d)",
                num_seqs, num_heads, num_kv_heads, max_blocks_per_seq, (long long)num_blocks, max_query_len);
  if (num_heads % num_kv_heads)
    return fail(PA_ERR_SHAPE, "prefill: num_heads (%d) is not a multiple of num_kv_heads (%d)", num_heads,
                num_kv_heads);
  if (q_dtype != PA_DTYPE_F16 && q_dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_DTYPE, "prefill: q dtype must be F16 or BF16 (matrix-core kernel)");
  const bool fp8 = cache_dtype == PA_DTYPE_FP8_E4M3;
  if (!(cache_dtype == q_dtype || fp8))
    return fail(PA_ERR_DTYPE, "prefill: cache dtype must equal the q dtype or be FP8_E4M3");
  if (out_dtype != q_dtype && out_dtype != PA_DTYPE_F32)
    return fail(PA_ERR_DTYPE, "prefill: out dtype must be the q dtype or F32");
  if (!std::isfinite(scale)) return fail(PA_ERR_SHAPE, "prefill: scale must be finite");
  if (fp8 && !(std::isfinite(k_scale) && std::isfinite(v_scale) && k_scale > 0.f && v_scale > 0.f))
    return fail(PA_ERR_SHAPE, "prefill: FP8 scales must be finite and positive");
  const int64_t group = num_heads / num_kv_heads;
  const int64_t row_tiles = ((int64_t)max_query_len * group + pa::kPrefillRows - 1) / pa::kPrefillRows;
  if (row_tiles * num_kv_heads > 0x7fffffffLL)
    return fail(PA_ERR_UNSUPPORTED, "prefill: max_query_len %d too large", max_query_len);
  if (num_seqs == 0 || max_query_len == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start_loc)
    return fail(PA_ERR_NULL, "prefill: NULL pointer argument");
  pa::PrefillArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  const double log2e = 1.4426950408889634;
  a.qk_scale = (float)((double)scale * log2e * (fp8 ? (double)k_scale : 1.0));
  a.out_scale = fp8 ? v_scale : 1.0f;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_size = head_size;
  a.group = (int)group;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.row_tiles = (int)row_tiles;
  a.max_query_len = max_query_len;
  a.out_kind = out_dtype;
  a.waves = pa::kPrefillRows / 16;
  a.wave_tiles = 1;
  const hipError_t e = pa::launch_prefill(a, q_dtype, cache_dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "prefill: launch failed: %s", hipGetErrorString(e));
  return ok();
}

int pa_decode_partition_blocks(int num_seqs, int num_heads, int num_kv_heads, int head_size,
                               int max_blocks_per_seq, int block_size) {
  if (!shapes_ok(num_seqs, num_heads, num_kv_heads, head_size, max_blocks_per_seq, block_size)) return 0;
  return choose_partition_blocks(num_seqs, num_heads, num_kv_heads, max_blocks_per_seq);
}

size_t pa_decode_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads, int head_size,
                                 int max_blocks_per_seq, int block_size, int partition_blocks) {
  if (!shapes_ok(num_seqs, num_heads, num_kv_heads, head_size, max_blocks_per_seq, block_size)) return 0;
  size_t balanced = 0;
  if (partition_blocks == 0) {
    // The kernel family depends on the query dtype and the balanced range
    // count on the cache dtype, neither of which this function sees: size for
    // the largest need the choice may have (FP8's range count is the larger).
    const int tile = balanced_tile(num_heads / num_kv_heads);
    if (tile && balanced_fits(num_seqs, max_blocks_per_seq) && num_seqs > 0)
      balanced = balanced_layout(num_seqs, num_heads, head_size,
                                 balanced_ranges(num_heads, tile, /*fp8_cache=*/true)).total;
    partition_blocks = choose_partition_blocks(num_seqs, num_heads, num_kv_heads, max_blocks_per_seq);
  }
  if (partition_blocks < 4 || partition_blocks > pa::kMaxPartitionBlocks || partition_blocks % 4) return 0;
  const size_t split = workspace_layout(num_seqs, num_heads, head_size, max_blocks_per_seq, partition_blocks).total;
  return split > balanced ? split : balanced;
}

}  // extern "C"

namespace {

// The new tokens of pa_decode_append (one per sequence). fused: the decode
// kernel writes them itself; otherwise the reshape kernel is queued first.
struct Append {
  const void* key;
  const void* value;
  void* k_cache;
  void* v_cache;
  const void* slots;
  int slots_int64;
  pa_dtype kv_dtype;
  bool fused;
};

// pa_decode_split, pa_decode_shared_prefix and pa_decode_append: validation,
// schedule choice, launch. groups (host, [num_groups][3]) name the
// shared-prefix groups, or are NULL; app, when set, holds the step's new
// tokens (the caller has checked them with reshape_check): a fused append
// asks the decode kernel to write them (the caller has checked that a kernel
// with one workgroup or wave per KV head and block runs), otherwise the
// reshape kernel is queued before the decode kernels. Every check runs
// before the first launch.
int decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                const int32_t* context_lens, float scale, int num_kv_heads, int block_size, int num_seqs,
                int num_heads, int head_size, int max_blocks_per_seq, int64_t num_blocks, pa_dtype q_dtype,
                pa_dtype cache_dtype, pa_dtype out_dtype, float k_scale, float v_scale, int partition_blocks,
                const int32_t* groups, int num_groups, void* workspace, size_t workspace_bytes, void* stream,
                const Append* app = nullptr) {
  if (block_size != 16) return fail(PA_ERR_UNSUPPORTED, "decode: block_size must be 16 (got %d)", block_size);
  if (head_size != 64 && head_size != 128)
    return fail(PA_ERR_UNSUPPORTED, "decode: head_size must be 64 or 128 (got %d)", head_size);
  if (num_seqs < 0 || num_seqs > 65535 || num_heads < 1 || num_kv_heads < 1 || max_blocks_per_seq < 1 ||
      num_blocks < 1)
    return fail(PA_ERR_SHAPE,
                "decode: bad sizes (num_seqs=%d in [0,65535], num_heads=%d, num_kv_heads=%d, "
                "max_blocks_per_seq=%d, num_blocks=%lld)",
                num_seqs, num_heads, num_kv_heads, max_blocks_per_seq, (long long)num_blocks);
  if (num_heads % num_kv_heads)
    return fail(PA_ERR_SHAPE, "decode: num_heads (%d) is not a multiple of num_kv_heads (%d)", num_heads,
                num_kv_heads);
  if (!activation_kind(q_dtype)) return fail(PA_ERR_DTYPE, "decode: q dtype must be F32, F16 or BF16");
  const bool fp8 = cache_dtype == PA_DTYPE_FP8_E4M3;
  if (!(cache_dtype == q_dtype || (fp8 && q_dtype != PA_DTYPE_F32)))
    return fail(PA_ERR_DTYPE, "decode: cache dtype must equal the q dtype, or be FP8_E4M3 with F16/BF16 queries");
  if (out_dtype != q_dtype && out_dtype != PA_DTYPE_F32)
    return fail(PA_ERR_DTYPE, "decode: out dtype must be the q dtype or F32");
  if (!std::isfinite(scale)) return fail(PA_ERR_SHAPE, "decode: scale must be finite");
  if (fp8 && !(std::isfinite(k_scale) && std::isfinite(v_scale) && k_scale > 0.f && v_scale > 0.f))
    return fail(PA_ERR_SHAPE, "decode: FP8 scales must be finite and positive");
  if (partition_blocks != 0 &&
      (partition_blocks < 4 || partition_blocks > pa::kMaxPartitionBlocks || partition_blocks % 4))
    return fail(PA_ERR_UNSUPPORTED, "decode: partition_blocks must be 0 or a multiple of 4 in [4, %d] (got %d)",
                pa::kMaxPartitionBlocks, partition_blocks);
  if (num_groups < 0 || num_groups > pa::kMaxPrefixGroups)
    return fail(PA_ERR_SHAPE, "decode: num_groups must be in [0, %d] (got %d)", pa::kMaxPrefixGroups, num_groups);
  if (num_groups > 0 && !groups) return fail(PA_ERR_NULL, "decode: NULL prefix_groups with num_groups > 0");
  int max_shared = 0;
  for (int i = 0; i < num_groups; ++i) {
    const int first = groups[3 * i], count = groups[3 * i + 1], blocks = groups[3 * i + 2];
    const int prev_end = i ? groups[3 * (i - 1)] + groups[3 * (i - 1) + 1] : 0;
    if (first < prev_end || count < 1 || (int64_t)first + count > num_seqs || blocks < 1 ||
        blocks > max_blocks_per_seq)
      return fail(PA_ERR_SHAPE,
                  "decode: prefix group %d (first %d, count %d, blocks %d) must lie in [0, %d) after the previous "
                  "group, with 1 <= blocks <= %d",
                  i, first, count, blocks, num_seqs, max_blocks_per_seq);
    if (blocks > max_shared) max_shared = blocks;
  }
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_ERR_NULL, "decode: NULL pointer argument");

  const int group = num_heads / num_kv_heads;
  const bool mfma = use_mfma(q_dtype, group);
  const bool wide = mfma && wide_group(group);
  const int group_tile = mfma ? pa::mfma_group_tile(group) : pa::group_tile_for(group);
  // The library's own choice for the matrix-core kernel is the balanced
  // schedule (below 32 query heads per KV head); an explicit partition length
  // selects the partitioned one. It needs a workspace; a caller that passes
  // none (or too small a one, as sized before this schedule existed) gets the
  // partitioned schedule.
  bool balanced = partition_blocks == 0 && mfma && !wide && balanced_fits(num_seqs, max_blocks_per_seq);
  const int64_t ranges = balanced ? balanced_ranges(num_heads, balanced_tile(group), fp8) : 0;
  if (balanced && (!workspace || workspace_bytes < balanced_layout(num_seqs, num_heads, head_size, ranges).total))
    balanced = false;
  if (ranges / 4 > 65535) return fail(PA_ERR_UNSUPPORTED, "decode: too many ranges (%lld)", (long long)ranges);
  const int pb = partition_blocks ? partition_blocks
                                  : choose_partition_blocks(num_seqs, num_heads, num_kv_heads, max_blocks_per_seq);
  const Layout L = balanced ? balanced_layout(num_seqs, num_heads, head_size, ranges)
                            : workspace_layout(num_seqs, num_heads, head_size, max_blocks_per_seq, pb);
  if (L.num_parts > 65535) return fail(PA_ERR_UNSUPPORTED, "decode: too many partitions (%d)", L.num_parts);
  // The shared-prefix pass runs with the balanced schedule when the group
  // size divides the 16 query columns of its tile; otherwise every block is
  // read per sequence, which gives the same result.
  const bool prefix = num_groups > 0 && balanced && group >= 4 && 16 % group == 0;
  int prefix_tiles = 0;  // tiles of 16 / group sequences over all groups
  if (prefix)
    for (int i = 0; i < num_groups; ++i) prefix_tiles += (groups[3 * i + 1] + 16 / group - 1) / (16 / group);
  const int prefix_part = prefix ? prefix_part_blocks_for(num_kv_heads, prefix_tiles, max_shared) : 0;
  const int prefix_parts = prefix ? (max_shared + prefix_part - 1) / prefix_part : 0;
  const PrefixLayout PL = prefix_layout(L.total, num_seqs, num_heads, head_size, prefix_parts);
  const size_t need = prefix ? PL.total : L.total;
  if (need > 0) {
    if (!workspace)
      return fail(PA_ERR_WORKSPACE, "decode: a workspace of %zu bytes is needed", need);
    if (workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, "decode: workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
                  need);
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
      return fail(PA_ERR_WORKSPACE, "decode: workspace must be 256-byte aligned");
  }

  if (wide) {
    // Groups of 32 and more (a multiple of 32): the prefill kernel's decode
    // mode, then decode_reduce for split contexts.
    pa::PrefillArgs w{};
    w.out = out;
    w.q = q;
    w.k_cache = k_cache;
    w.v_cache = v_cache;
    w.block_tables = block_tables;
    w.context_lens = context_lens;
    w.query_start_loc = nullptr;
    const double log2e = 1.4426950408889634;
    w.qk_scale = (float)((double)scale * log2e * (fp8 ? (double)k_scale : 1.0));
    w.out_scale = fp8 ? v_scale : 1.0f;
    w.num_seqs = num_seqs;
    w.num_heads = num_heads;
    w.num_kv_heads = num_kv_heads;
    w.head_size = head_size;
    w.group = group;
    w.max_blocks = max_blocks_per_seq;
    w.num_blocks = num_blocks;
    wide_shape(group, w.waves, w.wave_tiles);
    w.row_tiles = group / (16 * w.waves * w.wave_tiles);
    w.max_query_len = 1;
    w.out_kind = out_dtype;
    w.decode = 1;
    w.part_blocks = L.num_parts > 1 ? pb : 0;
    w.num_parts = L.num_parts;
    w.ws_out = L.total ? static_cast<float*>(workspace) : nullptr;
    w.ws_ml = L.total ? reinterpret_cast<float*>(static_cast<char*>(workspace) + L.ml_offset) : nullptr;
    if (app && !app->fused) {
      const int rc = reshape_launch(app->key, app->value, app->k_cache, app->v_cache, app->slots, app->slots_int64,
                                    num_seqs, num_kv_heads, head_size, num_blocks, app->kv_dtype, cache_dtype, k_scale,
                                    v_scale, stream);
      if (rc != PA_OK) return rc;
    }
    const hipError_t e = pa::launch_decode_wide(w, q_dtype, cache_dtype, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "decode: launch failed: %s", hipGetErrorString(e));
    return ok();
  }

  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.ws_out = L.total ? static_cast<float*>(workspace) : nullptr;
  a.ws_ml = L.total ? reinterpret_cast<float*>(static_cast<char*>(workspace) + L.ml_offset) : nullptr;
  a.ws_pref = balanced ? reinterpret_cast<int*>(static_cast<char*>(workspace) + L.pref_offset) : nullptr;
  const double log2e = 1.4426950408889634;
  a.qk_scale = (float)((double)scale * log2e * (fp8 ? (double)k_scale : 1.0));
  a.out_scale = fp8 ? v_scale : 1.0f;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_size = head_size;
  a.group = group;
  a.use_mfma = mfma ? 1 : 0;
  a.group_tile = balanced ? balanced_tile(group) : group_tile;
  a.balanced = balanced ? 1 : 0;
  a.cached_loads = cached_loads_requested() ? 1 : 0;
  a.ranges = balanced ? (int)ranges : 0;
  a.num_blocks = num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.partition_blocks = pb;
  a.num_parts = L.num_parts;
  a.out_kind = out_dtype;
  if (prefix) {
    char* ws = static_cast<char*>(workspace);
    a.shared_prefix = 1;
    a.prefix_groups = num_groups;
    a.prefix_parts = prefix_parts;
    a.prefix_part_blocks = prefix_part;
    a.ws_shared = reinterpret_cast<int*>(ws + PL.shared_offset);
    a.ws_sh_out = reinterpret_cast<float*>(ws + PL.out_offset);
    a.ws_sh_ml = reinterpret_cast<float*>(ws + PL.ml_offset);
    const int spt = 16 / group;  // sequences per tile of the prefix pass
    int tiles = 0;
    for (int i = 0; i < num_groups; ++i) {
      a.grp_first[i] = groups[3 * i];
      a.grp_count[i] = groups[3 * i + 1];
      a.grp_blocks[i] = groups[3 * i + 2];
      a.grp_tile0[i] = tiles;
      tiles += (groups[3 * i + 1] + spt - 1) / spt;
    }
    a.grp_tile0[num_groups] = tiles;
    if (prefix_parts > 65535) return fail(PA_ERR_UNSUPPORTED, "decode: shared prefix too long");
  }
  if (app && app->fused) {
    a.append = 1;
    a.new_key = app->key;
    a.new_value = app->value;
    a.new_slots = app->slots;
    a.new_slots_int64 = app->slots_int64;
    a.enc_k_scale = k_scale;
    a.enc_v_scale = v_scale;
  } else if (app) {
    const int rc = reshape_launch(app->key, app->value, app->k_cache, app->v_cache, app->slots, app->slots_int64,
                                  num_seqs, num_kv_heads, head_size, num_blocks, app->kv_dtype, cache_dtype, k_scale,
                                  v_scale, stream);
    if (rc != PA_OK) return rc;
  }
  const hipError_t e = pa::launch_decode(a, q_dtype, cache_dtype, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "decode: launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int pa_decode_split(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, float scale,
                    int num_kv_heads, int block_size, int num_seqs, int num_heads, int head_size,
                    int max_blocks_per_seq, int64_t num_blocks, pa_dtype q_dtype,
                    pa_dtype cache_dtype, pa_dtype out_dtype, float k_scale, float v_scale,
                    int partition_blocks, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, num_kv_heads, block_size, num_seqs,
                     num_heads, head_size, max_blocks_per_seq, num_blocks, q_dtype, cache_dtype, out_dtype, k_scale,
                     v_scale, partition_blocks, nullptr, 0, workspace, workspace_bytes, stream);
}

int pa_decode_shared_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens, float scale,
                            int num_kv_heads, int block_size, int num_seqs, int num_heads, int head_size,
                            int max_blocks_per_seq, int64_t num_blocks, pa_dtype q_dtype, pa_dtype cache_dtype,
                            pa_dtype out_dtype, float k_scale, float v_scale, const int32_t* prefix_groups,
                            int num_groups, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, num_kv_heads, block_size, num_seqs,
                     num_heads, head_size, max_blocks_per_seq, num_blocks, q_dtype, cache_dtype, out_dtype, k_scale,
                     v_scale, 0, prefix_groups, num_groups, workspace, workspace_bytes, stream);
}

size_t pa_decode_shared_prefix_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads, int head_size,
                                               int max_blocks_per_seq, int block_size, int max_shared_blocks) {
  const size_t base = pa_decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_size, max_blocks_per_seq,
                                                block_size, 0);
  if (!shapes_ok(num_seqs, num_heads, num_kv_heads, head_size, max_blocks_per_seq, block_size) ||
      max_shared_blocks < 0 || max_shared_blocks > max_blocks_per_seq)
    return 0;
  if (max_shared_blocks == 0 || !balanced_tile(num_heads / num_kv_heads) ||
      !balanced_fits(num_seqs, max_blocks_per_seq) || num_seqs == 0)
    return base;
  // The balanced layout for the larger (FP8) range count, then the prefix region.
  const size_t bal = balanced_layout(num_seqs, num_heads, head_size,
                                     balanced_ranges(num_heads, balanced_tile(num_heads / num_kv_heads), true)).total;
  const size_t total = prefix_layout(bal, num_seqs, num_heads, head_size, prefix_parts_for(max_shared_blocks)).total;
  return total > base ? total : base;
}

int pa_decode_append(void* out, const void* q, const void* key, const void* value, void* k_cache, void* v_cache,
                     const void* slot_mapping, int slot_is_int64, const int32_t* block_tables,
                     const int32_t* context_lens, float scale, int num_kv_heads, int block_size, int num_seqs,
                     int num_heads, int head_size, int max_blocks_per_seq, int64_t num_blocks, pa_dtype q_dtype,
                     pa_dtype cache_dtype, pa_dtype out_dtype, float k_scale, float v_scale, void* workspace,
                     size_t workspace_bytes, void* stream) {
  // The decode kernel writes the new rows itself where exactly one wave of the
  // launch reads the block holding a sequence's new row for a KV head: the
  // vector-ALU kernel with one workgroup per (sequence, KV head, partition)
  // (MHA or two query heads per KV head with 16-bit queries; groups of 1, 2,
  // 4 or 8 with float32 queries), and the matrix-core kernel with one head
  // tile per KV head (groups of 4, 8 or 16), in either schedule. Elsewhere the
  // reshape kernel runs first (two launches, same result).
  const int group = num_kv_heads >= 1 && num_heads % num_kv_heads == 0 ? num_heads / num_kv_heads : 0;
  const bool sixteen = q_dtype == PA_DTYPE_F16 || q_dtype == PA_DTYPE_BF16;
  const bool mfma = group > 0 && use_mfma(q_dtype, group);
  const bool fused = group > 0 && (mfma ? pa::mfma_group_tile(group) == group
                                        : pa::group_tile_for(group) == group && !(group >= 4 && sixteen));
  if (num_seqs < 0) return fail(PA_ERR_SHAPE, "decode_append: num_seqs must be >= 0 (got %d)", num_seqs);
  const int rc = reshape_check(key, value, k_cache, v_cache, slot_mapping, num_seqs, num_kv_heads, head_size,
                               num_blocks, block_size, q_dtype, cache_dtype, k_scale, v_scale);
  if (rc != PA_OK) return rc;
  const Append app{key, value, k_cache, v_cache, slot_mapping, slot_is_int64 ? 1 : 0, q_dtype, fused};
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, num_kv_heads, block_size, num_seqs,
                     num_heads, head_size, max_blocks_per_seq, num_blocks, q_dtype, cache_dtype, out_dtype, k_scale,
                     v_scale, 0, nullptr, 0, workspace, workspace_bytes, stream, &app);
}

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
              const int32_t* context_lens, float scale, int num_kv_heads, int block_size, int num_seqs,
              int num_heads, int head_size, int max_blocks_per_seq, int64_t num_blocks, pa_dtype q_dtype,
              pa_dtype cache_dtype, pa_dtype out_dtype, float k_scale, float v_scale, void* workspace,
              size_t workspace_bytes, void* stream) {
  return pa_decode_split(out, q, k_cache, v_cache, block_tables, context_lens, scale, num_kv_heads, block_size,
                         num_seqs, num_heads, head_size, max_blocks_per_seq, num_blocks, q_dtype, cache_dtype,
                         out_dtype, k_scale, v_scale, 0, workspace, workspace_bytes, stream);
}

}  // extern "C"

// --- pa_decode_scratch: pa_decode without a caller-provided workspace ---------
//
// For callers that cannot allocate device memory around a call (code under
// graph capture, tight serving loops): the workspace is a fixed array in the
// library's device code, one copy per GPU, held until the process ends.

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB per GPU

// In host code this name only stands for the device array: its address on a
// device comes from hipGetSymbolAddress, made with that device current.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's scratch array in *ptr, looked up
// once per device (with that device current) and kept. Returns a status.
int scratch_for_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "decode_scratch: hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(PA_ERR_UNSUPPORTED, "decode_scratch: device %d is past the %d devices served", dev,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PA_ERR_LAUNCH, "decode_scratch: hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" {

size_t pa_decode_scratch_bytes(void) { return kScratchBytes; }

int pa_decode_scratch(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale, int num_kv_heads,
                      int block_size, int num_seqs, int num_heads, int head_size, int max_blocks_per_seq,
                      int64_t num_blocks, pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype, float k_scale,
                      float v_scale, void* stream) {
  void* ws = nullptr;
  const int st = scratch_for_current_device(&ws);
  if (st != PA_OK) return st;
  // Same choice of schedule as pa_decode with a workspace of kScratchBytes: the
  // balanced schedule where its need fits, else the partitioned one. Every
  // element the kernels read from the workspace is written earlier in the same
  // call, so the array needs no clearing between calls.
  const int rc = decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, num_kv_heads, block_size,
                             num_seqs, num_heads, head_size, max_blocks_per_seq, num_blocks, q_dtype, cache_dtype,
                             out_dtype, k_scale, v_scale, 0, nullptr, 0, ws, kScratchBytes, stream);
  if (rc == PA_ERR_WORKSPACE) {
    const std::string why = pa_last_error();
    return fail(PA_ERR_WORKSPACE, "decode_scratch: these shapes need more than the fixed %zu-byte scratch (%s)",
                kScratchBytes, why.c_str());
  }
  return rc;
}

}  // extern "C"
