// Host-side declarations shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

struct ReshapeArgs {
  const void* key;
  const void* value;
  void* k_cache;
  void* v_cache;
  const void* slots;
  int64_t num_tokens;
  int64_t num_blocks;     // pool size; slots at or past num_blocks * 16 are skipped
  int num_kv_heads;
  int head_size;
  int slot_is_int64;
  float k_scale;
  float v_scale;
};

// Returns a hipError_t of the launch.
hipError_t launch_reshape(const ReshapeArgs& a, int src_kind, int cache_kind, hipStream_t stream);

// Groups a shared-prefix call may name, and the shortest part (in blocks) of
// the prefix kernel, for which the workspace is sized; a call takes parts of
// up to kMaxPartitionBlocks blocks (prefix_part_blocks).
constexpr int kMaxPrefixGroups = 16;
constexpr int kPrefixPartBlocks = 64;

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_out;          // [S, H, P, D] unnormalised partition outputs
  float* ws_ml;           // [S, H, P, 2] partition max (log2 domain) and sum
                          // (balanced schedule: [H, S + R, D] and [H, S + R, 2], slot s + r)
  int* ws_pref;           // balanced schedule: [S + 1] first flattened block of each sequence
  float qk_scale;         // scale * log2(e) (* k_scale for FP8 caches)
  float out_scale;        // v_scale for FP8 caches, else 1
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int head_size;
  int group;              // num_heads / num_kv_heads
  int group_tile;         // query heads handled by one workgroup (divides group)
  int64_t num_blocks;     // pool size (block ids outside [0, num_blocks) are clamped)
  int max_blocks;         // block table row length
  int partition_blocks;   // blocks per partition
  int num_parts;          // ceil(max_blocks / partition_blocks)
  int out_kind;           // Kind of out: F32 or the query kind
  int use_mfma;           // 1: matrix-core kernel (16-bit queries, group_tile 4, 8 or 16)
  int balanced;           // 1: balanced schedule (matrix-core kernel only): equal block ranges per wave
  int cached_loads;       // 1: the MHA vector kernel reads K/V with cached instead of nontemporal loads
                          //    (comparison runs only, PA_DECODE_LOADS=cached)
  int ranges;             // balanced schedule: number of ranges R (a multiple of 4)
  // Shared-prefix pass (balanced schedule only): groups of consecutive
  // sequences whose block tables start with the same full blocks. The prefix
  // kernel reads those blocks once per 16 query columns (16 / group sequences)
  // and leaves per-part partial results; the balanced kernel then streams
  // only the blocks past each sequence's shared prefix.
  int shared_prefix;      // 1: the pass runs (ws_shared, ws_sh_* and the group list are set)
  int prefix_groups;      // number of groups (<= kMaxPrefixGroups)
  int prefix_parts;       // P1: parts of prefix_part_blocks blocks of the longest shared prefix
  int prefix_part_blocks; // blocks per part (a power of two from kPrefixPartBlocks to kMaxPartitionBlocks)
  int* ws_shared;         // [S] shared blocks of each sequence (0 outside every group)
  float* ws_sh_out;       // [H, S, P1, D] unnormalised partial outputs over the shared blocks
  float* ws_sh_ml;        // [H, S, P1, 2] their max (log2 domain) and sum
  int grp_first[kMaxPrefixGroups];  // group g: sequences grp_first[g] .. grp_first[g] + grp_count[g] - 1
  int grp_count[kMaxPrefixGroups];
  int grp_blocks[kMaxPrefixGroups];     // shared full blocks of group g
  int grp_tile0[kMaxPrefixGroups + 1];  // first prefix-kernel tile of group g (tiles of 16 / group sequences)
  // Fused append (pa_decode_append, where one wave of the launch reads each
  // (sequence, KV head)'s last block: the vector-ALU kernel with one
  // workgroup per (sequence, KV head, partition), or the matrix-core kernel
  // with one head tile per KV head): that wave first writes the sequence's
  // new K/V row of its KV head into the cache (as pa_reshape_and_cache
  // would) and waits for the stores, then attends.
  int append;
  int new_slots_int64;    // slot type: int64 (1) or int32 (0)
  const void* new_key;    // [S, Hkv, D], the query dtype
  const void* new_value;
  const void* new_slots;  // [S]; a negative slot (or one outside the pool) writes nothing
  float enc_k_scale;      // FP8 caches: the E4M3 encoding scales
  float enc_v_scale;
};


// Queues the decode kernel(s) chosen by a.use_mfma, then the partition merge if needed.
hipError_t launch_decode(const DecodeArgs& a, int q_kind, int cache_kind, hipStream_t stream);
// The partition merge alone: for every (sequence, head) whose context spans
// several partitions of a.partition_blocks blocks, merges the a.num_parts
// slots of ws_out / ws_ml into out (reads out, context_lens, ws_*, sizes).
hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t stream);
// The matrix-core decode kernel alone (pa_decode_mfma.hip).
hipError_t launch_decode_mfma(const DecodeArgs& a, int q_kind, int cache_kind, hipStream_t stream);
// The shared-prefix pass of the matrix-core kernel (a.shared_prefix; 16-bit queries, group 4, 8 or 16).
hipError_t launch_decode_prefix(const DecodeArgs& a, int q_kind, int cache_kind, hipStream_t stream);

// Largest query-head tile (8, 4, 2 or 1) dividing the group size.
inline int group_tile_for(int group) {
  for (int t = 8; t > 1; t /= 2)
    if (group % t == 0) return t;
  return 1;
}

struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start_loc;  // [num_seqs + 1]
  float qk_scale;         // scale * log2(e) (* k_scale for FP8 caches)
  float out_scale;        // v_scale for FP8 caches, else 1
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int head_size;
  int group;
  int max_blocks;
  int64_t num_blocks;
  int row_tiles;          // workgroups per KV head and sequence: ceil(max_query_len * group / rows per workgroup)
  int max_query_len;      // rows of longer chunks past this many tokens are not computed
  int out_kind;
  // Decode through the same kernel (groups of 32 and more query heads per KV
  // head): sequence s has one query, row s of q, and its group's heads are the
  // rows; query_start_loc is not read. A context longer than part_blocks
  // blocks is split into partitions (grid z) whose (max, sum, unnormalised
  // output) go to ws_out / ws_ml in decode_reduce's layout; an empty context
  // gives zeros.
  int decode;             // 1: decode mode
  int waves;              // waves per workgroup (2, 4 or 8)
  int wave_tiles;         // 16-row tiles per wave (1; 2 with 4 waves)
  int part_blocks;        // decode: blocks per partition (0: whole contexts)
  int num_parts;          // decode: partitions per sequence (grid z)
  float* ws_out;          // decode, split contexts: [S, H, P, D]
  float* ws_ml;           // decode, split contexts: [S, H, P, 2]
};

// Rows ((token, head) pairs of one KV head) per prefill workgroup (16 per wave).
constexpr int kPrefillRows = 128;

hipError_t launch_prefill(const PrefillArgs& a, int q_kind, int cache_kind, hipStream_t stream);

// Decode for groups of 32 and more query heads per KV head on the prefill
// kernel (a.decode = 1), then, for split contexts, the partition merge.
hipError_t launch_decode_wide(const PrefillArgs& a, int q_kind, int cache_kind, hipStream_t stream);

// Copies whole (all KV heads) blocks src[i] -> dst[i] in both caches.
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst, int num_pairs,
                              int64_t block_bytes, int64_t num_blocks, hipStream_t stream);

// Query-head tile of the matrix-core kernel (16, 8 or 4 dividing the group), or 0 if none does.
inline int mfma_group_tile(int group) {
  for (int t = 16; t >= 4; t /= 2)
    if (group % t == 0) return t;
  return 0;
}

constexpr int kMaxPartitionBlocks = 512;

// Largest batch the balanced schedule serves (its block-count prefix lives in LDS).
constexpr int kBalancedMaxSeqs = 1024;

}  // namespace pa
