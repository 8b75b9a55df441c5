// Paged-attention decode for gfx950 (CDNA4).
//
// What is computed ("vLLM 前世今生" §3.2; "vLLM" note, sections "PagedAttention"
// and "内核优化"): for every sequence and query head, softmax(q·Kᵀ·scale)·V
// over the sequence's cached tokens, which sit in 16-token blocks scattered
// through a pool and are reached through the sequence's block table; a group
// of query heads shares one KV head.
//
// How (decode is a matrix-vector product, bound by HBM bandwidth, so no MFMA):
//  * one workgroup of 4 waves per (sequence, KV head, head tile, partition);
//    all query heads of the tile are served from one read of each K/V tile;
//  * the partition's slice of the block table is staged in LDS; each wave walks
//    its share of the blocks (wave w takes blocks w, w+4, ...), reading each
//    (block, KV head) tile of 16 rows with 16-byte loads: one wave-load moves
//    1 KiB of contiguous memory, and the next tile's loads are issued before
//    the current tile is consumed;
//  * a token row is split over LPR lanes; q·k is a packed dot product per lane
//    (v_dot2 for 16-bit data) followed by a DPP butterfly inside the lane group;
//  * every lane group keeps its own running max / sum / output (the online
//    softmax normaliser of Milakov & Gimelshein, 2018, also used by
//    FlashAttention, which the history page cites in §2.2); the groups and
//    the waves are merged once at the end through shuffles and LDS;
//  * a context longer than one partition is split: each partition leaves its
//    max, sum and unnormalised output in the workspace and decode_reduce merges
//    them in partition order (deterministic).
// Rows past the context (the tail of the last block) are removed by selection,
// never by multiplying with zero, so stale or NaN data there cannot leak.
#include <type_traits>

#include "pa_decode_common.h"

namespace pa {
namespace {

constexpr int kRing = 2;  // register ring depth: blocks per wave in flight, plus the one in use


template <int QK, int CK, int D> struct QFrag {
  static constexpr int kElems = TileGeo<CK, D>::E;                     // q elements per lane
  static constexpr int kWords = (QK == kF32) ? kElems : kElems / 2;    // 32-bit words per lane
};

// First term of a packed 16-bit dot product: the VOP3 form with an inline
// zero addend, so the accumulator needs no zeroing move (the compiler would
// otherwise pick the tied-accumulator form and zero a register first).
template <int QK>
__device__ __forceinline__ float dot2_first(uint32_t a, uint32_t b) {
  float r;
  if constexpr (QK == kBF16)
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  else
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

template <int QK>
__device__ __forceinline__ float dot2_acc(uint32_t a, uint32_t b, float acc) {
  if constexpr (QK == kBF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a), __builtin_bit_cast(bf162_t, b), acc, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), acc, false);
}

// Partial q·k over the E elements one lane holds of a token row.
template <int QK, int CK>
__device__ __forceinline__ float dot_chunk(const uint32_t* qw, const uint4& k) {
  const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
  float acc;
  if constexpr (CK == kF32) {
    acc = __uint_as_float(qw[0]) * __uint_as_float(kw[0]);
#pragma unroll
    for (int i = 1; i < 4; ++i) acc = __builtin_fmaf(__uint_as_float(qw[i]), __uint_as_float(kw[i]), acc);
  } else if constexpr (CK == kF16 || CK == kBF16) {
    acc = dot2_first<CK>(qw[0], kw[0]);
#pragma unroll
    for (int i = 1; i < 4; ++i) acc = dot2_acc<CK>(qw[i], kw[i], acc);
  } else {
    // FP8 codes widen exactly to the query's 16-bit type (scale 1), then dot2.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo, hi;
      if constexpr (QK == kBF16) {
        lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)kw[i], 1.0f, false));
        hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)kw[i], 1.0f, true));
      } else {
        lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)kw[i], 1.0f, false));
        hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)kw[i], 1.0f, true));
      }
      acc = (i == 0) ? dot2_first<QK>(qw[0], lo) : dot2_acc<QK>(qw[2 * i], lo, acc);
      acc = dot2_acc<QK>(qw[2 * i + 1], hi, acc);
    }
  }
  return acc;
}

// The E elements one lane holds of a V row, as float32.
template <int CK>
__device__ __forceinline__ void v_to_float(const uint4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (CK == kF32) {
      f[i] = __uint_as_float(w[i]);
    } else if constexpr (CK == kF16) {
      f[2 * i] = f16_lo(w[i]);
      f[2 * i + 1] = f16_hi(w[i]);
    } else if constexpr (CK == kBF16) {
      f[2 * i] = bf16_lo(w[i]);
      f[2 * i + 1] = bf16_hi(w[i]);
    } else {
      const float2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)w[i], 1.0f, false);
      const float2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)w[i], 1.0f, true);
      f[4 * i] = lo.x;
      f[4 * i + 1] = lo.y;
      f[4 * i + 2] = hi.x;
      f[4 * i + 3] = hi.y;
    }
  }
}

// One lane's K chunk as packed 16-bit pairs of the query's type: FP8 codes are
// widened exactly (scale 1) once, so every query head reuses the conversion.
template <int QK, int CK> constexpr int kKWords = (CK == kFP8) ? 8 : 4;

template <int QK, int CK>
__device__ __forceinline__ void k_words(const uint4& k, uint32_t* w) {
  const uint32_t kw[4] = {k.x, k.y, k.z, k.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (CK == kFP8) {
      if constexpr (QK == kBF16) {
        w[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)kw[i], 1.0f, false));
        w[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)kw[i], 1.0f, true));
      } else {
        w[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)kw[i], 1.0f, false));
        w[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)kw[i], 1.0f, true));
      }
    } else {
      w[i] = kw[i];
    }
  }
}

template <int QK, int N>
__device__ __forceinline__ float dot_words(const uint32_t* q, const uint32_t* k) {
  float acc = dot2_first<QK>(q[0], k[0]);
#pragma unroll
  for (int i = 1; i < N; ++i) acc = dot2_acc<QK>(q[i], k[i], acc);
  return acc;
}

// Transposing pair sums across the two 32-lane halves (v_permlane32_swap) and
// across 16-lane rows (v_permlane16_swap): lanes whose bit is 0 end with
// a(own) + a(partner), lanes whose bit is 1 with b(partner) + b(own).
__device__ __forceinline__ float swap_sum32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_sum16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
constexpr int kDppRowRor8 = 0x128;  // lane j <- lane (j - 8) mod 16, i.e. j ^ 8
constexpr int kDppRowRor4 = 0x124;  // lane j <- lane (j - 4) mod 16

template <int QK, int CK, int D, int GT, bool kCachedLoads = false>
__global__ __launch_bounds__(kThreads) void decode_main(const DecodeArgs a) {
  using Geo = TileGeo<CK, D>;
  constexpr int E = Geo::E, LPR = Geo::LPR, RPL = Geo::RPL, NL = Geo::NL;
  constexpr int QW = QFrag<QK, CK, D>::kWords;
  constexpr int kQBytes = KindBytes<QK>::value;
  constexpr int kTileBytes = 16 * D * Geo::kBytes;
  static_assert(RPL * D * Geo::kBytes == 1024, "a wave-load covers 1 KiB");

  __shared__ int s_blocks[kMaxPartitionBlocks];
  __shared__ float s_acc[kWaves][GT][D];
  __shared__ float s_ml[kWaves][GT][2];

  const int n_sub = a.group / GT;
  const int kvh = blockIdx.x / n_sub;
  const int h0 = kvh * a.group + (blockIdx.x - kvh * n_sub) * GT;  // first query head of the tile
  const int part = blockIdx.y;
  const int seq = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int ctx = context_len(a, seq);
  // Fused append: the new row (position ctx - 1) lies in the sequence's last
  // block, which for this KV head only one wave of the launch reads (one
  // workgroup per KV head; the last partition's wave (nblk - 1) % kWaves, at
  // the end of its stream). That wave writes the row and waits until its
  // stores have completed before it issues any load, so its later load of
  // the block returns the new row; the other waves start streaming at once.
  // An empty context's row goes out with partition 0.
  const bool writer = a.append && part == (ctx > 0 ? (((ctx + 15) >> 4) - 1) / a.partition_blocks : 0);
  if (ctx <= 0) {  // nothing to attend
    if (writer) append_row<QK, CK, D, kThreads>(a, seq, kvh, tid);
    write_zeros<GT, D>(a, seq, h0, part, tid);
    return;
  }
  const int seq_blocks = (ctx + 15) >> 4;
  const int blk0 = part * a.partition_blocks;
  if (blk0 >= seq_blocks) return;
  const int nblk = min(a.partition_blocks, seq_blocks - blk0);
  const int seq_parts = (seq_blocks + a.partition_blocks - 1) / a.partition_blocks;

  const int32_t* bt = a.block_tables + (int64_t)seq * a.max_blocks + blk0;
  for (int j = tid; j < nblk; j += kThreads) s_blocks[j] = bt[j];

  const int col = lane % LPR;  // which E-element slice of a row this lane holds
  const int row = lane / LPR;  // which of the RPL rows of a wave-load

  uint32_t qf[GT][QW];
  {
    const char* qp = static_cast<const char*>(a.q) + (((int64_t)seq * a.num_heads + h0) * D + col * E) * kQBytes;
#pragma unroll
    for (int g = 0; g < GT; ++g) {
#pragma unroll
      for (int c = 0; c < QW / 4; ++c) {
        const uint4 v = *reinterpret_cast<const uint4*>(qp + g * D * kQBytes + c * 16);
        qf[g][4 * c] = v.x;
        qf[g][4 * c + 1] = v.y;
        qf[g][4 * c + 2] = v.z;
        qf[g][4 * c + 3] = v.w;
      }
    }
  }
  __syncthreads();
  // (After the barrier, so that only the writing wave waits for its stores.)
  if (writer && wave == (nblk - 1) % kWaves) {
    append_row<QK, CK, D, 64>(a, seq, kvh, lane);
    wait_own_stores();
  }

  float m[GT], l[GT], acc[GT][E];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
  }

  const int64_t blk_stride = (int64_t)a.num_kv_heads * kTileBytes;
  const char* kbase = static_cast<const char*>(a.k_cache) + (int64_t)kvh * kTileBytes;
  const char* vbase = static_cast<const char*>(a.v_cache) + (int64_t)kvh * kTileBytes;
  const int lane_off = lane * 16;
  const float qk_scale = a.qk_scale;

  // The tile address is wave-uniform (scalar registers); each lane adds its
  // 16-byte offset, so the loads take the scalar-base + vector-offset form.
  struct Tile {
    uint4 k[NL], v[NL];
  };
  auto load_tile = [&](int j, Tile& t) {
    uint4(&kr)[NL] = t.k;
    uint4(&vr)[NL] = t.v;
    const int64_t off = pool_block(a, s_blocks, j) * blk_stride;
    const char* kt = kbase + off;
    const char* vt = vbase + off;
#pragma unroll
    for (int i = 0; i < NL; ++i) kr[i] = load_tile_chunk<kCachedLoads>(kt + lane_off + i * 1024);
#pragma unroll
    for (int i = 0; i < NL; ++i) vr[i] = load_tile_chunk<kCachedLoads>(vt + lane_off + i * 1024);
  };

  auto process = [&](int j, const Tile& t) {
    const uint4(&kr)[NL] = t.k;
    const uint4(&vin)[NL] = t.v;
    float sc[GT][NL];
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int g = 0; g < GT; ++g) sc[g][i] = group_sum<LPR>(dot_chunk<QK, CK>(qf[g], kr[i])) * qk_scale;
    uint4 vr[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) vr[i] = vin[i];
    const int tok0 = (blk0 + j) * 16;
    if (tok0 + 16 > ctx) {  // last, partial block: drop rows past the context
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const bool ok = tok0 + i * RPL + row < ctx;
#pragma unroll
        for (int g = 0; g < GT; ++g) sc[g][i] = ok ? sc[g][i] : kNegInf;
        vr[i].x = ok ? vr[i].x : 0u;  // all-zero bits are +0.0 in every storage type
        vr[i].y = ok ? vr[i].y : 0u;
        vr[i].z = ok ? vr[i].z : 0u;
        vr[i].w = ok ? vr[i].w : 0u;
      }
    }
    // With one query head the V elements are widened where they are used;
    // with several they are widened once and shared by all heads.
    float vf[GT == 1 ? 1 : NL][E];
    if constexpr (GT > 1) {
#pragma unroll
      for (int i = 0; i < NL; ++i) v_to_float<CK>(vr[i], vf[i]);
    }
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      float bm = sc[g][0];
#pragma unroll
      for (int i = 1; i < NL; ++i) bm = fmaxf(bm, sc[g][i]);
      const float mn = fmaxf(m[g], bm);
      const float ms = (mn == kNegInf) ? 0.f : mn;
      const float alpha = fast_exp2(m[g] - ms);
      float p[NL];
      float ls = 0.f;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        p[i] = fast_exp2(sc[g][i] - ms);
        ls += p[i];
      }
      l[g] = l[g] * alpha + ls;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[g][e] *= alpha;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        if constexpr (GT == 1) {
          float f[E];
          v_to_float<CK>(vr[i], f);
#pragma unroll
          for (int e = 0; e < E; ++e) acc[g][e] = __builtin_fmaf(p[i], f[e], acc[g][e]);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) acc[g][e] = __builtin_fmaf(p[i], vf[i][e], acc[g][e]);
        }
      }
      m[g] = mn;
    }
  };

  stream_blocks<kRing, Tile>(wave, kWaves, nblk, load_tile, process);

  // Merge the RPL lane groups of this wave (they saw disjoint tokens).
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    float mw = m[g];
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) mw = fmaxf(mw, __shfl_xor(mw, off, 64));
    const float f = fast_exp2(m[g] - ((mw == kNegInf) ? 0.f : mw));
    float lw = l[g] * f;
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) lw += __shfl_xor(lw, off, 64);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float t = acc[g][e] * f;
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) t += __shfl_xor(t, off, 64);
      acc[g][e] = t;
    }
    m[g] = mw;
    l[g] = lw;
  }
  if (row == 0) {
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int e = 0; e < E; ++e) s_acc[wave][g][col * E + e] = acc[g][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      s_ml[wave][g][0] = m[g];
      s_ml[wave][g][1] = l[g];
    }
  }
  __syncthreads();

  finish_partition<GT, D>(a, &s_acc[0][0][0], &s_ml[0][0][0], seq, h0, part, seq_parts, tid);
}

// Grouped-query decode for tiles of 4 or 8 query heads with 16-bit queries.
//
// Lane l holds 16 bytes of row r = l % RPL of every wave-load (rows i*RPL + r),
// at column slice c = l / RPL, so the LPR lanes sharing a row are spread over
// the high lane bits. The GT*NL partial q·k sums of a lane are reduced over
// those bits with two transposing swap steps (bits 5 and 4), which leave each
// lane the sums of GT/4 heads, and DPP rotations for the remaining bits. The
// online softmax then runs once per (row, head) instead of once per lane, with
// the running max moved only when a block's max exceeds it by more than
// kRescaleSlack (weights stay below 2^kRescaleSlack, so float32 is safe). The
// weights reach the lanes that hold V through a small per-wave LDS buffer.
constexpr float kRescaleSlack = 8.0f;

template <int QK, int CK, int D, int GT>
__global__ __launch_bounds__(kThreads) void decode_gqa(const DecodeArgs a) {
  using Geo = TileGeo<CK, D>;
  constexpr int E = Geo::E, RPL = Geo::RPL, NL = Geo::NL;
  constexpr int KW = kKWords<QK, CK>;  // q/K words per lane-load (16-bit pairs)
  constexpr int kRowBits = RPL == 4 ? 2 : RPL == 8 ? 3 : 4;
  constexpr int V0 = GT * NL;          // partial sums per lane per block
  constexpr int HL = GT / 4;           // heads per lane after the swaps
  constexpr int kQBytes = 2;
  constexpr int kTileBytes = 16 * D * Geo::kBytes;
  static_assert(GT == 4 || GT == 8, "GQA tile of 4 or 8 heads");
  static_assert(QK == kF16 || QK == kBF16, "16-bit queries");
  static_assert(KW * 2 == E, "q slice matches the K slice");

  __shared__ int s_blocks[kMaxPartitionBlocks];
  __shared__ float s_p[kWaves][RPL][NL][GT];
  __shared__ float s_alpha[kWaves][RPL][GT];
  __shared__ float s_rowml[kWaves][RPL][GT][2];
  __shared__ float s_acc[kWaves][GT][D];
  __shared__ float s_ml[kWaves][GT][2];

  const int n_sub = a.group / GT;
  const int kvh = blockIdx.x / n_sub;
  const int h0 = kvh * a.group + (blockIdx.x - kvh * n_sub) * GT;
  const int part = blockIdx.y;
  const int seq = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int ctx = context_len(a, seq);
  if (ctx <= 0) {
    write_zeros<GT, D>(a, seq, h0, part, tid);
    return;
  }
  const int seq_blocks = (ctx + 15) >> 4;
  const int blk0 = part * a.partition_blocks;
  if (blk0 >= seq_blocks) return;
  const int nblk = min(a.partition_blocks, seq_blocks - blk0);
  const int seq_parts = (seq_blocks + a.partition_blocks - 1) / a.partition_blocks;

  const int32_t* bt = a.block_tables + (int64_t)seq * a.max_blocks + blk0;
  for (int j = tid; j < nblk; j += kThreads) s_blocks[j] = bt[j];

  const int r = lane & (RPL - 1);      // row of each wave-load
  const int c = lane >> kRowBits;      // column slice
  const int hq = lane >> 4;            // head quarter kept through the swaps
  // One lane per (row, head quarter) publishes to LDS: the remaining column
  // bits below bit 4 hold copies.
  const bool writer = ((lane >> kRowBits) & ((1 << (4 - kRowBits)) - 1)) == 0;

  uint32_t qf[GT][KW];
  {
    const char* qp = static_cast<const char*>(a.q) + (((int64_t)seq * a.num_heads + h0) * D + c * E) * kQBytes;
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int w = 0; w < KW / 4; ++w) {
        const uint4 v = *reinterpret_cast<const uint4*>(qp + g * D * kQBytes + w * 16);
        qf[g][4 * w] = v.x;
        qf[g][4 * w + 1] = v.y;
        qf[g][4 * w + 2] = v.z;
        qf[g][4 * w + 3] = v.w;
      }
  }
  __syncthreads();

  float acc[GT][E];
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
  float mref[HL], lsum[HL];
#pragma unroll
  for (int jj = 0; jj < HL; ++jj) {
    mref[jj] = kNegInf;
    lsum[jj] = 0.f;
  }

  const int64_t blk_stride = (int64_t)a.num_kv_heads * kTileBytes;
  const char* kbase = static_cast<const char*>(a.k_cache) + (int64_t)kvh * kTileBytes;
  const char* vbase = static_cast<const char*>(a.v_cache) + (int64_t)kvh * kTileBytes;
  const int lane_off = r * (D * Geo::kBytes) + c * 16;
  const float qk_scale = a.qk_scale;

  struct Tile {
    uint4 k[NL], v[NL];
  };
  auto load_tile = [&](int j, Tile& t) {
    uint4(&kr)[NL] = t.k;
    uint4(&vr)[NL] = t.v;
    const int64_t off = pool_block(a, s_blocks, j) * blk_stride;
    const char* kt = kbase + off;
    const char* vt = vbase + off;
#pragma unroll
    for (int i = 0; i < NL; ++i) kr[i] = load_stream(kt + lane_off + i * 1024);
#pragma unroll
    for (int i = 0; i < NL; ++i) vr[i] = load_stream(vt + lane_off + i * 1024);
  };

  // kMasked: the block holds rows past the context (the last, partial block
  // of a sequence); only that instantiation pays for the selects.
  auto process = [&](auto masked, int j, const Tile& t) {
    constexpr bool kMasked = decltype(masked)::value;
    const uint4(&kr)[NL] = t.k;
    const uint4(&vin)[NL] = t.v;
    float x[V0];  // x[g*NL + i] = partial q_g . k_(i*RPL + r) over this lane's slice
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      uint32_t kw[KW];
      k_words<QK, CK>(kr[i], kw);
#pragma unroll
      for (int g = 0; g < GT; ++g) x[g * NL + i] = dot_words<QK, KW>(qf[g], kw);
    }
    float y[V0 / 2];
#pragma unroll
    for (int k = 0; k < V0 / 2; ++k) y[k] = swap_sum32(x[k], x[k + V0 / 2]);
    float z[V0 / 4];  // z[jj*NL + i]: head hq*HL + jj, token i*RPL + r
#pragma unroll
    for (int k = 0; k < V0 / 4; ++k) {
      float t = swap_sum16(y[k], y[k + V0 / 4]);
      if constexpr (RPL <= 8) t += dpp<kDppRowRor8>(t);
      if constexpr (RPL == 4) t += dpp<kDppRowRor4>(t);
      z[k] = t * qk_scale;
    }
    uint4 vr[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) vr[i] = vin[i];
    if constexpr (kMasked) {  // last, partial block: drop rows past the context
      const int tok0 = (blk0 + j) * 16;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const bool ok = tok0 + i * RPL + r < ctx;
#pragma unroll
        for (int jj = 0; jj < HL; ++jj) z[jj * NL + i] = ok ? z[jj * NL + i] : kNegInf;
        vr[i].x = ok ? vr[i].x : 0u;
        vr[i].y = ok ? vr[i].y : 0u;
        vr[i].z = ok ? vr[i].z : 0u;
        vr[i].w = ok ? vr[i].w : 0u;
      }
    }
    float bm[HL];
    bool need = false;
#pragma unroll
    for (int jj = 0; jj < HL; ++jj) {
      bm[jj] = z[jj * NL];
#pragma unroll
      for (int i = 1; i < NL; ++i) bm[jj] = fmaxf(bm[jj], z[jj * NL + i]);
      need |= bm[jj] > mref[jj] + kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(need) != 0) {  // move the reference max (wave-uniform branch)
#pragma unroll
      for (int jj = 0; jj < HL; ++jj) {
        const float mn = fmaxf(mref[jj], bm[jj]);
        const float al = fast_exp2(mref[jj] - ((mn == kNegInf) ? 0.f : mn));
        lsum[jj] *= al;
        mref[jj] = mn;
        if (writer) s_alpha[wave][r][hq * HL + jj] = al;
      }
      wave_lds_fence();
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        const float al = s_alpha[wave][r][g];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[g][e] *= al;
      }
    }
#pragma unroll
    for (int jj = 0; jj < HL; ++jj) {
      const float ms = (mref[jj] == kNegInf) ? 0.f : mref[jj];
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const float pv = fast_exp2(z[jj * NL + i] - ms);
        lsum[jj] += pv;
        if (writer) s_p[wave][r][i][hq * HL + jj] = pv;
      }
    }
    wave_lds_fence();
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float vf[E];
      v_to_float<CK>(vr[i], vf);
      float pg[GT];
#pragma unroll
      for (int g = 0; g < GT; ++g) pg[g] = s_p[wave][r][i][g];
#pragma unroll
      for (int g = 0; g < GT; ++g)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[g][e] = __builtin_fmaf(pg[g], vf[e], acc[g][e]);
    }
  };

  // Partition-relative index of the block holding rows past the context, if any.
  const int masked_j = (ctx & 15) && blk0 + nblk == seq_blocks ? nblk - 1 : -1;
  stream_blocks<kRing, Tile>(wave, kWaves, nblk, load_tile, [&](int j, const Tile& t) {
    if (j != masked_j)
      process(std::false_type{}, j, t);
    else
      process(std::true_type{}, j, t);
  });

  // Merge the RPL rows of this wave: publish each (row, head) max and sum,
  // rescale the accumulators to the wave's max, then sum over the row lanes.
  if (writer) {
#pragma unroll
    for (int jj = 0; jj < HL; ++jj) {
      s_rowml[wave][r][hq * HL + jj][0] = mref[jj];
      s_rowml[wave][r][hq * HL + jj][1] = lsum[jj];
    }
  }
  wave_lds_fence();
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    float mw = kNegInf;
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr) mw = fmaxf(mw, s_rowml[wave][rr][g][0]);
    const float mws = (mw == kNegInf) ? 0.f : mw;
    const float f = fast_exp2(s_rowml[wave][r][g][0] - mws);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float t = acc[g][e] * f;
      t += dpp<kDppQuadXor1>(t);
      t += dpp<kDppQuadXor2>(t);
      if constexpr (RPL >= 8) t += dpp<kDppRowHalfMirror>(t);
      if constexpr (RPL >= 16) t += dpp<kDppRowMirror>(t);
      acc[g][e] = t;
    }
    if (lane == 0) {
      float lw = 0.f;
#pragma unroll
      for (int rr = 0; rr < RPL; ++rr) lw += s_rowml[wave][rr][g][1] * fast_exp2(s_rowml[wave][rr][g][0] - mws);
      s_ml[wave][g][0] = mw;
      s_ml[wave][g][1] = lw;
    }
  }
  if (r == 0) {
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int e = 0; e < E; ++e) s_acc[wave][g][c * E + e] = acc[g][e];
  }
  __syncthreads();
  finish_partition<GT, D>(a, &s_acc[0][0][0], &s_ml[0][0][0], seq, h0, part, seq_parts, tid);
}

// Merge the partitions of every (sequence, head) whose context spans several:
// up to 64 partitions in one or two rounds of 16-byte loads (below), more one
// partition at a time. The merge order is fixed: deterministic.
template <int D>
__global__ __launch_bounds__(64) void decode_reduce(const DecodeArgs a) {
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int lane = threadIdx.x;
  const int ctx = context_len(a, seq);
  const int seq_parts = (((ctx + 15) >> 4) + a.partition_blocks - 1) / a.partition_blocks;
  if (seq_parts <= 1) return;  // written directly by the decode kernel
  const int64_t base = ((int64_t)seq * a.num_heads + h) * a.num_parts;
  const float* ml = a.ws_ml + 2 * base;
  const float* o = a.ws_out + base * D;
  const int64_t sh = (int64_t)seq * a.num_heads + h;
  if (seq_parts <= 64) {
    // Lane p holds partition p's (max, sum); the outputs are read as 16-byte
    // chunks, PPI partitions per wave instruction (lane (c, sp) takes chunk c
    // of partition PPI * j + sp), 4 or 16 instructions in flight at a time, so
    // that 64 partitions take two rounds of loads rather than one per
    // partition; lanes holding the same chunk then add up by shuffles.
    constexpr int CH = D / 4;       // 16-byte chunks per output row
    constexpr int PPI = 64 / CH;    // partitions per wave instruction
    const int c = lane % CH, sp = lane / CH;
    const bool mine = lane < seq_parts;
    const float2 mlv = mine ? *reinterpret_cast<const float2*>(ml + 2 * lane) : make_float2(kNegInf, 0.f);
    float M = mlv.x;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    const float f = mine ? fast_exp2(mlv.x - M) : 0.f;
    float L = mlv.y * f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off, 64);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const int nj = (seq_parts + PPI - 1) / PPI;  // instructions needed
    // Rounds of K instructions in flight: 4 when that covers every partition
    // (the common few-partition case issues no idle loads), else 16.
    auto rounds = [&](auto k_c) {
      constexpr int K = decltype(k_c)::value;
      for (int j0 = 0; j0 < nj; j0 += K) {
        float4 v[K];
        float w[K];
#pragma unroll
        for (int u = 0; u < K; ++u) {
          const int p = PPI * (j0 + u) + sp;
          const int pc = p < seq_parts ? p : 0;  // past the last partition: a valid row, weight 0
          v[u] = *reinterpret_cast<const float4*>(o + (int64_t)pc * D + 4 * c);
          w[u] = __shfl(f, pc, 64) * (p < seq_parts ? 1.f : 0.f);
        }
#pragma unroll
        for (int u = 0; u < K; ++u) {
          acc.x += v[u].x * w[u];
          acc.y += v[u].y * w[u];
          acc.z += v[u].z * w[u];
          acc.w += v[u].w * w[u];
        }
      }
    };
    if (nj <= 4) rounds(std::integral_constant<int, 4>{});
    else rounds(std::integral_constant<int, 16>{});
#pragma unroll
    for (int off = CH; off < 64; off <<= 1) {
      acc.x += __shfl_xor(acc.x, off, 64);
      acc.y += __shfl_xor(acc.y, off, 64);
      acc.z += __shfl_xor(acc.z, off, 64);
      acc.w += __shfl_xor(acc.w, off, 64);
    }
    if (sp == 0) {
      const float inv = 1.f / L;
      store_out4(a, sh * D + 4 * c, make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv));
    }
    return;
  }
  float O[D / 64];
#pragma unroll
  for (int k = 0; k < D / 64; ++k) O[k] = 0.f;
  float M = kNegInf, L = 0.f;
  for (int p = 0; p < seq_parts; ++p) M = fmaxf(M, ml[2 * p]);
  for (int p = 0; p < seq_parts; ++p) {
    const float f = fast_exp2(ml[2 * p] - M);
    L += ml[2 * p + 1] * f;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) O[k] += o[(int64_t)p * D + lane + 64 * k] * f;
  }
#pragma unroll
  for (int k = 0; k < D / 64; ++k) store_out(a, sh * D + lane + 64 * k, O[k] / L);
}

// Merge the pieces of every (sequence, head) that the balanced schedule of
// the matrix-core kernel cut: ranges r_lo .. r_hi (those of them that hold
// any block) each left one piece in slot seq + r. With the shared-prefix
// pass, a sequence inside a group also has one part per a.prefix_part_blocks
// shared blocks, merged in after the pieces. Sequences held by a single
// range and outside every group were written by the kernel itself; empty
// ones get zeros here.
template <int D>
__global__ __launch_bounds__(64) void decode_bal_reduce(const DecodeArgs a) {
  __shared__ float s_f[64];
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int lane = threadIdx.x;
  const int ps = a.ws_pref[seq];
  const int pe = a.ws_pref[seq + 1];
  const int64_t T = a.ws_pref[a.num_seqs];
  const int64_t sh = (int64_t)seq * a.num_heads + h;
  const int shb = a.shared_prefix ? a.ws_shared[seq] : 0;  // shared blocks, merged from the prefix pass
  // The prefix pass's first part (its only one for prefixes of at most
  // a.prefix_part_blocks blocks), loaded in the same round as the indices above
  // (its address does not depend on them; the slot exists for every sequence).
  float pm0 = kNegInf, pl0 = 0.f, po0[D / 64];
  if (a.shared_prefix) {
    const int64_t p0 = ((int64_t)h * a.num_seqs + seq) * a.prefix_parts;
    pm0 = a.ws_sh_ml[2 * p0];
    pl0 = a.ws_sh_ml[2 * p0 + 1];
#pragma unroll
    for (int k = 0; k < D / 64; ++k) po0[k] = a.ws_sh_out[p0 * D + lane + 64 * k];
  }
  if (ps >= pe && shb <= 0) {
#pragma unroll
    for (int k = 0; k < D / 64; ++k) store_out(a, sh * D + lane + 64 * k, 0.f);
    return;
  }
  // Range r holds positions [floor(r T / R), floor((r + 1) T / R)); r_lo and
  // r_hi are the last ranges starting at or before the first and the last
  // block of the sequence.
  const int64_t R = a.ranges;
  int r_lo = 0, pieces = 0;
  if (ps < pe) {
    r_lo = (int)(((int64_t)(ps + 1) * R + T - 1) / T) - 1;
    const int r_hi = (int)(((int64_t)pe * R + T - 1) / T) - 1;
    pieces = r_hi - r_lo + 1;
  }
  if (pieces <= 1 && shb <= 0) return;
  const int64_t slots = (int64_t)a.num_seqs + R;
  const float* ml = a.ws_ml + ((int64_t)h * slots + seq + r_lo) * 2;
  const float* o = a.ws_out + ((int64_t)h * slots + seq + r_lo) * D;
  auto held = [&](int i) { return (int64_t)(r_lo + i) * T / R < (int64_t)(r_lo + i + 1) * T / R; };
  float O[D / 64];
#pragma unroll
  for (int k = 0; k < D / 64; ++k) O[k] = 0.f;
  float M = kNegInf, L = 0.f;
  if (pieces == 0) {
    // Nothing past the shared prefix.
  } else if (pieces <= 64) {
    // Common case, one round of loads: lane i takes piece i's max and sum,
    // every lane its columns of the first kPre pieces' outputs; the weights
    // are then shared by lane reads.
    constexpr int kPre = 16;
    float ov[kPre][D / 64];
#pragma unroll
    for (int j = 0; j < kPre; ++j)
#pragma unroll
      for (int k = 0; k < D / 64; ++k) ov[j][k] = j < pieces ? o[(int64_t)j * D + lane + 64 * k] : 0.f;
    const bool mine = lane < pieces && held(lane);
    const float m = mine ? ml[2 * lane] : kNegInf;
    const float l = mine ? ml[2 * lane + 1] : 0.f;
    M = m;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    const float f = mine ? fast_exp2(m - M) : 0.f;
    L = l * f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off, 64);
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
      const float fj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), j));
#pragma unroll
      for (int k = 0; k < D / 64; ++k) O[k] += fj != 0.f ? ov[j][k] * fj : 0.f;
    }
#pragma unroll 4
    for (int j = kPre; j < pieces; ++j) {
      const float fj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), j));
#pragma unroll
      for (int k = 0; k < D / 64; ++k) {
        const float v = o[(int64_t)j * D + lane + 64 * k];
        O[k] += fj != 0.f ? v * fj : 0.f;
      }
    }
  } else {
    // Maxima and sums with the lanes across the pieces.
    for (int i = lane; i < pieces; i += 64)
      if (held(i)) M = fmaxf(M, ml[2 * i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    for (int i = lane; i < pieces; i += 64)
      if (held(i)) L += ml[2 * i + 1] * fast_exp2(ml[2 * i] - M);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off, 64);
    // Outputs: 64 pieces at a time, their weights staged in LDS (0 for ranges
    // that hold no block; their slots were never written and are skipped by
    // selection, not multiplied).
    for (int base = 0; base < pieces; base += 64) {
      const int i = base + lane;
      wave_lds_fence();
      s_f[lane] = (i < pieces && held(i)) ? fast_exp2(ml[2 * i] - M) : 0.f;
      wave_lds_fence();
      const int n = min(64, pieces - base);
#pragma unroll 8
      for (int j = 0; j < n; ++j) {
        const float f = s_f[j];
#pragma unroll
        for (int k = 0; k < D / 64; ++k) {
          const float v = o[(int64_t)(base + j) * D + lane + 64 * k];
          O[k] += f != 0.f ? v * f : 0.f;
        }
      }
    }
  }
  if (shb > 0) {
    // The prefix pass's parts: rescale what the pieces gave to the joint max.
    const int np = (shb + a.prefix_part_blocks - 1) / a.prefix_part_blocks;
    const int64_t p0 = ((int64_t)h * a.num_seqs + seq) * a.prefix_parts;
    const float* pml = a.ws_sh_ml + 2 * p0;
    const float* po = a.ws_sh_out + p0 * D;
    float Mp = pm0;
    for (int i = 1 + lane; i < np; i += 64) Mp = fmaxf(Mp, pml[2 * i]);
    if (np > 1) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) Mp = fmaxf(Mp, __shfl_xor(Mp, off, 64));
    }
    const float Mn = fmaxf(M, Mp);
    const float fo = M == kNegInf ? 0.f : fast_exp2(M - Mn);
    L *= fo;
    const float f0 = fast_exp2(pm0 - Mn);
    L += pl0 * f0;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) O[k] = O[k] * fo + po0[k] * f0;
    for (int i = 1; i < np; ++i) {
      const float f = fast_exp2(pml[2 * i] - Mn);
      L += pml[2 * i + 1] * f;
#pragma unroll
      for (int k = 0; k < D / 64; ++k) O[k] += po[(int64_t)i * D + lane + 64 * k] * f;
    }
  }
#pragma unroll
  for (int k = 0; k < D / 64; ++k) store_out(a, sh * D + lane + 64 * k, O[k] / L);
}

template <int QK, int CK, int D, int GT>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.num_kv_heads * (a.group / GT)), (unsigned)a.num_parts, (unsigned)a.num_seqs);
  if constexpr (GT >= 4 && QK != kF32)
    decode_gqa<QK, CK, D, GT><<<grid, dim3(kThreads), 0, stream>>>(a);
  else if constexpr (GT == 1)
    if (a.cached_loads)
      decode_main<QK, CK, D, GT, true><<<grid, dim3(kThreads), 0, stream>>>(a);
    else
      decode_main<QK, CK, D, GT><<<grid, dim3(kThreads), 0, stream>>>(a);
  else
    decode_main<QK, CK, D, GT><<<grid, dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

template <int QK, int CK, int D>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  switch (a.group_tile) {
    case 1: return launch_t<QK, CK, D, 1>(a, stream);
    case 2: return launch_t<QK, CK, D, 2>(a, stream);
    case 4: return launch_t<QK, CK, D, 4>(a, stream);
    case 8: return launch_t<QK, CK, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int QK, int CK>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  switch (a.head_size) {
    case 64: return launch_g<QK, CK, 64>(a, stream);
    case 128: return launch_g<QK, CK, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int q_kind, int cache_kind, hipStream_t stream) {
  hipError_t e;
  if (a.shared_prefix) {
    e = launch_decode_prefix(a, q_kind, cache_kind, stream);
    if (e != hipSuccess) return e;
  }
  if (a.use_mfma) {
    e = launch_decode_mfma(a, q_kind, cache_kind, stream);
  } else {
    switch (q_kind * 4 + cache_kind) {
      case kF32 * 4 + kF32: e = launch_d<kF32, kF32>(a, stream); break;
      case kF16 * 4 + kF16: e = launch_d<kF16, kF16>(a, stream); break;
      case kBF16 * 4 + kBF16: e = launch_d<kBF16, kBF16>(a, stream); break;
      case kF16 * 4 + kFP8: e = launch_d<kF16, kFP8>(a, stream); break;
      case kBF16 * 4 + kFP8: e = launch_d<kBF16, kFP8>(a, stream); break;
      default: return hipErrorInvalidValue;
    }
  }
  if (e != hipSuccess) return e;
  if (a.balanced) {
    const dim3 grid((unsigned)a.num_heads, (unsigned)a.num_seqs);
    switch (a.head_size) {
      case 64: decode_bal_reduce<64><<<grid, dim3(64), 0, stream>>>(a); break;
      case 128: decode_bal_reduce<128><<<grid, dim3(64), 0, stream>>>(a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (a.num_parts == 1) return e;
  return launch_decode_reduce(a, stream);
}

hipError_t launch_decode_reduce(const DecodeArgs& a, hipStream_t stream) {
  switch (a.head_size) {
    case 64: decode_reduce<64><<<dim3((unsigned)a.num_heads, (unsigned)a.num_seqs), dim3(64), 0, stream>>>(a); break;
    case 128: decode_reduce<128><<<dim3((unsigned)a.num_heads, (unsigned)a.num_seqs), dim3(64), 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
