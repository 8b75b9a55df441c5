// Chunked-prefill attention over the paged cache, on the gfx950 matrix cores.
//
// What is computed ("vLLM 前世今生" §5.4 and §7.3, chunked prefill; §3.2, the
// paged cache): a sequence's chunk of q_len new query tokens, the last q_len
// of its context_len tokens (whose K/V are already in the cache), attends
// causally: query i of the chunk, at position p = context_len - q_len + i,
// sees the tokens 0..p, reached through the sequence's block table. Per query
// head: softmax(q·Kᵀ·scale)·V over those tokens.
//
// How: this is the dense, compute-bound side of paged attention, so it runs
// as MFMA tiles, flash-attention style (online softmax over key blocks):
//  * the (token, head) pairs of one KV head form the rows of the problem;
//    a workgroup of 8 waves takes kPrefillRows = 128 consecutive rows (row =
//    token * G + head within the group, so grouped heads share every K/V
//    tile), one 16-row tile per wave (two tiles per wave measured no faster:
//    the cost per block is not the LDS reads);
//  * the workgroup streams the sequence's 16-token blocks, two per step, up
//    to the last position among its rows. Each block's K and V tile is loaded
//    once, by all eight waves together, into double-buffered LDS (rows padded
//    by 16 bytes against bank conflicts; FP8 widened exactly to the 16-bit
//    type), while the waves compute on the previous step;
//  * per wave and step, S = K·Qᵀ is 16x16x32 MFMAs on K read from LDS in the
//    A-operand layout; the lane layout of S is the A-operand layout of P, so
//    the online softmax (a lazily moved per-row reference max) runs in place;
//    O += P·V is one 16x16x32 MFMA per 16 output columns and P part (P split
//    into 16-bit hi + lo), its 32 keys being this lane group's four rows of
//    each of the two blocks, matched by two transposed reads of V from LDS
//    (on gfx950 the 16x16x32 form issues in the same time as 16x16x16);
//  * causality is a per-row limit on the key index, applied by selection; a
//    wave whose rows all end before a block skips its arithmetic.
// No split over keys is done for prefill: a chunk's rows already give many
// workgroups.
//
// Decode mode (groups of 32 and more query heads per KV head, "vLLM" note,
// section "内核优化": MQA / GQA kernels): the rows are the G query heads of one
// sequence's single query over one KV head, so every K/V tile loaded into LDS
// serves all of them; with one wave per 16 or 32 heads reading the tile for
// itself, each byte would be requested G/16 or G/32 times. The workgroup
// follows G (2 or 4 waves of 16 heads; from 128 heads on, 4 waves of two
// 16-head tiles), and a long context is split into partitions whose partial
// results decode_reduce merges.
#include "pa_decode_common.h"
#include "pa_mfma.h"

namespace pa {
namespace {

// Waves per workgroup for prefill: eight, each with one 16-row tile, so every
// K/V tile staged in LDS serves 128 rows (measured: 4 waves 392 TFLOP/s, 8
// waves 425, 16 waves 286 on 8 x 2048-token GQA prompts). Decode mode takes
// 2, 4 or 8 waves, one per 16 heads of the group.
constexpr int kPrefillWaves = kPrefillRows / 16;
constexpr int kSB = 2;                              // blocks per step (the P·V operands below pair two)
static_assert(kSB == 2, "one 16x16x32 P·V product spans two blocks");
constexpr float kPSlack = 8.0f;

template <int CK, int D, int PW> struct PGeo {
  static constexpr int kBytes = KindBytes<CK>::value;
  static constexpr int kRowBytes = D * kBytes;
  static constexpr int kTileBytes = 16 * kRowBytes;
  static constexpr int NL = kTileBytes / 1024;       // wave-loads of 1 KiB per tile (K or V)
  static constexpr int NLW = (2 * NL + PW - 1) / PW;  // loads per wave per block (K and V together)
  static constexpr int NKB = D / 32;
  static constexpr int NDB = D / 16;
  // LDS row strides of the staged tiles, 16-bit elements. K rows are read
  // 16 bytes per lane down 16 rows, V rows back transposed, 8 bytes per lane
  // from 4 rows x 4 column pairs. Both take a stride of 8 (mod 64) dwords,
  // the one measured free of bank conflicts for both reads (SQ_LDS_BANK_CONFLICT
  // 0 on the 8 x 2048 GQA prefill; a K stride of 4 (mod 64) dwords conflicted
  // on 1.2 cycles per LDS instruction, an unpadded one on 8.5).
  static constexpr int S = D + 16;   // K
  static constexpr int SV = D + 16;  // V
};

template <int QK, int CK, int D, int PW, int kRT = 1>
__global__ __launch_bounds__(64 * PW) void prefill_mfma(const PrefillArgs a) {
  using G = PGeo<CK, D, PW>;
  constexpr int NL = G::NL, NLW = G::NLW, NKB = G::NKB, NDB = G::NDB, S = G::S, SV = G::SV;
  constexpr int kRows = 16 * kRT * PW;  // rows per workgroup (kRT 16-row tiles per wave)
  static_assert(QK == kF16 || QK == kBF16, "16-bit queries");
  static_assert(PW == 2 || PW == 4 || PW == 8, "2, 4 or 8 waves");
  static_assert(kRT == 1 || kRT == 2, "one or two 16-row tiles per wave");

  __shared__ __align__(16) uint16_t s_k[2][kSB][16 * S];
  __shared__ __align__(16) uint16_t s_v[2][kSB][16 * SV];

  const int kvh = blockIdx.x / a.row_tiles;
  // Causal prefill: later rows see more keys, so the row tiles are dispatched
  // last-first (the longest workgroups start earliest).
  const int rt = a.decode ? blockIdx.x - kvh * a.row_tiles : a.row_tiles - 1 - (blockIdx.x - kvh * a.row_tiles);
  const int seq = blockIdx.y;
  const int part = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;

  const int ctx = min(a.context_lens[seq], a.max_blocks * 16);
  // Prefill: the chunk is positions ctx - qlen .. ctx - 1. Decode: one query, row seq of q.
  const int q0 = a.decode ? seq : a.query_start_loc[seq];
  const int qlen = a.decode ? (ctx > 0 ? 1 : 0) : min(a.query_start_loc[seq + 1] - q0, ctx);
  const int rows = min(qlen, a.max_query_len) * a.group;        // rows computed (the grid covers max_query_len)
  const int row0 = rt * kRows;
  if (a.decode && ctx <= 0) {  // nothing to attend: zeros (written once, by partition 0)
    if (part == 0)
      for (int idx = tid; idx < kRows * D; idx += 64 * PW) {
        const int r = row0 + idx / D;
        if (r < a.group) {
          const int64_t e = ((int64_t)seq * a.num_heads + kvh * a.group + r) * D + idx % D;
          if (a.out_kind == kF32) static_cast<float*>(a.out)[e] = 0.f;
          else static_cast<uint16_t*>(a.out)[e] = 0;
        }
      }
    return;
  }
  if (row0 >= rows) return;
  const int last_row = min(row0 + kRows, rows) - 1;
  const int nblk_all = (ctx - qlen + last_row / a.group + 1 + 15) >> 4;  // blocks up to the last row's position
  // Decode partitions: blocks [blk0, nblk) of the context (the whole of it when not split).
  const int blk0 = a.part_blocks ? part * a.part_blocks : 0;
  const int nblk = a.part_blocks ? min(nblk_all, blk0 + a.part_blocks) : nblk_all;
  if (blk0 >= nblk) return;
  const int seq_parts = a.part_blocks ? (nblk_all + a.part_blocks - 1) / a.part_blocks : 1;

  // This lane's S columns: row n of each of the wave's 16-row tiles.
  const int wrow0 = row0 + wave * 16 * kRT;
  int my_limit[kRT];  // keys visible to the row (0 for rows past the chunk)
  uint32_t qf[kRT][NKB][4];
#pragma unroll
  for (int t = 0; t < kRT; ++t) {
    const int r = wrow0 + t * 16 + n;
    const bool ok = r < rows;
    const int tok = ok ? r / a.group : 0;
    const int head = kvh * a.group + (ok ? r - tok * a.group : 0);
    my_limit[t] = ok ? ctx - qlen + tok + 1 : 0;
    const char* qp = static_cast<const char*>(a.q) + ((int64_t)(q0 + tok) * a.num_heads + head) * D * 2;
#pragma unroll
    for (int b = 0; b < NKB; ++b) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (ok) v = *reinterpret_cast<const uint4*>(qp + (32 * b + 8 * g) * 2);
      qf[t][b][0] = v.x;
      qf[t][b][1] = v.y;
      qf[t][b][2] = v.z;
      qf[t][b][3] = v.w;
    }
  }
  // The wave's largest limit (its last valid row): blocks at or past it are
  // skipped. Its smallest (its first row): steps wholly below it need no mask.
  const int wave_last = min(wrow0 + 16 * kRT - 1, rows - 1);
  const int wave_limit = wrow0 < rows ? ctx - qlen + wave_last / a.group + 1 : 0;
  const int wave_first_limit = wrow0 < rows ? ctx - qlen + wrow0 / a.group + 1 : 0;
  // Scores are scaled inside the exponent, exp2(s * c - m), which needs c >= 0:
  // a negative scale is moved into q (its sign flipped, exactly), and a zero
  // one is raised to 1e-30 (weights then equal to within float32 rounding, and
  // -inf scores stay -inf).
  if (a.qk_scale < 0.f) {
#pragma unroll
    for (int t = 0; t < kRT; ++t)
#pragma unroll
      for (int b = 0; b < NKB; ++b)
#pragma unroll
        for (int w = 0; w < 4; ++w) qf[t][b][w] ^= 0x80008000u;
  }
  const float qk_c = fmaxf(fabsf(a.qk_scale), 1e-30f);

  const int32_t* bt = a.block_tables + (int64_t)seq * a.max_blocks;
  const int64_t blk_stride = (int64_t)a.num_kv_heads * G::kTileBytes;
  const char* kbase = static_cast<const char*>(a.k_cache) + (int64_t)kvh * G::kTileBytes;
  const char* vbase = static_cast<const char*>(a.v_cache) + (int64_t)kvh * G::kTileBytes;

  // The tiles of step j (blocks blk0 + kSB*j .. blk0 + kSB*j + kSB - 1), as this wave's
  // share of the 2*NL wave-loads per block (K first, then V), into register
  // buffer rb; loads run two steps ahead of the arithmetic. The loads are
  // unconditional, so that the compiler's wait before staging a step counts
  // the newer step's loads and leaves them in flight: a block past the last
  // one needed (its table entry may lie past the row) reloads the last
  // block, and is staged as zeros (its keys are beyond every row's limit).
  uint4 pre[2][kSB][NLW];
  auto issue = [&](int j, int rb) {
#pragma unroll
    for (int p = 0; p < kSB; ++p) {
      const int blk = min(blk0 + kSB * j + p, nblk - 1);
      // A scalar load (the table is read-only here): waiting for it does not
      // wait for the vector loads of the steps in flight.
      const int phys = ((const __attribute__((address_space(4))) int32_t*)bt)[blk];
      const int64_t off = ((uint32_t)phys < (uint64_t)a.num_blocks ? phys : 0) * blk_stride;
#pragma unroll
      for (int u = 0; u < NLW; ++u) {
        const int L = (wave & (PW - 1)) + u * PW;  // wave < PW, stated for the compiler
        if (L < 2 * NL) {
          const char* base = L < NL ? kbase : vbase;
          pre[rb][p][u] = load_stream(base + off + (L % NL) * 1024 + lane * 16);
        }
      }
    }
  };
  auto stage = [&](int j, int buf, int rb) {
#pragma unroll
    for (int p = 0; p < kSB; ++p) {
      const int blk = blk0 + kSB * j + p;
      // Blocks before the last needed one lie wholly inside the context and
      // are stored as loaded; the last one (rows past the context may hold
      // anything: V rows there become zero, as a zero weight times NaN would
      // still be NaN; K rows are masked later) and blocks not needed (zero
      // throughout) go through selection.
      const bool inside = blk + 1 < nblk;
#pragma unroll
      for (int u = 0; u < NLW; ++u) {
        const int L = (wave & (PW - 1)) + u * PW;  // wave < PW, stated for the compiler
        if (L < 2 * NL) {
          const bool is_v = L >= NL;
          const int byte = (L % NL) * 1024 + lane * 16;
          const int row = byte / G::kRowBytes;
          const int col = (byte % G::kRowBytes) / G::kBytes;
          uint16_t* dst = is_v ? s_v[buf][p] + row * SV + col : s_k[buf][p] + row * S + col;
          uint4 v = pre[rb][p][u];
          if (!inside) {
            const bool zero = blk >= nblk || (is_v && blk * 16 + row >= ctx);
            if (zero) v = make_uint4(0u, 0u, 0u, 0u);
          }
          if constexpr (CK == kFP8) {
            uint4 w0, w1;
            fp8x4_to_16<QK>(v.x, w0.x, w0.y);
            fp8x4_to_16<QK>(v.y, w0.z, w0.w);
            fp8x4_to_16<QK>(v.z, w1.x, w1.y);
            fp8x4_to_16<QK>(v.w, w1.z, w1.w);
            *reinterpret_cast<uint4*>(dst) = w0;
            *reinterpret_cast<uint4*>(dst + 8) = w1;
          } else {
            *reinterpret_cast<uint4*>(dst) = v;
          }
        }
      }
    }
  };

  f32x4_t acc[kRT][NDB];
#pragma unroll
  for (int t = 0; t < kRT; ++t)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[t][db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float mref[kRT], lsum[kRT];
#pragma unroll
  for (int t = 0; t < kRT; ++t) {
    mref[t] = kNegInf;
    lsum[t] = 0.f;
  }
  auto compute = [&](int j, int buf) {
    const int key0 = (blk0 + kSB * j) * 16;  // first key of the step
    if (key0 >= wave_limit) return;  // every row of this wave ends before this step
    f32x4_t s[kRT][kSB];
#pragma unroll
    for (int t = 0; t < kRT; ++t)
#pragma unroll
      for (int p = 0; p < kSB; ++p) s[t][p] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < kSB; ++p) {
      const uint16_t* sk = s_k[buf][p];
#pragma unroll
      for (int b = 0; b < NKB; ++b) {
        const uint4 kw = *reinterpret_cast<const uint4*>(sk + n * S + 32 * b + 8 * g);
        const uint32_t w[4] = {kw.x, kw.y, kw.z, kw.w};
#pragma unroll
        for (int t = 0; t < kRT; ++t) s[t][p] = mma_k32<QK>(w, qf[t][b], s[t][p]);
      }
    }
    uint32_t ph[kRT][kSB][2], pl[kRT][kSB][2];
    // Steps wholly below every row's limit need no mask (a wave-uniform choice).
    const bool full = key0 + kSB * 16 <= wave_first_limit;
#pragma unroll
    for (int t = 0; t < kRT; ++t) {
      float x[kSB][4];  // unscaled scores
      float bm = kNegInf;
      if (full) {
#pragma unroll
        for (int p = 0; p < kSB; ++p)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[p][i] = s[t][p][i];
            bm = fmaxf(bm, x[p][i]);
          }
      } else {
#pragma unroll
        for (int p = 0; p < kSB; ++p)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[p][i] = s[t][p][i];
            // causal limit (and rows past the chunk), by selection
            if (key0 + 16 * p + 4 * g + i >= my_limit[t]) x[p][i] = kNegInf;
            bm = fmaxf(bm, x[p][i]);
          }
      }
      bm *= qk_c;  // the step's largest logit (c >= 0 keeps the order)
      if (__builtin_amdgcn_ballot_w64(bm > mref[t] + kPSlack) != 0) {
        float bmx = fmaxf(bm, __shfl_xor(bm, 16, 64));
        bmx = fmaxf(bmx, __shfl_xor(bmx, 32, 64));
        const float mn = fmaxf(mref[t], bmx);
        const float alpha = fast_exp2(mref[t] - ((mn == kNegInf) ? 0.f : mn));
        lsum[t] *= alpha;
        mref[t] = mn;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float al = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
          for (int db = 0; db < NDB; ++db) acc[t][db][i] *= al;
        }
      }
      const float ms = (mref[t] == kNegInf) ? 0.f : mref[t];
#pragma unroll
      for (int p = 0; p < kSB; ++p) {
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[i] = fast_exp2(__builtin_fmaf(x[p][i], qk_c, -ms));
          lsum[t] += pr[i];
        }
        ph[t][p][0] = pack2<QK>(pr[0], pr[1]);
        ph[t][p][1] = pack2<QK>(pr[2], pr[3]);
        pl[t][p][0] = pack2<QK>(pr[0] - lo16_to_f32<QK>(ph[t][p][0]), pr[1] - hi16_to_f32<QK>(ph[t][p][0]));
        pl[t][p][1] = pack2<QK>(pr[2] - lo16_to_f32<QK>(ph[t][p][1]), pr[3] - hi16_to_f32<QK>(ph[t][p][1]));
      }
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const u32x2_t b0 = v_operand_tr(s_v[buf][0], SV, db * 16, lane);
      const u32x2_t b1 = v_operand_tr(s_v[buf][1], SV, db * 16, lane);
      const uint32_t b[4] = {b0[0], b0[1], b1[0], b1[1]};
#pragma unroll
      for (int t = 0; t < kRT; ++t) {
        const uint32_t ah[4] = {ph[t][0][0], ph[t][0][1], ph[t][1][0], ph[t][1][1]};
        const uint32_t al[4] = {pl[t][0][0], pl[t][0][1], pl[t][1][0], pl[t][1][1]};
        acc[t][db] = mma_k32<QK>(ah, b, acc[t][db]);
        acc[t][db] = mma_k32<QK>(al, b, acc[t][db]);
      }
    }
  };

  const int nsteps = (nblk - blk0 + kSB - 1) / kSB;
  issue(0, 0);
  issue(1, 1);
  __builtin_amdgcn_sched_barrier(0);
  stage(0, 0, 0);
  __syncthreads();
  // Two steps per iteration, so that both register buffers have fixed names
  // (an indexed choice between them made the compiler wait for every load).
  for (int j = 0; j < nsteps; j += 2) {
    issue(j + 2, 0);  // step j's registers were staged last iteration
    __builtin_amdgcn_sched_barrier(0);
    compute(j, 0);
    __builtin_amdgcn_sched_barrier(0);
    stage(j + 1, 1, 1);  // past the last step: zeros, unused
    __syncthreads();
    if (j + 1 >= nsteps) break;
    issue(j + 3, 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(j + 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    stage(j + 2, 0, 0);
    __syncthreads();
  }

  // Normalise and write this wave's rows: lane (n, g) holds rows 4g + i of
  // each tile, column 16 db + n. A partition of a split decode context
  // leaves its running max (log2 units), sum and unnormalised output instead.
#pragma unroll
  for (int t = 0; t < kRT; ++t) {
    float ls = lsum[t];
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    if (seq_parts > 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wrow0 + t * 16 + 4 * g + i;  // decode: the row is the head within the group
        const float L = __shfl(ls, 4 * g + i, 64);
        const float M = __shfl(mref[t], 4 * g + i, 64);
        if (r < rows) {
          const int64_t pi = ((int64_t)seq * a.num_heads + kvh * a.group + r) * a.num_parts + part;
#pragma unroll
          for (int db = 0; db < NDB; ++db) a.ws_out[pi * D + db * 16 + n] = acc[t][db][i] * a.out_scale;
          if (n == 0) {
            a.ws_ml[2 * pi] = M;
            a.ws_ml[2 * pi + 1] = L;
          }
        }
      }
      continue;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wrow0 + t * 16 + 4 * g + i;
      const float L = __shfl(ls, 4 * g + i, 64);
      if (r < rows) {
        const int tok = r / a.group;
        const int head = kvh * a.group + (r - tok * a.group);
        const int64_t base = ((int64_t)(q0 + tok) * a.num_heads + head) * D;
        const float inv = L > 0.f ? a.out_scale / L : 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int64_t e = base + db * 16 + n;
          const float v = acc[t][db][i] * inv;
          if (a.out_kind == kF32) static_cast<float*>(a.out)[e] = v;
          else if (a.out_kind == kBF16) static_cast<uint16_t*>(a.out)[e] = f32_to_bf16_rne(v);
          else static_cast<uint16_t*>(a.out)[e] = f32_to_f16_rne(v);
        }
      }
    }
  }
}

template <int QK, int CK, int D>
hipError_t launch_w(const PrefillArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.row_tiles * a.num_kv_heads), (unsigned)a.num_seqs,
                  (unsigned)(a.decode && a.part_blocks ? a.num_parts : 1));
  switch (a.waves * 10 + a.wave_tiles) {
    case 21: prefill_mfma<QK, CK, D, 2><<<grid, dim3(64 * 2), 0, stream>>>(a); break;
    case 41: prefill_mfma<QK, CK, D, 4><<<grid, dim3(64 * 4), 0, stream>>>(a); break;
    case 81: prefill_mfma<QK, CK, D, 8><<<grid, dim3(64 * 8), 0, stream>>>(a); break;
    case 42: prefill_mfma<QK, CK, D, 4, 2><<<grid, dim3(64 * 4), 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int QK, int CK>
hipError_t launch_d(const PrefillArgs& a, hipStream_t stream) {
  switch (a.head_size) {
    case 64: return launch_w<QK, CK, 64>(a, stream);
    case 128: return launch_w<QK, CK, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int q_kind, int cache_kind, hipStream_t stream) {
  switch (q_kind * 4 + cache_kind) {
    case kF16 * 4 + kF16: return launch_d<kF16, kF16>(a, stream);
    case kBF16 * 4 + kBF16: return launch_d<kBF16, kBF16>(a, stream);
    case kF16 * 4 + kFP8: return launch_d<kF16, kFP8>(a, stream);
    case kBF16 * 4 + kFP8: return launch_d<kBF16, kFP8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_wide(const PrefillArgs& a, int q_kind, int cache_kind, hipStream_t stream) {
  const hipError_t e = launch_prefill(a, q_kind, cache_kind, stream);
  if (e != hipSuccess || !a.part_blocks || a.num_parts <= 1) return e;
  // Merge the partitions (the decode path's merge kernel, same workspace layout).
  DecodeArgs r{};
  r.out = a.out;
  r.context_lens = a.context_lens;
  r.ws_out = a.ws_out;
  r.ws_ml = a.ws_ml;
  r.num_seqs = a.num_seqs;
  r.num_heads = a.num_heads;
  r.head_size = a.head_size;
  r.max_blocks = a.max_blocks;
  r.partition_blocks = a.part_blocks;
  r.num_parts = a.num_parts;
  r.out_kind = a.out_kind;
  return launch_decode_reduce(r, stream);
}

}  // namespace pa
