// Grouped-query paged decode on the gfx950 matrix cores, for 16-bit queries.
//
// Same result as the vector-ALU kernels in pa_decode.hip: softmax(q·Kᵀ·scale)·V
// per query head over the sequence's cached tokens, reached through its block
// table ("vLLM 前世今生" §3.2; "vLLM" note, sections "PagedAttention" and
// "内核优化", where a group of query heads shares one KV head).
//
// With GT query heads per KV head, one (block, KV head) tile of 16 tokens is a
// small dense contraction, not a matrix-vector product: S = K·Qᵀ is
// [16 tokens × D]·[D × GT heads] and O += P·V is [GT × 16]·[16 × D]. On the
// vector ALU these products cost about 600 instructions per tile at GT = 8,
// which leaves the kernel ALU-bound below the HBM roofline; here they are
// issued as MFMA instructions, and the vector ALU only runs the online softmax.
//
// Three modes share the per-block arithmetic below:
//  * partitioned: one workgroup of 4 waves per (sequence, KV head, head tile
//    of GT <= 16, partition), wave w taking blocks w, w+4, ... of the
//    partition, with the block-table slice staged in LDS; the waves merge
//    through LDS at the end;
//  * balanced (kBalanced): the blocks of all sequences are laid end to end
//    and cut into equal ranges, one per wave, whatever the context lengths;
//    each wave streams its range piece by piece (a piece is the part of one
//    sequence inside the range) and leaves each piece's partial result for
//    decode_bal_reduce, or writes a sequence it holds whole. GT may be 32
//    here: two 16-head sub-tiles per wave share every K/V block it loads.
//    With the shared-prefix pass (a.shared_prefix) each sequence's first
//    ws_shared[s] blocks are left out of the ranges: that pass read them.
//  * shared-prefix pass (kPrefix, GT = 16): the 16 columns of a tile are the
//    (sequence, head) pairs of 16 / group consecutive sequences of one group
//    that share their first blocks ("vLLM 前世今生" §3.2: a common prompt in
//    the same physical blocks), so every shared K/V tile is read and
//    multiplied once for all of them; workgroups are (KV head, part of
//    a.prefix_part_blocks shared blocks, tile) and leave per-part partial
//    results for decode_bal_reduce.
// In all, a wave keeps the next blocks' K/V loads in flight while it works.
//
//  * K is loaded straight from HBM in the MFMA A-operand layout: lane l reads
//    16 bytes of token l % 16 (64 contiguous bytes per token per instruction),
//    so S needs no data movement at all. The head dimension may be taken in
//    any order as long as q is read in the same order (a dot product does not
//    care), which lets FP8 rows be read 16 bytes at a time. S is 16×16×32
//    MFMAs.
//  * S comes out with lane l holding head l % 16 for tokens 4·(l/16) + i,
//    which is exactly the A-operand layout of P in O += P·V: the softmax runs
//    in place, per lane, with no shuffle of P.
//  * V must be read token-major per lane, so each wave stages its V tiles in
//    LDS (rows padded by 32 bytes against bank conflicts; FP8 widened to the
//    16-bit type on the way) and reads the B operand back transposed, one
//    ds_read_b64_tr_b16 per 16 columns and block.
//  * Blocks go two per step: O += P·V for the pair is one 16×16×32 MFMA per 16
//    columns (its 32 tokens are this lane group's four rows of each block),
//    which issues in the time of one 16×16×16 MFMA. A leftover block and the
//    masked tail block form a peeled last step (16×16×16 for a single block).
//  * P is rounded to the 16-bit type as hi + lo (two MFMAs per D-slice), so the
//    weights keep about 16 significant bits and the output stays within float32
//    accumulation error of the exact weights; V, K and q are exact in the
//    16-bit type (FP8 codes widen exactly).
//  * When a KV head has several head tiles (more query heads per KV head than
//    one wave takes), their workgroups read the same K/V. Then K/V are loaded
//    with the ordinary (cached) hint and the workgroups are renumbered so that
//    the tiles of one (sequence or range, KV head) get consecutive numbers on
//    the same XCD: the hardware hands workgroups to the 8 XCDs in turn, so
//    dispatch index i runs on XCD i mod 8, and the tiles that share data then
//    run side by side behind one L2. With a single tile per KV head nothing is
//    reused and the loads stay streaming (nontemporal), in launch order.
//  * The running max is moved lazily: only when a step's max exceeds it by
//    more than kSlack (log2 units) is it raised and the accumulators rescaled;
//    all weights stay below 2^kSlack, which float32 sums hold easily.
// Rows past the context get a -inf logit by selection and a zero V row, so
// stale or NaN data there never reaches the output.
#include <type_traits>

#include "pa_decode_common.h"
#include "pa_mfma.h"

namespace pa {
namespace {

constexpr float kSlack = 8.0f;    // lazy-max slack, log2 units
constexpr int kRing = 2;          // register ring depth: blocks per wave in flight, plus the one in use
constexpr int kRingBalanced = 2;  // the same for the balanced schedule
constexpr int kRingWide = 2;      // the same for 32-head tiles (one wave per SIMD)

// Geometry of one (block, KV head) tile for the MFMA kernel.
template <int CK, int D> struct MGeo {
  static constexpr int kBytes = KindBytes<CK>::value;
  static constexpr int kRowBytes = D * kBytes;
  static constexpr int kTileBytes = 16 * kRowBytes;
  static constexpr int NKB = D / 32;                      // 32-wide k blocks of S
  static constexpr int NKL = (CK == kFP8) ? D / 64 : D / 32;  // K loads per lane (16 bytes each)
  static constexpr int NVL = kTileBytes / 1024;           // V loads per lane (16 bytes each)
  static constexpr int NDB = D / 16;                      // 16-wide column blocks of O
  // LDS row stride of the staged V tile (16-bit elements). V is read back
  // transposed, 8 bytes per lane from 4 rows x 4 column pairs: a stride of
  // 8 or 40 (mod 64) dwords puts the 32 lanes of a pass on distinct banks.
  static constexpr int kVStride = D + 16;
  static_assert(NVL >= 1, "tile smaller than one wave-load");
};

// Workgroup coordinates (x = KV head and head tile, y = partition, z =
// sequence). With kShared the linear dispatch index is renumbered so that each
// XCD gets one contiguous range of workgroups: XCD c receives dispatch
// indices c, c + 8, c + 16, ..., which become numbers start(c), start(c) + 1,
// ..., with start(c) = c * (total / 8) + min(c, total % 8); this is a
// bijection onto [0, total).
template <bool kShared> __device__ __forceinline__ void wg_coords(int& x, int& y, int& z) {
  if (!kShared) {
    x = blockIdx.x;
    y = blockIdx.y;
    z = blockIdx.z;
    return;
  }
  const unsigned nx = gridDim.x, ny = gridDim.y, total = nx * ny * gridDim.z;
  const unsigned lin = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  const unsigned xcd = lin % 8;
  const unsigned m = xcd * (total / 8) + min(xcd, total % 8) + lin / 8;
  x = (int)(m % nx);
  y = (int)(m / nx % ny);
  z = (int)(m / (nx * ny));
}

template <bool kShared> __device__ __forceinline__ uint4 load_kv(const char* p) {
  return kShared ? *reinterpret_cast<const uint4*>(p) : load_stream(p);
}

// First element (along D) of the 8 q/K elements lane group g supplies to k block b.
template <int CK> __device__ __forceinline__ constexpr int k_col(int b, int g) {
  return CK == kFP8 ? 64 * (b >> 1) + 16 * g + 8 * (b & 1) : 32 * b + 8 * g;
}

template <int QK, int CK, int D, int GT, bool kShared, bool kBalanced, bool kPrefix = false>
__global__ __launch_bounds__(kThreads) void decode_mfma(const DecodeArgs a) {
  using G = MGeo<CK, D>;
  constexpr int NKB = G::NKB, NKL = G::NKL, NVL = G::NVL, NDB = G::NDB, VS = G::kVStride;
  static_assert(QK == kF16 || QK == kBF16, "16-bit queries");
  static_assert(GT == 4 || GT == 8 || GT == 16 || (GT == 32 && kBalanced),
                "head tile of 4, 8 or 16; 32 (two sub-tiles per wave) in the balanced schedule only");
  static_assert(!kPrefix || (GT == 16 && !kBalanced && !kShared), "the shared-prefix pass takes 16 columns");
  constexpr int NT = GT > 16 ? GT / 16 : 1;  // 16-head sub-tiles of a wave, sharing each K/V tile
  constexpr int GS = GT > 16 ? 16 : GT;      // heads per sub-tile

  __shared__ int s_blocks[kMaxPartitionBlocks];
  __shared__ __align__(16) uint16_t s_v[kWaves][2 * 16 * VS];  // two staged V tiles per wave
  __shared__ float s_acc[kBalanced ? 1 : kWaves * GT * D];
  __shared__ float s_ml[kBalanced ? 1 : kWaves * GT * 2];
  __shared__ int s_pref[kBalanced ? kBalancedMaxSeqs + 1 : 1];
  __shared__ int s_shr[kBalanced ? kBalancedMaxSeqs : 1];  // shared-prefix blocks of each sequence
  __shared__ int s_len[kBalanced ? kBalancedMaxSeqs : 1];  // context length of each sequence
  __shared__ int s_scan[kBalanced ? kWaves : 1];

  const int n_sub = kPrefix ? 1 : a.group / GT;  // the prefix pass: x is the KV head
  int bx, part, seq;  // balanced: part is the group of four ranges, seq is set per piece
  wg_coords<kShared>(bx, part, seq);
  const int kvh = bx / n_sub;
  const int h0 = kvh * a.group + (bx - kvh * n_sub) * GT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;  // token of K rows / head of S columns and P rows / column of O
  const int g = lane >> 4;  // k group of the operands / row group of the results

  int ctx = 0;     // context length of the sequence in hand
  int blk0 = 0;    // its first block handled here (partition start, or start of the piece)
  int sb_off = 0;  // entry of s_blocks holding block blk0

  // q as the B operand of S = K·Qᵀ: for sub-tile t, lane (n, g) holds head
  // h0 + 16t + n, the 8 elements of k block b that group g supplies; heads
  // past the tile are zero.
  uint32_t qf[NT][NKB][4];
  auto load_q = [&](int s) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const char* qp = static_cast<const char*>(a.q) + ((int64_t)s * a.num_heads + h0 + 16 * t + n) * D * 2;
#pragma unroll
      for (int b = 0; b < NKB; ++b) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (n < GS) v = *reinterpret_cast<const uint4*>(qp + k_col<CK>(b, g) * 2);
        qf[t][b][0] = v.x;
        qf[t][b][1] = v.y;
        qf[t][b][2] = v.z;
        qf[t][b][3] = v.w;
      }
    }
  };

  f32x4_t acc[NT][NDB];
  float mref[NT];  // running reference max of head n (log2 units), equal on lanes n, n+16, n+32, n+48
  float lsum[NT];  // this lane's share of the running sum of head n
  auto reset = [&]() {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[t][db] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      mref[t] = kNegInf;
      lsum[t] = 0.f;
    }
  };

  const int64_t blk_stride = (int64_t)a.num_kv_heads * G::kTileBytes;
  const char* kbase = static_cast<const char*>(a.k_cache) + (int64_t)kvh * G::kTileBytes;
  const char* vbase = static_cast<const char*>(a.v_cache) + (int64_t)kvh * G::kTileBytes;
  const int k_off = n * G::kRowBytes + g * 16;  // + 64 * load
  const int v_off = lane * 16;                  // + 1024 * load
  const float qk_scale = a.qk_scale;
  uint16_t* sv = s_v[wave];

  struct Tile {
    uint4 k[NKL], v[NVL];
  };
  auto load_tile = [&](int j, Tile& t) {
    uint4(&kr)[NKL] = t.k;
    uint4(&vr)[NVL] = t.v;
    const int64_t off = pool_block(a, kBalanced ? s_blocks + wave * (kMaxPartitionBlocks / kWaves) : s_blocks,
                                   sb_off + j) * blk_stride;
    const char* kt = kbase + off;
    const char* vt = vbase + off;
#pragma unroll
    for (int c = 0; c < NKL; ++c) kr[c] = load_kv<kShared>(kt + k_off + c * 64);
#pragma unroll
    for (int c = 0; c < NVL; ++c) vr[c] = load_kv<kShared>(vt + v_off + c * 1024);
  };

  // One step over NP (1 or 2) tiles t0, t1 holding valid0, valid1 token rows
  // inside the context (16 unless kMasked; 0 marks a missing second tile,
  // whose registers are then t0's and are never used unmasked). With two
  // tiles the P·V products take both at once: the 32 tokens of a 16x16x32
  // MFMA are this lane group's four rows of t0 followed by its four rows of
  // t1 (a contraction does not care about the order of its terms), which
  // halves the P·V instructions and gives the softmax two independent chains.
  auto process = [&](auto masked, auto np_c, const Tile& t0, const Tile& t1, int valid0, int valid1) {
    constexpr bool kMasked = decltype(masked)::value;
    constexpr int NP = decltype(np_c)::value;
    const Tile* tl[2] = {&t0, &t1};
    const int valid[2] = {kMasked ? valid0 : 16, kMasked ? valid1 : 16};

    // Stage V (row-major, 16-bit) for the transposed operand reads.
    wave_lds_fence();  // the previous step's reads of sv are issued before it is overwritten
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      uint16_t* svp = sv + p * 16 * VS;
#pragma unroll
      for (int c = 0; c < NVL; ++c) {
        const int byte = c * 1024 + lane * 16;
        const int row = byte / G::kRowBytes;
        const int col = (byte % G::kRowBytes) / G::kBytes;
        const bool keep = !kMasked || row < valid[p];
        uint4 v = tl[p]->v[c];
        if constexpr (CK == kFP8) {
          uint4 w0, w1;
          fp8x4_to_16<QK>(v.x, w0.x, w0.y);
          fp8x4_to_16<QK>(v.y, w0.z, w0.w);
          fp8x4_to_16<QK>(v.z, w1.x, w1.y);
          fp8x4_to_16<QK>(v.w, w1.z, w1.w);
          if (!keep) w0 = w1 = make_uint4(0u, 0u, 0u, 0u);
          *reinterpret_cast<uint4*>(svp + row * VS + col) = w0;
          *reinterpret_cast<uint4*>(svp + row * VS + col + 8) = w1;
        } else {
          if (!keep) v = make_uint4(0u, 0u, 0u, 0u);
          *reinterpret_cast<uint4*>(svp + row * VS + col) = v;
        }
      }
    }

    // S = K·Qᵀ per sub-tile and tile: lane (n, g) ends with the logits of head
    // n for tokens 4g + i.
    f32x4_t sc[NT][NP];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int p = 0; p < NP; ++p) sc[t][p] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint4(&kr)[NKL] = tl[p]->k;
      if constexpr (CK == kFP8) {
#pragma unroll
        for (int c = 0; c < NKL; ++c) {
          uint32_t w[8];
          fp8x4_to_16<QK>(kr[c].x, w[0], w[1]);
          fp8x4_to_16<QK>(kr[c].y, w[2], w[3]);
          fp8x4_to_16<QK>(kr[c].z, w[4], w[5]);
          fp8x4_to_16<QK>(kr[c].w, w[6], w[7]);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            sc[t][p] = mma_k32<QK>(w, qf[t][2 * c], sc[t][p]);
            sc[t][p] = mma_k32<QK>(w + 4, qf[t][2 * c + 1], sc[t][p]);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < NKL; ++c) {
          const uint32_t w[4] = {kr[c].x, kr[c].y, kr[c].z, kr[c].w};
#pragma unroll
          for (int t = 0; t < NT; ++t) sc[t][p] = mma_k32<QK>(w, qf[t][c], sc[t][p]);
        }
      }
    }

    // Online softmax per sub-tile; P as hi + lo in the 16-bit type (the A
    // operand: head n, tokens 4g .. 4g+3 of each tile).
    uint32_t ph[NT][NP][2], pl[NT][NP][2];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float x[NP][4];
      float bm = kNegInf;
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[p][i] = sc[t][p][i] * qk_scale;
          if (n >= GS || (kMasked && 4 * g + i >= valid[p])) x[p][i] = kNegInf;
          bm = fmaxf(bm, x[p][i]);
        }
      if (__builtin_amdgcn_ballot_w64(bm > mref[t] + kSlack) != 0) {  // raise the reference max (wave-uniform)
        float bmx = fmaxf(bm, __shfl_xor(bm, 16, 64));
        bmx = fmaxf(bmx, __shfl_xor(bmx, 32, 64));
        const float mn = fmaxf(mref[t], bmx);
        const float alpha = fast_exp2(mref[t] - ((mn == kNegInf) ? 0.f : mn));
        lsum[t] *= alpha;
        mref[t] = mn;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float al = __shfl(alpha, 4 * g + i, 64);  // the factor of head 4g + i (rows of acc)
#pragma unroll
          for (int db = 0; db < NDB; ++db) acc[t][db][i] *= al;
        }
      }
      const float ms = (mref[t] == kNegInf) ? 0.f : mref[t];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[i] = fast_exp2(x[p][i] - ms);
          lsum[t] += pr[i];
        }
        ph[t][p][0] = pack2<QK>(pr[0], pr[1]);
        ph[t][p][1] = pack2<QK>(pr[2], pr[3]);
        pl[t][p][0] = pack2<QK>(pr[0] - lo16_to_f32<QK>(ph[t][p][0]), pr[1] - hi16_to_f32<QK>(ph[t][p][0]));
        pl[t][p][1] = pack2<QK>(pr[2] - lo16_to_f32<QK>(ph[t][p][1]), pr[3] - hi16_to_f32<QK>(ph[t][p][1]));
      }
    }

    wave_lds_fence();  // the staged V tiles are written
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      if constexpr (NP == 2) {
        const u32x2_t b0 = v_operand_tr(sv, VS, db * 16, lane);
        const u32x2_t b1 = v_operand_tr(sv + 16 * VS, VS, db * 16, lane);
        const uint32_t b[4] = {b0[0], b0[1], b1[0], b1[1]};
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint32_t ah[4] = {ph[t][0][0], ph[t][0][1], ph[t][1][0], ph[t][1][1]};
          const uint32_t al[4] = {pl[t][0][0], pl[t][0][1], pl[t][1][0], pl[t][1][1]};
          acc[t][db] = mma_k32<QK>(ah, b, acc[t][db]);
          acc[t][db] = mma_k32<QK>(al, b, acc[t][db]);
        }
      } else {
        const u32x2_t b = v_operand_tr(sv, VS, db * 16, lane);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          acc[t][db] = mma_k16<QK>(ph[t][0][0], ph[t][0][1], b[0], b[1], acc[t][db]);
          acc[t][db] = mma_k16<QK>(pl[t][0][0], pl[t][0][1], b[0], b[1], acc[t][db]);
        }
      }
    }
  };

  struct Pair {
    Tile a, b;
  };
  using One = std::integral_constant<int, 1>;
  using Two = std::integral_constant<int, 2>;

  // Blocks blk0 + first, blk0 + first + step, ... below blk0 + nblk of a
  // sequence holding seq_blocks blocks, two per step. The last step is run
  // apart, by the wave that owns it: the block holding rows past the context
  // (the last of the sequence, when its length is not a multiple of 16)
  // and/or a block left without a partner, so the stream's loop body holds
  // one unmasked pair per ring slot and the accumulators stay in place.
  auto run_blocks = [&](int first, int step, int nblk, int seq_blocks) {
    if (first >= nblk) return;
    const bool tail_masked = (ctx & 15) && blk0 + nblk == seq_blocks;
    const int cnt = (nblk - 1 - first) / step + 1;  // blocks of this wave
    const bool own_masked = tail_masked && (nblk - 1 - first) % step == 0;
    const int fin = own_masked ? 2 - (cnt & 1) : (cnt & 1);  // blocks of the last step
    const int pairs = (cnt - fin) / 2;
    const int j_fin = first + step * (cnt - fin);            // first block of the last step
    auto valid_of = [&](int j) { return min(16, ctx - (blk0 + j) * 16); };
    auto load_pair = [&](int q, Pair& pr) {
      load_tile(first + step * (2 * q), pr.a);
      load_tile(first + step * (2 * q + 1), pr.b);
    };
    auto proc_pair = [&](int, const Pair& pr) { process(std::false_type{}, Two{}, pr.a, pr.b, 16, 16); };
    auto run_fin = [&](const Pair& pr) {
      if (fin == 2)
        process(std::true_type{}, Two{}, pr.a, pr.b, valid_of(j_fin), valid_of(j_fin + step));
      else if (fin == 1)
        process(std::true_type{}, One{}, pr.a, pr.a, valid_of(j_fin), 0);
    };
    if constexpr (kBalanced) {
      // One wave per piece, registers to spare: the last step's loads go out
      // first, so they arrive with the stream's first pair instead of after
      // its last.
      Pair fp;
      if (fin >= 1) load_tile(j_fin, fp.a);
      if (fin == 2) load_tile(j_fin + step, fp.b);
      stream_blocks<(NT > 1 ? kRingWide : kRingBalanced), Pair>(0, 1, pairs, load_pair, proc_pair);
      run_fin(fp);
    } else {
      stream_blocks<kRing, Pair>(0, 1, pairs, load_pair, proc_pair);
      if (fin) {
        Pair fp;
        load_tile(j_fin, fp.a);
        if (fin == 2) load_tile(j_fin + step, fp.b);
        run_fin(fp);
      }
    }
  };

  if constexpr (kPrefix) {
    // Shared-prefix pass: workgroup (KV head, part, tile). The tile's 16
    // query columns are the (sequence, head) pairs of 16 / group consecutive
    // sequences of one group, which share the group's first blocks, so every
    // shared K/V tile is read once for all of them (their table rows agree
    // there; the first sequence's row is read). All shared blocks are full:
    // no row is masked. Each column leaves the part's max, sum and
    // unnormalised output for decode_bal_reduce.
    const int tile = seq;
    const int S = a.num_seqs;
    if (kvh == 0 && part == 0 && tile == 0) {  // the per-sequence shared block counts, for the kernels after
      for (int s = tid; s < S; s += kThreads) {
        int shb = 0;
        for (int gi = 0; gi < a.prefix_groups; ++gi)
          if (s >= a.grp_first[gi] && s < a.grp_first[gi] + a.grp_count[gi]) shb = a.grp_blocks[gi];
        a.ws_shared[s] = shb;
      }
    }
    int gi = 0;
    while (gi + 1 < a.prefix_groups && tile >= a.grp_tile0[gi + 1]) ++gi;
    const int spt = 16 / a.group;  // sequences per tile
    const int s0 = a.grp_first[gi] + (tile - a.grp_tile0[gi]) * spt;
    const int s_end = min(a.grp_first[gi] + a.grp_count[gi], s0 + spt);
    const int nshared = a.grp_blocks[gi];
    blk0 = part * a.prefix_part_blocks;
    if (blk0 >= nshared || s0 >= s_end) return;
    const int nblk = min(a.prefix_part_blocks, nshared - blk0);
    ctx = nshared * 16;
    const int32_t* bt = a.block_tables + (int64_t)a.grp_first[gi] * a.max_blocks + blk0;
    for (int j = tid; j < nblk; j += kThreads) s_blocks[j] = bt[j];
    // Column n: query head kvh * group + n % group of sequence s0 + n / group
    // (zero past the group's last sequence; such columns are not written).
    const int cs = s0 + n / a.group;
    {
      const char* qp = static_cast<const char*>(a.q) +
                       ((int64_t)cs * a.num_heads + kvh * a.group + n % a.group) * D * 2;
#pragma unroll
      for (int b = 0; b < NKB; ++b) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (cs < s_end) v = *reinterpret_cast<const uint4*>(qp + k_col<CK>(b, g) * 2);
        qf[0][b][0] = v.x;
        qf[0][b][1] = v.y;
        qf[0][b][2] = v.z;
        qf[0][b][3] = v.w;
      }
    }
    __syncthreads();

    reset();
    run_blocks(wave, kWaves, nblk, nshared);

    float ls = lsum[0] + __shfl_xor(lsum[0], 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    if (g == 0) {
      s_ml[(wave * 16 + n) * 2] = mref[0];
      s_ml[(wave * 16 + n) * 2 + 1] = ls;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int db = 0; db < NDB; ++db) s_acc[(wave * 16 + 4 * g + i) * D + db * 16 + n] = acc[0][db][i];
    __syncthreads();
    // Merge the waves per column (the part holds a block, so the max is finite).
    for (int idx = tid; idx < 16 * D; idx += kThreads) {
      const int c = idx / D;
      const int d = idx - c * D;
      const int s = s0 + c / a.group;
      if (s >= s_end) continue;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_ml[(w * 16 + c) * 2]);
      float Lw = 0.f, O = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = fast_exp2(s_ml[(w * 16 + c) * 2] - M);
        Lw += s_ml[(w * 16 + c) * 2 + 1] * f;
        O += s_acc[(w * 16 + c) * D + d] * f;
      }
      const int64_t pi = ((int64_t)(kvh * a.group + c % a.group) * S + s) * a.prefix_parts + part;
      a.ws_sh_out[pi * D + d] = O * a.out_scale;
      if (d == 0) {
        a.ws_sh_ml[2 * pi] = M;
        a.ws_sh_ml[2 * pi + 1] = Lw;
      }
    }
  } else if constexpr (!kBalanced) {
    // One partition of one sequence; the four waves take its blocks in turn.
    ctx = context_len(a, seq);
    // Fused append (one workgroup per KV head): the new row lies in the
    // sequence's last block, read only by wave (nblk - 1) % kWaves of the
    // last partition; that wave writes it and waits for its stores before it
    // loads anything. An empty context's row goes out with partition 0.
    const bool writer = a.append && part == (ctx > 0 ? (((ctx + 15) >> 4) - 1) / a.partition_blocks : 0);
    if (ctx <= 0) {
      if (writer) append_row<QK, CK, D, kThreads>(a, seq, kvh, tid);
      write_zeros<GT, D>(a, seq, h0, part, tid);
      return;
    }
    const int seq_blocks = (ctx + 15) >> 4;
    blk0 = part * a.partition_blocks;
    if (blk0 >= seq_blocks) return;
    const int nblk = min(a.partition_blocks, seq_blocks - blk0);
    const int seq_parts = (seq_blocks + a.partition_blocks - 1) / a.partition_blocks;

    const int32_t* bt = a.block_tables + (int64_t)seq * a.max_blocks + blk0;
    for (int j = tid; j < nblk; j += kThreads) s_blocks[j] = bt[j];
    load_q(seq);
    __syncthreads();
    if (writer && wave == (nblk - 1) % kWaves) {
      append_row<QK, CK, D, 64>(a, seq, kvh, lane);
      wait_own_stores();
    }

    reset();
    run_blocks(wave, kWaves, nblk, seq_blocks);

    // This wave's sum of head n over its four row groups; the max is already shared.
    float ls = lsum[0] + __shfl_xor(lsum[0], 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    if (g == 0 && n < GT) {
      s_ml[(wave * GT + n) * 2] = mref[0];
      s_ml[(wave * GT + n) * 2 + 1] = ls;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (4 * g + i < GT) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) s_acc[(wave * GT + 4 * g + i) * D + db * 16 + n] = acc[0][db][i];
      }
    }
    __syncthreads();
    finish_partition<GT, D>(a, s_acc, s_ml, seq, h0, part, seq_parts, tid);
  } else {
    // Balanced schedule. The blocks of all sequences, laid end to end in
    // sequence order, are T positions; range r of R holds positions
    // [B(r), B(r + 1)) with B(r) = floor(r * T / R), and wave w of this
    // workgroup takes range 4 * part + w whole, cutting sequences wherever
    // the ranges fall. The piece of a sequence that a range holds is
    // streamed like a partition; a sequence held entirely by one range is
    // written straight to the output, any other piece leaves its max, sum
    // and unnormalised output in slot s + r of the workspace for
    // decode_bal_reduce. Every workgroup first builds the block-count
    // prefix of the batch in LDS (one pass over context_lens).
    const int S = a.num_seqs;
    // Blocks per sequence and their exclusive prefix sum s_pref[0..S].
    constexpr int kPer = (kBalancedMaxSeqs + kThreads - 1) / kThreads;
    const int per = (S + kThreads - 1) / kThreads;
    int nb[kPer];
    int local = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int s = tid * per + k;
      int c = 0, shb = 0;
      if (k < per && s < S) {
        c = context_len(a, s);
        if (a.shared_prefix) shb = a.ws_shared[s];
        s_shr[s] = shb;
        s_len[s] = c;
      }
      // Blocks past the shared prefix (those inside it were read by the prefix pass).
      nb[k] = c > 0 ? max(0, ((c + 15) >> 4) - shb) : 0;
      local += nb[k];
    }
    // Inclusive scan of the per-thread sums: within each wave by shuffles,
    // then across the four waves through LDS.
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    if (lane == 63) s_scan[wave] = incl;
    __syncthreads();
    {
      int run = incl - local;
      for (int w = 0; w < wave; ++w) run += s_scan[w];
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int s = tid * per + k;
        if (k < per && s < S) s_pref[s] = run;
        run += nb[k];
      }
      if (tid == kThreads - 1) s_pref[S] = run;
    }
    __syncthreads();
    const int T = s_pref[S];
    const int64_t R = a.ranges;
    auto range_start = [&](int64_t r) { return (int)(r * T / R); };
    // Sequence holding position p < T: the last s with s_pref[s] <= p (empty
    // sequences share their successor's start and are passed over).
    auto seq_of = [&](int p) {
      int lo = 0, hi = S;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pref[mid] <= p) lo = mid;
        else hi = mid;
      }
      return lo;
    };
    if (blockIdx.x == 0 && blockIdx.y == 0)
      for (int k = tid; k <= S; k += kThreads) a.ws_pref[k] = s_pref[k];
    // Fused append (one wave per KV head and range): the wave whose range
    // holds a sequence's last block writes that sequence's new row below,
    // before it loads any block of it. Sequences with no block in any range
    // (empty contexts) are read by no wave; their rows are written here, by
    // the first workgroup of each KV head, one thread per sequence.
    if (a.append && part == 0)
      for (int s = tid; s < S; s += kThreads)
        if (s_pref[s] == s_pref[s + 1]) append_row<QK, CK, D, 1>(a, s, kvh, 0);

    // Each wave stages the block ids of its range in LDS, a window of
    // kWindow positions at a time (no workgroup barrier: the window is the
    // wave's own quarter of s_blocks).
    constexpr int kWindow = kMaxPartitionBlocks / kWaves;
    int* const wblocks = s_blocks + wave * kWindow;
    int win = 0, win_end = 0;
    auto stage = [&](int from, int to) {
      wave_lds_fence();  // the previous window's reads are issued
      for (int i = lane; i < to - from; i += 64) {
        const int p = from + i;
        const int s = seq_of(p);
        wblocks[i] = a.block_tables[(int64_t)s * a.max_blocks + (p - s_pref[s]) + s_shr[s]];
      }
      wave_lds_fence();
      win = from;
      win_end = to;
    };

    const int r = 4 * part + wave;
    const int r_end = range_start(r + 1);
    const int64_t slots = (int64_t)S + R;
    for (int pos = range_start(r); pos < r_end;) {
      seq = __builtin_amdgcn_readfirstlane(seq_of(pos));
      const int ps = s_pref[seq], pe = s_pref[seq + 1];
      const int piece_end = min(r_end, pe);
      const int shb = s_shr[seq];  // position ps is block shb of the sequence
      ctx = s_len[seq];
      if (a.append && piece_end == pe) {  // this range holds the sequence's last block
        append_row<QK, CK, D, 64>(a, seq, kvh, lane);
        wait_own_stores();
      }
      load_q(seq);
      reset();
      // The piece [pos, piece_end), window by window, accumulating throughout.
      for (int sub = pos; sub < piece_end;) {
        if (sub >= win_end) stage(sub, min(sub + kWindow, r_end));
        const int sub_end = min(piece_end, win_end);
        blk0 = sub - ps + shb;
        sb_off = sub - win;
        run_blocks(0, 1, sub_end - sub, pe - ps + shb);
        sub = sub_end;
      }

      // A sequence with a shared prefix always leaves a piece: the merge adds the prefix pass's parts.
      const bool whole = pos == ps && piece_end == pe && shb == 0;
      const int64_t slot = seq + r;
      // The results leave through the wave's V staging area (free between
      // steps): the MFMA layout puts head 4g + i, column 16 db + n on lane
      // (n, g), so direct stores would take NDB * 4 instructions of 16 to 64
      // lanes each, and every vector memory instruction waits its turn behind
      // the other waves' tile loads; restaged, each lane stores 16
      // consecutive bytes and a 16-head tile takes D / 16 instructions.
      float* const sf = reinterpret_cast<float*>(sv);
      constexpr int RS = D + 4;  // staged row stride in floats: the four row groups fall on different banks
      static_assert(GS * RS * 4 <= 2 * 16 * VS * 2, "staged rows fit the wave's V area");
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float ls = lsum[t] + __shfl_xor(lsum[t], 16, 64);
        ls += __shfl_xor(ls, 32, 64);
        const int hb = h0 + 16 * t;  // first head of the sub-tile
        float sc[4];  // the whole sequence: normalise; a piece: its unnormalised output
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = whole ? a.out_scale / __shfl(ls, 4 * g + i, 64) : a.out_scale;
        wave_lds_fence();  // the last step's reads of the area, and the previous sub-tile's, are done
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (4 * g + i < GS) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) sf[(4 * g + i) * RS + db * 16 + n] = acc[t][db][i] * sc[i];
          }
        }
        wave_lds_fence();
        constexpr int kChunks = GS * D / 4;  // float4 chunks of the tile
        static_assert(kChunks % 64 == 0, "whole rounds of the wave");
#pragma unroll
        for (int c = lane; c < kChunks; c += 64) {
          const int hh = c / (D / 4);
          const int col = (c - hh * (D / 4)) * 4;
          const float4 v = *reinterpret_cast<const float4*>(sf + hh * RS + col);
          if (whole) store_out4(a, ((int64_t)seq * a.num_heads + hb + hh) * D + col, v);
          else *reinterpret_cast<float4*>(a.ws_out + ((int64_t)(hb + hh) * slots + slot) * D + col) = v;
        }
        if (!whole && g == 0 && n < GS)
          *reinterpret_cast<float2*>(a.ws_ml + ((int64_t)(hb + n) * slots + slot) * 2) = make_float2(mref[t], ls);
      }
      pos = piece_end;
    }
  }
}

template <int QK, int CK, int D, int GT, bool kBalanced>
void launch_s(const DecodeArgs& a, dim3 grid, hipStream_t stream) {
  if (a.group > GT)
    decode_mfma<QK, CK, D, GT, true, kBalanced><<<grid, dim3(kThreads), 0, stream>>>(a);
  else
    decode_mfma<QK, CK, D, GT, false, kBalanced><<<grid, dim3(kThreads), 0, stream>>>(a);
}

template <int QK, int CK, int D, int GT>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const unsigned columns = (unsigned)(a.num_kv_heads * (a.group / GT));
  if (a.balanced) {
    launch_s<QK, CK, D, GT, true>(a, dim3(columns, (unsigned)(a.ranges / 4), 1u), stream);
  } else {
    if constexpr (GT > 16) return hipErrorInvalidValue;  // 32-head tiles exist in the balanced schedule only
    else launch_s<QK, CK, D, GT, false>(a, dim3(columns, (unsigned)a.num_parts, (unsigned)a.num_seqs), stream);
  }
  return hipGetLastError();
}

template <int QK, int CK, int D>
hipError_t launch_g(const DecodeArgs& a, hipStream_t stream) {
  switch (a.group_tile) {
    case 4: return launch_t<QK, CK, D, 4>(a, stream);
    case 8: return launch_t<QK, CK, D, 8>(a, stream);
    case 16: return launch_t<QK, CK, D, 16>(a, stream);
    case 32: return launch_t<QK, CK, D, 32>(a, stream);
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

template <int QK, int CK>
hipError_t launch_prefix_d(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.num_kv_heads, (unsigned)a.prefix_parts, (unsigned)a.grp_tile0[a.prefix_groups]);
  switch (a.head_size) {
    case 64: decode_mfma<QK, CK, 64, 16, false, false, true><<<grid, dim3(kThreads), 0, stream>>>(a); break;
    case 128: decode_mfma<QK, CK, 128, 16, false, false, true><<<grid, dim3(kThreads), 0, stream>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_prefix(const DecodeArgs& a, int q_kind, int cache_kind, hipStream_t stream) {
  switch (q_kind * 4 + cache_kind) {
    case kF16 * 4 + kF16: return launch_prefix_d<kF16, kF16>(a, stream);
    case kBF16 * 4 + kBF16: return launch_prefix_d<kBF16, kBF16>(a, stream);
    case kF16 * 4 + kFP8: return launch_prefix_d<kF16, kFP8>(a, stream);
    case kBF16 * 4 + kFP8: return launch_prefix_d<kBF16, kFP8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int q_kind, int cache_kind, hipStream_t stream) {
  switch (q_kind * 4 + cache_kind) {
    case kF16 * 4 + kF16: return launch_d<kF16, kF16>(a, stream);
    case kBF16 * 4 + kBF16: return launch_d<kBF16, kBF16>(a, stream);
    case kF16 * 4 + kFP8: return launch_d<kF16, kFP8>(a, stream);
    case kBF16 * 4 + kFP8: return launch_d<kBF16, kFP8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
