// Pieces shared by the decode kernels: workgroup shape, streaming tile loads,
// LDS ordering inside a wave, output rounding, and the per-workgroup epilogue
// that merges the waves' running (max, sum, unnormalised output).
#pragma once

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kNegInf = -__builtin_huge_valf();

// Orders LDS traffic between lanes of one wave: the LDS executes one wave's
// instructions in order, so only the compiler has to be kept from moving them.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// K/V tiles are read once per step: nontemporal loads keep them from
// displacing reusable lines in the caches.
__device__ __forceinline__ uint4 load_stream(const char* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// One 16-byte tile chunk: streaming (nontemporal) by default; an ordinary
// cached load where a comparison run asks for it.
template <bool kCached> __device__ __forceinline__ uint4 load_tile_chunk(const char* p) {
  if constexpr (kCached) return *reinterpret_cast<const uint4*>(p);
  else return load_stream(p);
}

__device__ __forceinline__ void store_out(const DecodeArgs& a, int64_t elem, float x) {
  if (a.out_kind == kF32) {
    static_cast<float*>(a.out)[elem] = x;
  } else if (a.out_kind == kBF16) {
    static_cast<uint16_t*>(a.out)[elem] = f32_to_bf16_rne(x);
  } else {
    static_cast<uint16_t*>(a.out)[elem] = f32_to_f16_rne(x);
  }
}

// Four consecutive output elements (elem a multiple of 4): one 16- or 8-byte
// store when the output is aligned for it (the pointer is a kernel argument,
// so the choice is uniform), else four element stores.
__device__ __forceinline__ void store_out4(const DecodeArgs& a, int64_t elem, float4 v) {
  if ((reinterpret_cast<uintptr_t>(a.out) & 15) != 0) {
    store_out(a, elem, v.x);
    store_out(a, elem + 1, v.y);
    store_out(a, elem + 2, v.z);
    store_out(a, elem + 3, v.w);
  } else if (a.out_kind == kF32) {
    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + elem) = v;
  } else {
    const bool bf = a.out_kind == kBF16;
    auto cv = [bf](float x) -> uint32_t { return bf ? f32_to_bf16_rne(x) : f32_to_f16_rne(x); };
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + elem) =
        make_uint2(cv(v.x) | (cv(v.y) << 16), cv(v.z) | (cv(v.w) << 16));
  }
}

// Merge the waves of a workgroup (each left its max, sum and unnormalised
// output in LDS: s_acc is [kWaves][GT][D], s_ml is [kWaves][GT][2]) and write
// the result, or the partition's partial result. The partition holds at least
// one token, so the merged max is finite.
template <int GT, int D>
__device__ __forceinline__ void finish_partition(const DecodeArgs& a, const float* s_acc, const float* s_ml, int seq,
                                                 int h0, int part, int seq_parts, int tid) {
  for (int idx = tid; idx < GT * D; idx += kThreads) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_ml[(w * GT + g) * 2]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(s_ml[(w * GT + g) * 2] - M);
      L += s_ml[(w * GT + g) * 2 + 1] * f;
      O += s_acc[(w * GT + g) * D + d] * f;
    }
    O *= a.out_scale;
    const int64_t sh = (int64_t)seq * a.num_heads + h0 + g;
    if (seq_parts == 1) {
      store_out(a, sh * D + d, O / L);
    } else {
      const int64_t pi = sh * a.num_parts + part;
      a.ws_out[pi * D + d] = O;
      if (d == 0) {
        a.ws_ml[2 * pi] = M;
        a.ws_ml[2 * pi + 1] = L;
      }
    }
  }
}

// Context length of a sequence, clamped to what its block-table row can hold,
// so a length past the row never sends a kernel beyond the table.
__device__ __forceinline__ int context_len(const DecodeArgs& a, int seq) {
  return min(a.context_lens[seq], a.max_blocks * 16);
}

// Physical block of table entry j (wave-uniform); an id outside the pool is
// clamped into it, so a corrupt table reads wrong data but no foreign memory.
__device__ __forceinline__ int64_t pool_block(const DecodeArgs& a, const int* s_blocks, int j) {
  const int phys = __builtin_amdgcn_readfirstlane(s_blocks[j]);
  return (uint32_t)phys < (uint64_t)a.num_blocks ? phys : 0;
}

// Streams blocks j = first, first + step, ... < n through a ring of N register
// buffers: the loads of the next N-1 blocks are in flight while a block is
// processed. The steady-state loop issues its loads unconditionally, so the
// compiler's wait for a block's registers counts the newer loads and leaves
// them in flight; a conditional prefetch would join two paths with different
// numbers of outstanding loads and force a wait for all of them. Scheduling
// barriers keep the compiler from hoisting work of a block just requested
// above the point where it is requested (which would again wait for it) or
// from sinking loads below the processing.
template <int N, class Buf, class Load, class Proc>
__device__ __forceinline__ void stream_blocks(int first, int step, int n, Load&& load, Proc&& proc) {
  static_assert(N >= 2, "ring of at least two buffers");
  if (first >= n) return;
  if constexpr (N == 2) {  // written out: fewer live registers than the general tail
    Buf b0, b1;
    int j = first;
    load(j, b0);
    for (; j + 2 * step < n; j += 2 * step) {
      load(j + step, b1);
      __builtin_amdgcn_sched_barrier(0);
      proc(j, b0);
      __builtin_amdgcn_sched_barrier(0);
      load(j + 2 * step, b0);
      __builtin_amdgcn_sched_barrier(0);
      proc(j + step, b1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (j + step < n) {
      load(j + step, b1);
      __builtin_amdgcn_sched_barrier(0);
      proc(j, b0);
      __builtin_amdgcn_sched_barrier(0);
      proc(j + step, b1);
    } else {
      proc(j, b0);
    }
    return;
  }
  Buf b[N];
#pragma unroll
  for (int d = 0; d < N - 1; ++d)
    if (first + d * step < n) load(first + d * step, b[d]);
  int j = first;
  for (; j + (2 * N - 2) * step < n; j += N * step) {
#pragma unroll
    for (int d = 0; d < N; ++d) {
      load(j + (d + N - 1) * step, b[(d + N - 1) % N]);
      __builtin_amdgcn_sched_barrier(0);
      proc(j + d * step, b[d]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // Tail: blocks j + d*step < n for d < 2N-2; those with d < N-1 are loaded.
#pragma unroll
  for (int d = 0; d < 2 * N - 2; ++d) {
    if (d + N - 1 < 2 * N - 2 && j + (d + N - 1) * step < n) load(j + (d + N - 1) * step, b[(d + N - 1) % N]);
    if (j + d * step < n) proc(j + d * step, b[d % N]);
  }
}

// Waits until every vector memory operation this wave has issued, stores
// included, has completed (s_waitcnt vmcnt(0); gfx9 counts stores in vmcnt).
// After it, a load by this wave of an address the wave just stored to returns
// the stored data: the store is complete at the L2 that serves the load, and
// the write-through L1 holds no older copy of a line this wave never read.
__device__ __forceinline__ void wait_own_stores() {
  // simm16 on gfx9: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14].
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt not waited for
}

// Fused append: write sequence seq's new K and V rows of KV head kvh into the
// cache slot a.new_slots[seq] (bit copy, or E4M3 after dividing by the scale,
// exactly as reshape_kernel does), one 16-byte source chunk per thread of
// the N taking part (thread index tid).
template <int QK, int CK, int D, int N>
__device__ __forceinline__ void append_row(const DecodeArgs& a, int seq, int kvh, int tid) {
  const int64_t slot = a.new_slots_int64 ? static_cast<const int64_t*>(a.new_slots)[seq]
                                         : (int64_t) static_cast<const int32_t*>(a.new_slots)[seq];
  if (slot < 0 || slot >= a.num_blocks * 16) return;
  constexpr int kSrc = KindBytes<QK>::value;
  constexpr int E = 16 / kSrc;  // source elements per chunk
  constexpr int NC = D / E;     // chunks per row
  const int64_t src = ((int64_t)seq * a.num_kv_heads + kvh) * D;
  const int64_t dst = (((slot >> 4) * a.num_kv_heads + kvh) * 16 + (slot & 15)) * D;
  for (int i = tid; i < 2 * NC; i += N) {
    const bool is_v = i >= NC;
    const int c = is_v ? i - NC : i;
    const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const char*>(is_v ? a.new_value : a.new_key) +
                                                     (src + (int64_t)c * E) * kSrc);
    char* cache = static_cast<char*>(const_cast<void*>(is_v ? a.v_cache : a.k_cache));
    if constexpr (CK == QK) {
      *reinterpret_cast<uint4*>(cache + (dst + (int64_t)c * E) * kSrc) = x;
    } else if constexpr (CK == kFP8 && QK == kF32) {
      *reinterpret_cast<uint32_t*>(cache + dst + (int64_t)c * E) = e4m3_chunk32(x, is_v ? a.enc_v_scale : a.enc_k_scale);
    } else if constexpr (CK == kFP8) {
      *reinterpret_cast<uint2*>(cache + dst + (int64_t)c * E) = e4m3_chunk16<QK>(x, is_v ? a.enc_v_scale : a.enc_k_scale);
    }
  }
}

// Zeros for a sequence with nothing to attend, written once (by partition 0).
template <int GT, int D>
__device__ __forceinline__ void write_zeros(const DecodeArgs& a, int seq, int h0, int part, int tid) {
  if (part == 0)
    for (int idx = tid; idx < GT * D; idx += kThreads) store_out(a, ((int64_t)seq * a.num_heads + h0) * D + idx, 0.f);
}

}  // namespace pa
