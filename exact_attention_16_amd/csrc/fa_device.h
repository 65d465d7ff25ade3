// Device-side building blocks shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace detail {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Buffer descriptor word 3 for gfx9-family raw (untyped) buffers.
constexpr int kRsrcWord3 = 0x00020000;
// s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt left at their maxima.
constexpr int kWaitVmcnt0 = 0x0F70;
// When the row max is taken (a tile's first visit of a row, or a tile whose
// weights exceed Elem<T>::kTileSumLimit), the partial output is rescaled only
// if the max grew by more than this many binary orders of magnitude.
constexpr float kRescaleMargin = 8.0f;
// XCDs (each with its own L2) that work-groups are dealt to round-robin.
constexpr int kXcds = 8;

template <typename T>
struct Elem;

template <>
struct Elem<__bf16> {
  static __device__ __forceinline__ f32x16 mma(i16x8 a, i16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack(float x, float y) {
    bf16x2 r = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(unsigned, r);
  }
  // The weights rounded to bf16 keep 8 significant bits, so the output is
  // normalised by the sum of the ROUNDED weights (acc + both halves of a
  // packed pair, one v_dot2): a weight's rounding error then cancels between
  // numerator and denominator instead of scaling the whole output row.
  static constexpr bool kRoundedSum = true;
  // A tile's weights are accepted without the row max while no lane's share
  // of the tile's row sum (32 weights) exceeds this (FwdWave::softmax_impl).
  // bf16 weights have fp32's exponent range, so only the fp32 output
  // accumulator bounds them: with weights up to 2^40, a million keys times
  // |V| up to 2^64 still fit.  (At least twice 32 * 2^kRescaleMargin, the
  // largest share a tile can have right after a rescale, so a retried tile
  // always passes.)
  static constexpr float kTileSumLimit = 1099511627776.0f;  // 2^40
  static __device__ __forceinline__ float add_packed(unsigned w, float acc) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, acc, false);
  }
};

template <>
struct Elem<_Float16> {
  static __device__ __forceinline__ f32x16 mma(i16x8 a, i16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack(float x, float y) {
    f16x2 r = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(unsigned, r);
  }
  // fp16 weights keep 11 significant bits: the exact fp32 row sum serves both
  // the output and the logsumexp.
  static constexpr bool kRoundedSum = false;
  // fp16 weights must stay below 65504: 2^14 bounds every weight of a share
  // (and is at least twice 32 * 2^kRescaleMargin, see the bf16 case).
  static constexpr float kTileSumLimit = 16384.0f;
  static __device__ __forceinline__ float add_packed(unsigned, float acc) { return acc; }
};

struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int BH;      // B * H
  int S;       // query rows per head
  int Sk;      // key rows per head (= S for self-attention)
  int shift;   // causal offset: query row i sits at key position i + shift (Sk - S)
  int nqb;     // query-row blocks per head
  int persist; // 1: persistent grid, each work-group walks its own list of query blocks
  float c;     // scale * log2(e): scores enter exp2 as c * s
  // Strided layouts only: heads per batch entry, the batch and head strides
  // (elements) of q, k, v, o, and their row strides (bytes).
  int H;
  long long qsb, qsh, ksb, ksh, vsb, vsh, osb, osh;
  uint32_t q_rs, k_rs, v_rs, o_rs;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

// Value of x held by lane l^32.  v_permlane32_swap exchanges the upper half
// of its first operand with the lower half of its second; called with x
// twice, lanes 0-31 find the partner's value in the second result and lanes
// 32-63 in the first.  Each result element is copied to a scalar before use:
// this compiler's __builtin_bit_cast applied directly to a vector element
// (bit_cast(float, r[1])) reads element 0 whatever the index.  No inline
// assembly is involved, so the compiler keeps the wait states that the
// producer of x requires (a v_dot2 result, for one).
__device__ __forceinline__ float partner_value(float x) {
  const unsigned xb = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(xb, xb, false, false);
  const unsigned lo = r[0], hi = r[1];
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? lo : hi);
}

__device__ __forceinline__ float max_with_partner(float x) { return fmaxf(x, partner_value(x)); }

__device__ __forceinline__ float sum_with_partner(float x) { return x + partner_value(x); }

// Work-group barrier.  It first waits for this wavefront's own LDS accesses
// (lgkmcnt(0)): an LDS read still in flight could otherwise see a buffer that
// another wavefront refills after the barrier, and an LDS write might not yet
// be visible to the wavefronts that read it after the barrier.  Waits for
// vector memory (vmcnt) are explicit at each call site, and the "memory"
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace detail
}  // namespace fa
