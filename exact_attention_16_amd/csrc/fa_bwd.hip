// gfx950 (CDNA4) kernels of the exact-attention backward pass.
//
// The pages describe the method as exact attention used for training
// (searcharxiv abstract page, "Abstract"), whose gradients match the plain
// calculation up to rounding (IPLEX blog "FlashAttention-2: making long-context
// attention run efficiently on GPUs", section "Tiling preserves the attention
// calculation").  They do not give the backward algorithm; this is our own,
// built from the chain rule of the forward definition and the same ideas the
// pages credit for the forward pass: the S x S matrices never reach HBM (each
// tile of P is recomputed from Q, K and the row logsumexp the forward pass
// saved), work is spread over the sequence dimension as well as (batch, head)
// (section "Three changes improve GPU utilisation"), and every wavefront owns
// its accumulators outright, so nothing is reduced through LDS or atomics.
//
// With c = scale * log2(e), lse2_i = LSE_i * log2(e) and D_i = dO_i . O_i:
//   P_ij  = 2^(c s_ij - lse2_i)        (s_ij = q_i . k_j; 0 for masked keys)
//   dP_ij = dO_i . v_j
//   dS_ij = P_ij (dP_ij - D_i)
//   dQ    = scale dS K,   dK = scale dS^T Q,   dV = P^T dO.
//
// Two kernels, launched in this order on one stream:
// * dq_kernel: one wavefront per 32 query rows (work-group = 8 wavefronts =
//   256 rows, as in the forward pass).  It first computes D_i from dO and O
//   and writes it to the caller's delta buffer, then walks the key tiles:
//   S^T = K Q^T and dP^T = V dO^T on the matrix cores (Q and dO held in
//   VGPRs, K and V from LDS), P, dS on the vector ALUs (each lane holds one
//   query, so LSE_i and D_i are per-lane scalars), and dQ^T += K^T dS^T (K^T
//   read through ds_read_b64_tr_b16).
// * dkdv_kernel: one wavefront per 32 keys; K and V stay in VGPRs while the
//   wavefront walks the query tiles: S = Q K^T and dP = dO V^T (each lane holds
//   one key; LSE and D of the tile's queries come from LDS), then
//   dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read transposed.
//   At d >= 128, dkdv16_kernel does the same with 16 keys per wavefront on
//   16x16x32 MFMAs, so that two or three wavefronts share each SIMD.
// Tiles move HBM -> LDS with direct-to-LDS buffer loads, double-buffered:
// in the forward kernel's fragment-major layouts, or for dkdv16_kernel in one
// swizzled layout per tile (Tile16).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_bwd_launch.h"

namespace fa {
namespace bwd {

using namespace fa::detail;

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;
  int BH;
  int S;        // query rows per head (q, o, dout, dq, lse, delta)
  int Sk;       // key rows per head (k, v, dk, dv)
  int shift;    // causal offset: key j is kept for query row i iff j <= i + shift (Sk - S)
  int nblk;     // row blocks per head (query blocks for dq_kernel, key blocks for dkdv_kernel)
  float scale;
  float c;      // scale * log2(e)
  // Strided layouts only: heads per batch entry, and per tensor (kQ .. kDV)
  // the batch and head strides (elements) and the row stride (bytes).
  int H;
  long long sb[8], sh[8];
  uint32_t rs[8];
};

enum { kQ, kK, kV, kO, kDO, kDQ, kDK, kDV };

// One head of one tensor: base, bytes between rows and the byte range that
// ends with the head's last row (rows past it read 0 / are dropped).
struct View {
  const char* base;
  uint32_t rs;
  uint32_t bytes;
};

template <int D, bool STRIDED>
__device__ __forceinline__ View head_view(const BwdParams& p, const void* ptr, int t, int bh) {
  const int rows = (t == kK || t == kV || t == kDK || t == kDV) ? p.Sk : p.S;
  View v;
  if (STRIDED) {
    const int b = bh / p.H, hh = bh - b * p.H;
    v.base = (const char*)ptr + (b * p.sb[t] + hh * p.sh[t]) * 2;
    v.rs = p.rs[t];
    v.bytes = rows > 0 ? (uint32_t)(rows - 1) * p.rs[t] + D * 2 : 0u;
  } else {
    v.base = (const char*)ptr + (size_t)bh * rows * D * 2;
    v.rs = D * 2;
    v.bytes = (uint32_t)rows * D * 2;
  }
  return v;
}

constexpr float kLog2e = 1.4426950408889634f;

// Tiles of ROWS rows x D columns, staged by NW wavefronts, in two LDS layouts:
//   A layout: 1 KiB block (rb, kk) holds, at lane l, row 32 rb + l%32,
//     columns 16 kk + 8 (l/32) .. +8: the A operand of a 32x32x16 MFMA whose
//     m index is the row and whose k index is the column;
//   T layout: the layout of the forward kernel's V tiles: two 512-byte halves
//     per block ((rb*2 + cc)*2 + tt)*(DB/2) + dp, read with ds_read_b64_tr_b16
//     into the A operand of an MFMA whose m index is the column (32 columns
//     per d-block) and whose k index is the row (16 rows per chunk cc).
template <int D, int NW, int ROWS>
struct Tile {
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int KSTEPS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int RB = ROWS / 32;
  static constexpr int BYTES = ROWS * ROW_BYTES;
  static constexpr int LOADS = BYTES / (NW * 64 * 16);
  static_assert(LOADS * NW * 64 * 16 == BYTES, "tile must split evenly over lanes");

  // rs: bytes between rows (ROW_BYTES for dense tensors); base: the tile's
  // first row offset in bytes.
  static __device__ __forceinline__ void issue_a(__amdgpu_buffer_rsrc_t r, uint32_t base, char* dst, int wave,
                                                 int lane, uint32_t rs = ROW_BYTES) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int f = i * NW + wave;  // block (rb, kk)
      const int rb = f / KSTEPS, kk = f % KSTEPS;
      const uint32_t off = base + (uint32_t)(rb * 32 + (lane & 31)) * rs + (kk * 2 + (lane >> 5)) * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + f * 1024), 16, off, 0, 0, 0);
    }
  }

  static __device__ __forceinline__ void issue_t(__amdgpu_buffer_rsrc_t r, uint32_t base, char* dst, int wave,
                                                 int lane, uint32_t rs = ROW_BYTES) {
    const int x = lane >> 5;
    const int lp = lane & 31;
    const int vg = lp >> 3;
    const int vrow = (vg >> 1) * 4 + ((lp & 7) >> 1);
    const int vcol = x * 32 + (vg & 1) * 16 + (lp & 1) * 8;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int f = i * NW + wave;  // block ((rb * 2 + cc) * 2 + tt) * (DB / 2) + dp
      const int dp = f % (DB / 2), rest = f / (DB / 2);
      const uint32_t off = base + (uint32_t)(rest * 8 + vrow) * rs + (dp * 64 + vcol) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + f * 1024), 16, off, 0, 0, 0);
    }
  }

  static __device__ __forceinline__ i16x8 frag_a(const char* t, int rb, int kk, int lane) {
    return *(const i16x8*)(t + (rb * KSTEPS + kk) * 1024 + lane * 16);
  }

  // A operand with m = columns 32 db .. +32 and k = rows 32 rb + 16 cc .. +16
  // (row order permuted within the chunk exactly as a C-layout tile packed by
  // pack_c puts it).
  static __device__ __forceinline__ i16x8 frag_t(const char* t, int db, int rb, int cc, int lane) {
    i16x4 half[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int blk = ((rb * 2 + cc) * 2 + tt) * (DB / 2) + (db >> 1);
      half[tt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(t + blk * 1024 + (db & 1) * 512 + lane * 8));
    }
    return __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

// Row fragments as the B operand (k = column, n = the lane's row): lane l
// holds columns 16 kk + 8 (l/32) .. +8 of its row; rows past the range read 0.
template <int D>
__device__ __forceinline__ void load_row_frags(i16x8 (&f)[D / 16], const char* head, uint32_t head_bytes, int row,
                                               int h, uint32_t rs = D * 2) {
  const __amdgpu_buffer_rsrc_t r = rsrc(head, head_bytes);
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const uint32_t off = (uint32_t)row * rs + (kk * 16 + h * 8) * 2;
    f[kk] = __builtin_bit_cast(i16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
}

template <typename T>
__device__ __forceinline__ float dot_pairs(i16x8 a, i16x8 b, float acc);

// sum over the 8 element pairs of a . b, accumulated in fp32 (v_dot2).  Each
// 32-bit word is copied to a scalar before its bit_cast: this compiler's
// __builtin_bit_cast applied directly to a vector element (v[i]) reads
// element 0 whatever the index.
template <>
__device__ __forceinline__ float dot_pairs<__bf16>(i16x8 a, i16x8 b, float acc) {
  const u32x4 ua = __builtin_bit_cast(u32x4, a), ub = __builtin_bit_cast(u32x4, b);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned xa = ua[i], xb = ub[i];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, xa), __builtin_bit_cast(bf16x2, xb), acc, false);
  }
  return acc;
}

template <>
__device__ __forceinline__ float dot_pairs<_Float16>(i16x8 a, i16x8 b, float acc) {
  const u32x4 ua = __builtin_bit_cast(u32x4, a), ub = __builtin_bit_cast(u32x4, b);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned xa = ua[i], xb = ub[i];
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, xa), __builtin_bit_cast(f16x2, xb), acc, false);
  }
  return acc;
}

// A C-layout 32x32 fp32 tile (16 values per lane) packed to T as the two B
// operands (k chunks cc = 0, 1) of an MFMA whose k index is the tile's row:
// value r of lane l sits at row 8 (r/4) + 4 (l/32) + r%4, and frag_t reads
// the matching rows in the same order.
template <typename T>
__device__ __forceinline__ void pack_c(const float (&e)[16], i16x8 (&out)[2]) {
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = Elem<T>::pack(e[8 * cc + 2 * i], e[8 * cc + 2 * i + 1]);
    out[cc] = __builtin_bit_cast(i16x8, w);
  }
}

// Store a transposed C-layout accumulator set (acc[db] holds rows
// 32 db + 8 (r/4) + 4 (l/32) + r%4 of the lane's output row's columns) times
// `mul` as the lane's row of a row-major [rows x D] tensor in T.
template <typename T, int D>
__device__ __forceinline__ void store_row(const f32x16 (&acc)[D / 32], float mul, char* head, uint32_t head_bytes,
                                          int row, int h, uint32_t rs = D * 2) {
  const __amdgpu_buffer_rsrc_t r = rsrc(head, head_bytes);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      u32x2 w;
      w[0] = Elem<T>::pack(acc[db][4 * rg + 0] * mul, acc[db][4 * rg + 1] * mul);
      w[1] = Elem<T>::pack(acc[db][4 * rg + 2] * mul, acc[db][4 * rg + 3] * mul);
      const int col = db * 32 + 8 * rg + 4 * h;
      __builtin_amdgcn_raw_buffer_store_b64(w, r, (uint32_t)row * rs + col * 2, 0, 0);
    }
}

// Work-group -> (row block, head), dealing each head's row blocks to one XCD
// (K/V or Q/dO tiles shared through that XCD's L2).  longest_first_reversed:
// the causal dq blocks with the most key tiles are the LAST row blocks, the
// causal dkdv blocks with the most query tiles are the FIRST; either way the
// longest blocks of all heads on the XCD go first.
__device__ __forceinline__ void map_block(int BH, int nblk, bool causal, bool last_is_longest, int& bh, int& blk) {
  if (BH % kXcds == 0) {
    const int local = blockIdx.x / kXcds;
    if (causal) {
      const int hpx = BH / kXcds;
      blk = local / hpx;
      bh = (local % hpx) * kXcds + blockIdx.x % kXcds;
    } else {
      blk = local % nblk;
      bh = (local / nblk) * kXcds + blockIdx.x % kXcds;
    }
  } else {
    blk = blockIdx.x % nblk;
    bh = blockIdx.x / nblk;
  }
  if (causal && last_is_longest) blk = nblk - 1 - blk;
}

// ---------------------------------------------------------------- dQ kernel

template <typename T, int D, bool CAUSAL, bool TAIL, int NW, int BN>
struct DqWave {
  using KT = Tile<D, NW, BN>;
  static constexpr int KSTEPS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int SB = BN / 32;

  int lane, h, qw, myq, Sk, shift;
  float c, lse2, dl;
  i16x8 qf[KSTEPS], dof[KSTEPS];
  f32x16 dq[DB];

  __device__ __forceinline__ bool active(int k0) const { return !(CAUSAL && k0 > qw + 31 + shift); }
  __device__ __forceinline__ bool masked(int k0) const {
    return (CAUSAL && k0 + BN - 1 > qw + shift) || (TAIL && k0 + BN > Sk);
  }

  // One key tile: kA = K (A layout), vA = V (A layout), kT = K (T layout).
  template <bool MASKED>
  __device__ __forceinline__ void step(const char* kA, const char* vA, const char* kT, int k0) {
    f32x16 s[SB], dp[SB];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) s[sb] = dp[sb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        s[sb] = Elem<T>::mma(KT::frag_a(kA, sb, kk, lane), qf[kk], s[sb]);
        dp[sb] = Elem<T>::mma(KT::frag_a(vA, sb, kk, lane), dof[kk], dp[sb]);
      }
      // wide heads: keep the scheduler from hoisting every k-step's LDS reads
      // to the top (they would not fit the register file)
      if constexpr (D > 128)
        if (kk % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
    i16x8 dsf[SB][2];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      float e[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][r], c, -lse2));
        if (MASKED) {
          const int key = k0 + sb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          // a select, not a product: a row that keeps no key has LSE = -inf
          // and p = +inf here
          p = (key < Sk && (!CAUSAL || key <= myq + shift)) ? p : 0.f;
        }
        e[r] = p * (dp[sb][r] - dl);
      }
      pack_c<T>(e, dsf[sb]);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int sb = 0; sb < SB; ++sb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) dq[db] = Elem<T>::mma(KT::frag_t(kT, db, sb, cc, lane), dsf[sb][cc], dq[db]);
      if constexpr (D > 128)
        if (db % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    }
  }
};

template <typename T, int D, bool CAUSAL, bool TAIL, int NW, int BN, bool STRIDED>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 1 : 2) void dq_kernel(BwdParams p) {
  using W = DqWave<T, D, CAUSAL, TAIL, NW, BN>;
  using KT = typename W::KT;
  constexpr int BM = NW * 32;
  __shared__ __attribute__((aligned(1024))) char ka0[KT::BYTES];
  __shared__ __attribute__((aligned(1024))) char ka1[KT::BYTES];
  __shared__ __attribute__((aligned(1024))) char va0[KT::BYTES];
  __shared__ __attribute__((aligned(1024))) char va1[KT::BYTES];
  __shared__ __attribute__((aligned(1024))) char kt0[KT::BYTES];
  __shared__ __attribute__((aligned(1024))) char kt1[KT::BYTES];

  W w;
  w.lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  w.h = w.lane >> 5;
  int bh, qb;
  map_block(p.BH, p.nblk, CAUSAL, true, bh, qb);
  const int q_lo = qb * BM;
  w.qw = q_lo + 32 * wave;
  w.myq = w.qw + (w.lane & 31);
  w.Sk = p.Sk;
  w.shift = p.shift;
  w.c = p.c;

  const View kv = head_view<D, STRIDED>(p, p.k, kK, bh), vv = head_view<D, STRIDED>(p, p.v, kV, bh);
  const View qv = head_view<D, STRIDED>(p, p.q, kQ, bh), dov = head_view<D, STRIDED>(p, p.dout, kDO, bh);
  const View ov = head_view<D, STRIDED>(p, p.o, kO, bh), dqv = head_view<D, STRIDED>(p, p.dq, kDQ, bh);
  const __amdgpu_buffer_rsrc_t rk = rsrc(kv.base, kv.bytes);
  const __amdgpu_buffer_rsrc_t rv = rsrc(vv.base, vv.bytes);

  // Q and dO rows of the lane's query; D_i = dO_i . O_i (each lane holds half
  // the columns, its partner lane l^32 the other half); LSE_i in log2 units.
  load_row_frags<D>(w.qf, qv.base, qv.bytes, w.myq, w.h, qv.rs);
  load_row_frags<D>(w.dof, dov.base, dov.bytes, w.myq, w.h, dov.rs);
  {
    i16x8 of[W::KSTEPS];
    load_row_frags<D>(of, ov.base, ov.bytes, w.myq, w.h, ov.rs);
    float part = 0.f;
#pragma unroll
    for (int kk = 0; kk < W::KSTEPS; ++kk) part = dot_pairs<T>(w.dof[kk], of[kk], part);
    w.dl = sum_with_partner(part);
  }
  const __amdgpu_buffer_rsrc_t rl = rsrc(p.lse + (size_t)bh * p.S, (uint32_t)p.S * 4);
  w.lse2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, (uint32_t)w.myq * 4, 0, 0)) * kLog2e;
  if (w.h == 0) {
    const __amdgpu_buffer_rsrc_t rd = rsrc(p.delta + (size_t)bh * p.S, (uint32_t)p.S * 4);
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, w.dl), rd, (uint32_t)w.myq * 4, 0, 0);
  }
#pragma unroll
  for (int db = 0; db < W::DB; ++db) w.dq[db] = f32x16{};

  // keys this work-group visits (causal: up to its last row's position)
  const int kv_end = CAUSAL ? min(p.Sk, q_lo + BM + p.shift) : p.Sk;
  const int n = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
  const uint32_t tk = (uint32_t)BN * kv.rs, tv = (uint32_t)BN * vv.rs;  // bytes per key tile

  if (n > 0) {
    KT::issue_a(rk, 0, ka0, wave, w.lane, kv.rs);
    KT::issue_a(rv, 0, va0, wave, w.lane, vv.rs);
    KT::issue_t(rk, 0, kt0, wave, w.lane, kv.rs);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  barrier();
  for (int k = 0; k < n; k += 2) {
    if (k + 1 < n) {
      KT::issue_a(rk, (k + 1) * tk, ka1, wave, w.lane, kv.rs);
      KT::issue_a(rv, (k + 1) * tv, va1, wave, w.lane, vv.rs);
      KT::issue_t(rk, (k + 1) * tk, kt1, wave, w.lane, kv.rs);
    }
    if (w.active(k * BN)) {
      if (w.masked(k * BN)) w.template step<true>(ka0, va0, kt0, k * BN);
      else w.template step<false>(ka0, va0, kt0, k * BN);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    barrier();
    if (k + 1 >= n) break;
    if (k + 2 < n) {
      KT::issue_a(rk, (k + 2) * tk, ka0, wave, w.lane, kv.rs);
      KT::issue_a(rv, (k + 2) * tv, va0, wave, w.lane, vv.rs);
      KT::issue_t(rk, (k + 2) * tk, kt0, wave, w.lane, kv.rs);
    }
    if (w.active((k + 1) * BN)) {
      if (w.masked((k + 1) * BN)) w.template step<true>(ka1, va1, kt1, (k + 1) * BN);
      else w.template step<false>(ka1, va1, kt1, (k + 1) * BN);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    barrier();
  }
  store_row<T, D>(w.dq, p.scale, (char*)dqv.base, dqv.bytes, w.myq, w.h, dqv.rs);
}

// ------------------------------------------------------------- dK/dV kernel

// Floats reserved in LDS for a query tile's LSE values, and again for its D
// values (one dword per lane of a wavefront).
constexpr int kStatFloats = 64;

template <typename T, int D, bool CAUSAL, int NW, int BQ>
struct DkvWave {
  using QT = Tile<D, NW, BQ>;
  static constexpr int KSTEPS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int QB = BQ / 32;

  int lane, h, kw, myk, shift;
  float c;
  i16x8 kf[KSTEPS], vf[KSTEPS];
  f32x16 dk[DB], dv[DB];

  __device__ __forceinline__ bool active(int q0) const { return !(CAUSAL && q0 + BQ - 1 + shift < kw); }
  __device__ __forceinline__ bool masked(int q0) const { return CAUSAL && q0 + shift < kw + 31; }

  // One query tile: qA, dA = Q, dO (A layout); qT, dT = Q, dO (T layout);
  // st = the tile's LSE (floats 0..BQ-1) and D (floats kStatFloats..).
  template <bool MASKED>
  __device__ __forceinline__ void step(const char* qA, const char* dA, const char* qT, const char* dT,
                                       const float* st, int q0) {
    if constexpr (D > 128) __builtin_amdgcn_sched_barrier(0);  // no overlap across tiles (registers)
    f32x16 s[QB], dp[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[qb] = dp[qb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        s[qb] = Elem<T>::mma(QT::frag_a(qA, qb, kk, lane), kf[kk], s[qb]);
        dp[qb] = Elem<T>::mma(QT::frag_a(dA, qb, kk, lane), vf[kk], dp[qb]);
      }
      if constexpr (D > 128)  // as in DqWave::step
        if (kk % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
    i16x8 pf[QB][2], dsf[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float pe[16], de[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // queries 32 qb + 8 j + 4 h + (0..3): four consecutive LSE and D values
        const int qi = qb * 32 + 8 * j + 4 * h;
        const float4 l4 = *(const float4*)(st + qi);
        const float4 d4 = *(const float4*)(st + kStatFloats + qi);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dvv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = 4 * j + t;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][r], c, -lv[t] * kLog2e));
          // a select: a row that keeps no key has LSE = -inf and p = +inf
          if (MASKED) p = (q0 + qi + t + shift >= myk) ? p : 0.f;
          pe[r] = p;
          de[r] = p * (dp[qb][r] - dvv[t]);
        }
      }
      pack_c<T>(pe, pf[qb]);
      pack_c<T>(de, dsf[qb]);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          dv[db] = Elem<T>::mma(QT::frag_t(dT, db, qb, cc, lane), pf[qb][cc], dv[db]);
          dk[db] = Elem<T>::mma(QT::frag_t(qT, db, qb, cc, lane), dsf[qb][cc], dk[db]);
        }
      if constexpr (D > 128)
        if (db % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (D > 128) __builtin_amdgcn_sched_barrier(0);
  }
};

// LSE and D of a query tile into LDS (kStatFloats floats each): wavefront 0
// fetches the LSE values, wavefront 1 the D values, one dword per lane, so
// each writes 64 dwords; lanes >= BQ and rows past the sequence read 0.
template <int BQ>
__device__ __forceinline__ void issue_stats(__amdgpu_buffer_rsrc_t rl, __amdgpu_buffer_rsrc_t rd, int q0, char* dst,
                                            int wave, int lane) {
  static_assert(BQ <= kStatFloats, "one dword per lane");
  const uint32_t off = (lane < BQ) ? (uint32_t)(q0 + lane) * 4 : 0x7FFFFFF0u;
  if (wave == 0) __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void*)dst, 4, off, 0, 0, 0);
  if (wave == 1) __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void*)(dst + kStatFloats * 4), 4, off, 0, 0, 0);
}

template <int D>
constexpr int dkdv_waves() { return D == 64 ? 8 : 4; }

template <typename T, int D, bool CAUSAL, int NW, int BQ, bool STRIDED>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 1 : 2) void dkdv_kernel(BwdParams p) {
  using W = DkvWave<T, D, CAUSAL, NW, BQ>;
  using QT = typename W::QT;
  constexpr int BK = NW * 32;
  __shared__ __attribute__((aligned(1024))) char qa0[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char qa1[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char da0[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char da1[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char qt0[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char qt1[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char dt0[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char dt1[QT::BYTES];
  __shared__ __attribute__((aligned(16))) char st0[2 * kStatFloats * 4];
  __shared__ __attribute__((aligned(16))) char st1[2 * kStatFloats * 4];

  W w;
  w.lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  w.h = w.lane >> 5;
  int bh, kb;
  map_block(p.BH, p.nblk, CAUSAL, false, bh, kb);
  const int k_lo = kb * BK;
  w.kw = k_lo + 32 * wave;
  w.myk = w.kw + (w.lane & 31);
  w.c = p.c;
  w.shift = p.shift;

  const View kv = head_view<D, STRIDED>(p, p.k, kK, bh), vv = head_view<D, STRIDED>(p, p.v, kV, bh);
  const View qv = head_view<D, STRIDED>(p, p.q, kQ, bh), dov = head_view<D, STRIDED>(p, p.dout, kDO, bh);
  const View dkv = head_view<D, STRIDED>(p, p.dk, kDK, bh), dvv = head_view<D, STRIDED>(p, p.dv, kDV, bh);
  load_row_frags<D>(w.kf, kv.base, kv.bytes, w.myk, w.h, kv.rs);
  load_row_frags<D>(w.vf, vv.base, vv.bytes, w.myk, w.h, vv.rs);
#pragma unroll
  for (int db = 0; db < W::DB; ++db) w.dk[db] = w.dv[db] = f32x16{};

  const __amdgpu_buffer_rsrc_t rq = rsrc(qv.base, qv.bytes);
  const __amdgpu_buffer_rsrc_t rdo = rsrc(dov.base, dov.bytes);
  const __amdgpu_buffer_rsrc_t rl = rsrc(p.lse + (size_t)bh * p.S, (uint32_t)p.S * 4);
  const __amdgpu_buffer_rsrc_t rd = rsrc(p.delta + (size_t)bh * p.S, (uint32_t)p.S * 4);

  // query tiles t0 .. n-1 (causal: only queries whose position i + shift
  // reaches the block's first key)
  const int t0 = CAUSAL ? max(0, k_lo - p.shift) / BQ : 0;
  const int n = (p.S + BQ - 1) / BQ;
  const uint32_t tq = (uint32_t)BQ * qv.rs, tdo = (uint32_t)BQ * dov.rs;  // bytes per query tile

  if (t0 < n) {
    QT::issue_a(rq, t0 * tq, qa0, wave, w.lane, qv.rs);
    QT::issue_a(rdo, t0 * tdo, da0, wave, w.lane, dov.rs);
    QT::issue_t(rq, t0 * tq, qt0, wave, w.lane, qv.rs);
    QT::issue_t(rdo, t0 * tdo, dt0, wave, w.lane, dov.rs);
    issue_stats<BQ>(rl, rd, t0 * BQ, st0, wave, w.lane);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  barrier();
  for (int t = t0; t < n; t += 2) {
    if (t + 1 < n) {
      QT::issue_a(rq, (t + 1) * tq, qa1, wave, w.lane, qv.rs);
      QT::issue_a(rdo, (t + 1) * tdo, da1, wave, w.lane, dov.rs);
      QT::issue_t(rq, (t + 1) * tq, qt1, wave, w.lane, qv.rs);
      QT::issue_t(rdo, (t + 1) * tdo, dt1, wave, w.lane, dov.rs);
      issue_stats<BQ>(rl, rd, (t + 1) * BQ, st1, wave, w.lane);
    }
    if (w.active(t * BQ)) {
      if (w.masked(t * BQ)) w.template step<true>(qa0, da0, qt0, dt0, (const float*)st0, t * BQ);
      else w.template step<false>(qa0, da0, qt0, dt0, (const float*)st0, t * BQ);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    barrier();
    if (t + 1 >= n) break;
    if (t + 2 < n) {
      QT::issue_a(rq, (t + 2) * tq, qa0, wave, w.lane, qv.rs);
      QT::issue_a(rdo, (t + 2) * tdo, da0, wave, w.lane, dov.rs);
      QT::issue_t(rq, (t + 2) * tq, qt0, wave, w.lane, qv.rs);
      QT::issue_t(rdo, (t + 2) * tdo, dt0, wave, w.lane, dov.rs);
      issue_stats<BQ>(rl, rd, (t + 2) * BQ, st0, wave, w.lane);
    }
    if (w.active((t + 1) * BQ)) {
      if (w.masked((t + 1) * BQ)) w.template step<true>(qa1, da1, qt1, dt1, (const float*)st1, (t + 1) * BQ);
      else w.template step<false>(qa1, da1, qt1, dt1, (const float*)st1, (t + 1) * BQ);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    barrier();
  }
  store_row<T, D>(w.dk, p.scale, (char*)dkv.base, dkv.bytes, w.myk, w.h, dkv.rs);
  store_row<T, D>(w.dv, 1.0f, (char*)dvv.base, dvv.bytes, w.myk, w.h, dvv.rs);
}

// ------------------------------------------ dK/dV kernel, 16 keys per wavefront

// At d = 128 the 32-key wavefront above holds 128 accumulator registers for
// dK and dV alone and needs more than half of a SIMD's register file, so a
// SIMD runs one wavefront and its exp / dS work never overlaps matrix work.
// dkdv16_kernel gives each wavefront 16 keys on v_mfma_f32_16x16x32: half
// the accumulator registers (154-158 VGPRs in all, no AGPRs), four
// wavefronts per work-group and three work-groups per CU, so each SIMD
// interleaves three wavefronts whose barriers are independent.  The price is
// twice the LDS operand bytes per FLOP.  The wide heads (d = 192, 256) run
// it too, at two wavefronts per SIMD (202-256 VGPRs) where the 32-key
// kernel fits only one.
//
// Lane layouts (checked on the MI355X with an in-bounds probe):
//   v_mfma_f32_16x16x32: A (16 x 32) lane l holds row l%16, k = 8 (l/16) ..
//     +8; B (32 x 16) lane l holds column l%16, the same k; C (16 x 16) lane l
//     holds column l%16, rows 4 (l/16) .. +4.
//   ds_read_b64_tr_b16: in each group of 16 lanes, lane u receives element
//     u%4 of the 4-element reads of lanes 4 j + u/4, j = 0..3 (the group's
//     reads as a 4 x 16 block, transposed).

template <typename T>
__device__ __forceinline__ f32x4 mma16(i16x8 a, i16x8 b, f32x4 c);

template <>
__device__ __forceinline__ f32x4 mma16<__bf16>(i16x8 a, i16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

template <>
__device__ __forceinline__ f32x4 mma16<_Float16>(i16x8 a, i16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}

// Q and dO tiles of ROWS rows x D columns, staged once in a swizzled layout
// that serves both the plain 16-byte operand reads of S and dP and the
// transposing reads of dV and dK.  Slot s (16 bytes) of 1 KiB block (rb, kk)
// holds row 16 rb + ((s % 16) ^ 12 ((s / 16) % 2)), columns 32 kk + 8 (s / 16)
// .. +8.  A transposing read fetches 4 consecutive columns of 4 rows per
// 16-lane group, in two 8-byte pieces 8 columns apart.  Without the swizzle
// those pieces share banks.  With XOR 12, 16-lane groups 0 and 3 use one
// half of the 64 banks and groups 1 and 2 the other, so the read is free of
// conflicts whether the LDS serves lanes 0-31 together or lanes 0-15 with
// 32-47 (XOR 8 left groups 0 and 2 on the same banks: SQ_LDS_BANK_CONFLICT
// was 30 % of the LDS cycles).
template <int D, int NW, int ROWS>
struct Tile16 {
  static constexpr int KS = D / 32;
  static constexpr int BYTES = ROWS * D * 2;
  static constexpr int LOADS = BYTES / (NW * 1024);
  static_assert(ROWS % 32 == 0 && LOADS * NW * 1024 == BYTES, "tile must split evenly over wavefronts");

  // each lane fetches the 16 bytes that belong at its slot
  static __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, uint32_t base, char* dst, int wave,
                                               int lane, uint32_t rs) {
    const int c = lane >> 4;
    const int q = (lane & 15) ^ (12 * (c & 1));
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int f = i * NW + wave;  // block (rb, kk)
      const int rb = f / KS, kk = f % KS;
      const uint32_t off = base + (uint32_t)(rb * 16 + q) * rs + (kk * 32 + c * 8) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + f * 1024), 16, off, 0, 0, 0);
    }
  }

  // byte offset of lane l's A operand in a block: row l % 16, columns
  // 8 (l / 16) .. +8
  static __device__ __forceinline__ int a_off(int lane) {
    const int c = lane >> 4;
    return 16 * (16 * c + ((lane & 15) ^ (12 * (c & 1))));
  }
  // byte offset of lane l = 16 g + u's transposing read in the first half of a
  // block: row 4 g + u / 4, columns 4 (u % 4) .. +4 (the second half, +512,
  // holds columns 16 .. 31)
  static __device__ __forceinline__ int t_off(int lane) {
    const int g = lane >> 4, u = lane & 15, a = u & 3, h = a >> 1;
    return 256 * h + 16 * ((4 * g + (u >> 2)) ^ (12 * h)) + 8 * (a & 1);
  }

  static __device__ __forceinline__ i16x8 frag_a(const char* t, int rb, int kk, int aoff) {
    return *(const i16x8*)(t + (rb * KS + kk) * 1024 + aoff);
  }

  // A operand with m = columns 16 db .. +16 and k = rows 32 ch + {4 (l/16)
  // .. +4, 16 + 4 (l/16) .. +4}: the order in which pack16 puts a pair of C
  // tiles into one B operand
  static __device__ __forceinline__ i16x8 frag_t(const char* t, int db, int ch, int toff) {
    i16x4 half[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int blk = (2 * ch + tt) * KS + (db >> 1);
      half[tt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(t + blk * 1024 + (db & 1) * 512 + toff));
    }
    return __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

// Two C-layout 16x16 tiles (4 values per lane each: rows 4 (l/16) + t) as one
// B operand whose k index runs over their 32 rows in the order frag_t reads.
template <typename T>
__device__ __forceinline__ i16x8 pack16(const float (&e)[8]) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = Elem<T>::pack(e[2 * i], e[2 * i + 1]);
  return __builtin_bit_cast(i16x8, w);
}

template <typename T, int D, bool CAUSAL, int NW, int BQ>
struct Dkv16Wave {
  using QT = Tile16<D, NW, BQ>;
  static constexpr int KS = D / 32;
  static constexpr int DB = D / 16;    // 16-column d-blocks of dK, dV
  static constexpr int QB = BQ / 16;   // 16-query blocks of S, dP
  static constexpr int NCH = BQ / 32;  // 32-query chunks of the dV, dK products

  int lane, g, kw, myk, shift, aoff, toff;
  float c;
  i16x8 kf[KS], vf[KS];
  f32x4 dk[DB], dv[DB];
  f32x4 s[QB], dp[QB];
  i16x8 pf[NCH], dsf[NCH];

  __device__ __forceinline__ bool active(int q0) const { return !(CAUSAL && q0 + BQ - 1 + shift < kw); }
  __device__ __forceinline__ bool masked(int q0) const { return CAUSAL && q0 + shift < kw + 15; }

  // S = Q K^T and dP = dO V^T of a query tile (qA, dA: Q, dO)
  __device__ __forceinline__ void scores(const char* qA, const char* dA) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[qb] = dp[qb] = f32x4{};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        s[qb] = mma16<T>(QT::frag_a(qA, qb, kk, aoff), kf[kk], s[qb]);
        dp[qb] = mma16<T>(QT::frag_a(dA, qb, kk, aoff), vf[kk], dp[qb]);
      }
  }

  // P and dS from the scores; st = the tile's LSE in log2 units (floats
  // 0..BQ-1), then D
  template <bool MASKED>
  __device__ __forceinline__ void weights(const float* st, int q0) {
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      float pe[8], de[8];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int qb = 2 * ch + tt;
        const int qi = qb * 16 + 4 * g;  // queries 16 qb + 4 g + (0..3)
        const float4 l4 = *(const float4*)(st + qi);
        const float4 d4 = *(const float4*)(st + BQ + qi);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dl[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][t], c, -lv[t]));
          // a select: a row that keeps no key has LSE = -inf and p = +inf
          if (MASKED) p = (q0 + qi + t + shift >= myk) ? p : 0.f;
          pe[4 * tt + t] = p;
          de[4 * tt + t] = p * (dp[qb][t] - dl[t]);
        }
      }
      pf[ch] = pack16<T>(pe);
      dsf[ch] = pack16<T>(de);
    }
  }

  // dV^T += dO^T P and dK^T += Q^T dS
  __device__ __forceinline__ void grads(const char* qA, const char* dA) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        dv[db] = mma16<T>(QT::frag_t(dA, db, ch, toff), pf[ch], dv[db]);
        dk[db] = mma16<T>(QT::frag_t(qA, db, ch, toff), dsf[ch], dk[db]);
      }
  }

  // One query tile.  The phases stay apart: letting the scheduler hoist one
  // phase's LDS operand reads into another raises the register count past
  // what three wavefronts per SIMD allow.
  __device__ __forceinline__ void step(const char* qA, const char* dA, const float* st, int q0) {
    scores(qA, dA);
    __builtin_amdgcn_sched_barrier(0);
    if (masked(q0)) weights<true>(st, q0);
    else weights<false>(st, q0);
    __builtin_amdgcn_sched_barrier(0);
    grads(qA, dA);
  }
};

// The lane's key row as the B operand of S = Q K^T (k = column): columns
// 32 kk + 8 g .. +8; rows past the range read 0.
template <int D>
__device__ __forceinline__ void load_row_frags16(i16x8 (&f)[D / 32], const View& v, int row, int g) {
  const __amdgpu_buffer_rsrc_t r = rsrc(v.base, v.bytes);
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const uint32_t off = (uint32_t)row * v.rs + (kk * 32 + g * 8) * 2;
    f[kk] = __builtin_bit_cast(i16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
}

// A C-layout accumulator set (acc[db] holds columns 16 db + 4 g .. +4 of the
// lane's row) times `mul`, stored as that row of a row-major tensor in T.
template <typename T, int D>
__device__ __forceinline__ void store_row16(const f32x4 (&acc)[D / 16], float mul, const View& v, int row, int g) {
  const __amdgpu_buffer_rsrc_t r = rsrc(v.base, v.bytes);
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    u32x2 w;
    w[0] = Elem<T>::pack(acc[db][0] * mul, acc[db][1] * mul);
    w[1] = Elem<T>::pack(acc[db][2] * mul, acc[db][3] * mul);
    __builtin_amdgcn_raw_buffer_store_b64(w, r, (uint32_t)row * v.rs + (db * 16 + 4 * g) * 2, 0, 0);
  }
}

// LSE and D of a query tile: wavefront 0 loads the LSE values, wavefront 1
// the D values, one per lane (rows past the sequence read 0); put_stats16
// writes them to LDS, the LSE times log2 e, once the loads have landed.
template <int BQ>
__device__ __forceinline__ float load_stats16(__amdgpu_buffer_rsrc_t rl, __amdgpu_buffer_rsrc_t rd, int q0, int wave,
                                              int lane) {
  static_assert(BQ <= 64, "one value per lane");
  const uint32_t off = (lane < BQ) ? (uint32_t)(q0 + lane) * 4 : 0x7FFFFFF0u;
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(wave == 0 ? rl : rd, off, 0, 0));
}

template <int BQ>
__device__ __forceinline__ void put_stats16(float* st, float v, int wave, int lane) {
  if (wave < 2 && lane < BQ) st[wave * BQ + lane] = wave == 0 ? v * kLog2e : v;
}

template <typename T, int D, bool CAUSAL, int NW, int BQ, bool STRIDED>
__global__ __launch_bounds__(NW * 64, D == 128 ? 3 : 2) void dkdv16_kernel(BwdParams p) {
  using W = Dkv16Wave<T, D, CAUSAL, NW, BQ>;
  using QT = typename W::QT;
  constexpr int BK = NW * 16;
  __shared__ __attribute__((aligned(1024))) char qa0[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char qa1[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char da0[QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char da1[QT::BYTES];
  __shared__ __attribute__((aligned(16))) float st0[2 * BQ];
  __shared__ __attribute__((aligned(16))) float st1[2 * BQ];

  W w;
  w.lane = threadIdx.x & 63;
  // uniform across the wavefront: keeps the per-wavefront choices and LDS
  // destinations below in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  w.g = w.lane >> 4;
  w.aoff = QT::a_off(w.lane);
  w.toff = QT::t_off(w.lane);
  int bh, kb;
  map_block(p.BH, p.nblk, CAUSAL, false, bh, kb);
  const int k_lo = kb * BK;
  w.kw = k_lo + 16 * wave;
  w.myk = w.kw + (w.lane & 15);
  w.c = p.c;
  w.shift = p.shift;

  const View kv = head_view<D, STRIDED>(p, p.k, kK, bh), vv = head_view<D, STRIDED>(p, p.v, kV, bh);
  const View qv = head_view<D, STRIDED>(p, p.q, kQ, bh), dov = head_view<D, STRIDED>(p, p.dout, kDO, bh);
  const View dkv = head_view<D, STRIDED>(p, p.dk, kDK, bh), dvv = head_view<D, STRIDED>(p, p.dv, kDV, bh);
  load_row_frags16<D>(w.kf, kv, w.myk, w.g);
  load_row_frags16<D>(w.vf, vv, w.myk, w.g);
#pragma unroll
  for (int db = 0; db < W::DB; ++db) w.dk[db] = w.dv[db] = f32x4{};

  const __amdgpu_buffer_rsrc_t rq = rsrc(qv.base, qv.bytes);
  const __amdgpu_buffer_rsrc_t rdo = rsrc(dov.base, dov.bytes);
  const __amdgpu_buffer_rsrc_t rl = rsrc(p.lse + (size_t)bh * p.S, (uint32_t)p.S * 4);
  const __amdgpu_buffer_rsrc_t rd = rsrc(p.delta + (size_t)bh * p.S, (uint32_t)p.S * 4);

  // query tiles t0 .. n-1 (causal: only queries whose position i + shift
  // reaches the block's first key)
  const int t0 = CAUSAL ? max(0, k_lo - p.shift) / BQ : 0;
  const int n = (p.S + BQ - 1) / BQ;
  const uint32_t tq = (uint32_t)BQ * qv.rs, tdo = (uint32_t)BQ * dov.rs;  // bytes per query tile

  float sv = 0.f;
  if (t0 < n) {
    QT::issue(rq, t0 * tq, qa0, wave, w.lane, qv.rs);
    QT::issue(rdo, t0 * tdo, da0, wave, w.lane, dov.rs);
    sv = load_stats16<BQ>(rl, rd, t0 * BQ, wave, w.lane);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  put_stats16<BQ>(st0, sv, wave, w.lane);
  barrier();
  // tile t in (cq, cd, cs); tile t + 1 loaded into (nq, nd, ns)
  auto step = [&](int t, const char* cq, const char* cd, const float* cs, char* nq, char* nd, float* ns) {
    if (t + 1 < n) {
      QT::issue(rq, (t + 1) * tq, nq, wave, w.lane, qv.rs);
      QT::issue(rdo, (t + 1) * tdo, nd, wave, w.lane, dov.rs);
      sv = load_stats16<BQ>(rl, rd, (t + 1) * BQ, wave, w.lane);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (w.active(t * BQ)) w.step(cq, cd, cs, t * BQ);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if (t + 1 < n) put_stats16<BQ>(ns, sv, wave, w.lane);
    barrier();
  };
  for (int t = t0; t < n; t += 2) {
    step(t, qa0, da0, st0, qa1, da1, st1);
    if (t + 1 >= n) break;
    step(t + 1, qa1, da1, st1, qa0, da0, st0);
  }
  store_row16<T, D>(w.dk, p.scale, dkv, w.myk, w.g);
  store_row16<T, D>(w.dv, 1.0f, dvv, w.myk, w.g);
}

// ------------------------------------------------------------------ launch

// Wavefronts per dq_kernel work-group: eight (two per SIMD) up to d = 128;
// wider heads need a SIMD's whole register file per wavefront.
template <int D>
constexpr int dq_waves() { return D > 128 ? 4 : 8; }
template <int D>
constexpr int dq_key_tile() { return D == 64 ? 64 : 32; }
template <int D>
constexpr int dkdv_query_tile() { return D == 64 ? 64 : 32; }
// The 16-key dK/dV kernel (d >= 128): four wavefronts (64 keys) per
// work-group, 32-query tiles; three work-groups per CU at d = 128, two at
// d = 192 and 256.
template <int D>
constexpr int dkdv16_waves() { return 4; }
template <int D>
constexpr int dkdv16_query_tile() { return 32; }

template <typename T, int D, bool CAUSAL, bool STRIDED>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  BwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.dout = a.dout;
  p.lse = a.lse;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.delta = a.delta;
  p.BH = a.B * a.H;
  p.S = a.S;
  p.Sk = a.Sk;
  // Non-causal: shift = Sk keeps every key (j < Sk <= i + Sk).  The
  // non-causal instantiations ignore it; wide heads run the causal ones with
  // it (see launch_bwd_s).
  p.shift = a.causal ? a.Sk - a.S : a.Sk;
  p.scale = a.scale;
  p.c = a.scale * kLog2e;
  p.H = a.H;
  if (STRIDED)  // q, k, v, o, dout, dq, dk, dv: batch, head, row (elements)
    for (int t = 0; t < 8; ++t) {
      p.sb[t] = a.strides[3 * t];
      p.sh[t] = a.strides[3 * t + 1];
      p.rs[t] = (uint32_t)(a.strides[3 * t + 2] * 2);
    }

  constexpr int kDqWaves = dq_waves<D>();
  constexpr int BM = kDqWaves * 32;
  constexpr int BN = dq_key_tile<D>();
  // no query rows: no dq_kernel (nothing to write); no key rows: no
  // dkdv_kernel (the dq_kernel then writes dq = 0 and delta)
  p.nblk = (a.S + BM - 1) / BM;
  const bool tail = a.Sk % BN != 0;
  // A ragged non-causal d = 128 problem runs the causal tail variant (shift
  // = Sk keeps every key): the non-causal one spills.
  constexpr bool kTailCausal = CAUSAL || D == 128;
  if (p.nblk > 0) {
    if (tail)
      hipLaunchKernelGGL((dq_kernel<T, D, kTailCausal, true, kDqWaves, BN, STRIDED>),
                         dim3((unsigned)(p.nblk * p.BH)), dim3(kDqWaves * 64), 0, stream, p);
    else
      hipLaunchKernelGGL((dq_kernel<T, D, CAUSAL, false, kDqWaves, BN, STRIDED>), dim3((unsigned)(p.nblk * p.BH)),
                         dim3(kDqWaves * 64), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  if constexpr (D >= 128) {
    // Non-causal problems run the causal code with shift = Sk (every key
    // kept): at d = 128 the non-causal instantiation needs more registers
    // than three wavefronts per SIMD allow (40-64 B of spill).
    constexpr int NW = dkdv16_waves<D>();
    constexpr int BK = NW * 16;
    p.nblk = (a.Sk + BK - 1) / BK;
    if (p.nblk == 0) return hipSuccess;
    hipLaunchKernelGGL((dkdv16_kernel<T, D, true, NW, dkdv16_query_tile<D>(), STRIDED>), dim3((unsigned)(p.nblk * p.BH)),
                       dim3(NW * 64), 0, stream, p);
    return hipGetLastError();
  } else {
    constexpr int NW = dkdv_waves<D>();
    constexpr int BK = NW * 32;
    p.nblk = (a.Sk + BK - 1) / BK;
    if (p.nblk == 0) return hipSuccess;
    hipLaunchKernelGGL((dkdv_kernel<T, D, CAUSAL, NW, dkdv_query_tile<D>(), STRIDED>),
                       dim3((unsigned)(p.nblk * p.BH)), dim3(NW * 64), 0, stream, p);
    return hipGetLastError();
  }
}

template <typename T, int D, bool STRIDED>
hipError_t launch_bwd_s(const BwdArgs& a, hipStream_t stream) {
  // Wide heads (d = 192, 256) have only causal instantiations: without a
  // mask the compiler keeps more fragments in flight than the register file
  // holds and spills, while the causal code with shift = Sk (every key kept,
  // so every tile takes the unmasked path) computes the same.
  if constexpr (D > 128)
    return launch_bwd_t<T, D, true, STRIDED>(a, stream);
  else
    return a.causal ? launch_bwd_t<T, D, true, STRIDED>(a, stream) : launch_bwd_t<T, D, false, STRIDED>(a, stream);
}

template <typename T, int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
  return a.strides ? launch_bwd_s<T, D, true>(a, stream) : launch_bwd_s<T, D, false>(a, stream);
}

template <typename T>
hipError_t launch_bwd_dtype(const BwdArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 64: return launch_bwd_d<T, 64>(a, stream);
    case 128: return launch_bwd_d<T, 128>(a, stream);
    case 192: return launch_bwd_d<T, 192>(a, stream);
    default: return launch_bwd_d<T, 256>(a, stream);
  }
}

}  // namespace bwd

long long bwd_grid_size(const BwdArgs& a) {
  const long long bh = (long long)a.B * a.H;
  const int bm = (a.d > 128 ? bwd::dq_waves<256>() : bwd::dq_waves<64>()) * 32;
  const long long dq = (long long)((a.S + bm - 1) / bm) * bh;
  const int bk = a.d == 64 ? bwd::dkdv_waves<64>() * 32 : bwd::dkdv16_waves<128>() * 16;
  const long long dkdv = (long long)((a.Sk + bk - 1) / bk) * bh;
  return dq > dkdv ? dq : dkdv;
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  return a.dtype == 1 ? bwd::launch_bwd_dtype<__bf16>(a, stream) : bwd::launch_bwd_dtype<_Float16>(a, stream);
}

}  // namespace fa
