// gfx950 kernels of the split-key forward pass for short query blocks
// (token-by-token decoding).
//
// The pages set decoding apart from the processing of a whole prompt: the two
// are bound by different things (IPLEX blog "FlashAttention-2: making
// long-context attention run efficiently on GPUs", section "Document the
// implementation difference").  With a handful of new queries over a long
// key sequence there is almost no arithmetic per byte of K and V (about Sq
// flops per byte), so the pass is bound by HBM bandwidth, and the prefill
// grid of one work-group per 256-row query block and head leaves most of the
// chip idle.  This path therefore also splits the KEYS, which is the
// FlashAttention-2 "sequence parallelism" applied to the other sequence axis:
//
// * decode_kernel: work-group = (head, 32-row query block, key split).  Its
//   NW wavefronts load shared tiles of 32*NW*BPW keys HBM -> LDS with
//   buffer_load ... lds; wavefront w takes the 32-key blocks w*BPW .. of each
//   tile and keeps its own online softmax over the keys it saw (the same MFMA
//   score / output products and softmax as the prefill kernel).  At the end the
//   wavefronts' results are merged through LDS and the work-group writes one
//   normalised partial output and partial LSE (fp32) per query row to a
//   caller-provided workspace: no atomics.
// * merge_kernel: one wavefront per (head, query row) combines the P
//   partials exactly: LSE = ln sum_p exp(LSE_p) and O = sum_p exp(LSE_p - LSE)
//   O_p.  Partials of key subsets a row cannot see have LSE_p = -inf and drop
//   out; a row that sees no key at all gets O = 0, LSE = -inf.
//
// The key subsets of the partials are disjoint and cover every key, so the
// merge gives the whole softmax: softmax over a union of disjoint sets is the
// LSE-weighted mix of the per-set softmaxes.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "fa_device.h"
#include "fa_fwd_wave.h"
#include "fa_launch.h"

namespace fa {
namespace detail {

struct DecParams {
  const void* q;
  const void* k;
  const void* v;
  float* po;        // partial outputs [BH][P][Sq][D]
  float* pl;        // partial LSEs    [BH][P][Sq]
  int Sq, Sk;
  int shift;        // causal offset Sk - Sq (0 when not causal)
  int nrb;          // 32-row query blocks per head
  int nsplit;       // key splits per head
  int split_tiles;  // key tiles per split
  float c;          // scale * log2(e)
  // strided layouts only: heads per batch entry, batch / head strides
  // (elements) and row strides (bytes) of q, k, v
  int H;
  long long qsb, qsh, ksb, ksh, vsb, vsh;
  uint32_t q_rs, k_rs, v_rs;
};

struct MergeParams {
  const float* po;
  const float* pl;
  void* o;
  float* lse;
  int rows;         // B * H * Sq
  int Sq;
  int P;            // partials per head
  int H;
  long long osb, osh, osr;  // element strides of o: batch, head, row
};

// Work-groups per compute unit that LDS allows (K and V tiles of
// 32 * NW * BPW keys, 160 KiB per compute unit); the register budget is set
// to match, at most 4
// wavefronts per SIMD (128 registers), or 3 for the masked d = 64 variants,
// which need about 132.
template <int D, int NW, int BPW>
constexpr int decode_groups_per_cu() { return (160 * 1024) / (2 * 32 * NW * BPW * D * 2); }
template <int D, int NW, int BPW, bool MASKS>
constexpr int decode_waves_per_simd() {
  return decode_groups_per_cu<D, NW, BPW>() * NW / 4 < (MASKS ? 3 : 8) ? decode_groups_per_cu<D, NW, BPW>() * NW / 4
                                                                       : (MASKS ? 3 : 8);
}

template <typename T, int D, bool CAUSAL, bool TAIL, int NW, int BPW, bool STRIDED>
__global__ __launch_bounds__(NW * 64, (decode_waves_per_simd<D, NW, BPW, CAUSAL || TAIL>())) void decode_kernel(
    DecParams p) {
  // one 32-key block per wavefront (its own loaders unused)
  using W = FwdWave<T, D, CAUSAL, TAIL, 1, 32, STRIDED>;
  constexpr int BN = 32 * NW * BPW;                        // keys per shared tile
  using L = FwdWave<T, D, CAUSAL, TAIL, NW, BN, STRIDED>;  // the tile loaders
  constexpr int BLOCK = 32 * W::ROW_BYTES;        // one wavefront's block of a tile
  __shared__ __attribute__((aligned(1024))) char k_lds[L::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds[L::TILE_BYTES];

  const int split = blockIdx.x % p.nsplit;
  const int rest = blockIdx.x / p.nsplit;
  const int rb = rest % p.nrb;
  const int bh = rest / p.nrb;

  W w;
  w.lane = threadIdx.x & 63;
  w.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar partial address
  w.h = w.lane >> 5;
  w.col = w.lane & 31;
  w.qw = rb * 32;
  w.myq = w.qw + w.col;
  w.S = p.Sq;
  w.Sk = p.Sk;
  w.shift = p.shift;
  w.c = p.c;
  L ld;
  if constexpr (STRIDED) {
    const int b = bh / p.H, hh = bh - b * p.H;
    w.q_rs = p.q_rs;
    w.head_bytes = (uint32_t)(p.Sq - 1) * p.q_rs + W::ROW_BYTES;
    ld.k_rs = p.k_rs;
    ld.v_rs = p.v_rs;
    ld.kv_head_bytes = p.Sk > 0 ? (uint32_t)(p.Sk - 1) * p.k_rs + W::ROW_BYTES : 0u;
    ld.v_bytes = p.Sk > 0 ? (uint32_t)(p.Sk - 1) * p.v_rs + W::ROW_BYTES : 0u;
    ld.kh = (const char*)p.k + (b * p.ksb + hh * p.ksh) * 2;
    ld.vh = (const char*)p.v + (b * p.vsb + hh * p.vsh) * 2;
    w.load_q((const char*)p.q + (b * p.qsb + hh * p.qsh) * 2);
  } else {
    w.head_bytes = (uint32_t)p.Sq * W::ROW_BYTES;
    ld.kv_head_bytes = (uint32_t)p.Sk * W::ROW_BYTES;
    const size_t kv_head_elems = (size_t)bh * p.Sk * D;
    ld.kh = (const char*)p.k + kv_head_elems * 2;
    ld.vh = (const char*)p.v + kv_head_elems * 2;
    w.load_q((const char*)p.q + (size_t)bh * p.Sq * D * 2);
  }
  ld.lane = w.lane;
  ld.wave = w.wave;

  // tiles [t_lo, t_hi) of this split; causal: none past the block's last row
  const int kv_end = CAUSAL ? min(p.Sk, w.qw + 32 + p.shift) : p.Sk;
  const int t_lo = split * p.split_tiles;
  const int t_hi = min(kv_end > 0 ? (kv_end + BN - 1) / BN : 0, t_lo + p.split_tiles);

  // One LDS stage: load a tile, wait, compute it, release it.  The compute is
  // short next to the load, and the other work-groups on the compute unit
  // keep HBM busy meanwhile, so a second stage would only halve the bytes in
  // flight per work-group.
  for (int t = t_lo; t < t_hi; ++t) {
    ld.issue_k(t, k_lds);
    ld.issue_v(t, v_lds);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    barrier();
#pragma unroll
    for (int b = 0; b < BPW; ++b) {
      const int blk = w.wave * BPW + b;  // this wavefront's blocks are adjacent
      const int k0 = t * BN + blk * 32;
      if (k0 < p.Sk && w.active(k0)) {
        w.scores(k_lds + blk * BLOCK);
        w.softmax(k0);
        w.pv(v_lds + blk * BLOCK);
      }
    }
    barrier();
  }

  // Combine the NW wavefronts' results in log2(NW) rounds through LDS (the
  // tiles are free now).  Each wavefront first normalises its own: O_w =
  // O_acc / l_w and LSE_w per row.  In a round with `half` active pairs,
  // wavefront w + half stages O_w and LSE_w lane-major (every lane writes and
  // its partner lane reads the same 16-byte slots, so no bank conflicts) and
  // wavefront w merges them into its registers:
  //   M = max(LSE_a, LSE_b), LSE = M + ln(e^(LSE_a - M) + e^(LSE_b - M)),
  //   O = (e^(LSE_a - M) O_a + e^(LSE_b - M) O_b) / (e^(LSE_a - M) + e^(LSE_b - M)).
  // Wavefront 0 ends with the work-group's result and writes it as this
  // split's partial.
  constexpr int DB = W::DB;
  static_assert((NW / 2) * 64 * DB * 16 * 4 <= L::TILE_BYTES, "staging fits a tile buffer");
  float lse_w;
  {
    const float ltot = sum_with_partner(w.lsum);
    const bool none = !(ltot > 0.f);
    const float inv = none ? 0.f : 1.0f / w.out_divisor();
#pragma unroll
    for (int db = 0; db < DB; ++db) w.oacc[db] *= inv;
    lse_w = none ? -__builtin_inff() : (w.mc + __builtin_amdgcn_logf(ltot)) * 0.69314718055994531f;
  }
#pragma unroll
  for (int half = NW / 2; half >= 1; half /= 2) {
    barrier();
    if (w.wave >= half && w.wave < 2 * half) {
      f32x4* so = (f32x4*)k_lds + (w.wave - half) * 64 * DB * 4;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = w.oacc[db][4 * rg + e];
          so[(db * 4 + rg) * 64 + w.lane] = x;
        }
      ((float*)v_lds)[(w.wave - half) * 64 + w.lane] = lse_w;
    }
    barrier();
    if (w.wave < half) {
      const f32x4* so = (const f32x4*)k_lds + w.wave * 64 * DB * 4;
      const float lse_p = ((const float*)v_lds)[w.wave * 64 + w.lane];
      const float m = fmaxf(lse_w, lse_p);
      const bool none = m == -__builtin_inff();
      const float a = none ? 0.f : __builtin_amdgcn_exp2f((lse_w - m) * 1.4426950408889634f);
      const float b = none ? 0.f : __builtin_amdgcn_exp2f((lse_p - m) * 1.4426950408889634f);
      const float inv = none ? 0.f : 1.0f / (a + b);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const f32x4 x = so[(db * 4 + rg) * 64 + w.lane];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w.oacc[db][4 * rg + e] = (a * w.oacc[db][4 * rg + e] + b * x[e]) * inv;
        }
      lse_w = none ? -__builtin_inff() : m + __builtin_amdgcn_logf(a + b) * 0.69314718055994531f;
    }
  }
  if (w.wave == 0) {
    // this split's partial: rows [qw, qw + 32) of [Sq][D] (rows >= Sq dropped
    // by the range checks)
    const size_t part = ((size_t)bh * p.nsplit + split) * p.Sq;
    const __amdgpu_buffer_rsrc_t ro = rsrc(p.po + part * D, (uint32_t)p.Sq * D * 4);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        // (a whole-vector bit_cast: bit_cast of a single vector element
        // miscompiles to element 0 with this toolchain)
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = w.oacc[db][4 * rg + e];
        const int dcol = db * 32 + 8 * rg + 4 * w.h;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, y), ro, ((uint32_t)w.myq * D + dcol) * 4, 0,
                                               0);
      }
    if (w.h == 0) {
      const __amdgpu_buffer_rsrc_t rl = rsrc(p.pl + part, (uint32_t)p.Sq * 4);
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, lse_w), rl, (uint32_t)w.myq * 4, 0, 0);
    }
  }
}

// One wavefront per (head, query row): LSE = M + ln sum_p exp(LSE_p - M) with
// M = max_p LSE_p, O = sum_p exp(LSE_p - LSE) O_p.  Lane l holds d-columns
// l * D/64 .. +D/64.
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  constexpr int E = D / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const int bh = row / p.Sq, i = row % p.Sq;
  const float* pl = p.pl + (size_t)bh * p.P * p.Sq + i;
  const float* po = p.po + ((size_t)bh * p.P * p.Sq + i) * D + lane * E;
  const size_t ostride = (size_t)p.Sq * D;

  float m = -__builtin_inff();
#pragma unroll 8
  for (int q = 0; q < p.P; ++q) m = fmaxf(m, pl[(size_t)q * p.Sq]);
  float acc[E] = {};
  float sum = 0.f;
  if (m != -__builtin_inff()) {
#pragma unroll 8
    for (int q = 0; q < p.P; ++q) {
      const float wq = __builtin_amdgcn_exp2f((pl[(size_t)q * p.Sq] - m) * 1.4426950408889634f);
      sum += wq;
      const float* src = po + q * ostride;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(wq, src[e], acc[e]);
    }
  }
  const bool none = !(sum > 0.f);
  const float inv = none ? 0.f : 1.0f / sum;
  const int b = bh / p.H, hh = bh - b * p.H;
  T* out = (T*)p.o + b * p.osb + hh * p.osh + i * p.osr + lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) out[e] = (T)(acc[e] * inv);
  if (lane == 0) p.lse[row] = none ? -__builtin_inff() : m + __builtin_amdgcn_logf(sum) * 0.69314718055994531f;
}

// ------------------------------------------------ one query row (S_q = 1)
//
// With a single query row the scores are a matrix-vector product, so the
// key and value rows go straight from HBM into registers (no LDS stage, no
// MFMA), with the split plan, partial layout and merge of the kernel above.
// Work-group = 4 wavefronts on one (head, key split).  One wavefront
// instruction loads 1 KiB of whole rows: lane l holds 16-byte chunk l % LPR
// of row l / LPR (LPR = lanes per row), U instructions each of K and V in
// flight.  A row's score is the sum of its lanes' v_dot2 partial products
// (DPP exchanges within the row's lanes).  Each lane keeps an online softmax
// over the rows it sees: a reference max that trails the running max by at
// most kDec1Margin binary orders (moved, with a rescale, only when a score
// passes it), its row sum and the 8 output columns of its chunk.  The
// 4 * (64 / LPR) streams of the work-group are merged through LDS at the end
// into the split's partial row and LSE.

constexpr float kDec1Margin = 8.0f;
// Cache policy of the row loads: non-temporal (each K / V byte is read once).
// Measured on the MI355X (1 GiB caches): 6.7 TB/s against 5.9 TB/s with the
// default policy.
constexpr int kDecode1LoadAux = 2;

template <typename T>
struct Dec1Elem;
template <>
struct Dec1Elem<__bf16> {
  static __device__ __forceinline__ float dot2(unsigned a, unsigned b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
  }
  static __device__ __forceinline__ float lo(unsigned x) { return __builtin_bit_cast(float, x << 16); }
  static __device__ __forceinline__ float hi(unsigned x) { return __builtin_bit_cast(float, x & 0xffff0000u); }
};
template <>
struct Dec1Elem<_Float16> {
  static __device__ __forceinline__ float dot2(unsigned a, unsigned b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
  }
  static __device__ __forceinline__ float lo(unsigned x) { return (float)__builtin_bit_cast(f16x2, x)[0]; }
  static __device__ __forceinline__ float hi(unsigned x) { return (float)__builtin_bit_cast(f16x2, x)[1]; }
};

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// Sum over each aligned group of LPR (8 or 16) lanes, in every lane of it:
// swaps within pairs and quads, then the half-row and row mirrors.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f32<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_f32<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_f32<0x141>(x);  // row_half_mirror: lane i <-> 7 - i of each 8
  if constexpr (LPR == 16) x += dpp_f32<0x140>(x);  // row_mirror: lane i <-> 15 - i of each 16
  return x;
}

template <typename T, int D, int U, bool STRIDED>
__global__ __launch_bounds__(256) void decode1_kernel(DecParams p) {
  constexpr int ROW = D * 2;         // bytes per key / value row
  constexpr int LPR = ROW / 16;      // lanes per row
  constexpr int RPI = 64 / LPR;      // rows per wavefront instruction
  constexpr int ITER = 4 * U * RPI;  // rows per work-group iteration
  constexpr int STREAMS = 4 * RPI;
  static_assert(LPR == 8 || LPR == 16, "d = 64 or 128");
  static_assert((decode_tile_keys(D) * 1) % ITER == 0, "a split is a whole number of iterations");
  using E = Dec1Elem<T>;
  __shared__ float s_m[STREAMS], s_l[STREAMS];
  __shared__ __attribute__((aligned(16))) float s_o[STREAMS * D];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int chunk = lane % LPR, sub = lane / LPR;
  const int split = blockIdx.x % p.nsplit;
  const int bh = blockIdx.x / p.nsplit;  // one 32-row query block per head (S_q = 1)

  const char* qh;
  const char* kh;
  const char* vh;
  uint32_t k_rs = ROW, v_rs = ROW, k_bytes, v_bytes;
  if constexpr (STRIDED) {
    const int b = bh / p.H, hh = bh - b * p.H;
    qh = (const char*)p.q + (b * p.qsb + hh * p.qsh) * 2;
    kh = (const char*)p.k + (b * p.ksb + hh * p.ksh) * 2;
    vh = (const char*)p.v + (b * p.vsb + hh * p.vsh) * 2;
    k_rs = p.k_rs;
    v_rs = p.v_rs;
    k_bytes = p.Sk > 0 ? (uint32_t)(p.Sk - 1) * k_rs + ROW : 0u;
    v_bytes = p.Sk > 0 ? (uint32_t)(p.Sk - 1) * v_rs + ROW : 0u;
  } else {
    qh = (const char*)p.q + (size_t)bh * D * 2;
    kh = (const char*)p.k + (size_t)bh * p.Sk * D * 2;
    vh = (const char*)p.v + (size_t)bh * p.Sk * D * 2;
    k_bytes = v_bytes = (uint32_t)p.Sk * ROW;
  }
  const __amdgpu_buffer_rsrc_t rk = rsrc(kh, k_bytes), rv = rsrc(vh, v_bytes);
  const u32x4 qc = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc(qh, ROW), chunk * 16, 0, 0));

  const int k_begin = split * p.split_tiles * decode_tile_keys(D);
  const int k_end = min(p.Sk, k_begin + p.split_tiles * decode_tile_keys(D));
  float m = -__builtin_inff();  // reference max, log2 units (scores times c)
  float l = 0.f;
  float o[8] = {};
  // rows of an iteration starting at r0 (past the split: an offset past the
  // range, so they read as 0 without touching memory, and are masked)
  auto load = [&](int r0, u32x4 (&kx)[U], u32x4 (&vx)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = r0 + (wave * U + u) * RPI + sub;
      const bool ok = row < k_end;
      kx[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rk, ok ? (uint32_t)row * k_rs + chunk * 16 : k_bytes, 0, kDecode1LoadAux));
      vx[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rv, ok ? (uint32_t)row * v_rs + chunk * 16 : v_bytes, 0, kDecode1LoadAux));
    }
  };
  auto compute = [&](int r0, const u32x4 (&kx)[U], const u32x4 (&vx)[U]) {
    float x[U];
    float xm = -__builtin_inff();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = r0 + (wave * U + u) * RPI + sub;
      float sp = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) sp = E::dot2(qc[j], kx[u][j], sp);
      const float sc = group_sum<LPR>(sp);
      x[u] = row < k_end ? sc * p.c : -__builtin_inff();
      xm = fmaxf(xm, x[u]);
    }
    const bool grow = xm > m + kDec1Margin;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float mn = grow ? xm : m;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m - mn) : 1.f;  // 0 for the first rows (m = -inf)
      l *= alpha;
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] *= alpha;
      m = mn;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float pu = x[u] != -__builtin_inff() ? __builtin_amdgcn_exp2f(x[u] - m) : 0.f;
      l += pu;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[2 * j] = __builtin_fmaf(pu, E::lo(vx[u][j]), o[2 * j]);
        o[2 * j + 1] = __builtin_fmaf(pu, E::hi(vx[u][j]), o[2 * j + 1]);
      }
    }
  };
  // two register buffers: the next iteration's rows load while this one is
  // computed (an iteration wholly past the split computes masked zeros)
  u32x4 ka[U], va[U], kb[U], vb[U];
  load(k_begin, ka, va);
  for (int r0 = k_begin; r0 < k_end; r0 += 2 * ITER) {
    load(r0 + ITER, kb, vb);
    compute(r0, ka, va);
    load(r0 + 2 * ITER, ka, va);
    compute(r0 + ITER, kb, vb);
  }

  // merge the streams: M = max of their references, L = sum 2^(m_s - M) l_s,
  // O = sum 2^(m_s - M) o_s / L, LSE = (M + log2 L) ln 2
  const int stream = wave * RPI + sub;
  if (chunk == 0) {
    s_m[stream] = m;
    s_l[stream] = l;
  }
  f32x4* dst = (f32x4*)(s_o + stream * D + chunk * 8);
  dst[0] = f32x4{o[0], o[1], o[2], o[3]};
  dst[1] = f32x4{o[4], o[5], o[6], o[7]};
  barrier();
  if (threadIdx.x < D) {
    const int col = threadIdx.x;
    float M = -__builtin_inff();
#pragma unroll
    for (int t = 0; t < STREAMS; ++t) M = fmaxf(M, s_l[t] > 0.f ? s_m[t] : -__builtin_inff());
    float L = 0.f, acc = 0.f;
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int t = 0; t < STREAMS; ++t) {
        const float wt = s_l[t] > 0.f ? __builtin_amdgcn_exp2f(s_m[t] - M) : 0.f;
        L = __builtin_fmaf(wt, s_l[t], L);
        acc = __builtin_fmaf(wt, s_o[t * D + col], acc);
      }
    }
    const bool none = !(L > 0.f);
    const size_t part = (size_t)bh * p.nsplit + split;
    p.po[part * D + col] = none ? 0.f : acc / L;
    if (col == 0) p.pl[part] = none ? -__builtin_inff() : (M + __builtin_amdgcn_logf(L)) * 0.69314718055994531f;
  }
}

// Wavefronts and blocks per wavefront; LDS per work-group is
// 2 * 32 * NW * BPW * D * 2 bytes (K and V tiles).
template <int D>
struct DecodeShape {
  static constexpr int NW = decode_waves(D);
  static constexpr int BPW = decode_blocks_per_wave(D);
};

template <typename T, int D, bool CAUSAL, bool TAIL, bool STRIDED>
hipError_t launch_decode_t(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream) {
  constexpr int NW = DecodeShape<D>::NW, BPW = DecodeShape<D>::BPW;
  // a single query row at d = 64 / 128 runs decode1_kernel (any mask keeps
  // every key of it; see launch_decode_s)
  constexpr bool kDec1 = (D == 64 || D == 128) && !CAUSAL;
  constexpr int kDec1Unroll = 4;
  DecParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.po = (float*)a.workspace;
  p.pl = (float*)((char*)a.workspace + plan.partial_o_bytes);
  p.Sq = a.Sq;
  p.Sk = a.Sk;
  p.shift = a.causal ? a.Sk - a.Sq : 0;
  p.nrb = plan.nrb;
  p.nsplit = plan.nsplit;
  p.split_tiles = plan.split_tiles;
  p.c = a.scale * 1.4426950408889634f;
  p.H = a.H;
  // o's element strides (batch, head, row), for the merge
  long long osb = (long long)a.H * a.Sq * D, osh = (long long)a.Sq * D, osr = D;
  if (STRIDED) {
    const long long* st = a.strides;  // q, k, v, o: batch, head, row (elements)
    p.qsb = st[0]; p.qsh = st[1]; p.q_rs = (uint32_t)(st[2] * 2);
    p.ksb = st[3]; p.ksh = st[4]; p.k_rs = (uint32_t)(st[5] * 2);
    p.vsb = st[6]; p.vsh = st[7]; p.v_rs = (uint32_t)(st[8] * 2);
    osb = st[9]; osh = st[10]; osr = st[11];
  }
  const long long grid = (long long)a.B * a.H * plan.nrb * plan.nsplit;
  bool one_row = false;
  if constexpr (kDec1) {
    if (a.Sq == 1) {
      one_row = true;
      hipLaunchKernelGGL((decode1_kernel<T, D, kDec1Unroll, STRIDED>), dim3((unsigned)grid), dim3(256), 0, stream, p);
    }
  }
  if (!one_row)
    hipLaunchKernelGGL((decode_kernel<T, D, CAUSAL, TAIL, NW, BPW, STRIDED>), dim3((unsigned)grid), dim3(NW * 64), 0,
                       stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MergeParams m;
  m.po = p.po;
  m.pl = p.pl;
  m.o = a.o;
  m.lse = a.lse;
  m.rows = a.B * a.H * a.Sq;
  m.Sq = a.Sq;
  m.P = plan.partials;
  m.H = a.H;
  m.osb = osb;
  m.osh = osh;
  m.osr = osr;
  hipLaunchKernelGGL((merge_kernel<T, D>), dim3((unsigned)((m.rows + 3) / 4)), dim3(256), 0, stream, m);
  return hipGetLastError();
}

template <typename T, int D, bool STRIDED>
hipError_t launch_decode_s(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream) {
  const bool tail = a.Sk % 32 != 0;
  // End-aligned, the causal mask keeps every key of a single query row, so
  // Sq = 1 (the usual decoding step) runs the unmasked kernel.
  if (a.causal && a.Sq > 1)
    return tail ? launch_decode_t<T, D, true, true, STRIDED>(a, plan, stream)
                : launch_decode_t<T, D, true, false, STRIDED>(a, plan, stream);
  return tail ? launch_decode_t<T, D, false, true, STRIDED>(a, plan, stream)
              : launch_decode_t<T, D, false, false, STRIDED>(a, plan, stream);
}

template <typename T, int D>
hipError_t launch_decode_d(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream) {
  return a.strides ? launch_decode_s<T, D, true>(a, plan, stream) : launch_decode_s<T, D, false>(a, plan, stream);
}

template <typename T>
hipError_t launch_decode_dt(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream) {
  switch (a.d) {
    case 64: return launch_decode_d<T, 64>(a, plan, stream);
    case 128: return launch_decode_d<T, 128>(a, plan, stream);
    case 192: return launch_decode_d<T, 192>(a, plan, stream);
    default: return launch_decode_d<T, 256>(a, plan, stream);
  }
}

}  // namespace detail

using namespace detail;

DecodePlan decode_plan(const DecodeArgs& a) {
  DecodePlan plan{};
  const int BN = decode_tile_keys(a.d);
  const long long heads = (long long)a.B * a.H;
  plan.nrb = (a.Sq + 31) / 32;
  const int tiles = (a.Sk + BN - 1) / BN;
  // Enough work-groups for several per compute unit, but at least
  // kMinSplitTiles tiles per split so the ring has something to overlap.
  const long long blocks = heads * plan.nrb;
  long long want = blocks > 0 ? (kDecodeTargetGroups + blocks - 1) / blocks : 1;
  const long long most = tiles / kMinSplitTiles > 1 ? tiles / kMinSplitTiles : 1;
  if (want > most) want = most;
  if (want < 1) want = 1;
  plan.split_tiles = tiles > 0 ? (int)((tiles + want - 1) / want) : 1;
  plan.nsplit = tiles > 0 ? (tiles + plan.split_tiles - 1) / plan.split_tiles : 1;
  plan.partials = plan.nsplit;
  plan.partial_o_bytes = (size_t)heads * plan.partials * a.Sq * a.d * 4;
  plan.workspace_bytes = plan.partial_o_bytes + (size_t)heads * plan.partials * a.Sq * 4;
  plan.grid = heads * plan.nrb * plan.nsplit;
  return plan;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream) {
  if (a.dtype == 1)
    return launch_decode_dt<__bf16>(a, plan, stream);
  return launch_decode_dt<_Float16>(a, plan, stream);
}

namespace {

// The partial results of fa_fwd_decode_noalloc.  Host code never uses this
// name as an address (on the host it is only a stand-in for the symbol):
// each device's copy is found with hipGetSymbolAddress and that pointer is
// what the kernels receive.
__device__ __align__(256) char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

void* decode_scratch(hipStream_t stream, hipError_t* err) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    // with the stream's device current, as the symbol lookup requires
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess || (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)) {
      *err = e;
      return nullptr;
    }
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess || !ptr) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *err = hipSuccess;
  return g_scratch_ptr[dev];
}

}  // namespace fa
