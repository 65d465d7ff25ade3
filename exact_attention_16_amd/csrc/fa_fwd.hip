// gfx950 (CDNA4) kernels of the exact-attention forward pass.
//
// Method (FlashAttention-2 pages): the output is exact attention (searcharxiv
// abstract page, "Abstract"), computed tile by tile with an online softmax
// that keeps running row statistics and rescales the partial output (IPLEX
// blog "FlashAttention-2: making long-context attention run efficiently on
// GPUs", section "Tiling preserves the attention calculation"), so the S x S
// scores never reach HBM.  The three FlashAttention-2 changes (same blog,
// section "Three changes improve GPU utilisation"; abstract items (1)-(3)):
//   (1) less non-matmul work: the 1/l normalisation is deferred to the
//       epilogue, the partial output is rescaled only when a row maximum has
//       grown by more than a fixed margin, key tiles wholly above the causal
//       diagonal are never loaded or computed, and mask arithmetic runs only on
//       tiles that cross the diagonal or the sequence end;
//   (2) the grid covers (query-row block, head, batch), so even one head is
//       spread over many compute units;
//   (3) the wavefronts of a work-group split the query rows and share the K/V
//       tiles staged in LDS; each wavefront owns its rows' statistics and
//       output outright, so nothing is reduced through LDS.
//
// MI355X mapping (own design, not the pages'): one wavefront owns 32 query
// rows.  It computes the transposed score tile S^T = K Q^T with
// v_mfma_f32_32x32x16_{bf16,f16} (A = K rows from LDS, B = Q rows held in
// VGPRs), so every lane holds scores of ONE query: the row max and row sum are
// in-lane, plus one exchange with lane l^32 (v_permlane32_swap).  The output
// is accumulated transposed too, O^T += V^T P^T: B = P straight from the score
// accumulator (no shuffle), A = V^T read with ds_read_b64_tr_b16 (gfx950's
// transposing LDS read), and the per-row rescale and 1/l are per-lane scalars.
// K and V tiles go HBM -> LDS with buffer_load_dwordx4 ... lds (no VGPR
// staging), double-buffered, XOR-swizzled in 16-byte chunks against LDS bank
// conflicts; out-of-range rows read as zero and out-of-range stores are
// dropped by the buffer descriptors' range checks.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_launch.h"

namespace fa {
namespace detail {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
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
// The partial output is rescaled only when a row max grows by more than this
// many binary orders of magnitude, so unnormalised weights stay <= 2^8.
constexpr float kRescaleMargin = 8.0f;

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
};

struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int BH;      // B * H
  int S;
  int nqb;     // query-row blocks per head
  float c;     // scale * log2(e): scores enter exp2 as c * s
};

// XOR swizzle of the 16-byte chunk index inside a tile row, per tile.
// K rows are read 16 B per lane (ds_read_b128) with 32 lanes on one logical
// chunk of 32 consecutive rows; V rows are read 8 B per lane by the
// transposing read, 4 rows x 64 B per half-wave.  Each swizzle spreads those
// accesses over distinct 16-byte bank groups of a 256-byte bank row.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

// Value of x held by lane l^32.  v_permlane32_swap exchanges the upper half
// of its first operand with the lower half of its second; called with two
// copies of x, lanes 0-31 find the partner's value in the second result and
// lanes 32-63 in the first.  The copy is made opaque because the compiler
// otherwise folds the two identical operands and returns the first result
// for both.
__device__ __forceinline__ float partner_value(float x) {
  float y;
  asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, y), false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ float max_with_partner(float x) { return fmaxf(x, partner_value(x)); }

__device__ __forceinline__ float sum_with_partner(float x) { return x + partner_value(x); }

// One wavefront's share of a work-group: 32 query rows of one (batch, head),
// their Q fragments, running statistics and output accumulator.  The
// work-group's NW wavefronts share the K/V tiles (BN keys each) in LDS.
template <typename T, int D, bool CAUSAL, int NW, int BN>
struct FwdWave {
  static constexpr int BM = NW * 32;
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int CPR = D / 8;        // 16-byte chunks per row
  static constexpr int KSTEPS = D / 16;    // MFMA k-steps of S^T over d
  static constexpr int DB = D / 32;        // 32-row blocks of O^T (over d)
  static constexpr int SB = BN / 32;       // 32-key blocks per tile
  static constexpr int TILE_BYTES = BN * ROW_BYTES;
  static constexpr int LOADS = TILE_BYTES / (NW * 64 * 16);  // 16-byte loads per lane per tile
  static_assert(LOADS * NW * 64 * 16 == TILE_BYTES, "tile must split evenly over lanes");
  static_assert(BN % 32 == 0, "BN must be a multiple of 32");

  int lane, wave, h, col;
  int qw;    // first query row of this wavefront
  int myq;   // the query row this lane holds
  int S;
  float c;   // scale * log2(e)
  const char* kh;
  const char* vh;
  uint32_t head_bytes;

  i16x8 qf[KSTEPS];
  f32x16 oacc[DB];
  float m_used;  // reference max (raw score units) the weights are taken against
  float mc;      // c * m_used
  float lsum;    // this lane's share of the row sum

  // Q rows -> VGPRs as the B operand of S^T = K Q^T (rows >= S read as 0).
  __device__ __forceinline__ void load_q(const char* qh) {
    const __amdgpu_buffer_rsrc_t rq = rsrc(qh, head_bytes);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const uint32_t off = (uint32_t)myq * ROW_BYTES + (kk * 16 + h * 8) * 2;
      qf[kk] = __builtin_bit_cast(i16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    m_used = -__builtin_inff();
    mc = 0.f;
    lsum = 0.f;
  }

  // Start HBM -> LDS copies of key tile `tile` (K and V, BN rows each).  Each
  // wave instruction fills 1 KiB of LDS in lane order; the lane picks the
  // global 16-byte chunk that belongs at its swizzled slot.  Rows >= S read 0.
  __device__ __forceinline__ void issue_tile(int tile, char* kd, char* vd) const {
    const __amdgpu_buffer_rsrc_t rk = rsrc(kh, head_bytes);
    const __amdgpu_buffer_rsrc_t rv = rsrc(vh, head_bytes);
#pragma unroll
    for (int n = 0; n < LOADS; ++n) {
      const int slot = (n * NW + wave) * 64 + lane;
      const int row = slot / CPR;
      const int pc = slot % CPR;
      const uint32_t grow = (uint32_t)(tile * BN + row) * ROW_BYTES;
      lds_void* dk = (lds_void*)(kd + (n * NW + wave) * 1024);
      lds_void* dv = (lds_void*)(vd + (n * NW + wave) * 1024);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, dk, 16, grow + ((pc ^ swz_k<D>(row)) << 4), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, dv, 16, grow + ((pc ^ swz_v<D>(row)) << 4), 0, 0, 0);
    }
  }

  // All of the online-softmax update for the key tile starting at k0.
  __device__ __forceinline__ void compute_tile(int k0, const char* ks, const char* vs) {
    // ---- S^T = K Q^T : lane holds 16 scores of query `myq` per 32-key block
    f32x16 sacc[SB];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      sacc[sb] = f32x16{};
      const int row = sb * 32 + col;
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const int pc = (kk * 2 + h) ^ swz_k<D>(row);
        const i16x8 kf = *(const i16x8*)(ks + row * ROW_BYTES + pc * 16);
        sacc[sb] = Elem<T>::mma(kf, qf[kk], sacc[sb]);
      }
    }

    // ---- mask (only tiles crossing the diagonal or the sequence end)
    const bool masked = (CAUSAL && k0 + BN - 1 > qw) || (k0 + BN > S);
    if (masked) {
#pragma unroll
      for (int sb = 0; sb < SB; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + sb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          const bool ok = key < S && (!CAUSAL || key <= myq);
          sacc[sb][r] = ok ? sacc[sb][r] : -__builtin_inff();
        }
    }

    // ---- online softmax statistics
    float mx = -__builtin_inff();
#pragma unroll
    for (int sb = 0; sb < SB; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[sb][r]);
    mx = max_with_partner(mx);
    const float m_new = fmaxf(m_used, mx);
    const bool grow = (m_used == -__builtin_inff()) || (c * (m_new - m_used) > kRescaleMargin);
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float alpha =
          (m_used == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(c * (m_used - m_new));
      m_used = m_new;
      mc = c * m_new;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }

    // ---- P = exp2(c s - c m), packed to T as the B operand of O^T += V^T P^T
    i16x8 pf[SB][2];
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      float e[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[sb][r], c, -mc));
        if (masked) e[r] = (sacc[sb][r] == -__builtin_inff()) ? 0.f : e[r];
        lsum += e[r];
      }
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = Elem<T>::pack(e[8 * cc + 2 * i], e[8 * cc + 2 * i + 1]);
        pf[sb][cc] = __builtin_bit_cast(i16x8, w);
      }
    }

    // ---- O^T += V^T P^T ; V^T fragments by transposing LDS reads.  For chunk
    // cc of 32-key block sb, MFMA k-index h*8 + 4*tt + e stands for key
    // 32*sb + 16*cc + 8*tt + 4*h + e, matching where the score accumulator
    // put that key's weight in pf.
    const int g = lane >> 4;  // 16-lane group
    const int s16 = lane & 15;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          i16x4 half[2];
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int row = sb * 32 + cc * 16 + tt * 8 + (g >> 1) * 4 + (s16 >> 2);
            const int cv = db * 32 + (g & 1) * 16 + (s16 & 3) * 4;  // element column
            const int pc = (cv >> 3) ^ swz_v<D>(row);
            const char* a = vs + row * ROW_BYTES + pc * 16 + (cv & 7) * 2;
            half[tt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a));
          }
          const i16x8 vf = __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[db] = Elem<T>::mma(vf, pf[sb][cc], oacc[db]);
        }
      }
    }
  }

  // O = O_acc / l and LSE = (c m + log2 l) ln 2; rows >= S are dropped by the
  // descriptors' range checks.
  __device__ __forceinline__ void store(void* o, float* lse, size_t head_elems, int bh) const {
    const float ltot = sum_with_partner(lsum);
    const float inv = 1.0f / ltot;
    const __amdgpu_buffer_rsrc_t ro = rsrc((const char*)o + head_elems * 2, head_bytes);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        u32x2 w;
        w[0] = Elem<T>::pack(oacc[db][4 * rg + 0] * inv, oacc[db][4 * rg + 1] * inv);
        w[1] = Elem<T>::pack(oacc[db][4 * rg + 2] * inv, oacc[db][4 * rg + 3] * inv);
        const int dcol = db * 32 + 8 * rg + 4 * h;
        __builtin_amdgcn_raw_buffer_store_b64(w, ro, (uint32_t)myq * ROW_BYTES + dcol * 2, 0, 0);
      }
    if (h == 0) {
      const __amdgpu_buffer_rsrc_t rl = rsrc(lse + (size_t)bh * S, (uint32_t)S * 4);
      const float v = (mc + __builtin_amdgcn_logf(ltot)) * 0.69314718055994531f;
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), rl, (uint32_t)myq * 4, 0, 0);
    }
  }
};

template <typename T, int D, bool CAUSAL, int NW, int BN>
__global__ __launch_bounds__(NW * 64, 2) void fwd_kernel(Params p) {
  using W = FwdWave<T, D, CAUSAL, NW, BN>;
  // Two stages of K and V tiles as four distinct LDS objects: the tile loop is
  // unrolled by two so each access names its buffer at compile time, which
  // lets the compiler see that reads of one stage never alias the
  // direct-to-LDS loads filling the other (no spurious vmcnt waits).
  __shared__ __attribute__((aligned(1024))) char k_lds0[W::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k_lds1[W::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds0[W::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds1[W::TILE_BYTES];

  W w;
  w.lane = threadIdx.x & 63;
  w.wave = threadIdx.x >> 6;
  w.h = w.lane >> 5;
  w.col = w.lane & 31;

  // Work-group -> (query block, head).  Consecutive ids walk the heads, so the
  // query blocks of one head land on the same XCD when B*H is a multiple of 8
  // (ids are dealt to the 8 XCDs round-robin) and share its L2.  Causal:
  // the longest rows (most key tiles) are dispatched first.
  const int bh = blockIdx.x % p.BH;
  int qb = blockIdx.x / p.BH;
  if (CAUSAL) qb = p.nqb - 1 - qb;
  const int q_lo = qb * W::BM;
  w.qw = q_lo + w.wave * 32;
  w.myq = w.qw + w.col;
  w.S = p.S;
  w.c = p.c;

  const size_t head_elems = (size_t)bh * p.S * D;
  w.head_bytes = (uint32_t)p.S * W::ROW_BYTES;
  w.kh = (const char*)p.k + head_elems * 2;
  w.vh = (const char*)p.v + head_elems * 2;
  w.load_q((const char*)p.q + head_elems * 2);

  const int kv_end = CAUSAL ? min(p.S, q_lo + W::BM) : p.S;
  const int ntiles = (kv_end + BN - 1) / BN;

  // Each step: wait for this tile's loads (own wave), barrier (everyone's
  // loads landed, everyone done with the other stage), start the next tile's
  // loads into the other stage, compute on this stage.
  if (ntiles > 0) w.issue_tile(0, k_lds0, v_lds0);
  for (int t = 0; t < ntiles; t += 2) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (t + 1 < ntiles) w.issue_tile(t + 1, k_lds1, v_lds1);
    if (!(CAUSAL && t * BN > w.qw + 31)) w.compute_tile(t * BN, k_lds0, v_lds0);
    if (t + 1 < ntiles) {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
      if (t + 2 < ntiles) w.issue_tile(t + 2, k_lds0, v_lds0);
      if (!(CAUSAL && (t + 1) * BN > w.qw + 31)) w.compute_tile((t + 1) * BN, k_lds1, v_lds1);
    }
  }
  w.store(p.o, p.lse, head_elems, bh);
}

constexpr int kWaves = 4;
constexpr int kBN = 64;

template <typename T, int D, bool CAUSAL>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
  constexpr int BM = kWaves * 32;
  Params p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.BH = a.B * a.H;
  p.S = a.S;
  p.nqb = (a.S + BM - 1) / BM;
  p.c = a.scale * 1.4426950408889634f;
  const long long grid = (long long)p.nqb * p.BH;
  hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL, kWaves, kBN>), dim3((unsigned)grid), dim3(kWaves * 64), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dtype(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 64) return a.causal ? launch_t<T, 64, true>(a, stream) : launch_t<T, 64, false>(a, stream);
  return a.causal ? launch_t<T, 128, true>(a, stream) : launch_t<T, 128, false>(a, stream);
}

}  // namespace detail

using namespace detail;

long long fwd_grid_size(const FwdArgs& a) {
  const int BM = kWaves * 32;
  return (long long)((a.S + BM - 1) / BM) * a.B * a.H;
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  // dtype 0 = fp16, 1 = bf16 (fa_dtype)
  return a.dtype == 1 ? launch_dtype<__bf16>(a, stream) : launch_dtype<_Float16>(a, stream);
}

}  // namespace fa
