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
