// gfx950 in-order forward kernel: wide heads (d = 192 and 256), and short
// causal problems at d = 64 and 128.
//
// Same method and wavefront code as the d = 64 / 128 kernel in fa_fwd.hip
// (tiled exact attention with an online softmax, IPLEX blog
// "FlashAttention-2: making long-context attention run efficiently on GPUs",
// sections "Tiling preserves the attention calculation" and "Three changes
// improve GPU utilisation"): one wavefront owns 32 query rows and computes
// S^T = K Q^T and O^T += V^T P^T on MFMA over K/V tiles staged in LDS.
//
// What differs is the schedule.  A wide head's Q fragments and output
// accumulator take about 200 VGPRs (d = 256: 64 for Q, 128 for O^T), so two
// wavefronts per SIMD, which the ping-pong schedule needs, do not fit.  Here
// a work-group is four wavefronts (128 query rows), one per SIMD with the
// whole 512-entry register file, and each wavefront runs its tile in order:
// scores, softmax, P V.  The MFMA work per score grows with d while the
// softmax work does not, so at these widths the in-order schedule loses
// little.  K/V tiles (64 keys) are double-buffered in four LDS objects and
// the next tile's loads are issued before the current tile is computed.
//
// At d = 64 and 128 the same kernel runs short causal problems (the host's
// uses_in_order_kernel), at four and two wavefronts per SIMD: with only a
// few key tiles per query block, its 128-row blocks split the triangle of
// causal work more evenly over the compute units than the ping-pong
// kernel's 256-row blocks, which outweighs the lost overlap.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"
#include "fa_fwd_wave.h"
#include "fa_launch.h"

namespace fa {
namespace detail {

constexpr int kWideWaves = 4;
constexpr int kWideKeys = 64;

// Wavefronts per SIMD the register budget is sized for.
template <int D>
constexpr int wide_waves_per_simd() { return D == 64 ? 4 : D == 128 ? 2 : 1; }

template <typename T, int D, bool CAUSAL, bool TAIL, bool STRIDED>
__global__ __launch_bounds__(kWideWaves * 64, wide_waves_per_simd<D>()) void fwd_wide_kernel(Params p) {
  using W = FwdWave<T, D, CAUSAL, TAIL, kWideWaves, kWideKeys, STRIDED>;
  __shared__ __attribute__((aligned(1024))) char k_lds0[W::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k_lds1[W::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds0[W::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds1[W::TILE_BYTES];

  W w;
  w.lane = threadIdx.x & 63;
  w.wave = threadIdx.x >> 6;
  w.h = w.lane >> 5;
  w.col = w.lane & 31;
  int bh, qb;
  map_query_block<CAUSAL>(blockIdx.x, p.BH, p.nqb, bh, qb);
  const int q_lo = qb * W::BM;
  w.qw = q_lo + 32 * w.wave;
  w.myq = w.qw + w.col;
  const size_t head_elems = w.setup(p, bh);

  // keys this work-group visits (causal: up to its last row's position)
  const int kv_end = CAUSAL ? min(p.Sk, q_lo + W::BM + p.shift) : p.Sk;
  const int n = kv_end > 0 ? (kv_end + kWideKeys - 1) / kWideKeys : 0;
  w.n = n;

  if (n > 0) {
    w.issue_k(0, k_lds0);
    w.issue_v(0, v_lds0);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  barrier();
  // Tile k in buffers k % 2; tile k + 1's loads are in flight meanwhile.  The
  // loop is unrolled by two so every LDS access names its buffer, and every
  // iteration ends with all loads landed (nothing in flight across the back
  // edge), so the compiler adds no waits of its own.
  for (int k = 0; k < n; k += 2) {
    if (k + 1 < n) {
      w.issue_k(k + 1, k_lds1);
      w.issue_v(k + 1, v_lds1);
    }
    if (w.active(k * kWideKeys)) {
      __builtin_amdgcn_sched_barrier(0);
      w.scores(k_lds0);
      __builtin_amdgcn_sched_barrier(0);
      w.softmax(k * kWideKeys);
      __builtin_amdgcn_sched_barrier(0);
      w.pv(v_lds0);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    barrier();
    if (k + 1 >= n) break;
    if (k + 2 < n) {
      w.issue_k(k + 2, k_lds0);
      w.issue_v(k + 2, v_lds0);
    }
    if (w.active((k + 1) * kWideKeys)) {
      __builtin_amdgcn_sched_barrier(0);
      w.scores(k_lds1);
      __builtin_amdgcn_sched_barrier(0);
      w.softmax((k + 1) * kWideKeys);
      __builtin_amdgcn_sched_barrier(0);
      w.pv(v_lds1);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    barrier();
  }
  // the output tiles staged in the K buffers (two wavefronts' 32-row tiles
  // per buffer; every LDS read happened before the last barrier)
  w.store_staged(p.o, p.lse, head_elems, bh, (w.wave < 2 ? k_lds0 : k_lds1) + (w.wave & 1) * 32 * W::ROW_BYTES);
}

template <typename T, int D, bool CAUSAL, bool TAIL, bool STRIDED>
hipError_t launch_wide_t(const FwdArgs& a, hipStream_t stream) {
  constexpr int BM = kWideWaves * 32;
  Params p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.BH = a.B * a.H;
  p.S = a.S;
  p.Sk = a.Sk;
  p.shift = a.causal ? a.Sk - a.S : a.Sk;  // non-causal wide heads: every key kept
  p.nqb = (a.S + BM - 1) / BM;
  p.persist = 0;
  p.c = a.scale * 1.4426950408889634f;
  p.H = a.H;
  if (STRIDED) {
    const long long* st = a.strides;  // q, k, v, o: batch, head, row (elements)
    p.qsb = st[0]; p.qsh = st[1]; p.q_rs = (uint32_t)(st[2] * 2);
    p.ksb = st[3]; p.ksh = st[4]; p.k_rs = (uint32_t)(st[5] * 2);
    p.vsb = st[6]; p.vsh = st[7]; p.v_rs = (uint32_t)(st[8] * 2);
    p.osb = st[9]; p.osh = st[10]; p.o_rs = (uint32_t)(st[11] * 2);
  }
  const long long grid = (long long)p.nqb * p.BH;
  hipLaunchKernelGGL((fwd_wide_kernel<T, D, CAUSAL, TAIL, STRIDED>), dim3((unsigned)grid), dim3(kWideWaves * 64), 0,
                     stream, p);
  return hipGetLastError();
}

// Only causal instantiations exist: a non-causal problem runs them with
// shift = Sk, which keeps every key (j < Sk <= i + Sk), so every tile but a
// ragged last one takes the unmasked path.  The non-causal instantiations
// spilled up to 500 B per lane at d = 256 and ran 4-5 % slower.
template <typename T, int D, bool STRIDED>
hipError_t launch_wide_s(const FwdArgs& a, hipStream_t stream) {
  const bool tail = a.Sk % kWideKeys != 0;
  if (!a.causal && D <= 128) return hipErrorInvalidValue;  // only causal problems come here at these widths
  return tail ? launch_wide_t<T, D, true, true, STRIDED>(a, stream)
              : launch_wide_t<T, D, true, false, STRIDED>(a, stream);
}

template <typename T, int D>
hipError_t launch_wide_d(const FwdArgs& a, hipStream_t stream) {
  return a.strides ? launch_wide_s<T, D, true>(a, stream) : launch_wide_s<T, D, false>(a, stream);
}

template <typename T>
hipError_t launch_wide_dtype(const FwdArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 64: return launch_wide_d<T, 64>(a, stream);
    case 128: return launch_wide_d<T, 128>(a, stream);
    case 192: return launch_wide_d<T, 192>(a, stream);
    default: return launch_wide_d<T, 256>(a, stream);
  }
}

}  // namespace detail

using namespace detail;

long long fwd_wide_grid_size(const FwdArgs& a) {
  const int BM = kWideWaves * 32;
  return (long long)((a.S + BM - 1) / BM) * a.B * a.H;
}

hipError_t launch_fwd_wide(const FwdArgs& a, hipStream_t stream) {
  return a.dtype == 1 ? launch_wide_dtype<__bf16>(a, stream) : launch_wide_dtype<_Float16>(a, stream);
}

}  // namespace fa
