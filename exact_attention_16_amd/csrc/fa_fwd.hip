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
// MI355X mapping (own design, not the pages'):
// * One wavefront owns 32 query rows.  It computes the transposed score tile
//   S^T = K Q^T with v_mfma_f32_32x32x16_{bf16,f16} (A = K from LDS, B = Q held
//   in VGPRs), so each lane holds scores of ONE query: the row max and row sum
//   are in-lane plus one exchange with lane l^32 (v_permlane32_swap).  The
//   output is accumulated transposed too, O^T += V^T P^T: B = P straight from
//   the score accumulator (no shuffle), A = V^T read with ds_read_b64_tr_b16
//   (gfx950's transposing LDS read); the rescale and 1/l are per-lane scalars.
// * Eight wavefronts per work-group (256 query rows), two per SIMD, in two
//   groups of four that run half a tile out of phase ("ping-pong"): while one
//   group's wavefront issues the MFMAs of P_{k-1} V_{k-1} and K_k Q^T, the
//   other group's wavefront on the same SIMD runs the softmax of its tile, so
//   the matrix cores and the vector ALUs work at the same time.  A work-group
//   barrier separates the steps and keeps the groups one phase apart.
// * K and V tiles go HBM -> LDS with buffer_load_dwordx4 ... lds (no VGPR
//   staging), double-buffered, in a fragment-major layout that makes every
//   LDS read linear and bank-conflict free.  Out-of-range rows read as zero
//   and out-of-range stores are dropped by the buffer descriptors' range
//   checks.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "fa_device.h"
#include "fa_fwd_wave.h"
#include "fa_launch.h"

namespace fa {
namespace detail {

// TAIL: Sk is not a multiple of BN, so the last key tile needs the
// sequence-end mask.
//
// Separate lengths.  Q / O heads hold S rows and K / V heads Sk rows.  The
// causal mask is aligned to the sequence end: query row i sits at key
// position i + shift with shift = Sk - S, so with S = Sk it is the square
// mask and a single query sees every key.
//
// Schedule.  With n key tiles, a wavefront's work is a sequence of phases:
//   MFMA(0) = K_0 Q^T;  SOFT(k) = softmax of tile k;
//   MFMA(k) = P_{k-1} V_{k-1} and K_k Q^T (k = 1..n; MFMA(n) is P V only).
// The kernel runs 2n+2 barrier-separated steps.  Group 0 (wavefronts 0-3)
// runs MFMA(k) in step 2k and SOFT(k) in step 2k+1; group 1 (wavefronts 4-7,
// one per SIMD beside a group-0 wavefront) runs SOFT(k-1) in step 2k and
// MFMA(k) in step 2k+1.  Loads: at the start of step 2k every wavefront
// issues its share of K_{k+1} and V_k into the buffers that the barrier after
// step 2k-1 has freed; they must land by step 2k+2, which the vmcnt(0) wait
// before the barrier ending step 2k+1 guarantees.  K_k lives in K buffer k%2
// and V_k in V buffer k%2.  Steps 2n and 2n+1 issue no load and read no K
// tile; they run after the step loop, where a persistent work-group loads
// its next block's Q rows.
// Occupancy: head dimension 128 runs one work-group per compute unit (two
// wavefronts per SIMD, at most 256 VGPRs each); head dimension 64 fits two
// (at most 128 VGPRs each), so one work-group's prologue, barriers and
// epilogue overlap the other's work.  (A ragged non-causal d = 64 problem
// runs the causal tail variant, see launch_s: the non-causal one did not fit
// 128 VGPRs.)
template <int D, bool CAUSAL, bool TAIL>
constexpr int waves_per_simd() { return D == 64 ? 4 : 2; }

// Variants launched as a persistent grid (see launch_t): d = 128 except the
// ragged non-causal one, which spilled 100-220 B with the block loop.  At
// d = 64 the loop spills registers (32-112 B in the non-causal variants; the
// causal ones lost 15-18 % at S >= 4096).
template <int D, bool CAUSAL, bool TAIL>
constexpr bool persistent_variant() { return D == 128 && (CAUSAL || !TAIL); }

// The 32-row block (0..7) of a work-group's rows that wavefront `wave` owns.
// Causal: group-0 wavefront w takes block w and its group-1 partner on the
// same SIMD (wavefront w + 4) block 7 - w, so every SIMD holds one early and
// one late block.  Near the diagonal the late blocks see more key tiles than
// the early ones; with this pairing the last two diagonal tiles leave at most
// one wavefront active per SIMD (its phases then run alone, without waiting
// for a partner's), where pairing neighbouring blocks left two SIMDs with
// both wavefronts active and two idle.  Measured on the MI355X against the
// neighbour pairing: mid_seq_causal and S = 1024 causal +4 %, S = 4096
// causal +2 %.  Non-causal rows all see the same keys: neighbouring blocks
// (which kept one ragged variant free of register spills).
template <bool CAUSAL>
__device__ __forceinline__ int row_block(int wave, int group) {
  if (CAUSAL) return group == 0 ? (wave & 3) : 7 - (wave & 3);
  return 2 * (wave & 3) + group;
}

// FAST: unmasked tiles take the softmax without the row max when the weights'
// range allows (FwdWave::softmax_impl).
template <typename T, int D, bool CAUSAL, bool TAIL, int NW, int BN, bool STRIDED, bool FAST>
__global__ __launch_bounds__(NW * 64, (waves_per_simd<D, CAUSAL, TAIL>())) void fwd_kernel(Params p) {
  static_assert(NW == 8, "the ping-pong schedule pairs wavefronts w and w+4 on one SIMD");
  using W = FwdWave<T, D, CAUSAL, TAIL, NW, BN, STRIDED, FAST>;
  // K and V double buffers as four distinct LDS objects; the step loop is
  // unrolled by two so each access names its buffer at compile time, which
  // lets the compiler see that reads of one buffer never alias the
  // direct-to-LDS loads filling another (no spurious vmcnt waits).
  __shared__ __attribute__((aligned(1024))) char k_lds0[W::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k_lds1[W::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds0[W::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds1[W::TILE_BYTES];

  W w;
  w.lane = threadIdx.x & 63;
  w.wave = threadIdx.x >> 6;
  w.h = w.lane >> 5;
  w.col = w.lane & 31;
  const int group = w.wave >> 2;

  // One query block per work-group, or (persistent grid) the work-group's
  // list of blocks one after the other.
  constexpr bool kPersist = persistent_variant<D, CAUSAL, TAIL>();
  BlockCursor<CAUSAL> cur;
  int bh, qb;
  bool more;
  if (kPersist && p.persist) {
    cur.init(p);
    more = cur.next(p, bh, qb);
  } else {
    map_query_block<CAUSAL>(blockIdx.x, p.BH, p.nqb, bh, qb);
    more = true;
  }
  // Persistent: the block after this one.  Its Q rows are fetched during
  // this block's last two steps and its output store (once the block's last
  // K Q^T has run, Q is not read again), so the next block's prologue loads
  // only its first key tile.
  int next_bh = 0, next_qb = 0;
  bool prefetched = false;
  while (more) {
    const int q_lo = qb * W::BM;
    w.qw = q_lo + 32 * row_block<CAUSAL>(w.wave, group);
    w.myq = w.qw + w.col;
    const size_t head_elems = w.setup(p, bh, kPersist && prefetched);

    // keys this work-group visits (causal: up to its last row's position)
    const int kv_end = CAUSAL ? min(p.Sk, q_lo + W::BM + p.shift) : p.Sk;
    const int n = kv_end > 0 ? (kv_end + BN - 1) / BN : 0;
    w.n = n;

    w.issue_k(0, k_lds0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    barrier();
    const bool has_next = (kPersist && p.persist) ? cur.next(p, next_bh, next_qb) : false;
    const int next_qw = next_qb * W::BM + 32 * row_block<CAUSAL>(w.wave, group);

    // Steps 0 .. 2n-1; then steps 2n and 2n+1 (P V of the last tile and the
    // softmax before it), which read neither Q nor a K buffer.
    for (int k = 0; k < n; k += 2) {
      // ---- even k: K_k in buffer 0, V_{k-1} in buffer 1
      if (k + 1 < n) w.issue_k(k + 1, k_lds1);
      w.issue_v(k, v_lds0);
      if (group == 0) w.mfma_phase(k, k_lds0, v_lds1); else w.soft_phase(k - 1);
      barrier();
      if (group == 0) w.soft_phase(k); else w.mfma_phase(k, k_lds0, v_lds1);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      barrier();
      if (k + 1 >= n) break;
      // ---- odd k+1: K_{k+1} in buffer 1, V_k in buffer 0
      if (k + 2 < n) w.issue_k(k + 2, k_lds0);
      w.issue_v(k + 1, v_lds1);
      if (group == 0) w.mfma_phase(k + 1, k_lds1, v_lds0); else w.soft_phase(k);
      barrier();
      if (group == 0) w.soft_phase(k + 1); else w.mfma_phase(k + 1, k_lds1, v_lds0);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      barrier();
    }
    // The next block's Q rows stay in flight through the last two steps and
    // the output store.  (Issued after the loop, so that no read of Q inside
    // it waits for them.  A load of the next key tile here would make the
    // compiler wait for it before the LDS accesses below, whose buffer it
    // cannot tell apart from K buffer 0.)
    if (kPersist && has_next) w.prefetch_q(p, next_bh, next_qw);
    {
      const char* const vl = (n & 1) ? v_lds0 : v_lds1;  // V_{n-1}: buffer (n-1) % 2
      if (group == 0) w.pv_phase(n, vl); else w.soft_phase(n - 1);
      barrier();
      if (group == 1) w.pv_phase(n, vl);
      barrier();
    }
    // Every LDS read of this block happened before the last barrier, so the
    // output tiles are staged in the K/V buffers (two wavefronts' 32-row
    // tiles per buffer); the barrier after the store frees them for the next
    // block's first K tile.  (The fast-softmax d = 64 variants, which run
    // only long rows where the store is a small share, keep the direct store:
    // staging cost them registers, 28 -> 44 B of spill, and 1-3 %.)
    if constexpr (D == 64 && FAST) {
      w.store(p.o, p.lse, head_elems, bh);
    } else {
      char* const buf = w.wave < 2 ? k_lds0 : w.wave < 4 ? k_lds1 : w.wave < 6 ? v_lds0 : v_lds1;
      w.store_staged(p.o, p.lse, head_elems, bh, buf + (w.wave & 1) * 32 * W::ROW_BYTES);
    }
    more = has_next;
    prefetched = has_next;
    bh = next_bh;
    qb = next_qb;
    if (more) barrier();
  }
}

constexpr int kWaves = 8;

// Compute units of the device `stream` runs on (the current device for the
// NULL stream), looked up once per device; 0 if the runtime cannot say.
int device_cus(hipStream_t stream) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if ((stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev)) != hipSuccess || dev < 0 ||
      dev >= kMaxDevices)
    return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
    cache[dev].store(n, std::memory_order_relaxed);
  return n > 0 ? n : 0;
}
// Keys per tile (chosen by measurement on the MI355X).
template <int D>
constexpr int key_tile() { return 64; }

template <typename T, int D, bool CAUSAL, bool TAIL, bool STRIDED>
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
  p.Sk = a.Sk;
  // non-causal: shift = Sk keeps every key (only the causal instantiations
  // read it; see launch_s)
  p.shift = a.causal ? a.Sk - a.S : a.Sk;
  p.nqb = (a.S + BM - 1) / BM;
  p.c = a.scale * 1.4426950408889634f;
  p.H = a.H;
  if (STRIDED) {
    const long long* st = a.strides;  // q, k, v, o: batch, head, row (elements)
    p.qsb = st[0]; p.qsh = st[1]; p.q_rs = (uint32_t)(st[2] * 2);
    p.ksb = st[3]; p.ksh = st[4]; p.k_rs = (uint32_t)(st[5] * 2);
    p.vsb = st[6]; p.vsh = st[7]; p.v_rs = (uint32_t)(st[8] * 2);
    p.osb = st[9]; p.osh = st[10]; p.o_rs = (uint32_t)(st[11] * 2);
  }
  long long grid = (long long)p.nqb * p.BH;
  // The persistent variants run one work-group per compute unit, each
  // working through its list of query blocks (causal: (long, short) pairs,
  // so every work-group gets the same number of key tiles; see BlockCursor)
  // and loading each block's Q rows during the previous block's last steps.
  // Measured on the MI355X against one block per work-group: S = 512
  // non-causal +9 %, S = 2048 causal +3 %, S = 8192 causal +2 %.
  p.persist = 0;
  if constexpr (persistent_variant<D, CAUSAL, TAIL>()) {
    // resident work-groups: (waves per SIMD x 4 SIMDs) / kWaves per compute unit
    const long long slots = (long long)device_cus(stream) * (waves_per_simd<D, CAUSAL, TAIL>() * 4 / kWaves);
    const long long units = (long long)p.BH * (CAUSAL ? (p.nqb + 1) / 2 : p.nqb);
    if (slots > 0 && units > slots) {
      p.persist = 1;
      grid = slots;
    }
  }
  // The fast softmax keeps each tile's scores live while it computes the
  // weights (for a possible retry): at d = 128 that fits the registers
  // except in the non-causal ragged variant.  At d = 64 it costs spilled
  // registers in the step loop, which long non-causal rows repay (S = 2048:
  // +2-4 %, S = 16384: +5-6 % on the MI355X) and short or causal ones do not
  // (S = 512: -2 to -7 %, causal S = 4096: -17 %).
  constexpr bool kFastOk = D == 128 ? (CAUSAL || !TAIL) : !CAUSAL;
  const bool fast = kFastOk && (D == 128 || a.Sk >= 2048);
  if (fast)
    hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL, TAIL, kWaves, key_tile<D>(), STRIDED, kFastOk>),
                       dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL, TAIL, kWaves, key_tile<D>(), STRIDED, false>),
                       dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

// A ragged non-causal d = 64 problem runs the causal tail variant with
// shift = Sk, which keeps every key: the non-causal tail variant needed more
// than 128 VGPRs, i.e. one work-group per compute unit instead of two
// (measured: 13-22 % slower at S = 300, 1000 and 4099).
template <typename T, int D, bool STRIDED>
hipError_t launch_s(const FwdArgs& a, hipStream_t stream) {
  const bool tail = a.Sk % key_tile<D>() != 0;
  if (a.causal || (D == 64 && tail))
    return tail ? launch_t<T, D, true, true, STRIDED>(a, stream) : launch_t<T, D, true, false, STRIDED>(a, stream);
  if constexpr (D == 64)
    return launch_t<T, D, false, false, STRIDED>(a, stream);
  else
    return tail ? launch_t<T, D, false, true, STRIDED>(a, stream) : launch_t<T, D, false, false, STRIDED>(a, stream);
}

template <typename T, int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
  return a.strides ? launch_s<T, D, true>(a, stream) : launch_s<T, D, false>(a, stream);
}

template <typename T>
hipError_t launch_dtype(const FwdArgs& a, hipStream_t stream) {
  return a.d == 64 ? launch_d<T, 64>(a, stream) : launch_d<T, 128>(a, stream);
}

}  // namespace detail

using namespace detail;

long long fwd_grid_size(const FwdArgs& a) {
  if (uses_in_order_kernel(a)) return fwd_wide_grid_size(a);
  const int BM = kWaves * 32;
  return (long long)((a.S + BM - 1) / BM) * a.B * a.H;
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  if (uses_in_order_kernel(a)) return launch_fwd_wide(a, stream);  // fa_fwd_wide.hip
  // dtype 0 = fp16, 1 = bf16 (fa_dtype)
  return a.dtype == 1 ? launch_dtype<__bf16>(a, stream) : launch_dtype<_Float16>(a, stream);
}

}  // namespace fa
