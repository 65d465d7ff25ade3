// One wavefront's share of the forward pass: 32 query rows of one head, the
// MFMA score and output products over LDS-staged key tiles, and the online
// softmax between them.  Used by the prefill kernel (fa_fwd.hip) and the
// split-key decode kernel (fa_decode.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_device.h"

namespace fa {
namespace detail {

// Work-group -> (query block, head).  The dispatcher deals work-group ids to
// the chip's XCDs round-robin (id % kXcds), each XCD with its own L2.  When
// B*H is a multiple of kXcds, the ids an XCD receives are remapped so that
// all of one head's query blocks run on one XCD.  Non-causal: an XCD runs a
// head's query blocks back to back; they stream the same K/V tiles at about
// the same time, so each tile comes from HBM once per head.  Causal: query
// block qb visits qb + 1 row blocks' worth of key tiles, so an XCD's queue
// is ordered longest first across its heads (all heads' last query blocks,
// then the next-to-last, ...) and the short blocks fill the tail (greedy
// longest-processing-time scheduling).
template <bool CAUSAL>
__device__ __forceinline__ void map_query_block(unsigned id, int BH, int nqb, int& bh, int& qb) {
  if (BH % kXcds == 0) {
    const int local = id / kXcds;  // position in this XCD's queue
    if (CAUSAL) {
      const int heads_per_xcd = BH / kXcds;
      qb = local / heads_per_xcd;
      bh = (local % heads_per_xcd) * kXcds + id % kXcds;
    } else {
      qb = local % nqb;
      bh = (local / nqb) * kXcds + id % kXcds;
    }
  } else {
    qb = id % nqb;
    bh = id / nqb;
  }
  if (CAUSAL) qb = nqb - 1 - qb;
}

// The query blocks one work-group of a persistent grid works through.
// Units are dealt to the work-groups of each XCD (work-group i runs on XCD
// i % kXcds): with B*H a multiple of kXcds, XCD x owns heads x, x + kXcds,
// ... and its work-groups take that list's units in turn, so the work-groups
// of an XCD work on the same few heads at a time and share their K/V tiles
// in the XCD's L2.  A causal unit is the pair of query blocks (nqb-1-u, u)
// of one head: nqb + 1 row blocks' worth of key tiles for every pair, so the
// work-groups finish together whatever the head length (one block alone in
// the middle when nqb is odd).  A non-causal unit is one query block.
template <bool CAUSAL>
struct BlockCursor {
  int u, stride, units, xcd, upe;
  bool xcd_map;
  int part;  // causal: 0 = the long block of the pair, 1 = the short one

  __device__ __forceinline__ void init(const Params& p) {
    const int G = gridDim.x;
    upe = CAUSAL ? (p.nqb + 1) / 2 : p.nqb;  // units per head
    xcd_map = (p.BH % kXcds == 0) && (G % kXcds == 0);
    if (xcd_map) {
      xcd = blockIdx.x % kXcds;
      u = blockIdx.x / kXcds;
      stride = G / kXcds;
      units = (p.BH / kXcds) * upe;
    } else {
      xcd = 0;
      u = blockIdx.x;
      stride = G;
      units = p.BH * upe;
    }
    part = 0;
  }

  // The next query block of this work-group, or false when none is left.
  __device__ __forceinline__ bool next(const Params& p, int& bh, int& qb) {
    while (u < units) {
      const int head = u / upe, unit = u % upe;
      bh = xcd_map ? head * kXcds + xcd : head;
      if (!CAUSAL) {
        qb = unit;
        u += stride;
        return true;
      }
      if (part == 0) {
        qb = p.nqb - 1 - unit;
        part = 1;
        if (qb == unit) {  // the middle block of an odd count: alone
          part = 0;
          u += stride;
        }
        return true;
      }
      qb = unit;
      part = 0;
      u += stride;
      return true;
    }
    return false;
  }
};

// One wavefront's share of a work-group: 32 query rows of one (batch, head),
// their Q fragments, running statistics and output accumulator, plus the
// score tile / weights of the key tile in flight.  The work-group's NW
// wavefronts share the K/V tiles (BN keys each) in LDS.
//
// Rows of a head are ROW_BYTES apart (dense [B][H][S][d] tensors), or, when
// STRIDED, q_rs / k_rs / v_rs / o_rs bytes apart (e.g. a [B][S][H][d]
// layout); the head bases and range sizes are set by the kernel either way.
template <typename T, int D, bool CAUSAL, bool TAIL, int NW, int BN, bool STRIDED = false, bool FAST = false>
struct FwdWave {
  static constexpr int BM = NW * 32;
  static constexpr int ROW_BYTES = D * 2;
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
  int S;     // query rows
  int Sk;    // key rows
  int shift; // causal offset: key j is kept for query i iff j <= i + shift
  int n;     // key tiles this work-group visits
  float c;   // scale * log2(e)
  const char* kh;
  const char* vh;
  uint32_t head_bytes;     // one head of q (and of o when dense)
  uint32_t kv_head_bytes;  // one head of k (and of v when dense)
  // STRIDED only: row strides in bytes, the v and o range sizes, o's head base
  uint32_t q_rs, k_rs, v_rs, o_rs;
  uint32_t v_bytes, o_bytes;
  const char* oh;

  __device__ __forceinline__ uint32_t q_row(int r) const { return (uint32_t)r * (STRIDED ? q_rs : ROW_BYTES); }
  __device__ __forceinline__ uint32_t k_row(int r) const { return (uint32_t)r * (STRIDED ? k_rs : ROW_BYTES); }
  __device__ __forceinline__ uint32_t v_row(int r) const { return (uint32_t)r * (STRIDED ? v_rs : ROW_BYTES); }
  __device__ __forceinline__ uint32_t o_row(int r) const { return (uint32_t)r * (STRIDED ? o_rs : ROW_BYTES); }

  i16x8 qf[KSTEPS];
  f32x16 oacc[DB];
  f32x16 sacc[SB];   // scores of the tile between its MFMA step and its softmax
  i16x8 pf[SB][2];   // its weights between the softmax and the P V MFMAs
  float m_used;      // reference max (raw score units) the weights are taken against
  float mc;          // c * m_used
  float lsum;        // this lane's share of the row sum (fp32 weights: the logsumexp)
  float lsum_o;      // bf16: its share of the sum of the rounded weights (the output's divisor)

  // Lengths, scale, the head's Q/K/V/O bases and ranges from the launch
  // parameters, then this lane's Q row (qw, myq and the lane fields must be
  // set), unless `q_loaded` (prefetch() has already issued it).  Returns the
  // dense head offset in elements (bh * S * D).
  __device__ __forceinline__ size_t setup(const Params& p, int bh, bool q_loaded = false) {
    S = p.S;
    Sk = p.Sk;
    shift = p.shift;
    c = p.c;
    const size_t head_elems = (size_t)bh * p.S * D;
    if constexpr (STRIDED) {
      // head bases from the batch and head strides; each range ends with the
      // head's last row, so rows past S (or Sk) read as 0 / are dropped
      const int b = bh / p.H, hh = bh - b * p.H;
      q_rs = p.q_rs;
      k_rs = p.k_rs;
      v_rs = p.v_rs;
      o_rs = p.o_rs;
      head_bytes = (uint32_t)(p.S - 1) * p.q_rs + ROW_BYTES;
      kv_head_bytes = p.Sk > 0 ? (uint32_t)(p.Sk - 1) * p.k_rs + ROW_BYTES : 0u;
      v_bytes = p.Sk > 0 ? (uint32_t)(p.Sk - 1) * p.v_rs + ROW_BYTES : 0u;
      o_bytes = (uint32_t)(p.S - 1) * p.o_rs + ROW_BYTES;
      kh = (const char*)p.k + (b * p.ksb + hh * p.ksh) * 2;
      vh = (const char*)p.v + (b * p.vsb + hh * p.vsh) * 2;
      oh = (const char*)p.o + (b * p.osb + hh * p.osh) * 2;
      if (q_loaded) reset_rows(); else load_q((const char*)p.q + (b * p.qsb + hh * p.qsh) * 2);
    } else {
      const size_t kv_head_elems = (size_t)bh * p.Sk * D;
      head_bytes = (uint32_t)p.S * ROW_BYTES;
      kv_head_bytes = (uint32_t)p.Sk * ROW_BYTES;
      kh = (const char*)p.k + kv_head_elems * 2;
      vh = (const char*)p.v + kv_head_elems * 2;
      if (q_loaded) reset_rows(); else load_q((const char*)p.q + head_elems * 2);
    }
    return head_elems;
  }

  // The Q rows of the work-group's next query block (head nbh, first row nqw
  // of this wavefront) into qf, issued while this block finishes (it reads
  // qf no more once its last K Q^T has run).  setup(p, nbh, true) completes
  // the switch (head strides and range sizes are the same for every head).
  __device__ __forceinline__ void prefetch_q(const Params& p, int nbh, int nqw) {
    const char* qh;
    if constexpr (STRIDED) {
      const int b = nbh / p.H, hh = nbh - b * p.H;
      qh = (const char*)p.q + (b * p.qsb + hh * p.qsh) * 2;
    } else {
      qh = (const char*)p.q + (size_t)nbh * p.S * D * 2;
    }
    load_qf(qh, nqw + col);
  }

  // Does this wavefront have any unmasked key in the tile starting at k0?
  __device__ __forceinline__ bool active(int k0) const { return !(CAUSAL && k0 > qw + 31 + shift); }

  // Q rows -> VGPRs as the B operand of S^T = K Q^T (rows >= S read as 0).
  __device__ __forceinline__ void load_q(const char* qh) {
    load_qf(qh, myq);
    reset_rows();
  }
  __device__ __forceinline__ void load_qf(const char* qh, int row) {
    const __amdgpu_buffer_rsrc_t rq = rsrc(qh, head_bytes);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const uint32_t off = q_row(row) + (kk * 16 + h * 8) * 2;
      qf[kk] = __builtin_bit_cast(i16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
    }
  }
  // A new block's running statistics and output accumulator.
  __device__ __forceinline__ void reset_rows() {
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    m_used = -__builtin_inff();
    mc = 0.f;
    lsum = 0.f;
    lsum_o = 0.f;
  }

  // The wavefront index for the load blocks below, made wavefront-uniform so
  // that each load's LDS destination is a scalar value rather than a vector
  // register kept live through the step loop.  (Measured on the MI355X:
  // short_seq_batch +1 %, long_seq_causal +1 %, S >= 4096 causal d = 64
  // +2 %, the rest within noise; the strided variants keep the plain index,
  // with which they allocate registers without spilling.)
  __device__ __forceinline__ int uniform_wave() const {
    return STRIDED ? wave : __builtin_amdgcn_readfirstlane(wave);
  }

  // HBM -> LDS copies of one key tile (BN rows of K, or of V), issued
  // cooperatively by all NW wavefronts.
  //
  // LDS holds each tile "fragment-major": every 1 KiB block is exactly what
  // one wave instruction later reads, so every LDS read is a linear,
  // bank-conflict-free access at lane * 16 (or lane * 8) plus an immediate.
  // A direct-to-LDS buffer load also fills 1 KiB in lane order, so each lane
  // simply fetches the global 16-byte chunk that belongs at its slot:
  //   K block (sb, kk): lane l holds K[32*sb + l%32][16*kk + 8*(l/32) .. +8],
  //     the A operand of one S^T MFMA;
  //   V block (sb, cc, tt, dp): two 512-byte halves for d-blocks 2dp, 2dp+1;
  //     in half x, bytes 8*l .. 8*l+8 are the 4 elements that lane l passes
  //     to ds_read_b64_tr_b16 for the V^T operand of d-block 2dp+x, key
  //     chunk (sb, cc), sub-step tt (see pv()).
  // Rows >= S read as 0 (buffer range check).
  __device__ __forceinline__ void issue_k(int tile, char* kd) const {
    const __amdgpu_buffer_rsrc_t rk = rsrc(kh, kv_head_bytes);
    const uint32_t base = k_row(tile * BN);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int f = i * NW + uniform_wave();  // block (sb, kk)
      const int ksb = f / KSTEPS, kk = f % KSTEPS;
      const uint32_t off = base + k_row(ksb * 32 + (lane & 31)) + (kk * 2 + (lane >> 5)) * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kd + f * 1024), 16, off, 0, 0, 0);
    }
  }

  __device__ __forceinline__ void issue_v(int tile, char* vd) const {
    const __amdgpu_buffer_rsrc_t rv = rsrc(vh, STRIDED ? v_bytes : kv_head_bytes);
    const uint32_t base = v_row(tile * BN);
    const int x = lane >> 5;         // which half (d-block parity)
    const int lp = lane & 31;
    const int vg = lp >> 3;          // 16-lane group of the reading lanes 2lp, 2lp+1
    const int vrow = (vg >> 1) * 4 + ((lp & 7) >> 1);
    const int vcol = x * 32 + (vg & 1) * 16 + (lp & 1) * 8;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int f = i * NW + uniform_wave();  // block ((sb * 2 + cc) * 2 + tt) * (DB / 2) + dp
      const int dp = f % (DB / 2), rest = f / (DB / 2);
      const uint32_t off = base + v_row(rest * 8 + vrow) + (dp * 64 + vcol) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vd + f * 1024), 16, off, 0, 0, 0);
    }
  }

  // S^T = K Q^T for the tile in `ks`: lane holds 16 scores of query `myq`
  // per 32-key block (keys 8*(r/4) + 4*h + r%4 of the block, r = 0..15).
  // The k-steps run in the outer loop so the SB accumulation chains
  // interleave instead of waiting on one another.
  // K fragment (A operand of S^T) of 32-key block sb, k-step kk.
  __device__ __forceinline__ i16x8 k_frag(const char* ks, int sb, int kk) const {
    return *(const i16x8*)(ks + (sb * KSTEPS + kk) * 1024 + lane * 16);
  }

  __device__ __forceinline__ void scores(const char* ks) {
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) sacc[sb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      i16x8 kf[SB];
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) kf[sb] = k_frag(ks, sb, kk);
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) sacc[sb] = Elem<T>::mma(kf[sb], qf[kk], sacc[sb]);
      // wide heads: keep the scheduler from hoisting every k-step's LDS reads
      // to the top (they would not fit the register file); four k-steps of
      // reads may run ahead of the MFMAs
      if constexpr (D > 128)
        if (kk % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
  }

  // O^T += V^T P^T for the tile in `vs` and the weights in pf.  For chunk cc
  // of 32-key block sb, MFMA k-index h*8 + 4*tt + e stands for key
  // 32*sb + 16*cc + 8*tt + 4*h + e, matching where the score accumulator put
  // that key's weight.  ds_read_b64_tr_b16 gives lane j of each 16-lane group
  // element j%4 of the 8 bytes addressed by lanes 4e + j/4 of its group
  // (e = 0..3); the V block layout puts there
  // V[32*sb + 16*cc + 8*tt + 4*(g/2) + e][32*db + 16*(g%2) + j] for group g,
  // i.e. lane l receives V^T[d = 32*db + l%32][its 4 keys].
  // V^T fragment (A operand of O^T += V^T P^T) of d-block db, key chunk
  // (sb, cc).
  __device__ __forceinline__ i16x8 v_frag(const char* vs, int db, int sb, int cc) const {
    i16x4 half[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int blk = ((sb * 2 + cc) * 2 + tt) * (DB / 2) + (db >> 1);
      const char* a = vs + blk * 1024 + (db & 1) * 512 + lane * 8;
      half[tt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a));
    }
    return __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7);
  }

  __device__ __forceinline__ void pv(const char* vs) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const i16x8 vf = v_frag(vs, db, sb, cc);
          oacc[db] = Elem<T>::mma(vf, pf[sb][cc], oacc[db]);
        }
      }
      if constexpr (D > 128)  // as in scores(): bound the reads in flight
        if (db % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Does the tile starting at k0 cross the causal diagonal or the sequence end?
  __device__ __forceinline__ bool tile_masked(int k0) const {
    return (CAUSAL && k0 + BN - 1 > qw + shift) || (TAIL && k0 + BN > Sk);
  }

  // Online-softmax update for the tile starting at k0 (scores in sacc):
  // mask, row max, lazy rescale of O and l, weights P packed to T.  Only tiles
  // that cross the causal diagonal or the sequence end are MASKED; the two
  // variants are separate instantiations so the selects never run elsewhere.
  __device__ __forceinline__ void softmax(int k0) {
    if (tile_masked(k0))
      softmax_impl<true>(k0);
    else
      softmax_impl<false>(k0);
  }

  template <bool MASKED>
  __device__ __forceinline__ void softmax_impl(int k0) {
    if (MASKED) {
      // key k0 + t + 4h (t below) is kept iff t < Sk - k0 - 4h and, when
      // causal, t <= myq + shift - k0 - 4h
      const int base = k0 + 4 * h;
      const int end = Sk - base;
      const int last = myq + shift - base;
#pragma unroll
      for (int sb = 0; sb < SB; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = sb * 32 + 8 * (r >> 2) + (r & 3);
          const bool ok = t < end && (!CAUSAL || t <= last);
          sacc[sb][r] = ok ? sacc[sb][r] : -__builtin_inff();
        }
    }

    // The row max only guards the weights' range (after the rescale below
    // every weight is at most 2^kRescaleMargin).  The weights are first taken
    // against the current reference without the max, and accepted when every
    // lane's share of the tile's row sum stays within the dtype's
    // kTileSumLimit; otherwise (a score grew too far past the reference, or
    // the row has none yet) the max and rescale run and the weights are taken
    // again.  The reference may thus trail the row max: weights above 1 are
    // exact in floating point, and the LSE adds log2 of the larger sum.
    // (Masked tiles, on the diagonal or at the sequence end, are few: they
    // always take the max first, which keeps their register use down.)
    float ts, to;
    if constexpr (MASKED || !FAST) {
      rescale_to_max<false>();
      weights<MASKED>(ts, to);
    } else {
      bool slow = __builtin_amdgcn_ballot_w64(m_used == -__builtin_inff()) != 0;
      while (true) {
        if (slow) rescale_to_max<true>();
        weights<MASKED>(ts, to);
        if (slow || __builtin_amdgcn_ballot_w64(!(ts <= Elem<T>::kTileSumLimit)) == 0) break;
        slow = true;
      }
    }
    lsum += ts;
    if constexpr (Elem<T>::kRoundedSum) lsum_o += to;
  }

  // Row max of the tile in sacc; when it exceeds the reference m_used by more
  // than kRescaleMargin binary orders (or the row had none), it becomes the
  // new reference and O and the sums are rescaled to it.
  template <bool RETRY>
  __device__ __forceinline__ void rescale_to_max() {
    // (in the fast path's retry loop, empty asm statements keep the compiler
    // from hoisting the max out of the loop, where it would run on every tile)
    if constexpr (RETRY) {
#pragma unroll
      for (int sb = 0; sb < SB; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(sacc[sb][r]));
    }
    // row max: two chains over the 16 * SB scores, each step taking two more
    // (one v_max3 per step; the earlier four-chain tree took 23 instructions
    // for 32 scores, this takes 17)
    float mc2[2];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int b0 = c2 * 8 * SB;  // first score of this chain (flat index sb * 16 + r)
      float m = fmaxf(fmaxf(sacc[b0 / 16][b0 % 16], sacc[(b0 + 1) / 16][(b0 + 1) % 16]), sacc[(b0 + 2) / 16][(b0 + 2) % 16]);
#pragma unroll
      for (int i = b0 + 3; i + 1 < b0 + 8 * SB; i += 2)
        m = fmaxf(fmaxf(m, sacc[i / 16][i % 16]), sacc[(i + 1) / 16][(i + 1) % 16]);
      if constexpr ((8 * SB - 3) % 2 == 1) m = fmaxf(m, sacc[(b0 + 8 * SB - 1) / 16][(b0 + 8 * SB - 1) % 16]);
      mc2[c2] = m;
    }
    float mx = fmaxf(mc2[0], mc2[1]);
    mx = max_with_partner(mx);
    const float m_new = fmaxf(m_used, mx);
    const bool grow = (m_used == -__builtin_inff()) || (c * (m_new - m_used) > kRescaleMargin);
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float alpha =
          (m_used == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(c * (m_used - m_new));
      m_used = m_new;
      mc = c * m_new;
      lsum *= alpha;
      if constexpr (Elem<T>::kRoundedSum) lsum_o *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
  }

  // The weights of 32-key block sb of the tile against the reference mc,
  // packed to T into out (the block's two P V operands); adds this lane's
  // shares of the row sum to ls (four partial sums, independent chains;
  // `first` starts them) and, for bf16, of the sum of the rounded weights to
  // lo (two partial sums).
  template <bool MASKED>
  __device__ __forceinline__ void weights_block(int sb, float (&ls)[4], float (&lo)[2], bool first,
                                                i16x8 (&out)[2]) {
    float e[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      e[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[sb][r], c, -mc));
      if (MASKED) e[r] = (sacc[sb][r] == -__builtin_inff()) ? 0.f : e[r];
      ls[r & 3] = (first && r < 4) ? e[r] : ls[r & 3] + e[r];
    }
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned x = Elem<T>::pack(e[8 * cc + 2 * i], e[8 * cc + 2 * i + 1]);
        w[i] = x;
        if constexpr (Elem<T>::kRoundedSum) lo[i & 1] = Elem<T>::add_packed(x, lo[i & 1]);
      }
      out[cc] = __builtin_bit_cast(i16x8, w);
    }
  }

  // The whole tile's weights (into pf); ts returns this lane's share of the
  // tile's row sum, to (bf16) its share of the sum of the rounded weights.
  template <bool MASKED>
  __device__ __forceinline__ void weights(float& ts, float& to) {
    float ls[4];
    float lo[2] = {0.f, 0.f};
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) weights_block<MASKED>(sb, ls, lo, sb == 0, pf[sb]);
    ts = (ls[0] + ls[1]) + (ls[2] + ls[3]);
    to = lo[0] + lo[1];
  }

  // Both products of one MFMA phase as a single software pipeline.  MFMA i
  // (i < NPV: O^T += V^T P^T, d-blocks innermost so that neighbours write
  // different accumulators; then K Q^T, k-steps outermost) takes its A
  // operand from LDS, and that fragment is read kAhead MFMAs before it is
  // used.  Scheduling groups (LDS reads, then one MFMA and the reads of the
  // fragment kAhead further on, ...) pin this order, so the LDS latency is
  // covered by the matrix core's work except once at the start.
  static constexpr int NPV = DB * SB * 2;
  static constexpr int NQK = KSTEPS * SB;
  // Only the causal d = 128 variants: elsewhere the deeper read-ahead spilled
  // registers in the step loop and measured slower on the MI355X.
  static constexpr int kAhead = (D == 128 && CAUSAL) ? 6 : 0;
  static constexpr int kGroupMfma = 0x008, kGroupDsRead = 0x100;  // sched_group_barrier masks

  __device__ __forceinline__ i16x8 op_frag(int i, const char* ks, const char* vs) const {
    if (i < NPV) {
      const int db = i % DB, sc = i / DB;
      return v_frag(vs, db, sc >> 1, sc & 1);
    }
    const int j = i - NPV;
    return k_frag(ks, j % SB, j / SB);
  }

  __device__ __forceinline__ void op_mfma(int i, i16x8 a) {
    if (i < NPV) {
      const int db = i % DB, sc = i / DB;
      oacc[db] = Elem<T>::mma(a, pf[sc >> 1][sc & 1], oacc[db]);
    } else {
      const int j = i - NPV, sb = j % SB, kk = j / SB;
      sacc[sb] = Elem<T>::mma(a, qf[kk], kk == 0 ? f32x16{} : sacc[sb]);
    }
  }

  // LDS reads of fragment i: two transposing 8-byte reads for V^T, one
  // 16-byte read for K
  __device__ __forceinline__ static void group_reads(int i) {
    if (i < NPV)
      __builtin_amdgcn_sched_group_barrier(kGroupDsRead, 2, 0);
    else
      __builtin_amdgcn_sched_group_barrier(kGroupDsRead, 1, 0);
  }

  __device__ __forceinline__ void pv_scores(const char* ks, const char* vs) {
    constexpr int N = NPV + NQK;
    i16x8 f[N];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) f[i] = op_frag(i, ks, vs);
#pragma unroll
    for (int i = 0; i < kAhead; ++i) group_reads(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (i + kAhead < N) f[i + kAhead] = op_frag(i + kAhead, ks, vs);
      op_mfma(i, f[i]);
      __builtin_amdgcn_sched_group_barrier(kGroupMfma, 1, 0);
      if (i + kAhead < N) group_reads(i + kAhead);
    }
  }

  // Phase MFMA(k): P_{k-1} V_{k-1} (V from vp) and K_k Q^T (K from kc).
  __device__ __forceinline__ void mfma_phase(int k, const char* kc, const char* vp) {
    __builtin_amdgcn_s_setprio(1);
    const bool do_pv = k >= 1 && active((k - 1) * BN);
    const bool do_qk = k < n && active(k * BN);
    if (kAhead > 0 && do_pv && do_qk) {
      pv_scores(kc, vp);
    } else {
      if (do_pv) pv(vp);
      if (do_qk) scores(kc);
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // Phase MFMA(n) alone: P V of the last tile (no K Q^T).
  __device__ __forceinline__ void pv_phase(int k, const char* vp) {
    __builtin_amdgcn_s_setprio(1);
    if (k >= 1 && active((k - 1) * BN)) pv(vp);
    __builtin_amdgcn_s_setprio(0);
  }

  // Phase SOFT(k): the softmax of tile k.
  __device__ __forceinline__ void soft_phase(int k) {
    if (k >= 0 && k < n && active(k * BN)) softmax(k * BN);
  }

  // The sum the output is divided by (the rounded weights' for bf16).
  __device__ __forceinline__ float out_divisor() const {
    return sum_with_partner(Elem<T>::kRoundedSum ? lsum_o : lsum);
  }

  // O = O_acc / out_divisor() and LSE = (c m + log2 l) ln 2 with the fp32 row
  // sum l; rows >= S are dropped by the descriptors' range checks.  A row
  // that saw no key (causal, more query rows than keys) has l = 0: it stores
  // O = 0 and LSE = -inf.
  __device__ __forceinline__ void store(void* o, float* lse, size_t head_elems, int bh) const {
    const float ltot = sum_with_partner(lsum);
    const bool none = !(ltot > 0.f);
    const float inv = none ? 0.f : 1.0f / out_divisor();
    const __amdgpu_buffer_rsrc_t ro =
        STRIDED ? rsrc(oh, o_bytes) : rsrc((const char*)o + head_elems * 2, head_bytes);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        u32x2 w;
        w[0] = Elem<T>::pack(oacc[db][4 * rg + 0] * inv, oacc[db][4 * rg + 1] * inv);
        w[1] = Elem<T>::pack(oacc[db][4 * rg + 2] * inv, oacc[db][4 * rg + 3] * inv);
        const int dcol = db * 32 + 8 * rg + 4 * h;
        __builtin_amdgcn_raw_buffer_store_b64(w, ro, o_row(myq) + dcol * 2, 0, 0);
      }
    if (h == 0) {
      const __amdgpu_buffer_rsrc_t rl = rsrc(lse + (size_t)bh * S, (uint32_t)S * 4);
      const float v = none ? -__builtin_inff() : (mc + __builtin_amdgcn_logf(ltot)) * 0.69314718055994531f;
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), rl, (uint32_t)myq * 4, 0, 0);
    }
  }

  // store() with the output tile staged through LDS.  Storing straight from
  // the accumulators, each instruction scatters 8-byte pieces over 32 rows,
  // and a wavefront took about 4000 cycles to issue its O tile.  Here the
  // lanes first write their pieces into `stage` (this wavefront's 32 x D
  // tile of LDS, free once the block's last barrier is passed), then the
  // wavefront stores whole rows, 16 contiguous bytes per lane.  The layout
  // keeps both LDS accesses free of bank conflicts: 16-byte chunk c of row r
  // sits at chunk c ^ f(r), and rows 16..31 swap the two 8-byte halves of
  // each chunk (rows r and r + 16 share f(r)).
  __device__ __forceinline__ void store_staged(void* o, float* lse, size_t head_elems, int bh, char* stage) const {
    const float ltot = sum_with_partner(lsum);
    const bool none = !(ltot > 0.f);
    const float inv = none ? 0.f : 1.0f / out_divisor();
    // f(r): rows of a multiple of 256 bytes start on the same bank, so
    // spread rows 0..15 over the 16 chunks; rows of 128 or 384 bytes
    // alternate between the two bank halves, so spread pairs of rows
    constexpr bool kRowAligned = (ROW_BYTES / 4) % 64 == 0;
    auto fr = [](int r) { return kRowAligned ? (r & 15) : ((r >> 1) & 7); };
    {
      const int r = col;
      const int f = fr(r), gsw = (r >> 4) & 1;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          u32x2 w;
          w[0] = Elem<T>::pack(oacc[db][4 * rg + 0] * inv, oacc[db][4 * rg + 1] * inv);
          w[1] = Elem<T>::pack(oacc[db][4 * rg + 2] * inv, oacc[db][4 * rg + 3] * inv);
          const int c = db * 4 + rg;  // columns 32 db + 8 rg .. +8
          *(u32x2*)(stage + r * ROW_BYTES + ((c ^ f) * 16) + 8 * (h ^ gsw)) = w;
        }
    }
    const __amdgpu_buffer_rsrc_t ro =
        STRIDED ? rsrc(oh, o_bytes) : rsrc((const char*)o + head_elems * 2, head_bytes);
#pragma unroll
    for (int i = 0; i < 32 * ROW_BYTES / 1024; ++i) {
      const int off = i * 1024 + lane * 16;
      const int r = off / ROW_BYTES, c = (off % ROW_BYTES) / 16;
      u32x4 v = *(const u32x4*)(stage + r * ROW_BYTES + ((c ^ fr(r)) * 16));
      if ((r >> 4) & 1) v = u32x4{v[2], v[3], v[0], v[1]};
      __builtin_amdgcn_raw_buffer_store_b128(v, ro, o_row(qw + r) + c * 16, 0, 0);
    }
    if (h == 0) {
      const __amdgpu_buffer_rsrc_t rl = rsrc(lse + (size_t)bh * S, (uint32_t)S * 4);
      const float v = none ? -__builtin_inff() : (mc + __builtin_amdgcn_logf(ltot)) * 0.69314718055994531f;
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), rl, (uint32_t)myq * 4, 0, 0);
    }
  }
};

}  // namespace detail
}  // namespace fa
