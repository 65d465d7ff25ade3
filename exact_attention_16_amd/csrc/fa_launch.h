// Internal interface between the C-ABI front end (fa_api.cpp) and the gfx950
// forward and decoding kernels (fa_fwd.hip, fa_fwd_wide.hip, fa_decode.hip);
// the backward's is fa_bwd_launch.h.  Not
// installed; callers use
// include/fa.h.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, S, d;
  int Sk;     // key rows per head (= S for self-attention)
  bool causal;
  float scale;
  int dtype;  // fa_dtype
  // NULL: dense [B][H][S][d] tensors.  Else 12 element strides (host memory,
  // read at launch): batch, head, row of q, k, v and o; d is contiguous.
  const long long* strides;
};

// Number of work-groups the forward launch of `a` uses (for the host-side
// grid-size check).  Requires a validated head dimension.
long long fwd_grid_size(const FwdArgs& a);

// Enqueue the forward kernels on `stream`; returns the launch status.
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);

// The same for the in-order kernel (fa_fwd_wide.hip), used by the two
// functions above for head dimensions 192 and 256 and for short causal
// problems at 64 and 128 (uses_in_order_kernel).
long long fwd_wide_grid_size(const FwdArgs& a);
hipError_t launch_fwd_wide(const FwdArgs& a, hipStream_t stream);

// Short causal problems run faster on the in-order kernel's 128-row blocks:
// with few key tiles per block, finer blocks balance the triangular work
// better than the ping-pong kernel's 256 rows (measured on the MI355X).  At
// d = 128 the persistent ping-pong grid pairs long and short blocks, which
// moves the crossover down: S = 1024 causal runs 8 % faster there, S = 512
// ties.
inline bool uses_in_order_kernel(const FwdArgs& a) {
  if (a.d > 128) return true;
  return a.causal && a.Sk <= (a.d == 64 ? 2048 : 512);
}

}  // namespace fa

namespace fa {

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  void* workspace;  // partial results, DecodePlan::workspace_bytes
  int B, H, Sq, Sk, d;
  bool causal;
  float scale;
  int dtype;  // fa_dtype
  const long long* strides;  // as FwdArgs::strides (NULL: dense)
};

// Shape of the split-key pass for head dimension d: wavefronts per
// work-group, 32-key blocks per wavefront in each shared key tile, the
// work-groups it aims for, and the fewest key tiles a split may hold.  Chosen
// by measurement on the MI355X (1 GiB K/V caches): tiles of 128 keys at
// d = 64 and 64 keys at d = 128 (32 KiB of K and V per work-group), and about
// two work-groups per compute unit, read the caches fastest; more resident
// work-groups (more concurrent streams) read them more slowly.
constexpr int decode_waves(int) { return 2; }
constexpr int decode_blocks_per_wave(int d) { return d == 64 ? 2 : 1; }
constexpr int decode_tile_keys(int d) { return 32 * decode_waves(d) * decode_blocks_per_wave(d); }
constexpr long long kDecodeTargetGroups = 512;
constexpr int kMinSplitTiles = 4;

// How the split-key pass divides one call (a pure function of the shapes).
struct DecodePlan {
  int nrb;               // 32-row query blocks per head
  int nsplit;            // key splits per head
  int split_tiles;       // key tiles (decode_tile_keys(d) keys each) per split
  int partials;          // partial results per head and query row (= nsplit)
  size_t partial_o_bytes;
  size_t workspace_bytes;
  long long grid;        // work-groups of the split kernel
};

DecodePlan decode_plan(const DecodeArgs& a);

// Enqueue the split kernel and the merge kernel on `stream`.
hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream);

// Bytes of the library-owned scratch array (fa_decode.hip) that
// fa_fwd_decode_noalloc uses as its workspace; one copy per device.
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;

// Device address of the scratch array's copy on the device that `stream`
// belongs to (the current device for the NULL stream).  Looked up once per
// device with hipGetSymbolAddress and kept; allocates nothing.  On failure
// returns nullptr and sets *err.
void* decode_scratch(hipStream_t stream, hipError_t* err);

}  // namespace fa
