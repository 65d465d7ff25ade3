// Internal interface between the C-ABI front end (fa_api.cpp) and the gfx950
// kernels (fa_fwd.hip).  Not installed; callers use include/fa.h.
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
};

// Number of work-groups the forward launch of `a` uses (for the host-side
// grid-size check).  Requires a validated head dimension.
long long fwd_grid_size(const FwdArgs& a);

// Enqueue the forward kernels on `stream`; returns the launch status.
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);

struct BwdArgs {
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
  int B, H, S, d;
  bool causal;
  float scale;
  int dtype;  // fa_dtype
};

// Largest work-group count of the backward launches (for the host-side
// grid-size check).  Requires a validated head dimension.
long long bwd_grid_size(const BwdArgs& a);

// Enqueue the backward kernels (dQ and D first, then dK and dV) on `stream`.
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);

}  // namespace fa
