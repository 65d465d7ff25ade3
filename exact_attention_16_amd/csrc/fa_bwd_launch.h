// Internal interface between the C-ABI front end (fa_api.cpp) and the gfx950
// backward kernels (fa_bwd.hip).  Not installed; callers use include/fa.h.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

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
  int Sk;       // key rows per head (= S for self-attention)
  bool causal;
  float scale;
  int dtype;  // fa_dtype
  // NULL: dense tensors.  Else 24 element strides (host memory, read at
  // launch): batch, head, row of q, k, v, o, dout, dq, dk, dv.
  const long long* strides;
};

// Largest work-group count of the backward launches (for the host-side
// grid-size check).  Requires a validated head dimension.
long long bwd_grid_size(const BwdArgs& a);

// Enqueue the backward kernels (dQ and D first, then dK and dV) on `stream`.
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);

}  // namespace fa
