// C-ABI front end of libfa.so: argument validation, status text and dispatch.
// Validation runs on the host before any HIP call, so every error below can be
// exercised without a GPU.

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fa.h"
#include "fa_bwd_launch.h"
#include "fa_launch.h"

namespace {

thread_local char g_last_hip_error[256] = "";

// Head dimensions of every entry point (forward, decoding and backward kernels).
bool supported_head_dim(int d) { return d == 64 || d == 128 || d == 192 || d == 256; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (na == 0 || nb == 0) return false;  // an empty range overlaps nothing
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Element strides of one tensor: batch, head, row (d is contiguous).
struct Layout {
  long long sb, sh, rs;
};

Layout dense_layout(int H, int rows, int d) { return {(long long)H * rows * d, (long long)rows * d, d}; }

// Bytes from the tensor's base to the end of its last element.
size_t extent_bytes(const Layout& l, int B, int H, int rows, int d) {
  return 2 * (size_t)((B - 1) * l.sb + (H - 1) * l.sh + (rows - 1) * l.rs + d);
}

// Do distinct (batch, head, row, column) positions map to distinct elements?
// Sufficient test: ordered by stride, every dimension steps past the whole
// extent of the smaller ones.
bool injective(const Layout& l, int B, int H, int rows, int d) {
  long long st[3] = {l.sb, l.sh, l.rs}, n[3] = {B, H, rows};
  for (int i = 0; i < 3; ++i)  // sort by stride (three elements)
    for (int j = i + 1; j < 3; ++j)
      if (st[j] < st[i]) {
        const long long a = st[i], b = n[i];
        st[i] = st[j], n[i] = n[j], st[j] = a, n[j] = b;
      }
  long long reach = d;  // elements spanned by the dimensions placed so far
  for (int i = 0; i < 3; ++i) {
    if (n[i] <= 1) continue;
    if (st[i] < reach) return false;
    reach = st[i] * (n[i] - 1) + reach;
  }
  return true;
}

// Checks of one strided tensor: strides >= 0, 16-byte rows, rows at least d
// apart (also with one row: the kernels address rows past the end, which the
// range checks must drop), and every such row offset within 32 bits.
int check_layout(const Layout& l, int rows, int d) {
  if (l.sb < 0 || l.sh < 0 || l.rs < 0) return FA_ERR_STRIDE;
  if (l.rs < d) return FA_ERR_STRIDE;
  if ((l.sb | l.sh | l.rs) & 7) return FA_ERR_ALIGN;
  if (((long long)rows + 512) * l.rs * 2 + 2 * d > 0xffffffffLL) return FA_ERR_TOO_LARGE;
  return FA_OK;
}

// Shared by fa_fwd (Sk = S), fa_fwd_kv and fa_fwd_strided (strides != NULL:
// q, k, v, o batch/head/row element strides).  With Sk = 0 the key tensors
// are never read, so k and v may be NULL.
// Byte extents of q, k, v, o and lse from their bases (filled by validate).
struct Extents {
  size_t q, k, v, o, l;
};

int validate(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H,
             int S, int Sk, int d, int causal, float scale, int dtype, const long long* strides = nullptr,
             bool strided = false, Extents* ext = nullptr) {
  if (B < 0 || H < 0 || S < 0 || Sk < 0 || (causal != 0 && causal != 1)) return FA_ERR_SHAPE;
  if (!supported_head_dim(d)) return FA_ERR_HEAD_DIM;
  if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (!isfinite(scale) || scale < 0.f) return FA_ERR_SCALE;
  if ((long long)B * H * S == 0) return FA_OK;  // empty problem: nothing to touch
  if (!q || !o || !lse || (Sk > 0 && (!k || !v)) || (strided && !strides)) return FA_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return FA_ERR_ALIGN;
  if ((uintptr_t)lse & 3u) return FA_ERR_ALIGN;
  if ((long long)S * d >= (1LL << 30) || (long long)Sk * d >= (1LL << 30)) return FA_ERR_TOO_LARGE;  // 32-bit buffer offsets
  fa::FwdArgs a{};
  a.B = B; a.H = H; a.S = S; a.Sk = Sk; a.d = d;
  a.causal = causal != 0;  // the kernel (and so the grid) depends on it
  if (fa::fwd_grid_size(a) > 0x7fffffffLL) return FA_ERR_TOO_LARGE;
  Layout lq = dense_layout(H, S, d), lk = dense_layout(H, Sk, d), lv = lk, lo = lq;
  if (strided) {
    lq = {strides[0], strides[1], strides[2]};
    lk = {strides[3], strides[4], strides[5]};
    lv = {strides[6], strides[7], strides[8]};
    lo = {strides[9], strides[10], strides[11]};
    int st;
    if ((st = check_layout(lq, S, d)) != FA_OK || (st = check_layout(lo, S, d)) != FA_OK) return st;
    if (Sk > 0 && ((st = check_layout(lk, Sk, d)) != FA_OK || (st = check_layout(lv, Sk, d)) != FA_OK)) return st;
    if (!injective(lo, B, H, S, d)) return FA_ERR_STRIDE;
  }
  const size_t nq = extent_bytes(lq, B, H, S, d), no = extent_bytes(lo, B, H, S, d);
  const size_t nk = Sk > 0 ? extent_bytes(lk, B, H, Sk, d) : 0, nv = Sk > 0 ? extent_bytes(lv, B, H, Sk, d) : 0;
  const size_t nl = (size_t)B * H * S * 4;  // bytes of lse
  if (ext) *ext = {nq, nk, nv, no, nl};
  if (overlaps(o, no, q, nq) || overlaps(o, no, k, nk) || overlaps(o, no, v, nv) ||
      overlaps(o, no, lse, nl) || overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nk) ||
      overlaps(lse, nl, v, nv))
    return FA_ERR_ALIAS;
  return FA_OK;
}

// fa_bwd, fa_bwd_kv and fa_bwd_strided.  q, o, dout, dq, lse and delta hold
// Sq rows per head, k, v, dk and dv Sk rows; strides != NULL: q, k, v, o,
// dout, dq, dk, dv batch/head/row element strides.  square: fa_bwd's
// contract (Sq = Sk = S; B*H*S == 0 is a no-op).  Otherwise a side with no
// rows is not touched, so its pointers may be NULL: with Sq = 0 the call
// writes dk = dv = 0, with Sk = 0 it writes dq = 0 and delta.
int validate_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                 void* dq, void* dk, void* dv, float* delta, int B, int H, int Sq, int Sk, int d, int causal,
                 float scale, int dtype, const long long* strides = nullptr, bool strided = false,
                 bool square = false) {
  if (B < 0 || H < 0 || Sq < 0 || Sk < 0 || (causal != 0 && causal != 1)) return FA_ERR_SHAPE;
  if (!supported_head_dim(d)) return FA_ERR_HEAD_DIM;  // the backward takes the same widths
  if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (!isfinite(scale) || scale < 0.f) return FA_ERR_SCALE;
  if ((long long)B * H == 0 || (square ? Sq == 0 : (Sq == 0 && Sk == 0))) return FA_OK;
  const bool qs = Sq > 0, ks = Sk > 0;  // which sides are touched
  if ((qs && (!q || !o || !lse || !dout || !dq || !delta)) || (ks && (!k || !v || !dk || !dv)) ||
      (strided && !strides))
    return FA_ERR_NULL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout | (uintptr_t)dq |
       (uintptr_t)dk | (uintptr_t)dv) & 15u)
    return FA_ERR_ALIGN;
  if (((uintptr_t)lse | (uintptr_t)delta) & 3u) return FA_ERR_ALIGN;
  if ((long long)Sq * d >= (1LL << 30) || (long long)Sk * d >= (1LL << 30)) return FA_ERR_TOO_LARGE;
  fa::BwdArgs a{};
  a.B = B; a.H = H; a.S = Sq; a.Sk = Sk; a.d = d;
  if (fa::bwd_grid_size(a) > 0x7fffffffLL) return FA_ERR_TOO_LARGE;
  // byte extents of q, k, v, o, dout, dq, dk, dv (dense, or from the strides)
  size_t ext[8];
  for (int t = 0; t < 8; ++t) {
    const bool key_side = t == 1 || t == 2 || t == 6 || t == 7;  // k, v, dk, dv
    const int rows = key_side ? Sk : Sq;
    if (rows == 0) {
      ext[t] = 0;
      continue;
    }
    Layout l = dense_layout(H, rows, d);
    if (strided) {
      l = {strides[3 * t], strides[3 * t + 1], strides[3 * t + 2]};
      const int st = check_layout(l, rows, d);
      if (st != FA_OK) return st;
      if (t >= 5 && !injective(l, B, H, rows, d)) return FA_ERR_STRIDE;  // dq, dk, dv
    }
    ext[t] = extent_bytes(l, B, H, rows, d);
  }
  const size_t nl = (size_t)B * H * Sq * 4;
  const void* ins[6] = {q, k, v, o, dout, lse};
  const size_t in_bytes[6] = {ext[0], ext[1], ext[2], ext[3], ext[4], nl};
  const void* outs[4] = {dq, dk, dv, delta};
  const size_t out_bytes[4] = {ext[5], ext[6], ext[7], nl};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

// fa_fwd_decode: validate() plus the workspace, which must be present, large
// enough, 16-byte aligned and disjoint from every tensor.
int validate_decode(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H,
                    int Sq, int Sk, int d, int causal, float scale, int dtype, const void* ws, size_t ws_bytes,
                    fa::DecodePlan* plan, const long long* strides = nullptr, bool strided = false) {
  Extents e{};
  const int st = validate(q, k, v, o, lse, B, H, Sq, Sk, d, causal, scale, dtype, strides, strided, &e);
  if (st != FA_OK || (long long)B * H * Sq == 0) return st;
  fa::DecodeArgs a{};
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk; a.d = d;
  *plan = fa::decode_plan(a);
  if (plan->grid > 0x7fffffffLL || (long long)B * H * Sq > 0x7fffffffLL) return FA_ERR_TOO_LARGE;
  if (!ws || ws_bytes < plan->workspace_bytes || ((uintptr_t)ws & 15u)) return FA_ERR_WORKSPACE;
  const size_t nw = plan->workspace_bytes;
  if (overlaps(ws, nw, q, e.q) || overlaps(ws, nw, k, e.k) || overlaps(ws, nw, v, e.v) || overlaps(ws, nw, o, e.o) ||
      overlaps(ws, nw, lse, e.l))
    return FA_ERR_ALIAS;
  return FA_OK;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  snprintf(g_last_hip_error, sizeof g_last_hip_error, "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
  return FA_ERR_HIP;
}

int forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int S, int Sk, int d,
            int causal, float scale, int dtype, void* stream, const long long* strides = nullptr,
            bool strided = false) {
  const int st = validate(q, k, v, o, lse, B, H, S, Sk, d, causal, scale, dtype, strides, strided);
  if (st != FA_OK) return st;
  if ((long long)B * H * S == 0) return FA_OK;
  fa::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.H = H; a.S = S; a.d = d; a.Sk = Sk;
  a.causal = causal != 0;
  a.scale = scale;
  a.dtype = dtype;
  a.strides = strided ? strides : nullptr;
  return hip_status(fa::launch_fwd(a, (hipStream_t)stream));
}

int decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Sq, int Sk, int d,
           int causal, float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream,
           const long long* strides = nullptr, bool strided = false) {
  fa::DecodePlan plan{};
  const int st = validate_decode(q, k, v, o, lse, B, H, Sq, Sk, d, causal, scale, dtype, workspace,
                                 workspace_bytes, &plan, strides, strided);
  if (st != FA_OK) return st;
  if ((long long)B * H * Sq == 0) return FA_OK;
  fa::DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.workspace = workspace;
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.causal = causal != 0;
  a.scale = scale;
  a.dtype = dtype;
  a.strides = strided ? strides : nullptr;
  return hip_status(fa::launch_decode(a, plan, (hipStream_t)stream));
}

static_assert(FA_DECODE_NOALLOC_MAX_BYTES == fa::kDecodeScratchBytes, "scratch size in fa.h and fa_launch.h");

// fa_fwd_decode with the library's scratch array as the workspace: the same
// validation (minus the workspace argument), a size check against the array,
// then the same kernels.
int decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Sq, int Sk,
                   int d, int causal, float scale, int dtype, void* stream) {
  const int st = validate(q, k, v, o, lse, B, H, Sq, Sk, d, causal, scale, dtype);
  if (st != FA_OK) return st;
  if ((long long)B * H * Sq == 0) return FA_OK;
  fa::DecodeArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk; a.d = d;
  a.causal = causal != 0;
  a.scale = scale;
  a.dtype = dtype;
  a.strides = nullptr;
  const fa::DecodePlan plan = fa::decode_plan(a);
  if (plan.grid > 0x7fffffffLL || (long long)B * H * Sq > 0x7fffffffLL) return FA_ERR_TOO_LARGE;
  if (plan.workspace_bytes > fa::kDecodeScratchBytes) return FA_ERR_SCRATCH;
  hipError_t err = hipSuccess;
  a.workspace = fa::decode_scratch((hipStream_t)stream, &err);
  if (!a.workspace) return hip_status(err);
  return hip_status(fa::launch_decode(a, plan, (hipStream_t)stream));
}

int backward(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
             void* dk, void* dv, float* delta, int B, int H, int Sq, int Sk, int d, int causal, float scale,
             int dtype, void* stream, const long long* strides, bool strided, bool square) {
  const int st = validate_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Sq, Sk, d, causal, scale, dtype,
                              strides, strided, square);
  if (st != FA_OK) return st;
  if ((long long)B * H == 0 || (Sq == 0 && Sk == 0) || (square && Sq == 0)) return FA_OK;
  fa::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv; a.delta = delta;
  a.B = B; a.H = H; a.S = Sq; a.Sk = Sk; a.d = d;
  a.causal = causal != 0;
  a.scale = scale;
  a.dtype = dtype;
  a.strides = strided ? strides : nullptr;
  return hip_status(fa::launch_bwd(a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int S, int d,
           int causal, float scale, int dtype, void* stream) {
  return forward(q, k, v, o, lse, B, H, S, S, d, causal, scale, dtype, stream);
}

int fa_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Sq, int Sk,
              int d, int causal, float scale, int dtype, void* stream) {
  return forward(q, k, v, o, lse, B, H, Sq, Sk, d, causal, scale, dtype, stream);
}

int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Sq, int Sk,
                   int d, const long long* strides, int causal, float scale, int dtype, void* stream) {
  return forward(q, k, v, o, lse, B, H, Sq, Sk, d, causal, scale, dtype, stream, strides, true);
}

size_t fa_fwd_decode_workspace_size(int B, int H, int Sq, int Sk, int d) {
  if (B <= 0 || H <= 0 || Sq <= 0 || Sk < 0 || !supported_head_dim(d)) return 0;
  fa::DecodeArgs a{};
  a.B = B; a.H = H; a.Sq = Sq; a.Sk = Sk; a.d = d;
  return fa::decode_plan(a).workspace_bytes;
}

int fa_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Sq, int Sk,
                  int d, int causal, float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return decode(q, k, v, o, lse, B, H, Sq, Sk, d, causal, scale, dtype, workspace, workspace_bytes, stream);
}

int fa_fwd_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Sq,
                          int Sk, int d, int causal, float scale, int dtype, void* stream) {
  return decode_noalloc(q, k, v, o, lse, B, H, Sq, Sk, d, causal, scale, dtype, stream);
}

int fa_fwd_decode_strided(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Sq,
                          int Sk, int d, const long long* strides, int causal, float scale, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return decode(q, k, v, o, lse, B, H, Sq, Sk, d, causal, scale, dtype, workspace, workspace_bytes, stream,
                strides, true);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
           void* dk, void* dv, float* delta, int B, int H, int S, int d, int causal, float scale, int dtype,
           void* stream) {
  return backward(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, S, S, d, causal, scale, dtype, stream, nullptr,
                  false, true);
}

int fa_bwd_kv(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
              void* dq, void* dk, void* dv, float* delta, int B, int H, int Sq, int Sk, int d, int causal,
              float scale, int dtype, void* stream) {
  return backward(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Sq, Sk, d, causal, scale, dtype, stream, nullptr,
                  false, false);
}

int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, float* delta, int B, int H, int Sq, int Sk, int d,
                   const long long* strides, int causal, float scale, int dtype, void* stream) {
  return backward(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Sq, Sk, d, causal, scale, dtype, stream, strides,
                  true, false);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a pointer argument is NULL";
    case FA_ERR_SHAPE: return "B, H, S or Sk is negative, or causal is not 0 or 1";
    case FA_ERR_HEAD_DIM: return "head dimension d must be 64, 128, 192 or 256";
    case FA_ERR_DTYPE: return "dtype must be FA_DTYPE_FP16 or FA_DTYPE_BF16";
    case FA_ERR_SCALE: return "scale must be finite and >= 0";
    case FA_ERR_ALIGN:
      return "tensors must be 16-byte aligned (strides multiples of 8 elements), and lse and delta 4-byte aligned";
    case FA_ERR_ALIAS: return "an output overlaps an input or another output";
    case FA_ERR_TOO_LARGE: return "problem too large: S*d and Sk*d must be < 2^30 and the grid < 2^31 work-groups";
    case FA_ERR_HIP: return "the HIP runtime rejected the launch";
    case FA_ERR_STRIDE:
      return "a stride is negative, a row stride is below d, or the output's strides map two positions to one "
             "element";
    case FA_ERR_WORKSPACE:
      return "workspace is NULL, smaller than fa_fwd_decode_workspace_size() or not 16-byte aligned";
    case FA_ERR_SCRATCH:
      return "fa_fwd_decode_noalloc: these shapes need more than FA_DECODE_NOALLOC_MAX_BYTES of scratch "
             "(fa_fwd_decode_workspace_size() bytes); use fa_fwd_decode with a workspace";
    default: return "unknown status";
  }
}

const char* fa_last_hip_error(void) { return g_last_hip_error; }

int fa_version(void) { return 300; }  // 0.3.0

}  // extern "C"
