// fa_api.cpp -- the exported C ABI (include/fa.h): argument validation,
// workspace layout and dispatch to the kernel launchers. Every check runs on
// the host before anything is enqueued, so a rejected call touches no device
// state.
#include "../../include/fa.h"

#include <float.h>
#include <math.h>
#include <stdint.h>

#include "fa_internal.hpp"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// The kernels' exponent multiplier scale*log2(e). It is kept >= FLT_MIN so
// that a hidden score (-inf) always maps to exp2(-inf) = 0; for scale = 0 the
// finite scores then give exp2(~1e-35) = 1 exactly, as they should.
float exp2_scale(float scale) { return fmaxf(scale * kLog2e, FLT_MIN); }

size_t elem_size(int dtype) { return dtype == FA_F32 ? 4 : 2; }

bool dtype_ok(int dtype) { return dtype == FA_F32 || dtype == FA_F16 || dtype == FA_BF16; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [p, p+n) and [q, q+m) intersect.
bool overlap(const void* p, size_t n, const void* q, size_t m) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + m && b < a + n;
}

constexpr size_t kAlign = 256;
constexpr int kMaxSplits = 64;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Shared shape checks. Returns FA_OK or the status to report.
int check_shape(int B, int H, int N, int d, float scale, int causal, int dtype) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale < 0.f) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // One head's slab is addressed with 32-bit byte offsets (plus one tile of
  // overrun past N); the whole problem with 64-bit ones.
  const long long total = (long long)B * H * N * d;
  if ((long long)N * d * elem_size(dtype) > (1ll << 31) - (1ll << 20) || total >= (1ll << 40))
    return FA_ERR_UNSUPPORTED;
  if (fa::fwd_grid_size(B, H, N) >= (1ll << 31)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// Options with defaults filled in; FA_OK or FA_ERR_INVALID_ARG.
struct Opts {
  int Hkv, wl, wr;
};
// A window bound of N - 1 or more hides nothing on its side, so it is the
// same as no bound; mapping it to -1 keeps the kernels' index sums (query
// +/- bound) within int for every accepted bound up to INT_MAX.
int window_bound(int b, int N) { return b < 0 || b >= N - 1 ? -1 : b; }

int read_opts(const fa_options* o, int H, int N, Opts* out) {
  out->Hkv = H;
  out->wl = out->wr = -1;
  if (!o) return FA_OK;
  if (o->kv_heads < 0 || (o->kv_heads > 0 && H % o->kv_heads != 0)) return FA_ERR_INVALID_ARG;
  out->Hkv = o->kv_heads == 0 ? H : o->kv_heads;
  out->wl = window_bound(o->window_left, N);
  out->wr = window_bound(o->window_right, N);
  return FA_OK;
}

// Block-sparse calls: the mask's side in blocks (N <= 65536, 16-bit types),
// or the status to report (as a negative number).
int mask_blocks(const void* mask, int N, int dtype) {
  if (!mask) return FA_ERR_INVALID_ARG;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  const int nmb = (N + fa::kMaskBlock - 1) / fa::kMaskBlock;
  if (nmb > fa::kMaxMaskBlocks) return FA_ERR_UNSUPPORTED;
  return nmb;
}

// key_split: 0 = the library's choice (fa_fwd, fa_fwd_ex, fa_fwd_sparse),
// 1 = the key-split kernel (fa_fwd_keysplit; 16-bit, dense).
int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int N, int d, float scale, int causal, int dtype, const fa_options* opts,
             const void* mask, void* stream, int key_split = 0) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  int st = check_shape(B, H, N, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  if (key_split && dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  Opts op;
  if ((st = read_opts(opts, H, N, &op)) != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  const size_t tb = (size_t)B * H * N * d * elem_size(dtype);
  const size_t kb = (size_t)B * op.Hkv * N * d * elem_size(dtype);
  const size_t lb = (size_t)B * H * N * sizeof(float);
  struct Range { const void* p; size_t n; };
  const Range ins[] = {{q, tb}, {k, kb}, {v, kb}};
  for (const Range& in : ins)
    if (overlap(o, tb, in.p, in.n) || overlap(lse, lb, in.p, in.n)) return FA_ERR_INVALID_ARG;
  if (overlap(o, tb, lse, lb)) return FA_ERR_INVALID_ARG;

  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, scale, exp2_scale(scale), causal, dtype,
                op.Hkv, op.wl, op.wr};
  if (mask) {
    const int nmb = mask_blocks(mask, N, dtype);
    if (nmb < 0) return nmb;
    const size_t mb = (size_t)nmb * nmb;
    if (overlap(mask, mb, o, tb) || overlap(mask, mb, lse, lb)) return FA_ERR_INVALID_ARG;
    a.block_mask = static_cast<const uint8_t*>(mask);
    a.nmb = nmb;
  }
  a.key_split = !mask && (key_split || fa::fwd_auto_key_split(B, H, N, d, dtype, causal));
  return hip_status(fa::launch_fwd(a, reinterpret_cast<hipStream_t>(stream)));
}

// Scratch bytes of the plain backward (no grouped K/V heads) when the
// library supplies them: D, plus the float32 dQ accumulator for FA_F32 (the
// 16-bit kernels write dQ directly; without grouped heads nothing is split).
size_t plain_scratch_bytes(int B, int H, int N, int d, int dtype) {
  const size_t rows = (size_t)B * H * N;
  return round_up(rows * sizeof(float)) + (dtype == FA_F32 ? round_up(rows * d * sizeof(float)) : 0);
}

// workspace == nullptr with static_ws: the library's static scratch
// (fa_bwd_noalloc; opts and mask are then NULL).
int bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dO,
             const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
             float scale, int causal, int dtype, const fa_options* opts, const void* mask,
             void* workspace, size_t workspace_bytes, void* stream, bool static_ws = false) {
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv || (!workspace && !static_ws))
    return FA_ERR_INVALID_ARG;
  int st = check_shape(B, H, N, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  Opts op;
  if ((st = read_opts(opts, H, N, &op)) != FA_OK) return st;
  const void* ptrs[] = {q, k, v, o, dO, lse, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  size_t need = 0;
  if (static_ws) {
    if (plain_scratch_bytes(B, H, N, d, dtype) > fa::kStaticScratchBytes) return FA_ERR_SCRATCH;
  } else {
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return FA_ERR_ALIGN;
    need = fa_bwd_workspace_size(B, H, N, d);
    if (workspace_bytes < need) return FA_ERR_WORKSPACE;
  }

  const size_t tb = (size_t)B * H * N * d * elem_size(dtype);
  const size_t kb = (size_t)B * op.Hkv * N * d * elem_size(dtype);
  const size_t lb = (size_t)B * H * N * sizeof(float);
  struct Range { const void* p; size_t n; };
  const Range ins[] = {{q, tb}, {k, kb}, {v, kb}, {o, tb}, {dO, tb}, {lse, lb}};
  const Range outs[] = {{dq, tb}, {dk, kb}, {dv, kb}, {workspace, need}};
  for (const Range& w : outs) {
    for (const Range& r : ins)
      if (overlap(w.p, w.n, r.p, r.n)) return FA_ERR_INVALID_ARG;
    for (const Range& x : outs)
      if (&x != &w && overlap(w.p, w.n, x.p, x.n)) return FA_ERR_INVALID_ARG;
  }
  if (static_ws) {  // validated: now look up this GPU's scratch (no allocation)
    const hipError_t e = fa::static_scratch(&workspace);
    if (e != hipSuccess) return FA_ERR_HIP;
  }

  char* ws = static_cast<char*>(workspace);
  float* dsum = reinterpret_cast<float*>(ws);
  float* scratch = reinterpret_cast<float*>(ws + round_up(lb));
  fa::BwdArgs a{q, k, v, o, dO, lse, dq, dk, dv, dsum, scratch,
                B, H, N, d, scale, exp2_scale(scale), causal, dtype, op.Hkv, op.wl, op.wr,
                scratch};
  if (mask) {
    const int nmb = mask_blocks(mask, N, dtype);
    if (nmb < 0) return nmb;
    const size_t mb = (size_t)nmb * nmb;
    for (const Range& w : outs)
      if (overlap(mask, mb, w.p, w.n)) return FA_ERR_INVALID_ARG;
    a.block_mask = static_cast<const uint8_t*>(mask);
    a.nmb = nmb;
  }
  return hip_status(fa::launch_bwd(a, reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int N, int d, float scale, int causal, int dtype, const fa_options* opts,
              void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, opts, nullptr, stream);
}

int fa_fwd_keysplit(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int H, int N, int d, float scale, int causal, int dtype,
                    const fa_options* opts, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, opts, nullptr, stream, 1);
}

int fa_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int H, int N, int d, float scale, int causal, int dtype,
                  const fa_options* opts, const void* block_mask, void* stream) {
  if (!block_mask) return FA_ERR_INVALID_ARG;
  return fwd_impl(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, opts, block_mask, stream);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
           int N, int d, float scale, int causal, int dtype, void* stream) {
  return fa_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, nullptr, stream);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int N, int d, float scale, int causal, float q_descale, float k_descale,
               float v_descale, int out_dtype, const fa_options* opts, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (out_dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (out_dtype != FA_F16 && out_dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  int st = check_shape(B, H, N, d, scale, causal, out_dtype);
  if (st != FA_OK) return st;
  const float descales[] = {q_descale, k_descale, v_descale};
  for (float x : descales)
    if (!isfinite(x) || !(x > 0.f)) return FA_ERR_INVALID_ARG;
  const float score_scale = scale * q_descale * k_descale;
  if (!isfinite(score_scale)) return FA_ERR_INVALID_ARG;
  Opts op;
  if ((st = read_opts(opts, H, N, &op)) != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  const size_t qb = (size_t)B * H * N * d;
  const size_t kb = (size_t)B * op.Hkv * N * d;
  const size_t ob = qb * elem_size(out_dtype);
  const size_t lb = (size_t)B * H * N * sizeof(float);
  struct Range { const void* p; size_t n; };
  const Range ins[] = {{q, qb}, {k, kb}, {v, kb}};
  for (const Range& in : ins)
    if (overlap(o, ob, in.p, in.n) || overlap(lse, lb, in.p, in.n)) return FA_ERR_INVALID_ARG;
  if (overlap(o, ob, lse, lb)) return FA_ERR_INVALID_ARG;

  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, score_scale, exp2_scale(score_scale), causal,
                out_dtype, op.Hkv, op.wl, op.wr};
  a.v_descale = v_descale;
  return hip_status(fa::launch_fwd_fp8(a, reinterpret_cast<hipStream_t>(stream)));
}

int fa_fwd_num_splits(int B, int H, int N, int d, int dtype) {
  if (check_shape(B, H, N, d, 1.f, 0, dtype) != FA_OK) return 0;
  return fa::fwd_auto_splits(B, H, N, dtype);
}

size_t fa_fwd_splitkv_workspace_size(int B, int H, int N, int d, int dtype, int num_splits) {
  if (check_shape(B, H, N, d, 1.f, 0, dtype) != FA_OK) return 0;
  if (num_splits < 0 || num_splits > kMaxSplits) return 0;
  const int s = num_splits == 0 ? fa::fwd_auto_splits(B, H, N, dtype) : num_splits;
  if (s == 1) return 0;
  const size_t rows = (size_t)s * B * H * N;
  return round_up(rows * d * sizeof(float)) + round_up(rows * sizeof(float));
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int H, int N, int d, float scale, int causal, int dtype,
                   const fa_options* opts, int num_splits, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  int st = check_shape(B, H, N, d, scale, causal, dtype);
  if (st != FA_OK) return st;
  Opts op;
  if ((st = read_opts(opts, H, N, &op)) != FA_OK) return st;
  if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_INVALID_ARG;
  const int ns = num_splits == 0 ? fa::fwd_auto_splits(B, H, N, dtype) : num_splits;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  const size_t need = fa_fwd_splitkv_workspace_size(B, H, N, d, dtype, ns);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0) return FA_ERR_ALIGN;
  }
  const size_t tb = (size_t)B * H * N * d * elem_size(dtype);
  const size_t kb = (size_t)B * op.Hkv * N * d * elem_size(dtype);
  const size_t lb = (size_t)B * H * N * sizeof(float);
  struct Range { const void* p; size_t n; };
  const Range ins[] = {{q, tb}, {k, kb}, {v, kb}};
  const Range outs[] = {{o, tb}, {lse, lb}, {workspace, need}};
  for (const Range& w : outs) {
    if (w.n == 0) continue;
    for (const Range& r : ins)
      if (overlap(w.p, w.n, r.p, r.n)) return FA_ERR_INVALID_ARG;
    for (const Range& x : outs)
      if (&x != &w && x.n > 0 && overlap(w.p, w.n, x.p, x.n)) return FA_ERR_INVALID_ARG;
  }
  if (fa::fwd_grid_size(B, H, N) * ns >= (1ll << 31)) return FA_ERR_UNSUPPORTED;

  fa::FwdArgs a{q, k, v, o, lse, B, H, N, d, scale, exp2_scale(scale), causal, dtype,
                op.Hkv, op.wl, op.wr};
  if (ns > 1) {
    char* ws = static_cast<char*>(workspace);
    a.num_splits = ns;
    a.o_part = reinterpret_cast<float*>(ws);
    a.lse_part = reinterpret_cast<float*>(ws + round_up((size_t)ns * B * H * N * d * sizeof(float)));
  }
  return hip_status(fa::launch_fwd(a, reinterpret_cast<hipStream_t>(stream)));
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || (d != 64 && d != 128)) return 0;
  const size_t rows = (size_t)B * H * N;
  return round_up(rows * sizeof(float)) + round_up(2 * rows * d * sizeof(float));
}

int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dO,
              const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
              float scale, int causal, int dtype, const fa_options* opts, void* workspace,
              size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, opts,
                  nullptr, workspace, workspace_bytes, stream);
}

int fa_bwd_sparse(const void* q, const void* k, const void* v, const void* o, const void* dO,
                  const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                  float scale, int causal, int dtype, const fa_options* opts,
                  const void* block_mask, void* workspace, size_t workspace_bytes,
                  void* stream) {
  if (!block_mask) return FA_ERR_INVALID_ARG;
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, opts,
                  block_mask, workspace, workspace_bytes, stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
           const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
           float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
           void* stream) {
  return fa_bwd_ex(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, nullptr,
                   workspace, workspace_bytes, stream);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                   const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                   float scale, int causal, int dtype, void* stream) {
  return bwd_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, nullptr,
                  nullptr, nullptr, 0, stream, true);
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension or size";
    case FA_ERR_ALIGN: return "pointer not sufficiently aligned";
    case FA_ERR_WORKSPACE: return "workspace too small";
    case FA_ERR_HIP: return "HIP runtime error at launch";
    case FA_ERR_SCRATCH: return "problem too large for the library's static scratch";
    default: return "unknown status";
  }
}

}  // extern "C"
