// fa_internal.hpp -- argument blocks and launchers shared between the C-ABI
// layer (fa_api.cpp) and the kernel translation units. Host-visible only
// through this header; nothing here is exported from libfa.so.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Forward: contiguous [B,H,N,d] tensors, [B,H,N] float32 LSE.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N, d;
  float scale;       // softmax scale (>= 0)
  float scale_log2;  // scale * log2(e)
  int causal;
  int dtype;         // fa_dtype
  int Hkv;           // K/V heads (divides H)
  int wl, wr;        // window bounds (negative: unbounded)
  // Split-KV: with num_splits > 1 every workgroup covers one of num_splits
  // slices of its key tiles and writes float32 partials -- O normalized over
  // its slice's keys into o_part [num_splits][B,H,N,d] and that slice's LSE
  // (-inf where a row sees none of its keys) into lse_part
  // [num_splits][B,H,N] -- and a second kernel merges them into o and lse.
  int num_splits = 1;
  float* o_part = nullptr;
  float* lse_part = nullptr;
  // 8-bit inputs (launch_fwd_fp8): O is multiplied by this dequantization
  // factor of V; scale / scale_log2 then already hold the product of the
  // softmax scale and the factors of Q and K.
  float v_descale = 1.f;
  // Block-sparse attention: nonzero bytes of block_mask [nmb][nmb] (64-row
  // query block x 64-key block, shared by all batches and heads) mark the
  // blocks whose scores are kept; nullptr = dense.
  const uint8_t* block_mask = nullptr;
  int nmb = 0;
  // 16-bit inputs, dense, one slice: split the key tiles of each workgroup's
  // rows over its waves (fwd_ks_kernel) instead of one workgroup per 256
  // query rows.
  bool key_split = false;
};

// Backward: forward tensors plus dO and the gradient outputs. `dsum` is the
// float32 [B,H,N] row term D, `dq_acc` the float32 [B,H,N,d] dQ accumulator.
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
  float* dsum;
  float* dq_acc;
  int B, H, N, d;
  float scale;
  float scale_log2;
  int causal;
  int dtype;
  int Hkv;     // K/V heads (divides H)
  int wl, wr;  // window bounds (negative: unbounded)
  // float32 scratch of 2 * B*H*N*d elements (16-bit types, grouped K/V
  // heads): when the query heads of a group are split over several
  // workgroups, each part's dK and dV land here before being summed.
  float* dkv_part = nullptr;
  int kv_parts = 1;  // workgroups per key tile (set by the launcher)
  const uint8_t* block_mask = nullptr;  // as in FwdArgs
  int nmb = 0;
};

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);

// fa_bwd_noalloc's scratch: the device address, on the current GPU, of the
// library's static device array of kStaticScratchBytes bytes (looked up once
// per GPU, then cached). Allocates nothing.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
hipError_t static_scratch(void** ptr);
// E4M3 q, k, v (bytes); a.dtype is the output type (fp16 or bf16).
hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);

// Forward tile sizes, shared with the host-side grid arithmetic
// (fa_host.cpp): query rows per workgroup (float32 kernel, 16-bit kernel)
// and keys per tile.
constexpr int kFwdRowsF32 = 128;
constexpr int kFwdRows16 = 256;
constexpr int kFwdRowsKeySplitMin = 64;  // the key-split kernel: 64 (d = 64) or 128 rows
constexpr int kFwdKeyTile = 64;

// Workgroups of the largest forward grid any kernel launches for a shape.
long long fwd_grid_size(int B, int H, int N);

constexpr int kMaskBlock = 64;        // block-sparse mask granularity (rows and keys)
constexpr int kMaxMaskBlocks = 1024;  // block-sparse calls: N <= 65536

// Rows per forward workgroup and the split count the library picks for a
// shape: enough workgroups to occupy every compute unit once, with at least
// four 64-key tiles per slice, at most 16 slices.
int fwd_rows_per_workgroup(int dtype);
int fwd_auto_splits(int B, int H, int N, int dtype);
// Whether fa_fwd / fa_fwd_ex use the key-split kernel for a dense 16-bit
// shape: when one workgroup per 256 query rows would leave compute units
// idle, or (causal) fill them for one uneven round.
bool fwd_auto_key_split(int B, int H, int N, int d, int dtype, int causal);

}  // namespace fa
