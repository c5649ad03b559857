// fa_fwd_fp8.hip -- forward exact attention over 8-bit float inputs (gfx950).
//
// What it computes: the attention forward of fa_fwd (softmax of the scaled
// scores, causal rule and local window as options, grouped K/V heads) over
// inputs stored as OCP FP8 E4M3 codes, each tensor with one dequantization
// factor: Q = q_descale * Q8, K = k_descale * K8, V = v_descale * V8. O is
// written in bf16 or fp16, the LSE in float32. The pages name lower-precision
// data types (FP8, INT8) only as a direction for the method (section
// "应用展望" of "FlashAttention与新一代硬件架构融合：解锁大模型训练新高度")
// and give no scaling scheme; per-tensor
// factors are the plainest one, and they fold into the exponent multiplier
// and the epilogue, so the matrix products run on raw codes.
//
// Design: the 16-bit forward's ping-pong structure (8 waves = 256 query rows
// per workgroup; groups A and B one barrier apart, alternating a matrix phase
// -- O^T += V^T P^T for the previous 64-key tile, then S^T = K Q^T for the
// current one -- with a vector phase, the online softmax). What changes:
//   * both products run on v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3, float32
//     accumulate, K depth 64: 32 bytes of each operand per lane), at twice
//     the 16-bit rate; a 32x32 score block at d = 128 is two instructions.
//   * V stays row-major in LDS (16-byte units XOR-swizzled by key) and the
//     V^T operand is read with ds_read_b64_tr_b8, eight keys of one head-dim
//     column per lane and read.
//   * the probabilities enter the PV product as E4M3 codes. They are taken
//     as 2^3 * exp2(scaled score - reference), where the reference moves to
//     the row max whenever some value could exceed 448 (E4M3's largest
//     finite value), and the normal range of E4M3 (>= 2^-6) covers
//     probabilities down to 2^-9 of the max at the last move. The
//     row sum is accumulated from the unrounded float32 values, so the LSE
//     is exact to float32 and O carries only the probabilities' rounding
//     (relative 2^-4 per probability, an average over the keys).
#include <float.h>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(8))) uint32_t u32x8;
typedef __attribute__((ext_vector_type(2))) int i32x2;

constexpr int kF8Waves = 8;
constexpr int kF8Threads = kF8Waves * 64;
constexpr int kF8Group = kF8Threads / 2;  // threads per wave group
constexpr int kF8BM = kF8Waves * 32;      // query rows per workgroup
constexpr int kF8BN = 64;                 // keys per K/V tile
constexpr float kPLog2 = 3.f;             // probabilities enter the PV product as 2^3 * p
constexpr float kPMax = 448.f;            // largest finite E4M3 value

// S += A B on the FP8 matrix cores: A and B are E4M3 (format code 0 for
// both); zero scale operands select the unscaled instruction.
__device__ inline f32x16 mma8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Transposing LDS read of 8-bit elements (ds_read_b64_tr_b8). Within each
// group of 16 lanes, lane 2r + q addresses 8 bytes -- row R_r, columns
// [c + 8q, c + 8q + 8) of a row-major byte tile -- and output lane i receives
// column c + i of rows R_0 .. R_7 (byte r from row R_r).
__device__ inline u32x2 lds_read_tr8(const void* p) {
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Four probabilities as one word of E4M3 codes (round to nearest even).
__device__ inline uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

template <int D>
struct F8Shape {
  static constexpr int NQK = D / 64;           // MFMAs per 32x32 score block
  static constexpr int NMT = kF8BN / 32;       // 32-key blocks per tile
  static constexpr int NDT = D / 32;           // 32-wide head-dim blocks of O
  static constexpr int KS = D + 16;            // K row stride in LDS (bytes)
  static constexpr int K_BYTES = kF8BN * KS;
  static constexpr int V_BYTES = kF8BN * D;
  static constexpr int LDS_BYTES = 2 * K_BYTES + 2 * V_BYTES;
  static constexpr int UPR = D / 16;           // 16-byte units per row
  static constexpr int ROWS = kF8Group / UPR;  // tile rows per staging step
  static constexpr int VECS = kF8BN / ROWS;    // 16-byte units per thread per tile
  static_assert(kF8BN % ROWS == 0, "tile must split evenly over a group");
};

// Swizzle of the 16-byte units of V row `key`: the transposing reads of a
// half-wave (8 keys x two units) and the row writes then hit distinct banks.
template <int D>
__device__ constexpr int v8_swz(int key) {
  return D == 128 ? ((((key >> 1) & 1) | (((key >> 3) & 1) << 1)) << 1) : (((key >> 3) & 1) << 1);
}

// One wave group's share of a 64-key tile between its global load (matrix
// phase) and its LDS store (vector phase). Unit i of a thread is tile row
// ROWS*i + gtid/UPR, bytes 16*(gtid % UPR) .. +16.
template <int D>
struct F8Stage {
  using S = F8Shape<D>;
  static constexpr int K_STRIDE = S::ROWS * S::KS;
  static constexpr int V_STRIDE = S::ROWS * D;
  u32x4 r[S::VECS];

  // Rows past N read as zeros (buffer range check).
  __device__ inline void load(const HeadBuf& X, int k0, int gtid) {
#pragma unroll
    for (int i = 0; i < S::VECS; ++i) r[i] = X.ld16((gtid + kF8Group * i) * 16, k0 * D);
  }
  __device__ inline void store(char* dst, int off0, int stride) const {
#pragma unroll
    for (int i = 0; i < S::VECS; ++i) st<u32x4>(dst + off0 + i * stride, r[i]);
  }
  __device__ static inline int k_off(int gtid) {
    return (gtid / S::UPR) * S::KS + (gtid % S::UPR) * 16;
  }
  // The swizzle depends on key bits 1 and 3 only, so it is the same for
  // every unit of a thread (rows step by ROWS, a multiple of 16).
  __device__ static inline int v_off(int gtid) {
    const int row = gtid / S::UPR;
    return row * D + (((gtid % S::UPR) ^ v8_swz<D>(row)) << 4);
  }
};

template <int D, bool CAUSAL, typename TO>
__global__ __launch_bounds__(kF8Threads, 1) void fwd_fp8_kernel(FwdArgs a) {
  using S = F8Shape<D>;
  using E = Elem<TO>;

  __shared__ __attribute__((aligned(16))) char lds[S::LDS_BYTES];
  char* const kbuf = lds;                   // 2 x K tile
  char* const vbuf = lds + 2 * S::K_BYTES;  // 2 x V tile

  const int N = a.N;
  const int nqt = (N + kF8BM - 1) / kF8BM;
  const int lin = CAUSAL ? xcd_remap_ranked(blockIdx.x, gridDim.x, nqt, 1)
                         : xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lin / nqt;
  const int qi = lin % nqt;
  const int q0 = (CAUSAL ? nqt - 1 - qi : qi) * kF8BM;

  const size_t head = (size_t)bh * N * D;
  // Query head h attends with K/V head h / (H / Hkv).
  const size_t kvhead = (size_t)((bh / a.H) * a.Hkv + (bh % a.H) / (a.H / a.Hkv)) * N * D;
  const uint32_t head_bytes = (uint32_t)N * D;
  const HeadBuf Q(reinterpret_cast<const uint8_t*>(a.q) + head, head_bytes);
  const HeadBuf K(reinterpret_cast<const uint8_t*>(a.k) + kvhead, head_bytes);
  const HeadBuf V(reinterpret_cast<const uint8_t*>(a.v) + kvhead, head_bytes);
  TO* O = reinterpret_cast<TO*>(a.o) + head;
  float* L = a.lse + (size_t)bh * N;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;  // 0: A, 1: B (one phase behind)
  const int gtid = tid & (kF8Group - 1);
  const int col = lane & 31, half = lane >> 5;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + col;

  // Key tiles the workgroup streams (t0 .. t0+nkv-1) and the steps
  // [w_lo, w_end) on which this wave computes, as in the 16-bit kernel.
  const int qlast = min(q0 + kF8BM, N) - 1;
  const int t0 = first_visible_key(q0, a.wl) / kF8BN;
  const int nkv = last_visible_key(qlast, N, CAUSAL, a.wr) / kF8BN - t0 + 1;
  int w_lo = nkv + 1, w_end = -1;
  if (qw0 < N) {
    const int lo = max(first_visible_key(qw0, a.wl) / kF8BN - t0, 0);
    const int hi = min(last_visible_key(min(qw0 + 31, N - 1), N, CAUSAL, a.wr) / kF8BN - t0 + 1, nkv);
    if (lo < hi) w_lo = lo, w_end = hi;
  }

  // Q^T as MFMA B operands: operand u covers head-dim bytes [64u, 64u + 64);
  // lane half h holds its row's bytes [64u + 32h, 64u + 32h + 32). The K
  // operands use the same assignment, so the contraction pairs them up.
  i32x8 qf[S::NQK];
#pragma unroll
  for (int u = 0; u < S::NQK; ++u) {
    const u32x4 lo = Q.ld16(qrow * D + 64 * u + 32 * half);
    const u32x4 hi = Q.ld16(qrow * D + 64 * u + 32 * half + 16);
    qf[u] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  const int koff = col * S::KS + 32 * half;

  // V^T operand reads. The P^T operand of lane half h holds, as byte
  // b = 16*mt + r, the probability of key 32*mt + 8*(r>>2) + 4*h + (r&3) (the
  // score accumulator's row order), so V^T byte b of that half must be the
  // same key: read u (bytes 8u .. 8u+7) takes keys 16u + 8*(j>>2) + 4h + (j&3)
  // for j = 0..7. Lane 2j + q of 16-lane group g addresses key row j of that
  // list, head-dim unit 2*dt + (g&1), bytes 8q .. 8q+7.
  int voff[S::NDT];
  {
    const int g = lane >> 4, jq = lane & 15, j = jq >> 1, q = jq & 1, h = g >> 1;
    const int key = 8 * (j >> 2) + 4 * h + (j & 3);
#pragma unroll
    for (int dt = 0; dt < S::NDT; ++dt)
      voff[dt] = key * D + (((2 * dt + (g & 1)) ^ v8_swz<D>(key)) << 4) + 8 * q;
  }

  const float c = a.scale_log2;  // effective score scale * log2(e)
  float m = -FLT_MAX;            // reference (raw score units)
  float l = 0.f;                 // running sum of 2^3 * probabilities
  f32x16 o[S::NDT];
#pragma unroll
  for (int dt = 0; dt < S::NDT; ++dt) o[dt] = f32x16{};
  // Scores of a tile, then (words 0..7 of s[0]) its E4M3 probabilities.
  f32x16 s[S::NMT];
#pragma unroll
  for (int mt = 0; mt < S::NMT; ++mt) s[mt] = f32x16{};

  // Matrix phase: PV of the previous tile, then QK of the current one, in
  // chunks of two MFMAs whose LDS operands are read while the previous chunk
  // computes. MFMA index i < NPV is PV for head-dim block i; the rest are QK
  // for key block (i - NPV) / NQK, head-dim operand (i - NPV) % NQK.
  auto mphase = [&](const char* vt, const char* kt, auto pv_c, auto qk_c) {
    constexpr bool PV = decltype(pv_c)::value, QK = decltype(qk_c)::value;
    constexpr int NPV = PV ? S::NDT : 0;
    constexpr int NM = NPV + (QK ? S::NMT * S::NQK : 0);
    constexpr int NC = NM / 2;
    static_assert(NM % 2 == 0, "chunks of two MFMAs");
    const f32x16 x = s[0];
    const i32x8 pf = __builtin_bit_cast(i32x8, __builtin_shufflevector(x, x, 0, 1, 2, 3, 4, 5, 6, 7));
    i32x8 op[2][2];
    auto fetch = [&](int i, i32x8& dst) {
      if (i < NPV) {
        const char* vp = vt + voff[i];
        const u32x2 r0 = lds_read_tr8(vp);
        const u32x2 r1 = lds_read_tr8(vp + 16 * D);
        const u32x2 r2 = lds_read_tr8(vp + 32 * D);
        const u32x2 r3 = lds_read_tr8(vp + 48 * D);
        const u32x4 lo = __builtin_shufflevector(r0, r1, 0, 1, 2, 3);
        const u32x4 hi = __builtin_shufflevector(r2, r3, 0, 1, 2, 3);
        dst = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      } else {
        const int mt = (i - NPV) / S::NQK, u = (i - NPV) % S::NQK;
        const char* kp = kt + koff + mt * 32 * S::KS + 64 * u;
        const u32x4 lo = ld<u32x4>(kp), hi = ld<u32x4>(kp + 16);
        dst = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    auto compute = [&](int i, const i32x8& src) {
      if (i < NPV) {
        o[i] = mma8(src, pf, o[i]);
      } else {
        const int mt = (i - NPV) / S::NQK, u = (i - NPV) % S::NQK;
        s[mt] = mma8(src, qf[u], u == 0 ? f32x16{} : s[mt]);
      }
    };
    __builtin_amdgcn_s_setprio(1);
    fetch(0, op[0][0]);
    fetch(1, op[0][1]);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      if (cc + 1 < NC) {
        fetch(2 * cc + 2, op[(cc + 1) & 1][0]);
        fetch(2 * cc + 3, op[(cc + 1) & 1][1]);
      }
      __builtin_amdgcn_sched_barrier(0);
      compute(2 * cc, op[cc & 1][0]);
      compute(2 * cc + 1, op[cc & 1][1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Online softmax of one tile: scores s -> E4M3 probabilities in s[0].
  auto softmax = [&](int k0) {
    if (!block_all_visible(qw0, qw0 + 31, k0, k0 + kF8BN - 1, N, CAUSAL, a.wl, a.wr)) {
#pragma unroll
      for (int mt = 0; mt < S::NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (!key_visible(key, qrow, N, CAUSAL, a.wl, a.wr)) s[mt][r] = -INFINITY;
        }
    }
    // 2^3 * exp2((s - m) * c) against the current reference m, kept while no
    // lane's sum over its 32 values exceeds 448 (so none does, and every
    // value has a finite E4M3 code; a row whose 32 values all equal the max
    // sums to 256); otherwise, and while a row has no reference, the
    // reference moves to the row max (values <= 2^3), O and l are rescaled
    // and the values taken again (as in the 16-bit kernel, exact either way).
    float p[2 * 16];
    float ls;
    auto exps = [&]() {
      // Clamped: -FLT_MAX * c overflows for c > 1, and -inf + inf is NaN.
      const float mc = fmaxf(m * c, -FLT_MAX) - kPLog2;
#pragma unroll
      for (int mt = 0; mt < S::NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) p[mt * 16 + r] = __builtin_amdgcn_exp2f(fmaf(s[mt][r], c, -mc));
      float t[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) t[j] = p[2 * j] + p[2 * j + 1];
#pragma unroll
      for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
        for (int j = 0; j < w; ++j) t[j] = t[2 * j] + t[2 * j + 1];
      ls = t[0];
    };
    exps();
    if (wave_any(!(ls <= kPMax) || m == -FLT_MAX)) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < S::NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
      mx = max_with_other_half(mx);
      const float m_new = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < S::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      exps();
    }
    l += ls;
    // Word k of the P^T operand: values 4k .. 4k+3, straight into s[0].
#pragma unroll
    for (int k = 0; k < 8; ++k)
      s[0][k] = __builtin_bit_cast(float, pack4_e4m3(p[4 * k], p[4 * k + 1], p[4 * k + 2], p[4 * k + 3]));
  };

  if (nkv <= 0) return;  // (no tile: cannot happen for N >= 1)

  using GS = F8Stage<D>;
  GS stg;
  if (group == 0 || nkv > 1) {
    stg.load(K, (t0 + group) * kF8BN, gtid);
    stg.store(kbuf + group * S::K_BYTES, GS::k_off(gtid), GS::K_STRIDE);
  }
#pragma unroll
  for (int u = 0; u < S::NQK; ++u) {
    settle(__builtin_shufflevector(qf[u], qf[u], 0, 1, 2, 3));
    settle(__builtin_shufflevector(qf[u], qf[u], 4, 5, 6, 7));
  }
  __syncthreads();

  // Group A streams V tile i, group B K tile i + 2 (K tile i in kbuf[i % 2],
  // V tile i in vbuf[i % 2]); the same barrier schedule as the 16-bit kernel.
  const bool kgrp = group == 1;
  const HeadBuf& X = kgrp ? K : V;
  const int soff = kgrp ? GS::k_off(gtid) : GS::v_off(gtid);
  const int sstride = kgrp ? GS::K_STRIDE : GS::V_STRIDE;
  if (kgrp) __syncthreads();
  {
    const int lt = kgrp ? 2 : 0;
    if (lt < nkv) stg.load(X, (t0 + lt) * kF8BN, gtid);
    if (w_lo == 0 && w_end > 0) mphase(vbuf, kbuf, BoolC<false>{}, BoolC<true>{});
    __syncthreads();
    if (w_lo == 0 && w_end > 0) softmax(t0 * kF8BN);
    if (lt < nkv) stg.store(kgrp ? kbuf : vbuf, soff, sstride);
    __syncthreads();
  }
  for (int i = 1; i < nkv; ++i) {
    const int lt = kgrp ? i + 2 : i;
    if (lt < nkv) stg.load(X, (t0 + lt) * kF8BN, gtid);
    if (w_lo <= i && i <= w_end)
      mphase(vbuf + ((i - 1) & 1) * S::V_BYTES, kbuf + (i & 1) * S::K_BYTES, BoolC<true>{},
             BoolC<true>{});
    __syncthreads();
    if (w_lo <= i && i < w_end) softmax((t0 + i) * kF8BN);
    if (lt < nkv) stg.store(kgrp ? kbuf + (i & 1) * S::K_BYTES : vbuf + (i & 1) * S::V_BYTES, soff, sstride);
    __syncthreads();
  }
  if (w_end == nkv) mphase(vbuf + ((nkv - 1) & 1) * S::V_BYTES, kbuf, BoolC<true>{}, BoolC<false>{});
  __syncthreads();
  if (!kgrp) __syncthreads();

  if (qrow >= N) return;
  const float lt = l + __shfl_xor(l, 32);
  // O = v_descale * (sum of 2^3 p V8) / (sum of 2^3 p).
  const float inv = a.v_descale / lt;
  TO* orow = O + (size_t)qrow * D;
#pragma unroll
  for (int dt = 0; dt < S::NDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = dt * 32 + 8 * g + 4 * half;
      const uint32_t w0 = E::bits(o[dt][4 * g] * inv) | ((uint32_t)E::bits(o[dt][4 * g + 1] * inv) << 16);
      const uint32_t w1 = E::bits(o[dt][4 * g + 2] * inv) | ((uint32_t)E::bits(o[dt][4 * g + 3] * inv) << 16);
      st<u32x2>(orow + d0, u32x2{w0, w1});
    }
  // ln(sum p) = ln(l) - 3 ln 2 (l holds 2^3 * p).
  if (half == 0) L[qrow] = m * a.scale + (logf(lt) - kPLog2 * 0.69314718055994531f);
}

template <int D, bool CAUSAL, typename TO>
hipError_t launch8(const FwdArgs& a, hipStream_t stream) {
  const int nqt = (a.N + kF8BM - 1) / kF8BM;
  const dim3 grid((unsigned)((long long)a.B * a.H * nqt));
  FwdArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_fp8_kernel<D, CAUSAL, TO>), grid,
                         dim3(kF8Threads), kargs, 0, stream);
}

template <typename TO>
hipError_t dispatch8(const FwdArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? launch8<64, true, TO>(a, s) : launch8<64, false, TO>(a, s);
  return a.causal ? launch8<128, true, TO>(a, s) : launch8<128, false, TO>(a, s);
}

}  // namespace

hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t stream) {
  return a.dtype == 1 ? dispatch8<_Float16>(a, stream) : dispatch8<__bf16>(a, stream);
}

}  // namespace fa
