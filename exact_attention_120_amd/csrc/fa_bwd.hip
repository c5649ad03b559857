// fa_bwd.hip -- backward IO-aware exact attention for gfx950.
//
// Gradients of the loss sum(dO * O) with respect to Q, K and V, with the
// attention probabilities recomputed on chip from Q, K and the stored per-row
// LSE instead of being read back ("FlashAttention原理：从原始Attention到
// FlashAttention" §一.2 and the embedded answer "写一个flashattention算子",
// step 6). The pages give no gradient formulas; these are the derivatives of
// the definition:
//   P = exp(scale*Q K^T - LSE)          dV = P^T dO
//   dP = dO V^T                         D_i = sum_k dO_ik O_ik
//   dS = P * (dP - D)                   dK = scale * dS^T Q,  dQ = scale * dS K
//
// Three kernels on the caller's stream:
//   1. bwd_pre:  D (float32, workspace) and a zeroed float32 dQ accumulator.
//   2. bwd_main: one workgroup per 128-key tile of one head (4 waves x 32
//      keys); the query tiles are the inner loop (causal: only tiles at or
//      below the diagonal). Each wave keeps its K and V rows as MFMA
//      operands and its dK^T, dV^T accumulators in registers for the whole
//      loop. S = Q K^T and dP = dO V^T put one key per lane, so P and dS feed
//      dV^T += dO^T P and dK^T += Q^T dS straight from registers (Q^T and
//      dO^T are staged transposed in LDS next to Q and dO). dS goes through
//      LDS once so the workgroup can form its whole 128-key contribution to
//      dQ (dS K) and add it with one float32 atomic per element.
//   3. bwd_dq:   dQ accumulator * scale -> dtype.
#include <float.h>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kBN = 128;       // keys per workgroup (32 per wave)

template <typename T, int D>
struct BwdShape {
  using E = Elem<T>;
  static constexpr int KH = E::KH;
  static constexpr int ES = sizeof(T);
  static constexpr int EPV = 16 / ES;
  static constexpr int DH = D / 2;
  static constexpr int BM = ES == 2 ? 64 : 32;  // query rows per inner step
  static constexpr int NQB = BM / 32;           // 32-row query blocks per step
  static constexpr int NQK = DH / KH;           // MFMAs over the head dim
  static constexpr int NDT = D / 32;            // 32-wide head-dim blocks
  static constexpr int NPQ = BM / (2 * KH);     // MFMAs over the step's queries
  static constexpr int NKQ = kBN / (2 * KH);    // MFMAs over the workgroup's keys
  static constexpr int RS = D + EPV;            // row-major tile stride (elements)
  static constexpr int TS = BM + EPV;           // transposed tile stride (elements)
  static constexpr int ROW_BYTES = BM * RS * ES;
  static constexpr int TR_BYTES = D * TS * ES;
  static constexpr int OFF_QT = ROW_BYTES;
  static constexpr int OFF_DO = ROW_BYTES + TR_BYTES;
  static constexpr int OFF_DOT = 2 * ROW_BYTES + TR_BYTES;
  static constexpr int OFF_LSE = 2 * (ROW_BYTES + TR_BYTES);
  static constexpr int OFF_DSUM = OFF_LSE + BM * 4;
  static constexpr int STAGE = OFF_DSUM + BM * 4;
  static constexpr int DSS = kBN + EPV;         // dS [BM][kBN] row stride
  static constexpr int DS_BYTES = BM * DSS * ES;
  static constexpr int KTS = kBN + EPV;         // K^T [D][kBN] row stride
  static constexpr int KT_BYTES = D * KTS * ES;
  static constexpr int LDS = 2 * STAGE + DS_BYTES;
  static constexpr int ITEMS = (BM / 4) * (D / EPV);  // 4 rows x 16 B per item
  static constexpr int ITEMS_PER_T = (ITEMS + kThreads - 1) / kThreads;
  static constexpr int K_ITEMS = (kBN / 4) * (D / EPV);
  static constexpr int K_ITEMS_PER_T = (K_ITEMS + kThreads - 1) / kThreads;
  static constexpr int DQ_UNITS = NDT * NQB;    // 32x32 dQ tiles per step
  static_assert(KT_BYTES <= STAGE, "K^T staging must fit in one stage");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Write 4 rows x EPV elements (one item, rows r0..r0+3 of a tile, head-dim
// elements c..c+EPV) transposed into a [D][stride] LDS array at row
// positions pos(r0..r0+3).
template <typename T, bool PERMUTE>
__device__ inline void store_transposed(char* base, int stride, int c, int r0, const u32x4* v) {
  constexpr int KH = Elem<T>::KH;
  if constexpr (sizeof(T) == 2) {
    const int pos = PERMUTE ? vt_pos<KH>(r0) : r0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1, sh = (e & 1) * 16;
      const uint32_t a0 = (v[0][w] >> sh) & 0xffffu, a1 = (v[1][w] >> sh) & 0xffffu;
      const uint32_t a2 = (v[2][w] >> sh) & 0xffffu, a3 = (v[3][w] >> sh) & 0xffffu;
      st<u32x2>(base + ((c + e) * stride + pos) * 2, u32x2{a0 | (a1 << 16), a2 | (a3 << 16)});
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int pos = PERMUTE ? vt_pos<KH>(r0 + kk) : r0 + kk;
#pragma unroll
      for (int e = 0; e < 4; ++e) st<uint32_t>(base + ((c + e) * stride + pos) * 4, v[kk][e]);
    }
  }
}

// Loads one query tile (Q, dO rows q0..q0+BM-1 plus their LSE and D) into
// registers, then stores it to an LDS stage: Q and dO row-major and
// transposed (rows permuted by vt_pos), LSE pre-multiplied by log2(e).
template <typename T, int D>
struct QTile {
  using S = BwdShape<T, D>;
  u32x4 q[S::ITEMS_PER_T][4];
  u32x4 g[S::ITEMS_PER_T][4];
  float stat;

  __device__ inline void load(const T* Q, const T* dO, const float* lse, const float* dsum,
                              int q0, int N, int tid) {
#pragma unroll
    for (int i = 0; i < S::ITEMS_PER_T; ++i) {
      const int item = tid + kThreads * i;
      if (S::ITEMS % kThreads == 0 || item < S::ITEMS) {
        const int rg = item / (D / S::EPV);
        const int c = (item % (D / S::EPV)) * S::EPV;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int row = q0 + 4 * rg + kk;
          const bool in = row < N;
          q[i][kk] = in ? ld<u32x4>(Q + (size_t)row * D + c) : u32x4{0, 0, 0, 0};
          g[i][kk] = in ? ld<u32x4>(dO + (size_t)row * D + c) : u32x4{0, 0, 0, 0};
        }
      }
    }
    // Threads [0, BM) fetch LSE, [BM, 2*BM) fetch D. Rows past N get
    // LSE = +inf so that their probabilities are exactly 0.
    stat = 0.f;
    if (tid < S::BM) {
      const int row = q0 + tid;
      stat = row < N ? lse[row] * kLog2e : INFINITY;
    } else if (tid < 2 * S::BM) {
      const int row = q0 + tid - S::BM;
      stat = row < N ? dsum[row] : 0.f;
    }
  }

  __device__ inline void store(char* stage, int tid) const {
#pragma unroll
    for (int i = 0; i < S::ITEMS_PER_T; ++i) {
      const int item = tid + kThreads * i;
      if (S::ITEMS % kThreads == 0 || item < S::ITEMS) {
        const int rg = item / (D / S::EPV);
        const int c = (item % (D / S::EPV)) * S::EPV;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          st<u32x4>(stage + ((4 * rg + kk) * S::RS + c) * S::ES, q[i][kk]);
          st<u32x4>(stage + S::OFF_DO + ((4 * rg + kk) * S::RS + c) * S::ES, g[i][kk]);
        }
        store_transposed<T, true>(stage + S::OFF_QT, S::TS, c, 4 * rg, q[i]);
        store_transposed<T, true>(stage + S::OFF_DOT, S::TS, c, 4 * rg, g[i]);
      }
    }
    if (tid < 2 * S::BM) st<float>(stage + S::OFF_LSE + tid * 4, stat);
  }
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_main_kernel(BwdArgs a) {
  using S = BwdShape<T, D>;
  using E = Elem<T>;
  using Raw = typename E::Raw;
  constexpr int KH = S::KH;

  __shared__ __attribute__((aligned(16))) char lds[S::LDS];
  char* dsl = lds + 2 * S::STAGE;  // dS [BM][kBN] in T

  const int N = a.N;
  const int nkt = (N + kBN - 1) / kBN;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lin / nkt;
  const int ktile = lin % nkt;  // causal: low tiles have the most work, run first
  const int k0 = ktile * kBN;

  const size_t head = (size_t)bh * N * D;
  const T* Q = reinterpret_cast<const T*>(a.q) + head;
  const T* K = reinterpret_cast<const T*>(a.k) + head;
  const T* V = reinterpret_cast<const T*>(a.v) + head;
  const T* dO = reinterpret_cast<const T*>(a.dout) + head;
  T* dK = reinterpret_cast<T*>(a.dk) + head;
  T* dV = reinterpret_cast<T*>(a.dv) + head;
  float* dQacc = a.dq_acc + head;
  const float* lse = a.lse + (size_t)bh * N;
  const float* dsum = a.dsum + (size_t)bh * N;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int kw0 = k0 + wave * 32;  // first key of this wave
  const int key = kw0 + col;       // the key this lane serves in S and dP

  // This wave's K and V rows as B operands (K^T, V^T over the head dim).
  Raw kb[S::NQK], vb[S::NQK];
#pragma unroll
  for (int i = 0; i < S::NQK; ++i) {
    const size_t off = (size_t)key * D + half * S::DH + i * KH;
    kb[i] = key < N ? ld<Raw>(K + off) : Raw{};
    vb[i] = key < N ? ld<Raw>(V + off) : Raw{};
  }

  // K^T of the whole 128-key tile (natural key order) through LDS, then each
  // wave keeps the head-dim block it reduces dQ over as B operands.
  {
    char* kt = lds + S::STAGE;
#pragma unroll
    for (int i = 0; i < S::K_ITEMS_PER_T; ++i) {
      const int item = tid + kThreads * i;
      if (S::K_ITEMS % kThreads == 0 || item < S::K_ITEMS) {
        const int rg = item / (D / S::EPV);
        const int c = (item % (D / S::EPV)) * S::EPV;
        u32x4 v[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int row = k0 + 4 * rg + kk;
          v[kk] = row < N ? ld<u32x4>(K + (size_t)row * D + c) : u32x4{0, 0, 0, 0};
        }
        store_transposed<T, false>(kt, S::KTS, c, 4 * rg, v);
      }
    }
  }
  __syncthreads();
  const int dblk = wave % S::NDT;  // fixed per wave: units are wave + 4*k
  Raw kq[S::NKQ];
  {
    const char* kt = lds + S::STAGE + ((dblk * 32 + col) * S::KTS + half * KH) * S::ES;
#pragma unroll
    for (int t = 0; t < S::NKQ; ++t) kq[t] = ld<Raw>(kt + t * 2 * KH * S::ES);
  }
  __syncthreads();

  const int nq = (N + S::BM - 1) / S::BM;
  const int it0 = CAUSAL ? k0 / S::BM : 0;  // first query tile reaching these keys
  const float c = a.scale_log2;

  f32x16 dkt[S::NDT], dvt[S::NDT];
#pragma unroll
  for (int dt = 0; dt < S::NDT; ++dt) {
    dkt[dt] = f32x16{};
    dvt[dt] = f32x16{};
  }

  QTile<T, D> qt;
  qt.load(Q, dO, lse, dsum, it0 * S::BM, N, tid);
  qt.store(lds, tid);
  __syncthreads();

  for (int it = it0; it < nq; ++it) {
    const char* stage = lds + ((it - it0) & 1) * S::STAGE;
    const int q0 = it * S::BM;
    if (it + 1 < nq) qt.load(Q, dO, lse, dsum, q0 + S::BM, N, tid);

    // S = Q K^T and dP = dO V^T (lane = key, registers = queries).
    f32x16 s[S::NQB], dp[S::NQB];
#pragma unroll
    for (int qb = 0; qb < S::NQB; ++qb) {
      s[qb] = f32x16{};
      dp[qb] = f32x16{};
      const char* qa = stage + ((qb * 32 + col) * S::RS + half * S::DH) * S::ES;
      const char* ga = qa + S::OFF_DO;
#pragma unroll
      for (int i = 0; i < S::NQK; ++i) {
        s[qb] = E::mma(ld<Raw>(qa + i * KH * S::ES), kb[i], s[qb]);
        dp[qb] = E::mma(ld<Raw>(ga + i * KH * S::ES), vb[i], dp[qb]);
      }
    }

    // P = exp(S*scale - LSE), dS = P * (dP - D); masked entries are 0.
    const bool need_mask = (CAUSAL && q0 < kw0 + 31) || (kw0 + 31 >= N);
    Raw pf[S::NPQ], sf[S::NPQ];
#pragma unroll
    for (int qb = 0; qb < S::NQB; ++qb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ql = qb * 32 + 8 * g + 4 * half;  // first of 4 query rows
        const f32x4 l2 = ld<f32x4>(stage + S::OFF_LSE + ql * 4);
        const f32x4 dd = ld<f32x4>(stage + S::OFF_DSUM + ql * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float p = __builtin_amdgcn_exp2f(fmaf(s[qb][r], c, -l2[e]));
          if (need_mask) {
            const int qrow = q0 + ql + e;
            if (key >= N || (CAUSAL && key > qrow)) p = 0.f;
          }
          s[qb][r] = p;
          dp[qb][r] = p * (dp[qb][r] - dd[e]);
        }
      }
      float unused = 0.f;
#pragma unroll
      for (int u = 0; u < 16 / KH; ++u) {
        float tp[KH], ts[KH];
#pragma unroll
        for (int j = 0; j < KH; ++j) {
          tp[j] = s[qb][u * KH + j];
          ts[j] = dp[qb][u * KH + j];
        }
        pf[qb * (16 / KH) + u] = E::pack_sum(tp, unused);
        sf[qb * (16 / KH) + u] = E::pack_sum(ts, unused);
      }
    }

    // dS -> LDS as [query][key] (natural order) for the dQ product.
#pragma unroll
    for (int qb = 0; qb < S::NQB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = qb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        char* dst = dsl + (ql * S::DSS + wave * 32 + col) * S::ES;
        if constexpr (S::ES == 2)
          st<uint16_t>(dst, E::bits(dp[qb][r]));
        else
          st<float>(dst, dp[qb][r]);
      }

    // dV^T += dO^T P and dK^T += Q^T dS (A operands from the transposed copies).
#pragma unroll
    for (int dt = 0; dt < S::NDT; ++dt) {
      const char* ga = stage + S::OFF_DOT + ((dt * 32 + col) * S::TS + half * KH) * S::ES;
      const char* qa = stage + S::OFF_QT + ((dt * 32 + col) * S::TS + half * KH) * S::ES;
#pragma unroll
      for (int u = 0; u < S::NPQ; ++u) {
        dvt[dt] = E::mma(ld<Raw>(ga + u * 2 * KH * S::ES), pf[u], dvt[dt]);
        dkt[dt] = E::mma(ld<Raw>(qa + u * 2 * KH * S::ES), sf[u], dkt[dt]);
      }
    }
    __syncthreads();  // dS of all four waves is in LDS

    // dQ[q, d] += sum over the 128 keys of dS[q, key] K[key, d] (unscaled).
#pragma unroll
    for (int unit = wave; unit < S::DQ_UNITS; unit += 4) {
      const int qb = unit / S::NDT;
      f32x16 acc = f32x16{};
      const char* da = dsl + ((qb * 32 + col) * S::DSS + half * KH) * S::ES;
#pragma unroll
      for (int t = 0; t < S::NKQ; ++t) acc = E::mma(ld<Raw>(da + t * 2 * KH * S::ES), kq[t], acc);
      float* dst = dQacc + dblk * 32 + col;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qrow = q0 + qb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (qrow < N) unsafeAtomicAdd(dst + (size_t)qrow * D, acc[r]);
      }
    }

    if (it + 1 < nq) qt.store(lds + ((it + 1 - it0) & 1) * S::STAGE, tid);
    __syncthreads();
  }

  // Epilogue: lane = key, registers = head-dim rows of dK^T / dV^T.
  if (key >= N) return;
  T* dkrow = dK + (size_t)key * D;
  T* dvrow = dV + (size_t)key * D;
  const float sc = a.scale;
#pragma unroll
  for (int dt = 0; dt < S::NDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = dt * 32 + 8 * g + 4 * half;
      if constexpr (S::ES == 2) {
        const f32x16& kk = dkt[dt];
        const f32x16& vv = dvt[dt];
        st<u32x2>(dkrow + d0,
                  u32x2{E::bits(kk[4 * g] * sc) | ((uint32_t)E::bits(kk[4 * g + 1] * sc) << 16),
                        E::bits(kk[4 * g + 2] * sc) | ((uint32_t)E::bits(kk[4 * g + 3] * sc) << 16)});
        st<u32x2>(dvrow + d0,
                  u32x2{E::bits(vv[4 * g]) | ((uint32_t)E::bits(vv[4 * g + 1]) << 16),
                        E::bits(vv[4 * g + 2]) | ((uint32_t)E::bits(vv[4 * g + 3]) << 16)});
      } else {
        st<f32x4>(dkrow + d0, f32x4{dkt[dt][4 * g] * sc, dkt[dt][4 * g + 1] * sc,
                                    dkt[dt][4 * g + 2] * sc, dkt[dt][4 * g + 3] * sc});
        st<f32x4>(dvrow + d0, f32x4{dvt[dt][4 * g], dvt[dt][4 * g + 1], dvt[dt][4 * g + 2],
                                    dvt[dt][4 * g + 3]});
      }
    }
}

// D_i = sum_k dO_ik O_ik (float32) and dQ accumulator rows cleared.
// TPR threads per row, 16 bytes of O and dO each.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(BwdArgs a) {
  constexpr int EPV = 16 / sizeof(T);
  constexpr int TPR = D / EPV;
  constexpr int RPB = kThreads / TPR;
  const long long rows = (long long)a.B * a.H * a.N;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int sub = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * D + sub * EPV;
    const u32x4 o = ld<u32x4>(reinterpret_cast<const T*>(a.o) + off);
    const u32x4 g = ld<u32x4>(reinterpret_cast<const T*>(a.dout) + off);
    const T* op = reinterpret_cast<const T*>(&o);
    const T* gp = reinterpret_cast<const T*>(&g);
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc = fmaf((float)op[e], (float)gp[e], acc);
    float* z = a.dq_acc + off;
#pragma unroll
    for (int e = 0; e < EPV; e += 4) st<f32x4>(z + e, f32x4{0.f, 0.f, 0.f, 0.f});
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (row < rows && sub == 0) a.dsum[row] = acc;
}

// dQ = scale * accumulator, rounded to T; 4 elements per thread.
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_dq_kernel(BwdArgs a, long long n4) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n4) return;
  const f32x4 x = ld<f32x4>(a.dq_acc + 4 * i);
  const float s = a.scale;
  if constexpr (sizeof(T) == 2) {
    const uint32_t w0 = Elem<T>::bits(x[0] * s) | ((uint32_t)Elem<T>::bits(x[1] * s) << 16);
    const uint32_t w1 = Elem<T>::bits(x[2] * s) | ((uint32_t)Elem<T>::bits(x[3] * s) << 16);
    st<u32x2>(reinterpret_cast<T*>(a.dq) + 4 * i, u32x2{w0, w1});
  } else {
    st<f32x4>(reinterpret_cast<float*>(a.dq) + 4 * i, f32x4{x[0] * s, x[1] * s, x[2] * s, x[3] * s});
  }
}

template <typename T, int D>
hipError_t launch_all(const BwdArgs& a, hipStream_t stream) {
  BwdArgs args = a;
  const long long rows = (long long)a.B * a.H * a.N;
  constexpr int RPB = kThreads / (D / (16 / (int)sizeof(T)));
  {
    void* kargs[] = {&args};
    const dim3 grid((unsigned)((rows + RPB - 1) / RPB));
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_pre_kernel<T, D>), grid,
                                   dim3(kThreads), kargs, 0, stream);
    if (e != hipSuccess) return e;
  }
  {
    void* kargs[] = {&args};
    const int nkt = (a.N + kBN - 1) / kBN;
    const dim3 grid((unsigned)((long long)a.B * a.H * nkt));
    const void* fn = a.causal ? reinterpret_cast<const void*>(&bwd_main_kernel<T, D, true>)
                              : reinterpret_cast<const void*>(&bwd_main_kernel<T, D, false>);
    hipError_t e = hipLaunchKernel(fn, grid, dim3(kThreads), kargs, 0, stream);
    if (e != hipSuccess) return e;
  }
  {
    long long n4 = rows * D / 4;
    void* kargs[] = {&args, &n4};
    const dim3 grid((unsigned)((n4 + kThreads - 1) / kThreads));
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dq_kernel<T>), grid,
                           dim3(kThreads), kargs, 0, stream);
  }
}

template <typename T>
hipError_t dispatch_d(const BwdArgs& a, hipStream_t s) {
  return a.d == 64 ? launch_all<T, 64>(a, s) : launch_all<T, 128>(a, s);
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  switch (a.dtype) {
    case 0: return dispatch_d<float>(a, stream);
    case 1: return dispatch_d<_Float16>(a, stream);
    default: return dispatch_d<__bf16>(a, stream);
  }
}

}  // namespace fa
