// fa_fwd.hip -- forward IO-aware exact attention for gfx950.
//
// What it computes: O = softmax(scale * Q K^T [causal]) V and the per-row
// LSE, equal (up to rounding) to the standard unfused pipeline of
// "FlashAttention原理：从原始Attention到FlashAttention" §二.2, computed the way
// §二.5-二.7 of that page describe: inputs split into blocks, the softmax
// reduced incrementally block by block (the online update of the embedded
// answer "写一个flashattention算子", steps 4-5), query blocks in the outer
// dimension and key/value blocks in the inner loop, blocks above the causal
// diagonal never visited, and only O plus the normalizer written to HBM.
//
// gfx950 design (one workgroup = 4 waves = 128 query rows of one head):
//   * grid: B*H*ceil(N/128) workgroups, remapped so the query tiles of a head
//     share one XCD's L2; causal grids run the longest rows first.
//   * each wave owns 32 query rows; its Q tile stays in registers as MFMA B
//     operands for the whole key loop.
//   * per 64-key tile, K is staged in LDS row-major and V transposed (V^T,
//     keys contiguous, permuted to the order in which the score registers
//     feed the PV product), both double-buffered and padded by 16 bytes per
//     row against bank conflicts; the next tile's global loads are in flight
//     while the current tile computes.
//   * S^T = K Q^T on MFMA 32x32x16 (bf16/fp16) or 32x32x2 (fp32): each lane
//     then holds 16 scores of a single query row, so the row max is lane-local
//     plus one exchange with lane^32, and the probabilities feed O^T += V^T P^T
//     straight from registers with no LDS round trip.
//   * softmax in float32 with exp2 and scale*log2(e) folded into one FMA per
//     score, tracking the raw-score max (valid because scale >= 0); 1/l is
//     applied once in the epilogue (the FA2 reduction of non-matmul work).
#include <float.h>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;  // query rows per workgroup
constexpr int kBN = 64;           // keys per K/V tile

template <typename T, int D>
struct FwdShape {
  using E = Elem<T>;
  static constexpr int KH = E::KH;
  static constexpr int ES = sizeof(T);
  static constexpr int EPV = 16 / ES;        // elements per 16-byte vector
  static constexpr int DH = D / 2;           // head-dim elements per lane half
  static constexpr int NQK = DH / KH;        // MFMAs per 32x32 score tile
  static constexpr int NMT = kBN / 32;       // 32-key blocks per tile
  static constexpr int NDT = D / 32;         // 32-wide head-dim blocks of O
  static constexpr int NPV = kBN / (2 * KH); // PV MFMAs per head-dim block
  static constexpr int KS = D + EPV;         // K row stride in LDS (elements)
  static constexpr int VS = kBN + EPV;       // V^T row stride in LDS (elements)
  static constexpr int K_BYTES = kBN * KS * ES;
  static constexpr int V_BYTES = D * VS * ES;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int K_VECS = kBN * D / EPV / kThreads;   // 16B K loads / thread
  static constexpr int V_ITEMS = (kBN / 4) * (D / EPV);      // (4 keys x 16B) items
  static constexpr int V_PER_T = (V_ITEMS + kThreads - 1) / kThreads;
  static_assert(kBN * D / EPV % kThreads == 0, "K tile must split evenly");
};

template <typename T, int D>
struct TileLoader {
  using S = FwdShape<T, D>;
  u32x4 kreg[S::K_VECS];
  u32x4 vreg[S::V_PER_T][4];

  __device__ inline void load(const T* K, const T* V, int k0, int N, int tid) {
#pragma unroll
    for (int i = 0; i < S::K_VECS; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx / (D / S::EPV);
      const int c = (idx % (D / S::EPV)) * S::EPV;
      const int key = k0 + row;
      kreg[i] = key < N ? ld<u32x4>(K + (size_t)key * D + c) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < S::V_PER_T; ++i) {
      const int item = tid + kThreads * i;
      if (S::V_ITEMS % kThreads == 0 || item < S::V_ITEMS) {
        const int kg = item / (D / S::EPV);
        const int c = (item % (D / S::EPV)) * S::EPV;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int key = k0 + 4 * kg + kk;
          vreg[i][kk] = key < N ? ld<u32x4>(V + (size_t)key * D + c) : u32x4{0, 0, 0, 0};
        }
      }
    }
  }

  __device__ inline void store(char* stage, int tid) const {
    char* Kl = stage;
    char* Vl = stage + S::K_BYTES;
#pragma unroll
    for (int i = 0; i < S::K_VECS; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx / (D / S::EPV);
      const int c = (idx % (D / S::EPV)) * S::EPV;
      st<u32x4>(Kl + (row * S::KS + c) * S::ES, kreg[i]);
    }
#pragma unroll
    for (int i = 0; i < S::V_PER_T; ++i) {
      const int item = tid + kThreads * i;
      if (S::V_ITEMS % kThreads == 0 || item < S::V_ITEMS) {
        const int kg = item / (D / S::EPV);
        const int c = (item % (D / S::EPV)) * S::EPV;
        if constexpr (S::ES == 2) {
          // 4 keys x 8 head-dim elements -> 8 rows of V^T, 4 adjacent keys each.
          const int pos = vt_pos<S::KH>(4 * kg);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int w = e >> 1, sh = (e & 1) * 16;
            const uint32_t a0 = (vreg[i][0][w] >> sh) & 0xffffu;
            const uint32_t a1 = (vreg[i][1][w] >> sh) & 0xffffu;
            const uint32_t a2 = (vreg[i][2][w] >> sh) & 0xffffu;
            const uint32_t a3 = (vreg[i][3][w] >> sh) & 0xffffu;
            st<u32x2>(Vl + ((c + e) * S::VS + pos) * 2, u32x2{a0 | (a1 << 16), a2 | (a3 << 16)});
          }
        } else {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const int pos = vt_pos<S::KH>(4 * kg + kk);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              st<uint32_t>(Vl + ((c + e) * S::VS + pos) * 4, vreg[i][kk][e]);
          }
        }
      }
    }
  }
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, sizeof(T) == 2 ? 2 : 1) void fwd_kernel(FwdArgs a) {
  using S = FwdShape<T, D>;
  using E = Elem<T>;
  using Raw = typename E::Raw;
  constexpr int KH = S::KH;

  __shared__ __attribute__((aligned(16))) char lds[2 * S::STAGE];

  const int N = a.N;
  const int nqt = (N + kBM - 1) / kBM;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lin / nqt;
  const int qtile = CAUSAL ? nqt - 1 - lin % nqt : lin % nqt;
  const int q0 = qtile * kBM;

  const size_t head = (size_t)bh * N * D;
  const T* Q = reinterpret_cast<const T*>(a.q) + head;
  const T* K = reinterpret_cast<const T*>(a.k) + head;
  const T* V = reinterpret_cast<const T*>(a.v) + head;
  T* O = reinterpret_cast<T*>(a.o) + head;
  float* L = a.lse + (size_t)bh * N;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int qw0 = q0 + wave * 32;  // first query row of this wave
  const int qrow = qw0 + col;      // the query row this lane serves
  const bool wave_active = qw0 < N;

  // Q^T as MFMA B operands: lane half h holds head-dim elements
  // [h*D/2, h*D/2 + D/2) of its row, KH per MFMA.
  Raw qf[S::NQK];
#pragma unroll
  for (int i = 0; i < S::NQK; ++i)
    qf[i] = qrow < N ? ld<Raw>(Q + (size_t)qrow * D + half * S::DH + i * KH) : Raw{};

  // Key tiles this workgroup visits: all of them, or (causal) only those
  // holding a key <= the last query row of the tile.
  const int nkv_all = (N + kBN - 1) / kBN;
  const int nkv = CAUSAL ? min(nkv_all, (min(q0 + kBM, N) - 1) / kBN + 1) : nkv_all;

  const float c = a.scale_log2;  // scale * log2(e)
  float m = -FLT_MAX;            // running max of raw scores (this row)
  float l = 0.f;                 // running sum of probabilities (this lane's keys)
  f32x16 o[S::NDT];
#pragma unroll
  for (int dt = 0; dt < S::NDT; ++dt) o[dt] = f32x16{};

  TileLoader<T, D> tl;
  tl.load(K, V, 0, N, tid);
  tl.store(lds, tid);
  __syncthreads();

  for (int j = 0; j < nkv; ++j) {
    const char* stage = lds + (j & 1) * S::STAGE;
    if (j + 1 < nkv) tl.load(K, V, (j + 1) * kBN, N, tid);
    const int k0 = j * kBN;

    if (wave_active && (!CAUSAL || k0 <= qw0 + 31)) {
      // S^T = K Q^T for 64 keys x 32 queries.
      f32x16 s[S::NMT];
#pragma unroll
      for (int mt = 0; mt < S::NMT; ++mt) {
        s[mt] = f32x16{};
        const char* kp = stage + ((mt * 32 + col) * S::KS + half * S::DH) * S::ES;
#pragma unroll
        for (int i = 0; i < S::NQK; ++i) s[mt] = E::mma(ld<Raw>(kp + i * KH * S::ES), qf[i], s[mt]);
      }

      const bool need_mask = (CAUSAL && k0 + kBN - 1 > qw0) || (k0 + kBN > N);
      if (need_mask) {
#pragma unroll
        for (int mt = 0; mt < S::NMT; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            const bool vis = key < N && (!CAUSAL || key <= qrow);
            if (!vis) s[mt][r] = -INFINITY;
          }
      }

      // Online softmax update (row max over this lane's 32 scores, then the
      // partner lane half).
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < S::NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);
      const float mc = m_new * c;
      const float alpha = __builtin_amdgcn_exp2f(m * c - mc);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < S::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;

      // Probabilities -> MFMA B operands (P^T), in register order.
      Raw pf[S::NMT * (16 / KH)];
#pragma unroll
      for (int mt = 0; mt < S::NMT; ++mt)
#pragma unroll
        for (int u = 0; u < 16 / KH; ++u) {
          float p[KH];
#pragma unroll
          for (int jj = 0; jj < KH; ++jj) {
            const float sv = s[mt][u * KH + jj];
            float t = __builtin_amdgcn_exp2f(fmaf(sv, c, -mc));
            if (need_mask) t = sv == -INFINITY ? 0.f : t;
            p[jj] = t;
          }
          pf[mt * (16 / KH) + u] = E::pack_sum(p, l);
        }

      // O^T += V^T P^T.
      const char* vbase = stage + S::K_BYTES;
#pragma unroll
      for (int dt = 0; dt < S::NDT; ++dt) {
        const char* vp = vbase + ((dt * 32 + col) * S::VS + half * KH) * S::ES;
#pragma unroll
        for (int u = 0; u < S::NPV; ++u)
          o[dt] = E::mma(ld<Raw>(vp + u * 2 * KH * S::ES), pf[u], o[dt]);
      }
    }

    if (j + 1 < nkv) tl.store(lds + ((j + 1) & 1) * S::STAGE, tid);
    __syncthreads();
  }

  if (!wave_active || qrow >= N) return;
  const float lt = l + __shfl_xor(l, 32);
  const float inv = 1.0f / lt;
  T* orow = O + (size_t)qrow * D;
#pragma unroll
  for (int dt = 0; dt < S::NDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = dt * 32 + 8 * g + 4 * half;
      if constexpr (S::ES == 2) {
        const uint32_t w0 = E::bits(o[dt][4 * g] * inv) | ((uint32_t)E::bits(o[dt][4 * g + 1] * inv) << 16);
        const uint32_t w1 = E::bits(o[dt][4 * g + 2] * inv) | ((uint32_t)E::bits(o[dt][4 * g + 3] * inv) << 16);
        st<u32x2>(orow + d0, u32x2{w0, w1});
      } else {
        st<f32x4>(orow + d0, f32x4{o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv,
                                   o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv});
      }
    }
  if (half == 0) L[qrow] = m * a.scale + logf(lt);
}

template <typename T, int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int nqt = (a.N + kBM - 1) / kBM;
  const dim3 grid((unsigned)((long long)a.B * a.H * nqt));
  FwdArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_kernel<T, D, CAUSAL>), grid,
                         dim3(kThreads), kargs, 0, stream);
}

template <typename T>
hipError_t dispatch_d(const FwdArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? launch<T, 64, true>(a, s) : launch<T, 64, false>(a, s);
  return a.causal ? launch<T, 128, true>(a, s) : launch<T, 128, false>(a, s);
}

}  // namespace

long long fwd_grid_size(int B, int H, int N) {
  return (long long)B * H * ((N + kBM - 1) / kBM);
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  switch (a.dtype) {
    case 0: return dispatch_d<float>(a, stream);
    case 1: return dispatch_d<_Float16>(a, stream);
    default: return dispatch_d<__bf16>(a, stream);
  }
}

}  // namespace fa
