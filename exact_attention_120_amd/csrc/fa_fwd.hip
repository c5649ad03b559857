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
  static constexpr bool TRV = ES == 2;       // V read with transposing LDS loads
  static constexpr int DH = D / 2;           // head-dim elements per lane half
  static constexpr int NQK = DH / KH;        // MFMAs per 32x32 score tile
  static constexpr int NMT = kBN / 32;       // 32-key blocks per tile
  static constexpr int NDT = D / 32;         // 32-wide head-dim blocks of O
  static constexpr int NPV = kBN / (2 * KH); // PV MFMAs per head-dim block
  static constexpr int KS = D + EPV;         // K row stride in LDS (elements, +16 B)
  // V: row-major, unpadded, 16-byte units XOR-swizzled by key (16-bit types);
  // fp32 keeps a transposed V^T copy (keys contiguous, permuted by vt_pos).
  static constexpr int VS = TRV ? D : kBN + EPV;
  static constexpr int K_BYTES = kBN * KS * ES;
  static constexpr int V_BYTES = TRV ? kBN * D * ES : D * VS * ES;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int VECS = kBN * D / EPV / kThreads;     // 16 B loads per thread per tensor
  static_assert(kBN * D / EPV % kThreads == 0, "tile must split evenly");
};

// Swizzle of the 16-byte units of V row `key` (16-bit types). With it, the
// transposing reads of one wave (8 rows x 64 B) and the row writes (16 B per
// lane) are free of LDS bank conflicts (measured with SQ_LDS_BANK_CONFLICT).
template <int D>
__device__ constexpr int v_swz(int key) {
  return D == 128 ? (0xCA60 >> (4 * (key & 3))) & 15 : 2 * (key & 3);
}

template <typename T, int D>
struct TileLoader {
  using S = FwdShape<T, D>;
  u32x4 kreg[S::VECS];
  u32x4 vreg[S::VECS];

  // Rows past N read as zeros (buffer range check).
  __device__ inline void load(const HeadBuf& K, const HeadBuf& V, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < S::VECS; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx / (D / S::EPV);
      const int c = (idx % (D / S::EPV)) * S::EPV;
      const int off = ((k0 + row) * D + c) * S::ES;
      kreg[i] = K.ld16(off);
      vreg[i] = V.ld16(off);
    }
  }

  __device__ inline void store(char* stage, int tid) const {
    char* Kl = stage;
    char* Vl = stage + S::K_BYTES;
#pragma unroll
    for (int i = 0; i < S::VECS; ++i) {
      const int idx = tid + kThreads * i;
      const int row = idx / (D / S::EPV);
      const int c = (idx % (D / S::EPV)) * S::EPV;
      st<u32x4>(Kl + (row * S::KS + c) * S::ES, kreg[i]);
      if constexpr (S::TRV) {
        st<u32x4>(Vl + row * D * 2 + (((c >> 3) ^ v_swz<D>(row)) << 4), vreg[i]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          st<uint32_t>(Vl + ((c + e) * S::VS + vt_pos<S::KH>(row)) * 4, vreg[i][e]);
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
  const uint32_t head_bytes = (uint32_t)N * D * S::ES;
  const HeadBuf Q(reinterpret_cast<const T*>(a.q) + head, head_bytes);
  const HeadBuf K(reinterpret_cast<const T*>(a.k) + head, head_bytes);
  const HeadBuf V(reinterpret_cast<const T*>(a.v) + head, head_bytes);
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
  for (int i = 0; i < S::NQK; ++i) {
    const int off = (qrow * D + half * S::DH + i * KH) * S::ES;
    if constexpr (S::ES == 2)
      qf[i] = Q.ld16(off);
    else
      qf[i] = Q.ld4(off);
  }

  // Per-lane byte offsets of the V^T operand reads within a stage's V tile.
  // Transposing reads: lane 4r+q of 16-lane group g fetches key row 4h + r
  // (h = g/2) and head-dim columns 32*dt + 16*(g&1) + 4q .. +4.
  int voff[S::NDT];
  {
    const int g = lane >> 4, jf = lane & 15, r = jf >> 2, q = jf & 3, h = g >> 1;
    const int b = 2 * (g & 1) + (q >> 1);  // 16-byte unit within a 32-wide block
#pragma unroll
    for (int dt = 0; dt < S::NDT; ++dt) {
      if constexpr (S::TRV)
        voff[dt] = (4 * h + r) * D * 2 + (((4 * dt) ^ (b ^ v_swz<D>(r))) << 4) + (q & 1) * 8;
      else
        voff[dt] = ((dt * 32 + col) * S::VS + half * KH) * S::ES;
    }
  }

  // Key tiles this workgroup visits: all of them, or (causal) only those
  // holding a key <= the last query row of the tile.
  const int nkv_all = (N + kBN - 1) / kBN;
  const int nkv = CAUSAL ? min(nkv_all, (min(q0 + kBM, N) - 1) / kBN + 1) : nkv_all;

  const float c = a.scale_log2;  // scale * log2(e)
  // Reference max (raw scores) the exponentials are taken against; it only
  // moves when a row's max exceeds it by more than 2^8 in probability
  // (exact: O and l are always relative to the same reference).
  float m = -FLT_MAX;
  float l = 0.f;  // running sum of probabilities (this lane's keys)
  f32x16 o[S::NDT];
#pragma unroll
  for (int dt = 0; dt < S::NDT; ++dt) o[dt] = f32x16{};

  auto tile = [&](const char* stage, int k0, bool need_mask) {
    // S^T = K Q^T for 64 keys x 32 queries.
    f32x16 s[S::NMT];
#pragma unroll
    for (int mt = 0; mt < S::NMT; ++mt) {
      s[mt] = f32x16{};
      const char* kp = stage + ((mt * 32 + col) * S::KS + half * S::DH) * S::ES;
#pragma unroll
      for (int i = 0; i < S::NQK; ++i) s[mt] = E::mma(ld<Raw>(kp + i * KH * S::ES), qf[i], s[mt]);
    }
    if (need_mask) {  // diagonal or tail tile: hidden scores -> -inf (probability 0)
#pragma unroll
      for (int mt = 0; mt < S::NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool vis = key < N && (!CAUSAL || key <= qrow);
          if (!vis) s[mt][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < S::NMT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
    mx = max_with_other_half(mx);
    const float m_new = fmaxf(m, mx);
    if (wave_any((m_new - m) * c > 8.f || m == -FLT_MAX)) {
      const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < S::NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
    const float mc = m * c;

    // Probabilities -> MFMA B operands (P^T), in register order.
    Raw pf[S::NMT * (16 / KH)];
#pragma unroll
    for (int mt = 0; mt < S::NMT; ++mt)
#pragma unroll
      for (int u = 0; u < 16 / KH; ++u) {
        float p[KH];
#pragma unroll
        for (int jj = 0; jj < KH; ++jj) {
          // c > 0 always (the host passes max(scale*log2(e), FLT_MIN)), so
          // a hidden score (-inf) gives exactly 0.
          p[jj] = __builtin_amdgcn_exp2f(fmaf(s[mt][u * KH + jj], c, -mc));
        }
        pf[mt * (16 / KH) + u] = E::pack_sum(p, l);
      }

    // O^T += V^T P^T.
    const char* vbase = stage + S::K_BYTES;
#pragma unroll
    for (int dt = 0; dt < S::NDT; ++dt) {
      const char* vp = vbase + voff[dt];
#pragma unroll
      for (int u = 0; u < S::NPV; ++u) {
        Raw va;
        if constexpr (S::TRV) {
          const u32x2 lo = lds_read_tr16(vp + (16 * u) * D * 2);
          const u32x2 hi = lds_read_tr16(vp + (16 * u + 8) * D * 2);
          va = Raw{lo[0], lo[1], hi[0], hi[1]};
        } else {
          va = ld<Raw>(vp + u * 2 * KH * S::ES);
        }
        o[dt] = E::mma(va, pf[u], o[dt]);
      }
    }
  };

  TileLoader<T, D> tl;
  tl.load(K, V, 0, tid);
  tl.store(lds, tid);
  __syncthreads();

  for (int j = 0; j < nkv; ++j) {
    const char* stage = lds + (j & 1) * S::STAGE;
    if (j + 1 < nkv) tl.load(K, V, (j + 1) * kBN, tid);
    const int k0 = j * kBN;
    if (wave_active && (!CAUSAL || k0 <= qw0 + 31)) {
      tile(stage, k0, (CAUSAL && k0 + kBN - 1 > qw0) || (k0 + kBN > N));
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
