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
// gfx950 design, 16-bit inputs (bf16, fp16): one workgroup = 8 waves = 256
// query rows of one head, in two groups of four waves (A = waves 0-3,
// B = waves 4-7; waves 0-3 run on four different SIMDs and wave w + 4 on the
// SIMD of wave w, so each SIMD holds one wave of each group).
// For small grids, a key-split kernel (fwd_ks_kernel) deals each
// workgroup's key tiles over its waves and merges their partials in LDS.
//   * grid: B*H*ceil(N/256) workgroups, remapped so the query tiles of a head
//     share one XCD's L2; causal grids run the longest rows first.
//   * each wave owns 32 query rows; its Q tile stays in registers as MFMA B
//     operands for the whole key loop.
//   * work per 64-key tile i is split into a matrix phase M(i) -- O += P V
//     for tile i-1, then S^T = K Q^T for tile i -- and a vector phase V(i),
//     the online softmax of tile i. Phases end at workgroup barriers and
//     group B runs one phase behind group A, so on every SIMD one wave's
//     MFMA phase overlaps the other wave's softmax ("ping-pong").
//   * K and V tiles (64 keys) are double-buffered in LDS, K row-major padded
//     by 16 bytes per row, V row-major with its 16-byte units XOR-swizzled by
//     key and read transposed (ds_read_b64_tr_b16) as the V^T operand. Global
//     loads are issued in a wave's matrix phase into registers and written to
//     LDS in its vector phase: group A streams V tile i, group B K tile i+2.
//   * S^T = K Q^T leaves each lane 16 scores of a single query row, so the
//     row max is lane-local plus one exchange with lane^32, and P^T feeds
//     O^T += V^T P^T straight from registers with no LDS round trip.
//   * softmax in float32 with exp2 and scale*log2(e) folded into one FMA per
//     score, tracking the raw-score max (valid because scale >= 0); 1/l is
//     applied once in the epilogue (the FA2 reduction of non-matmul work).
//
// float32 inputs use a plainer kernel (4 waves = 128 rows per workgroup, one
// loop doing all three steps per tile) on the 32x32x2 fp32 MFMA.
#include <float.h>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;  // query rows per workgroup
constexpr int kBN = 64;           // keys per K/V tile

// Split-KV: slice `split` of `nsplit` of the key tiles [t0, t0 + nkv), an
// even share in order (empty when there are more slices than tiles).
__device__ inline void split_slice(int split, int nsplit, int& t0, int& nkv) {
  if (nsplit == 1) return;
  const int a0 = split * nkv / nsplit, a1 = (split + 1) * nkv / nsplit;
  t0 += a0;
  nkv = a1 - a0;
}

// One row's split-KV partial (this lane's half of the head dim, in the
// accumulator layout of the epilogues): O normalized over the slice's keys,
// in float32, and the slice's LSE. A row that saw no key of the slice
// (lt == 0) gets O = 0 and LSE = -inf, which the merge weighs with
// exp(-inf) = 0.
template <int NDT>
__device__ inline void write_partial(const FwdArgs& a, int split, int bh, int qrow, int half,
                                     const f32x16 (&o)[NDT], float m, float lt) {
  constexpr int D = NDT * 32;
  const size_t rows = (size_t)a.B * a.H * a.N;
  const size_t row = (size_t)split * rows + (size_t)bh * a.N + qrow;
  const bool empty = !(lt > 0.f);
  const float inv = empty ? 0.f : 1.0f / lt;
  float* orow = a.o_part + row * D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      st<f32x4>(orow + dt * 32 + 8 * g + 4 * half,
                f32x4{o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv, o[dt][4 * g + 2] * inv,
                      o[dt][4 * g + 3] * inv});
  if (half == 0) a.lse_part[row] = empty ? -INFINITY : m * a.scale + logf(lt);
}

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

// One 64-key tile of a wave's 32 query rows, all three steps in order (the
// float32 kernel's step; 16-bit types use attend_tile16 below):
// S^T = K Q^T from the stage's K tile, the online softmax (hidden scores set
// to -inf when need_mask), O^T += V^T P^T from the stage's V tile. m is the
// reference max the exponentials are taken against (raw scores): it moves to
// the row max only when that max has grown by more than 2^8 in probability,
// and O and l are rescaled with it, so O and l always share one reference.
template <typename T, int D, bool CAUSAL>
__device__ __forceinline__ void attend_tile(const char* stage, const int (&voff)[FwdShape<T, D>::NDT],
                                            const typename Elem<T>::Raw (&qf)[FwdShape<T, D>::NQK],
                                            int k0, bool need_mask, int qrow, int half, int col,
                                            int N, float c, int wl, int wr, float& m, float& l,
                                            f32x16 (&o)[FwdShape<T, D>::NDT]) {
  using S = FwdShape<T, D>;
  using E = Elem<T>;
  using Raw = typename E::Raw;
  constexpr int KH = S::KH;
  // S^T = K Q^T for 64 keys x 32 queries.
  f32x16 s[S::NMT];
#pragma unroll
  for (int mt = 0; mt < S::NMT; ++mt) {
    s[mt] = f32x16{};
    const char* kp = stage + ((mt * 32 + col) * S::KS + half * S::DH) * S::ES;
#pragma unroll
    for (int i = 0; i < S::NQK; ++i) s[mt] = E::mma(ld<Raw>(kp + i * KH * S::ES), qf[i], s[mt]);
  }
  if (need_mask) {  // diagonal, window edge or tail: hidden scores -> -inf (probability 0)
#pragma unroll
    for (int mt = 0; mt < S::NMT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (!key_visible(key, qrow, N, CAUSAL, wl, wr)) s[mt][r] = -INFINITY;
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
  // Clamped: with no visible key yet (m = -FLT_MAX) and c > 1 the product
  // overflows, and -inf + inf would turn hidden scores into NaN.
  const float mc = fmaxf(m * c, -FLT_MAX);

  // Probabilities -> MFMA B operands (P^T), in register order.
  Raw pf[S::NMT * (16 / KH)];
#pragma unroll
  for (int mt = 0; mt < S::NMT; ++mt)
#pragma unroll
    for (int u = 0; u < 16 / KH; ++u) {
      float p[KH];
#pragma unroll
      for (int jj = 0; jj < KH; ++jj) {
        // c > 0 always (the host passes max(scale*log2(e), FLT_MIN)), so a
        // hidden score (-inf) gives exactly 0.
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
}

// The same three steps for 16-bit types, with the ping-pong kernel's online
// softmax: the exponentials are taken against the current reference m and
// kept while no lane's sum over its 32 probabilities exceeds 2^8 (so no
// single one does); otherwise, and while a row has no reference yet, m moves
// to the row max, O and l are rescaled and the exponentials are taken again.
// The row sum is a tree of float32 adds over the unrounded probabilities.
template <typename T, int D, bool CAUSAL>
__device__ __forceinline__ void attend_tile16(const char* stage, const int (&voff)[FwdShape<T, D>::NDT],
                                              const typename Elem<T>::Raw (&qf)[FwdShape<T, D>::NQK],
                                              int k0, bool need_mask, int qrow, int half, int col,
                                              int N, float c, int wl, int wr, float& m, float& l,
                                              f32x16 (&o)[FwdShape<T, D>::NDT]) {
  using S = FwdShape<T, D>;
  using E = Elem<T>;
  using Raw = typename E::Raw;
  constexpr int KH = S::KH;
  static_assert(S::ES == 2 && S::NMT == 2 && KH == 8, "16-bit, 64-key tiles");
  f32x16 s[S::NMT];
#pragma unroll
  for (int mt = 0; mt < S::NMT; ++mt) {
    s[mt] = f32x16{};
    const char* kp = stage + ((mt * 32 + col) * S::KS + half * S::DH) * S::ES;
#pragma unroll
    for (int i = 0; i < S::NQK; ++i) s[mt] = E::mma(ld<Raw>(kp + i * KH * S::ES), qf[i], s[mt]);
  }
  if (need_mask) {
#pragma unroll
    for (int mt = 0; mt < S::NMT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (!key_visible(key, qrow, N, CAUSAL, wl, wr)) s[mt][r] = -INFINITY;
      }
  }
  float p[2 * 16];
  float ls;
  auto exps = [&]() {
    const float mc = fmaxf(m * c, -FLT_MAX);
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
  if (wave_any(!(ls <= 256.f) || m == -FLT_MAX)) {
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
  Raw pf[S::NMT * 2];
#pragma unroll
  for (int k = 0; k < S::NMT * 2; ++k)
#pragma unroll
    for (int w = 0; w < 4; ++w) pf[k][w] = E::pack_pair(p[8 * k + 2 * w], p[8 * k + 2 * w + 1]);
  const char* vbase = stage + S::K_BYTES;
#pragma unroll
  for (int dt = 0; dt < S::NDT; ++dt) {
    const char* vp = vbase + voff[dt];
#pragma unroll
    for (int u = 0; u < S::NPV; ++u) {
      const u32x2 lo = lds_read_tr16(vp + (16 * u) * D * 2);
      const u32x2 hi = lds_read_tr16(vp + (16 * u + 8) * D * 2);
      o[dt] = E::mma(Raw{lo[0], lo[1], hi[0], hi[1]}, pf[u], o[dt]);
    }
  }
}

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
  const int nsplit = a.num_splits;
  const int bh = lin / (nqt * nsplit);
  const int qi = lin % (nqt * nsplit) / nsplit, split = lin % nsplit;
  const int qtile = CAUSAL ? nqt - 1 - qi : qi;
  const int q0 = qtile * kBM;

  const size_t head = (size_t)bh * N * D;
  // Query head h attends with K/V head h / (H / Hkv).
  const size_t kvhead = (size_t)((bh / a.H) * a.Hkv + (bh % a.H) / (a.H / a.Hkv)) * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * S::ES;
  const HeadBuf Q(reinterpret_cast<const T*>(a.q) + head, head_bytes);
  const HeadBuf K(reinterpret_cast<const T*>(a.k) + kvhead, head_bytes);
  const HeadBuf V(reinterpret_cast<const T*>(a.v) + kvhead, head_bytes);
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

  // Key tiles t0 .. t0+nkv-1 this workgroup visits: those holding a key some
  // of its rows can see (all of them, or fewer under the causal rule and a
  // window), or its slice of them under split-KV; a wave computes on the
  // tiles its own rows can see.
  const int qlast = min(q0 + kBM, N) - 1;
  int t0 = first_visible_key(q0, a.wl) / kBN;
  int nkv = last_visible_key(qlast, N, CAUSAL, a.wr) / kBN - t0 + 1;
  split_slice(split, nsplit, t0, nkv);
  const int wk_lo = first_visible_key(qw0, a.wl);
  const int wk_hi = last_visible_key(min(qw0 + 31, N - 1), N, CAUSAL, a.wr);

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
    attend_tile<T, D, CAUSAL>(stage, voff, qf, k0, need_mask, qrow, half, col, N, c, a.wl, a.wr,
                              m, l, o);
  };

  if (nkv == 0) {  // an empty slice: nothing to visit, an empty partial
    if (wave_active && qrow < N) write_partial(a, split, bh, qrow, half, o, -FLT_MAX, 0.f);
    return;
  }
  TileLoader<T, D> tl;
  tl.load(K, V, t0 * kBN, tid);
  tl.store(lds, tid);
#pragma unroll
  for (int i = 0; i < S::NQK; ++i) settle(qf[i]);
  __syncthreads();

  for (int j = 0; j < nkv; ++j) {
    const char* stage = lds + (j & 1) * S::STAGE;
    if (j + 1 < nkv) tl.load(K, V, (t0 + j + 1) * kBN, tid);
    const int k0 = (t0 + j) * kBN;
    if (wave_active && k0 <= wk_hi && k0 + kBN - 1 >= wk_lo) {
      tile(stage, k0, !block_all_visible(qw0, qw0 + 31, k0, k0 + kBN - 1, N, CAUSAL, a.wl, a.wr));
    }
    if (j + 1 < nkv) tl.store(lds + ((j + 1) & 1) * S::STAGE, tid);
    __syncthreads();
  }

  if (!wave_active || qrow >= N) return;
  const float lt = l + __shfl_xor(l, 32);
  if (nsplit > 1) {
    write_partial(a, split, bh, qrow, half, o, m, lt);
    return;
  }
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

// ---------------------------------------------------------------------------
// 16-bit kernel: 8 waves, ping-pong between matrix and vector phases.

constexpr int kPPWaves = 8;
constexpr int kPPThreads = kPPWaves * 64;
constexpr int kPPGroup = kPPThreads / 2;  // threads per wave group
constexpr int kPPBM = kPPWaves * 32;      // query rows per workgroup

template <typename T, int D>
struct PPShape {
  static constexpr int KH = 8;               // operand elements per lane per MFMA
  static constexpr int NQK = D / 2 / KH;     // MFMAs per 32x32 score tile
  static constexpr int NMT = kBN / 32;       // 32-key blocks per tile
  static constexpr int NDT = D / 32;         // 32-wide head-dim blocks of O
  static constexpr int NPV = kBN / 16;       // PV MFMAs per head-dim block
  static constexpr int NPF = NMT * 2;        // P^T operands per tile
  static constexpr int KS = D + 8;           // K row stride in LDS (elements, +16 B)
  static constexpr int K_BYTES = kBN * KS * 2;
  static constexpr int V_BYTES = kBN * D * 2;
  static constexpr int LDS_BYTES = 2 * K_BYTES + 2 * V_BYTES;
  static constexpr int VECS = kBN * D / 8 / kPPGroup;  // 16 B per thread per tile
  static_assert(kBN * D / 8 % kPPGroup == 0, "tile must split evenly over a group");
};

// One wave group's share of a 64-key tile, staged in registers between the
// global load (matrix phase) and the LDS store (vector phase). Vector i of a
// thread is tile row ROWS*i + gtid/(D/8), columns 8*(gtid % (D/8)) .. +8, so
// the global offsets are contiguous and the LDS offsets step by a constant.
template <int D>
struct GroupStage {
  static constexpr int VECS = PPShape<__bf16, D>::VECS;
  static constexpr int ROWS = kPPGroup / (D / 8);  // tile rows per vector step
  static constexpr int K_STRIDE = ROWS * (D + 8) * 2;
  static constexpr int V_STRIDE = ROWS * D * 2;
  u32x4 r[VECS];

  // Rows past N read as zeros (buffer range check).
  __device__ inline void load(const HeadBuf& X, int k0, int gtid) {
#pragma unroll
    for (int i = 0; i < VECS; ++i) r[i] = X.ld16((gtid + kPPGroup * i) * 16, k0 * D * 2);
  }
  __device__ inline void store(char* dst, int off0, int stride) const {
#pragma unroll
    for (int i = 0; i < VECS; ++i) st<u32x4>(dst + off0 + i * stride, r[i]);
  }
  // LDS byte offset of vector 0: K row-major with rows padded by 16 bytes;
  // V row-major with 16-byte units XOR-swizzled by key.
  __device__ static inline int k_off(int gtid) {
    const int row = gtid / (D / 8), c = (gtid % (D / 8)) * 8;
    return (row * (D + 8) + c) * 2;
  }
  __device__ static inline int v_off(int gtid) {
    const int row = gtid / (D / 8), c = (gtid % (D / 8)) * 8;
    return row * D * 2 + (((c >> 3) ^ v_swz<D>(row)) << 4);
  }
};

template <typename T, int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(kPPThreads, 1) void fwd_pp_kernel(FwdArgs a) {
  using S = PPShape<T, D>;
  using E = Elem<T>;
  using Raw = typename E::Raw;
  constexpr int KH = S::KH;

  __shared__ __attribute__((aligned(16))) char lds[S::LDS_BYTES];
  char* const kbuf = lds;                     // 2 x K tile
  char* const vbuf = lds + 2 * S::K_BYTES;    // 2 x V tile

  const int N = a.N;
  const int nqt = (N + kPPBM - 1) / kPPBM;
  const int nsplit = a.num_splits;
  const int lin = CAUSAL ? xcd_remap_ranked(blockIdx.x, gridDim.x, nqt * nsplit, nsplit)
                         : xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lin / (nqt * nsplit);
  const int qi = lin % (nqt * nsplit) / nsplit, split = lin % nsplit;
  const int qtile = CAUSAL ? nqt - 1 - qi : qi;
  const int q0 = qtile * kPPBM;

  const size_t head = (size_t)bh * N * D;
  // Query head h attends with K/V head h / (H / Hkv).
  const size_t kvhead = (size_t)((bh / a.H) * a.Hkv + (bh % a.H) / (a.H / a.Hkv)) * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const HeadBuf Q(reinterpret_cast<const T*>(a.q) + head, head_bytes);
  const HeadBuf K(reinterpret_cast<const T*>(a.k) + kvhead, head_bytes);
  const HeadBuf V(reinterpret_cast<const T*>(a.v) + kvhead, head_bytes);
  T* O = reinterpret_cast<T*>(a.o) + head;
  float* L = a.lse + (size_t)bh * N;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;         // 0: A, 1: B (one phase behind)
  const int gtid = tid & (kPPGroup - 1);
  const int col = lane & 31, half = lane >> 5;
  const int qw0 = q0 + wave * 32;      // first query row of this wave
  const int qrow = qw0 + col;          // the query row this lane serves

  // Key tiles: the workgroup streams tiles t0 .. t0+nkv-1, those holding a
  // key some of its rows can see (all of them, or fewer under the causal rule
  // and a window), or its slice of them under split-KV; this wave computes on
  // its steps [w_lo, w_end), the tiles its own rows can see (none if its rows
  // are all past N or see no key of the slice).
  const int qlast = min(q0 + kPPBM, N) - 1;
  int t0 = first_visible_key(q0, a.wl) / kBN;
  int nkv = last_visible_key(qlast, N, CAUSAL, a.wr) / kBN - t0 + 1;
  split_slice(split, nsplit, t0, nkv);
  int w_lo = nkv + 1, w_end = -1;
  if (qw0 < N) {
    const int lo = max(first_visible_key(qw0, a.wl) / kBN - t0, 0);
    const int hi = min(last_visible_key(min(qw0 + 31, N - 1), N, CAUSAL, a.wr) / kBN - t0 + 1, nkv);
    if (lo < hi) w_lo = lo, w_end = hi;
  }
  // Block-sparse: the streamed tiles are those of [t0, t0 + nkv) that some
  // 64-row query block of the workgroup keeps, in order (an LDS list whose
  // entries also flag which of the four blocks keep the tile); every wave
  // runs every listed tile and hides all scores of a tile its block drops.
  const uint16_t* tlist = nullptr;
  if constexpr (SPARSE) {
    static_assert(kBN == kMaskBlock && kPPBM == 4 * kMaskBlock, "tiles of one mask block, four per workgroup");
    __shared__ uint16_t sl[kMaxMaskBlocks];
    __shared__ int sw[kPPWaves];
    const int qb0 = q0 / kMaskBlock;
    const int nyb = min(kPPBM / kMaskBlock, a.nmb - qb0);
    nkv = compact_blocks<kPPThreads, 4>(a.block_mask, (long long)qb0 * a.nmb + t0, 1, a.nmb, nyb,
                                        nkv, sl, sw);
    tlist = sl;
    if (qw0 < N) w_lo = 0, w_end = nkv;
  }
  // Stream position x -> key tile, and whether this wave's block keeps it.
  auto ktile = [&](int x) -> int {
    if constexpr (SPARSE) return t0 + (__builtin_amdgcn_readfirstlane(tlist[x]) >> 4);
    return t0 + x;
  };
  auto kept = [&](int x) -> bool {
    if constexpr (SPARSE) return (__builtin_amdgcn_readfirstlane(tlist[x]) >> ((qw0 - q0) / kMaskBlock)) & 1;
    return true;
  };

  // Q^T as MFMA B operands: lane half h holds head-dim elements
  // [h*D/2, h*D/2 + D/2) of its row, KH per MFMA.
  Raw qf[S::NQK];
#pragma unroll
  for (int i = 0; i < S::NQK; ++i) qf[i] = Q.ld16((qrow * D + half * (D / 2) + i * KH) * 2);

  // Per-lane byte offsets of the transposing V^T operand reads: lane 4r+q of
  // 16-lane group g fetches key row 4h + r (h = g/2) and head-dim columns
  // 32*dt + 16*(g&1) + 4q .. +4.
  int voff[S::NDT];
  {
    const int g = lane >> 4, jf = lane & 15, r = jf >> 2, q = jf & 3, h = g >> 1;
    const int b = 2 * (g & 1) + (q >> 1);
#pragma unroll
    for (int dt = 0; dt < S::NDT; ++dt)
      voff[dt] = (4 * h + r) * D * 2 + (((4 * dt) ^ (b ^ v_swz<D>(r))) << 4) + (q & 1) * 8;
  }
  const int koff = (col * S::KS + half * (D / 2)) * 2;

  const float c = a.scale_log2;  // scale * log2(e)
  // Reference max (raw scores) the exponentials are taken against; it only
  // moves when a row's max exceeds it by more than 2^8 in probability
  // (exact: O and l are always relative to the same reference).
  float m = -FLT_MAX;
  float l = 0.f;  // running sum of probabilities (this lane's keys)
  f32x16 o[S::NDT];
#pragma unroll
  for (int dt = 0; dt < S::NDT; ++dt) o[dt] = f32x16{};
  // Scores of a tile (from its matrix phase to its vector phase), then its
  // packed probabilities (to the next matrix phase): never live together, so
  // they share registers -- P^T operand k lives in words [4k, 4k+4) of s.
  // (Operands are taken out with constant-index shuffles: rebuilding a
  // vector element by element from another vector's elements mis-compiles.)
  f32x16 s[S::NMT];
#pragma unroll
  for (int mt = 0; mt < S::NMT; ++mt) s[mt] = f32x16{};
  static_assert(S::NPF == 4, "P^T operands of a 64-key tile fill s[0]");

  // Matrix phase: O^T += V^T P^T for the previous tile (PV), then
  // S^T = K Q^T for the current one (QK). The MFMAs run in chunks of four;
  // the LDS operands of chunk c + 1 are read while chunk c computes, so the
  // phase hides its own LDS latency (the other wave on this SIMD is in its
  // vector phase and issues no MFMAs to fill the gaps). PV chunk dt covers
  // head-dim block dt; QK chunk (mt, h) covers key block mt and head-dim
  // operands 4h .. 4h + 3. The P^T operands sit in s[0] and are consumed by
  // the PV chunks before the QK chunks overwrite s.
  auto mphase = [&](const char* vt, const char* kt, auto pv_c, auto qk_c) {
    constexpr bool PV = decltype(pv_c)::value, QK = decltype(qk_c)::value;
    constexpr int QKH = S::NQK / 4;  // QK chunks per key block
    constexpr int NPVC = PV ? S::NDT : 0;
    constexpr int NC = NPVC + (QK ? S::NMT * QKH : 0);
    const f32x16 x = s[0];
    const Raw pf[4] = {
        __builtin_bit_cast(Raw, __builtin_shufflevector(x, x, 0, 1, 2, 3)),
        __builtin_bit_cast(Raw, __builtin_shufflevector(x, x, 4, 5, 6, 7)),
        __builtin_bit_cast(Raw, __builtin_shufflevector(x, x, 8, 9, 10, 11)),
        __builtin_bit_cast(Raw, __builtin_shufflevector(x, x, 12, 13, 14, 15))};
    Raw op[2][4];
    auto fetch = [&](int c, Raw(&dst)[4]) {
      if (c < NPVC) {
        const char* vp = vt + voff[c];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const u32x2 lo = lds_read_tr16(vp + (16 * u) * D * 2);
          const u32x2 hi = lds_read_tr16(vp + (16 * u + 8) * D * 2);
          dst[u] = Raw{lo[0], lo[1], hi[0], hi[1]};
        }
      } else {
        const int mt = (c - NPVC) / QKH, h = (c - NPVC) % QKH;
        const char* kp = kt + koff + mt * 32 * S::KS * 2 + h * 4 * KH * 2;
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[j] = ld<Raw>(kp + j * KH * 2);
      }
    };
    auto compute = [&](int c, const Raw(&src)[4]) {
      if (c < NPVC) {
#pragma unroll
        for (int u = 0; u < 4; ++u) o[c] = E::mma(src[u], pf[u], o[c]);
      } else {
        const int mt = (c - NPVC) / QKH, h = (c - NPVC) % QKH;
        if (h == 0) s[mt] = f32x16{};
#pragma unroll
        for (int j = 0; j < 4; ++j) s[mt] = E::mma(src[j], qf[h * 4 + j], s[mt]);
      }
    };
    static_assert(S::NPV == 4 && S::NQK % 4 == 0, "chunks of four MFMAs");
    __builtin_amdgcn_s_setprio(1);
    fetch(0, op[0]);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c + 1 < NC) fetch(c + 1, op[(c + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      compute(c, op[c & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Online softmax of one tile: scores s -> probabilities pf.
  auto softmax = [&](int k0, bool keep) {
    if (SPARSE && !keep) {  // a block this wave's rows do not see
#pragma unroll
      for (int mt = 0; mt < S::NMT; ++mt) s[mt] = f32x16{} - INFINITY;
    } else if (!block_all_visible(qw0, qw0 + 31, k0, k0 + kBN - 1, N, CAUSAL, a.wl, a.wr)) {
      // Diagonal, window edge or tail tile: hidden scores -> -inf (probability 0).
#pragma unroll
      for (int mt = 0; mt < S::NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (!key_visible(key, qrow, N, CAUSAL, a.wl, a.wr)) s[mt][r] = -INFINITY;
        }
    }
    // Exponentials against the current reference m, without a row max:
    // as long as no lane's sum over its 32 scores exceeds 2^8 (so no single
    // probability does), they are kept. Otherwise (a row max that grew, an
    // overflow) and while a row has no reference yet, the reference moves to
    // the row max, O and l are rescaled, and the exponentials are taken
    // again. Either way O and l stay relative to one reference, so the
    // result is exact. (The no-reference case must not take the fast path:
    // m * c then differs from m * scale * log2(e) when scale is 0.)
    float p[2 * 16];
    float ls;
    auto exps = [&]() {
      // Clamped: with no visible key yet (m = -FLT_MAX) and c > 1 the product
      // overflows, and -inf + inf would turn hidden scores into NaN.
      const float mc = fmaxf(m * c, -FLT_MAX);
#pragma unroll
      for (int mt = 0; mt < S::NMT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          // c > 0 always (the host passes max(scale*log2(e), FLT_MIN)), so a
          // hidden score (-inf) gives exactly 0.
          p[mt * 16 + r] = __builtin_amdgcn_exp2f(fmaf(s[mt][r], c, -mc));
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
    if (wave_any(!(ls <= 256.f) || m == -FLT_MAX)) {
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
    // Operand k = 2*mt + u packs probabilities 8u .. 8u+8 of key block mt
    // into words [4k, 4k+4) of s, all of which were read above. Each packed
    // pair goes straight to its word: reading words back out of a vector
    // assembled from packed 16-bit pairs mis-compiles.
#pragma unroll
    for (int k = 0; k < S::NPF; ++k)
#pragma unroll
      for (int w = 0; w < 4; ++w)
        s[k / 4][(k % 4) * 4 + w] = __builtin_bit_cast(float, E::pack_pair(p[8 * k + 2 * w], p[8 * k + 2 * w + 1]));
  };

  if (nkv == 0) {  // an empty slice: nothing to visit, an empty partial
    if constexpr (SPARSE) {  // no kept block: O = 0, LSE = -inf
      if (qrow < N) {
#pragma unroll
        for (int dt = 0; dt < S::NDT; ++dt)
#pragma unroll
          for (int g = 0; g < 4; ++g) st<u32x2>(O + (size_t)qrow * D + dt * 32 + 8 * g + 4 * half, u32x2{0u, 0u});
        if (half == 0) L[qrow] = -INFINITY;
      }
      return;
    }
    if (qrow < N) write_partial(a, split, bh, qrow, half, o, -FLT_MAX, 0.f);
    return;
  }

  // Prologue: K tiles 0 and 1 (group A stages tile 0, group B tile 1).
  using GS = GroupStage<D>;
  GS stg;
  if (group == 0 || nkv > 1) {
    stg.load(K, ktile(group) * kBN, gtid);
    stg.store(kbuf + group * S::K_BYTES, GS::k_off(gtid), GS::K_STRIDE);
  }
#pragma unroll
  for (int i = 0; i < S::NQK; ++i) settle(qf[i]);
  __syncthreads();

  // Step i is a matrix phase M(i) then a vector phase V(i), each ending at a
  // barrier; group B runs one phase behind group A (one extra barrier first,
  // A one extra at the end), so the phases of the two groups alternate.
  // Group A streams V tile i (global load in M(i), LDS store in V(i)), group
  // B K tile i + 2. K tile i lives in kbuf[i % 2] and V tile i in vbuf[i % 2];
  // each store lands in a buffer whose last readers passed an earlier barrier.
  const bool kgrp = group == 1;
  const HeadBuf& X = kgrp ? K : V;
  const int soff = kgrp ? GS::k_off(gtid) : GS::v_off(gtid);
  const int sstride = kgrp ? GS::K_STRIDE : GS::V_STRIDE;
  // Where a group issues the global load of the next tile it stores: at
  // d = 128 right after its previous store, before the barrier (the staging
  // registers are free from there, and the load gets the barrier wait on top
  // of a matrix phase to land: measured +2% non-causal, +7% causal); at
  // d = 64 at the start of the matrix phase that precedes the store
  // (measured 4% faster there).
  constexpr bool kEarlyLoad = D == 128;
  if (kEarlyLoad && (kgrp ? 2 < nkv : true)) stg.load(X, ktile(kgrp ? 2 : 0) * kBN, gtid);
  if (kgrp) __syncthreads();
  // Step 0 (no PV yet).
  {
    const int lt = kgrp ? 2 : 0;
    if (!kEarlyLoad && lt < nkv) stg.load(X, ktile(lt) * kBN, gtid);
    if (w_lo == 0 && w_end > 0) mphase(vbuf, kbuf, BoolC<false>{}, BoolC<true>{});
    __syncthreads();
    if (w_lo == 0 && w_end > 0) softmax(ktile(0) * kBN, kept(0));
    if (lt < nkv) stg.store(kgrp ? kbuf : vbuf, soff, sstride);
    if (kEarlyLoad && lt + 1 < nkv) stg.load(X, ktile(lt + 1) * kBN, gtid);
    __syncthreads();
  }
  // Steps 1 .. nkv-1, one code path. At step w_lo (a wave whose first
  // visible tile is not the workgroup's first) the PV half multiplies the
  // previous V tile by probabilities that are still all zero, and at step
  // w_end (a wave past its last visible tile) the QK half is unused.
  for (int i = 1; i < nkv; ++i) {
    const int lt = kgrp ? i + 2 : i;  // the tile this group streams
    if (!kEarlyLoad && lt < nkv) stg.load(X, ktile(lt) * kBN, gtid);
    if (w_lo <= i && i <= w_end)
      mphase(vbuf + ((i - 1) & 1) * S::V_BYTES, kbuf + (i & 1) * S::K_BYTES, BoolC<true>{},
             BoolC<true>{});
    __syncthreads();
    if (w_lo <= i && i < w_end) softmax(ktile(i) * kBN, kept(i));
    if (lt < nkv) stg.store(kgrp ? kbuf + (i & 1) * S::K_BYTES : vbuf + (i & 1) * S::V_BYTES, soff, sstride);
    if (kEarlyLoad && lt + 1 < nkv) stg.load(X, ktile(lt + 1) * kBN, gtid);
    __syncthreads();
  }
  // Final matrix phase: PV of the last tile.
  if (w_end == nkv) mphase(vbuf + ((nkv - 1) & 1) * S::V_BYTES, kbuf, BoolC<true>{}, BoolC<false>{});
  __syncthreads();
  if (!kgrp) __syncthreads();

  if (qrow >= N) return;
  const float lt = l + __shfl_xor(l, 32);
  if (nsplit > 1) {
    write_partial(a, split, bh, qrow, half, o, m, lt);
    return;
  }
  // (Block-sparse: a row that kept no key has l = 0: O = 0, LSE = -inf.)
  const float inv = SPARSE && !(lt > 0.f) ? 0.f : 1.0f / lt;
  T* orow = O + (size_t)qrow * D;
#pragma unroll
  for (int dt = 0; dt < S::NDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = dt * 32 + 8 * g + 4 * half;
      const uint32_t w0 = E::bits(o[dt][4 * g] * inv) | ((uint32_t)E::bits(o[dt][4 * g + 1] * inv) << 16);
      const uint32_t w1 = E::bits(o[dt][4 * g + 2] * inv) | ((uint32_t)E::bits(o[dt][4 * g + 3] * inv) << 16);
      st<u32x2>(orow + d0, u32x2{w0, w1});
    }
  if (half == 0) L[qrow] = SPARSE && !(lt > 0.f) ? -INFINITY : m * a.scale + logf(lt);
}

// ---------------------------------------------------------------------------
// 16-bit kernel for grids too small to fill the GPU: the key tiles of a
// workgroup's rows are split over its waves, and the waves' partial results
// are combined in LDS at the end -- the blockwise softmax merge within one
// workgroup, so no float32 partials reach HBM and no second launch is needed.
//   * 8 waves = P key parts x RG groups of 32 query rows (d = 64: 4 x 2, a
//     workgroup of 64 rows; d = 128: 2 x 4, 128 rows). Part p takes the
//     workgroup's key tiles p, p + P, p + 2P, ... (interleaved, so the parts
//     stay even under the causal rule), streamed through its own pair of LDS
//     stages by its RG waves; one workgroup barrier per step.
//   * Each wave runs the three steps of a tile in order (attend_tile16, with
//     the ping-pong kernel's online softmax); the two waves of a SIMD overlap
//     each other's MFMAs and softmax by themselves.
//   * At the end the waves of parts 1 .. P-1 write their O, reference max m
//     and sum l to LDS; the part-0 wave of each row group rescales all P
//     partials to the largest reference and adds them (every wave holds the
//     same (row, column) elements per lane, so the merge is elementwise).
constexpr int kKSWaves = 8;
constexpr int kKSThreads = kKSWaves * 64;

template <int D>
struct KSShape {
  static constexpr int P = D == 64 ? 4 : 2;       // key parts
  static constexpr int RG = kKSWaves / P;         // 32-row groups
  static constexpr int BM = 32 * RG;              // query rows per workgroup
  static constexpr int PT = RG * 64;              // threads per part
  static constexpr int K_BYTES = kBN * (D + 8) * 2;
  static constexpr int STAGE = K_BYTES + kBN * D * 2;
  static constexpr int VECS = kBN * D / 8 / PT;   // 16-byte vectors per thread, per tensor
  static constexpr int LDS_BYTES = 2 * P * STAGE;
  static constexpr int NDT = D / 32;
  static constexpr int MW = NDT * 16 + 2;         // words per lane of a wave's partial: O, m, l
  static_assert(kBN * D / 8 % PT == 0, "tile must split evenly over a part");
  static_assert(kKSWaves * MW * 64 * 4 <= LDS_BYTES, "partials fit in the stages");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kKSThreads, 1) void fwd_ks_kernel(FwdArgs a) {
  using S = FwdShape<T, D>;
  using KS = KSShape<D>;
  using E = Elem<T>;
  using Raw = typename E::Raw;
  constexpr int KH = S::KH;
  static_assert(S::ES == 2 && S::STAGE == KS::STAGE && S::K_BYTES == KS::K_BYTES, "16-bit layout");

  __shared__ __attribute__((aligned(16))) char lds[KS::LDS_BYTES];

  const int N = a.N;
  const int nqt = (N + KS::BM - 1) / KS::BM;
  const int lin = CAUSAL ? xcd_remap_ranked(blockIdx.x, gridDim.x, nqt, 1)
                         : xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lin / nqt, qi = lin % nqt;
  const int q0 = (CAUSAL ? nqt - 1 - qi : qi) * KS::BM;

  const size_t head = (size_t)bh * N * D;
  // Query head h attends with K/V head h / (H / Hkv).
  const size_t kvhead = (size_t)((bh / a.H) * a.Hkv + (bh % a.H) / (a.H / a.Hkv)) * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const HeadBuf Q(reinterpret_cast<const T*>(a.q) + head, head_bytes);
  const HeadBuf K(reinterpret_cast<const T*>(a.k) + kvhead, head_bytes);
  const HeadBuf V(reinterpret_cast<const T*>(a.v) + kvhead, head_bytes);
  T* O = reinterpret_cast<T*>(a.o) + head;
  float* L = a.lse + (size_t)bh * N;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave % KS::RG, kp = wave / KS::RG;
  const int ptid = rg * 64 + lane;     // thread index within the part
  const int col = lane & 31, half = lane >> 5;
  const int qw0 = q0 + 32 * rg;        // first query row of this wave
  const int qrow = qw0 + col;          // the query row this lane serves
  const bool wave_active = qw0 < N;

  // Q^T as MFMA B operands: lane half h holds head-dim elements
  // [h*D/2, h*D/2 + D/2) of its row, KH per MFMA.
  Raw qf[S::NQK];
#pragma unroll
  for (int i = 0; i < S::NQK; ++i) qf[i] = Q.ld16((qrow * D + half * S::DH + i * KH) * 2);

  // Transposing V^T operand reads (the layout of the other 16-bit kernels):
  // lane 4r+q of 16-lane group g fetches key row 4h + r (h = g/2) and
  // head-dim columns 32*dt + 16*(g&1) + 4q .. +4.
  int voff[S::NDT];
  {
    const int g = lane >> 4, jf = lane & 15, r = jf >> 2, q = jf & 3, h = g >> 1;
    const int b = 2 * (g & 1) + (q >> 1);
#pragma unroll
    for (int dt = 0; dt < S::NDT; ++dt)
      voff[dt] = (4 * h + r) * D * 2 + (((4 * dt) ^ (b ^ v_swz<D>(r))) << 4) + (q & 1) * 8;
  }

  // Key tiles t0 .. t0+nkv-1 (those holding a key some row of the workgroup
  // can see); this part's are t0 + kp + P*j. A wave computes on those its
  // own rows can see.
  const int qlast = min(q0 + KS::BM, N) - 1;
  const int t0 = first_visible_key(q0, a.wl) / kBN;
  const int nkv = last_visible_key(qlast, N, CAUSAL, a.wr) / kBN - t0 + 1;
  const int wk_lo = first_visible_key(qw0, a.wl);
  const int wk_hi = last_visible_key(min(qw0 + 31, N - 1), N, CAUSAL, a.wr);

  // The part's staging: vector i of a thread is tile row idx/(D/8), columns
  // 8*(idx % (D/8)) .. +8 with idx = ptid + PT*i (rows past N read as zeros).
  u32x4 kr[KS::VECS], vr[KS::VECS];
  auto load = [&](int x) {
    const int k0 = (t0 + x) * kBN;
#pragma unroll
    for (int i = 0; i < KS::VECS; ++i) {
      const int off = (k0 * D + (ptid + KS::PT * i) * 8) * 2;
      kr[i] = K.ld16(off);
      vr[i] = V.ld16(off);
    }
  };
  auto stage_of = [&](int buf) { return lds + (kp * 2 + buf) * KS::STAGE; };
  auto store = [&](int buf) {
    char* Kl = stage_of(buf);
    char* Vl = Kl + KS::K_BYTES;
#pragma unroll
    for (int i = 0; i < KS::VECS; ++i) {
      const int idx = ptid + KS::PT * i;
      const int row = idx / (D / 8), c8 = (idx % (D / 8)) * 8;
      st<u32x4>(Kl + (row * (D + 8) + c8) * 2, kr[i]);
      st<u32x4>(Vl + row * D * 2 + (((c8 >> 3) ^ v_swz<D>(row)) << 4), vr[i]);
    }
  };

  const float c = a.scale_log2;  // scale * log2(e)
  float m = -FLT_MAX;  // reference max (raw scores)
  float l = 0.f;       // running sum of probabilities (this lane's keys)
  f32x16 o[S::NDT];
#pragma unroll
  for (int dt = 0; dt < S::NDT; ++dt) o[dt] = f32x16{};

  if (kp < nkv) {
    load(kp);
    store(0);
  }
#pragma unroll
  for (int i = 0; i < S::NQK; ++i) settle(qf[i]);
  __syncthreads();

  const int nit = (nkv + KS::P - 1) / KS::P;
  for (int j = 0; j < nit; ++j) {
    const int x = kp + KS::P * j, xn = x + KS::P;
    if (xn < nkv) load(xn);
    const int k0 = (t0 + x) * kBN;
    if (x < nkv && wave_active && k0 <= wk_hi && k0 + kBN - 1 >= wk_lo)
      attend_tile16<T, D, CAUSAL>(stage_of(j & 1), voff, qf, k0,
                                !block_all_visible(qw0, qw0 + 31, k0, k0 + kBN - 1, N, CAUSAL,
                                                   a.wl, a.wr),
                                qrow, half, col, N, c, a.wl, a.wr, m, l, o);
    if (xn < nkv) store((j + 1) & 1);
    __syncthreads();
  }

  // Merge the parts' partials (the stages are free: every wave passed the
  // last barrier). Lane-major words: conflict-free writes and reads.
  float* const part = reinterpret_cast<float*>(lds);
  auto word = [&](int w, int i) -> float& { return part[(w * KS::MW + i) * 64 + lane]; };
  if (kp > 0) {
#pragma unroll
    for (int dt = 0; dt < S::NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) word(wave, dt * 16 + r) = o[dt][r];
    word(wave, S::NDT * 16) = m;
    word(wave, S::NDT * 16 + 1) = l;
  }
  __syncthreads();
  if (kp > 0 || !wave_active) return;
  float mp[KS::P];
  mp[0] = m;
  float mmax = m;
#pragma unroll
  for (int p = 1; p < KS::P; ++p) {
    mp[p] = word(rg + KS::RG * p, S::NDT * 16);
    mmax = fmaxf(mmax, mp[p]);
  }
  // Rescale every partial to the largest reference (a part that saw no key
  // of these rows has O = 0, l = 0 and m = -FLT_MAX: weight 0).
  const float a0 = __builtin_amdgcn_exp2f(fmaxf((m - mmax) * c, -FLT_MAX));
  l *= a0;
#pragma unroll
  for (int dt = 0; dt < S::NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] *= a0;
#pragma unroll
  for (int p = 1; p < KS::P; ++p) {
    const int w = rg + KS::RG * p;
    const float ap = __builtin_amdgcn_exp2f(fmaxf((mp[p] - mmax) * c, -FLT_MAX));
    l += ap * word(w, S::NDT * 16 + 1);
#pragma unroll
    for (int dt = 0; dt < S::NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] += ap * word(w, dt * 16 + r);
  }

  if (qrow >= N) return;
  const float lt = l + __shfl_xor(l, 32);
  const float inv = 1.0f / lt;
  T* orow = O + (size_t)qrow * D;
#pragma unroll
  for (int dt = 0; dt < S::NDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = dt * 32 + 8 * g + 4 * half;
      const uint32_t w0 = E::bits(o[dt][4 * g] * inv) | ((uint32_t)E::bits(o[dt][4 * g + 1] * inv) << 16);
      const uint32_t w1 = E::bits(o[dt][4 * g + 2] * inv) | ((uint32_t)E::bits(o[dt][4 * g + 3] * inv) << 16);
      st<u32x2>(orow + d0, u32x2{w0, w1});
    }
  if (half == 0) L[qrow] = mmax * a.scale + logf(lt);
}

// Split-KV merge of the partials of every row: with M = max_s LSE_s and
// w_s = exp(LSE_s - M), O = sum_s w_s O_s / sum_s w_s and
// LSE = M + ln(sum_s w_s) -- the softmax over the union of the slices' keys,
// rebuilt from each slice's normalized output and normalizer. D/4 threads
// per row, 4 head-dim columns each.
template <typename T, int D>
__global__ __launch_bounds__(256) void fwd_merge_kernel(FwdArgs a) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const long long rows = (long long)a.B * a.H * a.N;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  if (row >= rows) return;
  const int c = (threadIdx.x % TPR) * 4;
  const int ns = a.num_splits;
  float mx = -INFINITY;
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, a.lse_part[s * rows + row]);
  const float mref = mx == -INFINITY ? 0.f : mx;
  float den = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < ns; ++s) {
    const float w = __builtin_amdgcn_exp2f((a.lse_part[s * rows + row] - mref) * kLog2e);
    const f32x4 x = ld<f32x4>(a.o_part + ((size_t)s * rows + row) * D + c);
    den += w;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(w, x[e], acc[e]);
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  T* orow = reinterpret_cast<T*>(a.o) + row * D + c;
  if constexpr (sizeof(T) == 2) {
    using E = Elem<T>;
    st<u32x2>(orow, u32x2{E::bits(acc[0] * inv) | ((uint32_t)E::bits(acc[1] * inv) << 16),
                          E::bits(acc[2] * inv) | ((uint32_t)E::bits(acc[3] * inv) << 16)});
  } else {
    st<f32x4>(orow, f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv});
  }
  if (c == 0) a.lse[row] = den > 0.f ? mref + logf(den) : -INFINITY;
}

template <typename T, int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  constexpr bool kPP = sizeof(T) == 2;
  const int bm = kPP ? kPPBM : kBM;
  const int nqt = (a.N + bm - 1) / bm;
  const dim3 grid((unsigned)((long long)a.B * a.H * nqt * a.num_splits));
  FwdArgs args = a;
  void* kargs[] = {&args};
  const void* fn;
  if constexpr (kPP) {
    if (a.key_split && a.num_splits == 1 && !a.block_mask) {
      const int nqk = (a.N + KSShape<D>::BM - 1) / KSShape<D>::BM;
      return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_ks_kernel<T, D, CAUSAL>),
                             dim3((unsigned)((long long)a.B * a.H * nqk)), dim3(kKSThreads), kargs,
                             0, stream);
    }
    fn = a.block_mask ? reinterpret_cast<const void*>(&fwd_pp_kernel<T, D, CAUSAL, true>)
                      : reinterpret_cast<const void*>(&fwd_pp_kernel<T, D, CAUSAL, false>);
  } else {
    fn = reinterpret_cast<const void*>(&fwd_kernel<T, D, CAUSAL>);
  }
  hipError_t e = hipLaunchKernel(fn, grid, dim3(kPP ? kPPThreads : kThreads), kargs, 0, stream);
  if (e != hipSuccess || a.num_splits == 1) return e;
  constexpr int RPB = 256 / (D / 4);
  const long long rows = (long long)a.B * a.H * a.N;
  return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_merge_kernel<T, D>),
                         dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), kargs, 0, stream);
}

template <typename T>
hipError_t dispatch_d(const FwdArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? launch<T, 64, true>(a, s) : launch<T, 64, false>(a, s);
  return a.causal ? launch<T, 128, true>(a, s) : launch<T, 128, false>(a, s);
}

}  // namespace

static_assert(kBM == kFwdRowsF32 && kPPBM == kFwdRows16 && kBN == kFwdKeyTile &&
                  KSShape<64>::BM == kFwdRowsKeySplitMin && KSShape<128>::BM >= kFwdRowsKeySplitMin,
              "host-side grid arithmetic (fa_host.cpp) uses these tile sizes");

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  switch (a.dtype) {
    case 0: return dispatch_d<float>(a, stream);
    case 1: return dispatch_d<_Float16>(a, stream);
    default: return dispatch_d<__bf16>(a, stream);
  }
}

}  // namespace fa
