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
// bf16/fp16: three kernels on the caller's stream, none with atomics:
//   1. bwd_pre:   D (float32, workspace).
//   2. bwd_kv16:  keys outer (128 per workgroup), query steps inner; dK and
//      dV accumulate in registers. Each 32-key slice is shared by two waves
//      of one SIMD, one forming P and dV, the other dP, dS and dK, in
//      alternating matrix and vector phases.
//   3. bwd_dq16:  queries outer (256 per workgroup), 32-key tiles inner (the
//      forward's decomposition); S and dP are recomputed and dQ accumulates
//      in registers, written once.
//   Grids of at most four rounds run 2 and 3 side by side in one launch
//   (bwd_fused16). With grouped K/V heads split over several workgroups per
//   key tile, a fourth kernel (bwd_kvsum) adds their float32 dK/dV partials
//   in a fixed order.
// float32: bwd_pre (also zeroes a float32 dQ accumulator), bwd_main (keys
// outer, dK/dV in registers, dQ added with one float32 atomic per element
// per key tile), bwd_dq (accumulator * scale -> dQ).
#include <float.h>

#include <mutex>

#include "fa_device.hpp"
#include "fa_internal.hpp"

namespace fa {

namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kCUs = 256;      // compute units of the part (grid sizing)
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
  const int bkv = lin / nkt;  // batch * Hkv + K/V head
  const int k0 = (lin % nkt) * kBN;
  const int grp = a.H / a.Hkv;  // query heads sharing this K/V head
  const int bq0 = (bkv / a.Hkv) * a.H + (bkv % a.Hkv) * grp;  // the first of them

  const size_t kvhead = (size_t)bkv * N * D;
  const T* K = reinterpret_cast<const T*>(a.k) + kvhead;
  const T* V = reinterpret_cast<const T*>(a.v) + kvhead;
  T* dK = reinterpret_cast<T*>(a.dk) + kvhead;
  T* dV = reinterpret_cast<T*>(a.dv) + kvhead;
  // Query-head arrays of query head g of the group.
  auto qhead = [&](int g) { return (size_t)(bq0 + g) * N; };

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

  // Query tiles [it0, it0 + ns) hold every row that sees a key of the tile;
  // step j covers query head j / ns, tile it0 + j % ns.
  const int it0 = first_query_seeing(k0, CAUSAL, a.wr) / S::BM;
  const int ns = last_query_seeing(min(k0 + kBN, N) - 1, N, a.wl) / S::BM - it0 + 1;
  const int nsteps = grp * ns;
  const float c = a.scale_log2;
  auto load_step = [&](QTile<T, D>& t, int j) {
    const int g = j / ns;
    const size_t qh = qhead(g);
    t.load(reinterpret_cast<const T*>(a.q) + qh * D, reinterpret_cast<const T*>(a.dout) + qh * D,
           a.lse + qh, a.dsum + qh, (it0 + j - g * ns) * S::BM, N, tid);
  };

  f32x16 dkt[S::NDT], dvt[S::NDT];
#pragma unroll
  for (int dt = 0; dt < S::NDT; ++dt) {
    dkt[dt] = f32x16{};
    dvt[dt] = f32x16{};
  }

  QTile<T, D> qt;
  load_step(qt, 0);
  qt.store(lds, tid);
  __syncthreads();

  for (int j = 0; j < nsteps; ++j) {
    const char* stage = lds + (j & 1) * S::STAGE;
    const int g = j / ns;
    const int q0 = (it0 + j - g * ns) * S::BM;
    if (j + 1 < nsteps) load_step(qt, j + 1);

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
    const bool need_mask =
        !block_all_visible(q0, q0 + S::BM - 1, kw0, kw0 + 31, N, CAUSAL, a.wl, a.wr);
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
            if (!key_visible(key, qrow, N, CAUSAL, a.wl, a.wr)) p = 0.f;
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
      float* dst = a.dq_acc + qhead(g) * D + dblk * 32 + col;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qrow = q0 + qb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (qrow < N) unsafeAtomicAdd(dst + (size_t)qrow * D, acc[r]);
      }
    }

    if (j + 1 < nsteps) qt.store(lds + ((j + 1) & 1) * S::STAGE, tid);
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

// ---------------------------------------------------------------------------
// 16-bit (bf16, fp16) kernels: shared tile layout.
//
// Q and dO (dK/dV kernel) and K and V (dQ kernel) tiles are stored
// row-major with their 16-byte units XOR-swizzled by row (tile_off). The
// swizzle makes both access patterns free of bank conflicts: 16-byte row
// reads (A operands of the score products) and transposing 8-byte reads
// (ds_read_b64_tr_b16, the transposed A operands of the gradient products).

constexpr int kStepQ = 64;  // query rows per inner step of the dK/dV kernel

// XOR swizzle of the 16-byte units of a tile row (ROWB bytes per row, 256 or
// 128), for LDS's 64 four-byte banks (one 256-byte bank line per cycle).
// Conflict-free for 16 lanes reading 16 bytes from 16 consecutive rows (a
// bijection on row mod 16, or on row pair mod 8, over the units of a bank
// line), and for the transposing 8-byte reads, which the LDS serves 32 lanes
// at a time: those lanes read 4 consecutive 4-aligned rows x 64 bytes, and
// the swizzle puts the four rows' 4-unit groups on disjoint banks. (A swizzle
// that separated only 16-lane groups left 2-way conflicts there, measured as
// about a fifth of the backward kernels' LDS-busy cycles.)
template <int ROWB>
__device__ constexpr int row_swz(int row) {
  if constexpr (ROWB == 256) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    const int m = row >> 1;  // two 128-byte rows share a bank line
    return ((m & 1) << 2) | ((m >> 1) & 3);
  }
}

// Byte offset of `byte` (within its row) of row `row` in a swizzled tile.
template <int ROWB>
__device__ constexpr int tile_off(int row, int byte) {
  return row * ROWB + (((byte >> 4) ^ row_swz<ROWB>(row)) << 4) + (byte & 15);
}

// Transposed 16-bit MFMA operand from a swizzled row-major tile: lane
// (c = lane & 31, h = lane >> 5) receives column col0 + c of 8 rows, as
// the K elements of a 32x32x16 operand. NATURAL: rows row0 + 8h + 0..7;
// otherwise the order in which a 32x32 C tile's registers hand rows to the
// next product: row0 + 4h + 0..3, then row0 + 8 + 4h + 0..3.
template <int ROWB, bool NATURAL>
__device__ inline u32x4 tr_operand(const char* tile, int row0, int col0, int lane) {
  const int g = lane >> 4, r = (lane >> 2) & 3, q = lane & 3, h = g >> 1;
  const int col = col0 + 16 * (g & 1) + 4 * q;
  const int ra = NATURAL ? row0 + 8 * h + r : row0 + 4 * h + r;
  const int rb = NATURAL ? ra + 4 : ra + 8;
  const u32x2 lo = lds_read_tr16(tile + tile_off<ROWB>(ra, col * 2));
  const u32x2 hi = lds_read_tr16(tile + tile_off<ROWB>(rb, col * 2));
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// ---------------------------------------------------------------------------
// 16-bit dK/dV kernel with 8 waves: keys outer (128 keys per workgroup),
// query steps of 64 rows inner. Each 32-key slice of the workgroup's keys is
// shared by the two waves of one SIMD, split by role:
//   role A (waves 0-3): S = Q K^T, P = exp2(S*scale*log2e - LSE*log2e) and
//                       dV^T += dO^T P; holds K and dV^T in registers;
//   role B (waves 4-7): dP = dO V^T, dS = P * (dP - D) and dK^T += Q^T dS;
//                       holds V and dK^T.
// P goes from A to B through LDS (bf16, lane-private slots). Each wave runs
// a matrix phase then a vector phase per step, each ending at a barrier,
// with role B one phase behind role A, so that on every SIMD one role's
// MFMAs overlap the other role's vector work (the ping-pong of the forward
// kernel). Q/dO/LSE/D stages live in three LDS buffers.

constexpr int kKVThreads = 512;

template <int D>
struct KVShape {
  static constexpr int ROWB = D * 2;
  static constexpr int TILE = kStepQ * ROWB;          // Q or dO of one step
  static constexpr int NSTAGE = 3;
  // Tensor-major regions, so that a step's stage adds at most 2 * TILE to a
  // region base (within the 16-bit offset of LDS instructions).
  static constexpr int REG_Q = 0;                     // Q tiles of the stages
  static constexpr int REG_DO = NSTAGE * TILE;        // dO tiles
  static constexpr int REG_LSE = 2 * NSTAGE * TILE;   // LSE * log2(e), float32
  static constexpr int REG_DSUM = REG_LSE + NSTAGE * kStepQ * 4;
  static constexpr int OFF_PX = REG_DSUM + NSTAGE * kStepQ * 4;  // P exchange: 4 slices x 4 KB
  static constexpr int LDS = OFF_PX + 4 * 4096;
  // Block-sparse: the list of query blocks and the compaction scratch.
  static constexpr int OFF_TL = LDS;
  static constexpr int LDS_SPARSE = OFF_TL + 2 * kMaxMaskBlocks + 4 * 8;
  static constexpr int UNITS = D / 8;
  static constexpr int NLD = kStepQ * UNITS / 256;    // loads per thread (one tensor, one role)
  static constexpr int NQK = D / 16;
  static constexpr int NDT = D / 32;
  static constexpr int NP = kStepQ / 16;              // P / dS operands per step
  static_assert(NLD * 256 == kStepQ * UNITS, "even split");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <int K>
struct IntC {
  static constexpr int value = K;
};

// One role's whole program. The role and, inside the main loop, the stage
// buffer of each step are compile-time constants, so every LDS address is a
// loop-invariant per-lane base plus an immediate offset: with a runtime
// stage index the matrix phase re-added the stage and role offsets to each
// of its address registers (about as many VALU instructions as MFMAs).
template <typename T, int D, bool CAUSAL, bool SPARSE, bool ROLE_A>
__device__ __forceinline__ void kv16_role(const BwdArgs& a, char* lds, int bid, int nblk) {
  using S = KVShape<D>;
  using E = Elem<T>;
  using Raw = u32x4;
  constexpr int ROWB = S::ROWB;
  constexpr bool roleA = ROLE_A;

  const int N = a.N;
  const int nkt = (N + kBN - 1) / kBN;
  const int parts = a.kv_parts;  // workgroups sharing one key tile's query heads
  const int lin = CAUSAL ? xcd_remap_ranked(bid, nblk, nkt * parts, parts) : xcd_remap(bid, nblk);
  const int bkv = lin / (nkt * parts);  // batch * Hkv + K/V head
  const int k0 = lin % (nkt * parts) / parts * kBN;
  const int part = lin % parts;
  const int grp = a.H / a.Hkv / parts;  // query heads of this workgroup
  // The first of them: the K/V head's group starts at query head
  // b*H + kvh*(H/Hkv); this part takes the grp heads after part*grp.
  const int bq0 = (bkv / a.Hkv) * a.H + (bkv % a.Hkv) * (a.H / a.Hkv) + part * grp;

  const size_t kvhead = (size_t)bkv * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const HeadBuf K(reinterpret_cast<const T*>(a.k) + kvhead, head_bytes);
  const HeadBuf V(reinterpret_cast<const T*>(a.v) + kvhead, head_bytes);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slice = wave & 3;       // the 32-key slice this wave serves
  const int col = lane & 31, half = lane >> 5;
  const int kw0 = k0 + slice * 32;  // first key of the slice
  const int key = kw0 + col;        // the key this lane serves in S and dP

  // K (role A) or V (role B) rows of the slice as B operands over the head
  // dim (rows past N read as zeros): lane half h holds elements
  // [h*D/2 + 8i, +8) for MFMA i.
  Raw kvb[S::NQK];
  {
    const HeadBuf& X = roleA ? K : V;
#pragma unroll
    for (int i = 0; i < S::NQK; ++i) kvb[i] = X.ld16((key * D + half * (D / 2) + i * 8) * 2);
  }
  // Byte offsets of the 16-byte A-operand reads of a Q or dO tile: row
  // `col` (plus 32 per query block), unit h*D/16 + i.
  int aoff[S::NQK];
#pragma unroll
  for (int i = 0; i < S::NQK; ++i) aoff[i] = tile_off<ROWB>(col, (half * (D / 2) + 8 * i) * 2);

  // Query steps [it0, it0 + ns) hold every row that sees a key of the tile;
  // step j covers query head j / ns, step it0 + j % ns. Block-sparse: the
  // steps are the query blocks of that range that keep one of the
  // workgroup's two 64-key blocks (an LDS list, entries flagging which); a
  // wave whose key block a step's block drops hides all its scores there.
  const int it0 = first_query_seeing(k0, CAUSAL, a.wr) / kStepQ;
  int ns = last_query_seeing(min(k0 + kBN, N) - 1, N, a.wl) / kStepQ - it0 + 1;
  const uint16_t* qlist = nullptr;
  if constexpr (SPARSE) {
    uint16_t* sl = reinterpret_cast<uint16_t*>(lds + S::OFF_TL);
    int* sw = reinterpret_cast<int*>(lds + S::OFF_TL + 2 * kMaxMaskBlocks);
    const int kb0 = k0 / kMaskBlock;
    const int nxb = min(kBN / kMaskBlock, a.nmb - kb0);
    ns = compact_blocks<kKVThreads, 2>(a.block_mask, (long long)it0 * a.nmb + kb0, a.nmb, 1, nxb,
                                       ns, sl, sw);
    qlist = sl;
  }
  const int nsteps = grp * ns;
  auto step_q0 = [&](int j) -> int {
    if constexpr (SPARSE) return (it0 + (__builtin_amdgcn_readfirstlane(qlist[j % ns]) >> 2)) * kStepQ;
    return (it0 + j % ns) * kStepQ;
  };
  auto kept = [&](int j) -> bool {
    if constexpr (SPARSE) return (__builtin_amdgcn_readfirstlane(qlist[j % ns]) >> (slice >> 1)) & 1;
    return true;
  };
  const float c = a.scale_log2;

  f32x16 acc[S::NDT];  // role A: dV^T, role B: dK^T (rows = head dim, lane = key)
#pragma unroll
  for (int dt = 0; dt < S::NDT; ++dt) acc[dt] = f32x16{};
  f32x16 sc[2];        // role A: S of the step's two 32-query blocks; role B: dP
  sc[0] = sc[1] = f32x16{};
  Raw pf[S::NP];       // role A: P^T operands; role B: dS^T operands
#pragma unroll
  for (int p = 0; p < S::NP; ++p) pf[p] = Raw{0u, 0u, 0u, 0u};

  // Stage staging, split by role: role A streams Q and LSE, role B dO and
  // D (each 256 threads; rows past N read as zeros, LSE = +inf there so
  // their probabilities are exactly 0).
  // Region offsets of this role: the tile it reads row-wise (and stages),
  // the tile it reads transposed, and its row statistics. Kept opaque so
  // that the compiler adds them into the loop-invariant per-lane base
  // addresses and leaves only stage and operand offsets for the immediates.
  int ts_off = roleA ? S::REG_Q : S::REG_DO;
  int ta_off = roleA ? S::REG_DO : S::REG_Q;
  int stat_off = roleA ? S::REG_LSE : S::REG_DSUM;
  asm volatile("" : "+s"(ts_off), "+s"(ta_off), "+s"(stat_off));
  const int rtid = tid & 255;
  u32x4 sx[S::NLD];
  // The row statistic as loaded (clamped row), and whether the row is real.
  // The scaling and the past-N select happen at the store, in the vector
  // phase: applied at the load they made the loading wave wait for the
  // global load inside its matrix phase.
  float stat = 0.f;
  bool stat_ok = false;
  auto load = [&](int j) {
    const int q0 = step_q0(j);
    const size_t qh = (size_t)(bq0 + j / ns) * N;  // query head of the step
    const HeadBuf X(reinterpret_cast<const T*>(roleA ? a.q : a.dout) + qh * D, head_bytes);
#pragma unroll
    for (int i = 0; i < S::NLD; ++i) {
      const int idx = rtid + 256 * i, row = idx / S::UNITS, u = idx % S::UNITS;
      sx[i] = X.ld16(((q0 + row) * D + u * 8) * 2);
    }
    if (rtid < kStepQ) {
      const int row = q0 + rtid;
      stat = (roleA ? a.lse : a.dsum)[qh + min(row, N - 1)];
      stat_ok = row < N;
    }
  };
  auto store = [&](auto kc) {  // into stage buffer kc
    char* stage = lds + ts_off + decltype(kc)::value * S::TILE;
#pragma unroll
    for (int i = 0; i < S::NLD; ++i) {
      const int idx = rtid + 256 * i, row = idx / S::UNITS, u = idx % S::UNITS;
      st<u32x4>(stage + tile_off<ROWB>(row, u * 16), sx[i]);
    }
    if (rtid < kStepQ)
      // (A row whose LSE is -inf -- it sees no key -- gets +inf: P = 0.)
      st<float>(lds + stat_off + decltype(kc)::value * (kStepQ * 4) + rtid * 4,
                roleA ? (stat_ok && (!SPARSE || stat > -INFINITY) ? stat * kLog2e : INFINITY) : (stat_ok ? stat : 0.f));
  };
  auto stats_at = [&](auto kc) -> const char* { return lds + stat_off + decltype(kc)::value * (kStepQ * 4); };
  char* const px = lds + S::OFF_PX + slice * 4096 + lane * 16;  // this lane's P slots

  // Matrix phase of either role: first dV^T += dO^T P (role A) or
  // dK^T += Q^T dS (role B) for step ja, with the transposed A operands read
  // from that step's tile; then S (role A, from Q) or dP (role B, from dO)
  // for step js (lane = key, registers = query rows of block qb). The MFMAs
  // run in chunks of four; the LDS operands of chunk c + 1 are read while
  // chunk c computes. Chunk c < NDT is head-dim block c of the accumulation,
  // chunk NDT + 2 qb + h is query block qb, head-dim operands 4h .. 4h + 3.
  auto mphase = [&](auto ka, auto ks, auto acc_c, auto sc_c) {
    constexpr int QKH = S::NQK / 4;
    constexpr int NC = S::NDT + 2 * QKH;
    const char* ta = lds + ta_off + decltype(ka)::value * S::TILE;
    const char* ts = lds + ts_off + decltype(ks)::value * S::TILE;
    constexpr int c0 = decltype(acc_c)::value ? 0 : S::NDT;
    constexpr int c1 = decltype(sc_c)::value ? NC : S::NDT;
    Raw op[2][4];
    auto fetch = [&](int cc, Raw(&dst)[4]) {
      if (cc < S::NDT) {
#pragma unroll
        for (int p = 0; p < 4; ++p) dst[p] = tr_operand<ROWB, false>(ta, 16 * p, 32 * cc, lane);
      } else {
        const int qb = (cc - S::NDT) / QKH, h = (cc - S::NDT) % QKH;
#pragma unroll
        for (int u = 0; u < 4; ++u) dst[u] = ld<Raw>(ts + aoff[4 * h + u] + 32 * qb * ROWB);
      }
    };
    auto compute = [&](int cc, const Raw(&src)[4]) {
      if (cc < S::NDT) {
#pragma unroll
        for (int p = 0; p < 4; ++p) acc[cc] = E::mma(src[p], pf[p], acc[cc]);
      } else {
        const int qb = (cc - S::NDT) / QKH, h = (cc - S::NDT) % QKH;
        f32x16 x = h == 0 ? f32x16{} : sc[qb];
#pragma unroll
        for (int u = 0; u < 4; ++u) x = E::mma(src[u], kvb[4 * h + u], x);
        sc[qb] = x;
      }
    };
    static_assert(S::NP == 4 && S::NQK % 4 == 0, "chunks of four MFMAs");
    __builtin_amdgcn_s_setprio(1);
    fetch(c0, op[0]);
#pragma unroll
    for (int cc = c0; cc < c1; ++cc) {
      if (cc + 1 < c1) fetch(cc + 1, op[(cc - c0 + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      compute(cc, op[(cc - c0) & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // Role A, step j: P from S (hidden scores -> probability 0), packed as
  // P^T operands (operand p = 2*qb + u covers registers [8u, 8u+8) of block
  // qb: queries 16p + 4h + 0..3 and 16p + 8 + 4h + 0..3), also stored to the
  // lane's slots for role B.
  auto probabilities = [&](int j, auto kc) {
    const char* lse2 = stats_at(kc);
    const int q0 = step_q0(j);
    const bool keep = kept(j);
    const bool need_mask =
        !block_all_visible(q0, q0 + kStepQ - 1, kw0, kw0 + 31, N, CAUSAL, a.wl, a.wr);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if (SPARSE && !keep) {
        sc[qb] = f32x16{} - INFINITY;
      } else if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qrow = q0 + 32 * qb + 8 * (r >> 2) + 4 * half + (r & 3);
          if (!key_visible(key, qrow, N, CAUSAL, a.wl, a.wr)) sc[qb][r] = -INFINITY;
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int ql = 32 * qb + 16 * u + 8 * k + 4 * half;  // first of 4 query rows
          const f32x4 l2 = ld<f32x4>(lse2 + ql * 4);
          float pe[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) pe[e] = __builtin_amdgcn_exp2f(fmaf(sc[qb][8 * u + 4 * k + e], c, -l2[e]));
          w[2 * k] = E::pack_pair(pe[0], pe[1]);
          w[2 * k + 1] = E::pack_pair(pe[2], pe[3]);
        }
        pf[2 * qb + u] = Raw{w[0], w[1], w[2], w[3]};
        st<Raw>(px + (2 * qb + u) * 1024, pf[2 * qb + u]);
      }
    }
  };
  // Role B, step j: dS = P * (dP - D) with P read back from role A's slots,
  // packed as dS^T operands (the same operand layout).
  auto score_grads = [&](auto kc) {
    const char* dsum = stats_at(kc);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const Raw pw = ld<Raw>(px + (2 * qb + u) * 1024);
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int ql = 32 * qb + 16 * u + 8 * k + 4 * half;
          const f32x4 dd = ld<f32x4>(dsum + ql * 4);
          float pe[4], de[4];
          E::unpack_pair(pw[2 * k], pe[0], pe[1]);
          E::unpack_pair(pw[2 * k + 1], pe[2], pe[3]);
#pragma unroll
          for (int e = 0; e < 4; ++e) de[e] = pe[e] * (sc[qb][8 * u + 4 * k + e] - dd[e]);
          w[2 * k] = E::pack_pair(de[0], de[1]);
          w[2 * k + 1] = E::pack_pair(de[2], de[3]);
        }
        pf[2 * qb + u] = Raw{w[0], w[1], w[2], w[3]};
      }
    // Computed here, in the vector phase: otherwise the compiler sinks this
    // work past the barrier to its first use, the next matrix phase, where
    // it delays the MFMAs (about 110 VALU instructions per step).
#pragma unroll
    for (int p = 0; p < S::NP; ++p) settle(pf[p]);
  };

  auto epilogue = [&]() {
    // Epilogue: lane = key, registers = head-dim rows of dV^T (A) / dK^T (B).
    // With several parts per key tile, float32 partials go to the scratch
    // ([part][B*Hkv][N][d], dK then dV) for bwd_kvsum to add up.
    if (key >= N) return;
    const float sc_out = roleA ? 1.f : a.scale;
    if (parts > 1) {
      const size_t plane = (size_t)a.B * a.Hkv * N * D;
      float* prow = a.dkv_part + (roleA ? (size_t)parts * plane : 0) + part * plane + kvhead + (size_t)key * D;
#pragma unroll
      for (int dt = 0; dt < S::NDT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& v = acc[dt];
          st<f32x4>(prow + dt * 32 + 8 * g + 4 * half,
                    f32x4{v[4 * g] * sc_out, v[4 * g + 1] * sc_out, v[4 * g + 2] * sc_out, v[4 * g + 3] * sc_out});
        }
      return;
    }
    T* row_p = reinterpret_cast<T*>(roleA ? a.dv : a.dk) + kvhead + (size_t)key * D;
#pragma unroll
    for (int dt = 0; dt < S::NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = dt * 32 + 8 * g + 4 * half;
        const f32x16& v = acc[dt];
        st<u32x2>(row_p + d0, u32x2{E::bits(v[4 * g] * sc_out) | ((uint32_t)E::bits(v[4 * g + 1] * sc_out) << 16),
                                    E::bits(v[4 * g + 2] * sc_out) | ((uint32_t)E::bits(v[4 * g + 3] * sc_out) << 16)});
      }

  };
  if (SPARSE && nsteps == 0) {  // no query block keeps these keys: dK = dV = 0
    epilogue();
    return;
  }

  // Prologue: stages 0 and 1 in LDS.
  load(0);
  store(IntC<0>{});
  if (nsteps > 1) {
    load(1);
    store(IntC<1>{});
  }
#pragma unroll
  for (int i = 0; i < S::NQK; ++i) settle(kvb[i]);
  __syncthreads();

  // Step j of a wave is its matrix phase M(j) then its vector phase V(j),
  // each ending at a barrier; role B runs one phase behind role A (one extra
  // barrier first, A one extra at the end), so one role's MFMAs overlap the
  // other's vector work:
  //   A: M(j) = dV of step j-1, S of step j;   V(j) = P of step j (to LDS);
  //   B: M(j) = dK of step j-1, dP of step j;  V(j) = dS of step j (P from LDS).
  // Stage j is read from A's M(j) to B's M(j+1). Role A loads Q/LSE of stage
  // j+1 in M(j) and stores them in V(j); role B loads dO/D of stage j+2 in
  // M(j) and stores them in V(j). Stage j lives in buffer j % 3; each store
  // lands in a buffer whose last readers passed an earlier barrier.
  constexpr int ahead = roleA ? 1 : 2;
  auto vphase = [&](int j, auto kc) {
    if constexpr (roleA)
      probabilities(j, kc);
    else
      score_grads(kc);
  };
  if (!roleA) __syncthreads();
  {
    if (roleA ? false : 2 < nsteps) load(2);
    mphase(IntC<0>{}, IntC<0>{}, BoolC<false>{}, BoolC<true>{});
    __syncthreads();
    vphase(0, IntC<0>{});
    if (!roleA && 2 < nsteps) store(IntC<2>{});
    __syncthreads();
  }
  // Step j (stage buffer kc = j % 3).
  auto step = [&](int j, auto kc) {
    constexpr int K = decltype(kc)::value;
    const int ls = j + ahead;
    if (ls < nsteps) load(ls);
    mphase(IntC<(K + 2) % 3>{}, kc, BoolC<true>{}, BoolC<true>{});
    __syncthreads();
    vphase(j, kc);
    if (ls < nsteps) store(IntC<(K + ahead) % 3>{});
    __syncthreads();
  };
  // Unrolled by the three stage buffers, straight-line, so that loop-carried
  // registers need no copies where differently compiled steps would meet.
  static_assert(S::NSTAGE == 3, "three stage buffers");
  int j = 1;
  for (; j + 2 < nsteps; j += 3) {
    step(j, IntC<1>{});
    step(j + 1, IntC<2>{});
    step(j + 2, IntC<0>{});
  }
  if (j < nsteps) step(j++, IntC<1>{});
  if (j < nsteps) step(j++, IntC<2>{});
  {
    const int k = (nsteps - 1) % 3;
    if (k == 0)
      mphase(IntC<0>{}, IntC<0>{}, BoolC<true>{}, BoolC<false>{});
    else if (k == 1)
      mphase(IntC<1>{}, IntC<0>{}, BoolC<true>{}, BoolC<false>{});
    else
      mphase(IntC<2>{}, IntC<0>{}, BoolC<true>{}, BoolC<false>{});
  }
  __syncthreads();
  if (roleA) __syncthreads();

  epilogue();
}

// Workgroup `bid` of `nblk` of the dK/dV grid (the XCD of bid is bid % 8).
template <typename T, int D, bool CAUSAL, bool SPARSE>
__device__ __forceinline__ void kv16_body(const BwdArgs& a, char* lds, int bid, int nblk) {
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < 4)
    kv16_role<T, D, CAUSAL, SPARSE, true>(a, lds, bid, nblk);
  else
    kv16_role<T, D, CAUSAL, SPARSE, false>(a, lds, bid, nblk);
}

template <typename T, int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(kKVThreads, 1) void bwd_kv16_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[SPARSE ? KVShape<D>::LDS_SPARSE : KVShape<D>::LDS];
  kv16_body<T, D, CAUSAL, SPARSE>(a, lds, blockIdx.x, gridDim.x);
}

// dK, dV = the sum of the parts' float32 partials (in part order, so the
// result does not depend on scheduling), rounded to T. 4 elements per
// thread; the first half of the grid does dK, the second dV.
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_kvsum_kernel(BwdArgs a, long long n4) {
  const long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= 2 * n4) return;
  const bool is_v = i >= n4;
  const long long e = (is_v ? i - n4 : i) * 4;
  const size_t plane = (size_t)n4 * 4;
  const float* src = a.dkv_part + (is_v ? (size_t)a.kv_parts * plane : 0) + e;
  f32x4 s = ld<f32x4>(src);
  for (int p = 1; p < a.kv_parts; ++p) {
    const f32x4 x = ld<f32x4>(src + p * plane);
    s = f32x4{s[0] + x[0], s[1] + x[1], s[2] + x[2], s[3] + x[3]};
  }
  const uint32_t w0 = Elem<T>::bits(s[0]) | ((uint32_t)Elem<T>::bits(s[1]) << 16);
  const uint32_t w1 = Elem<T>::bits(s[2]) | ((uint32_t)Elem<T>::bits(s[3]) << 16);
  st<u32x2>(reinterpret_cast<T*>(is_v ? a.dv : a.dk) + e, u32x2{w0, w1});
}

// ---------------------------------------------------------------------------
// 16-bit dQ kernel: query tiles outer, key tiles inner (the forward's
// decomposition), so dQ accumulates in registers and is written once, with
// no atomics. Per 32-key tile it recomputes S^T = K Q^T and dP^T = V dO^T,
// forms dS = P * (dP - D) with P = exp2(S*scale*log2e - LSE*log2e), and
// adds dQ^T += K^T dS^T (K^T read transposed from the same K tile).
//
// A workgroup has 8 waves covering 256 query rows of one head. As in the
// forward kernel, the waves form two groups of four (one wave of each group
// per SIMD) and alternate a matrix phase (MFMAs) and a vector phase (dS),
// one barrier per phase, group B one phase behind group A. K and V tiles of
// 32 keys use the swizzled row layout of the key-outer kernel (conflict-free
// for both 16-byte row reads and transposing reads). K tile i is read in the
// matrix phases of steps i (S) and i + 1 (dQ), so K has three buffers (and
// V three as well, so that both use buffer i % 3).
// Group A streams K (tile i + 1 loaded in its matrix phase i, stored in its
// vector phase i); group B streams V (tile i + 2 loaded in its matrix phase
// i, stored in its vector phase i, which comes before the matrix phase i + 1
// of group A).

constexpr int kDQThreads = 512;
constexpr int kDQGroup = 256;  // threads per wave group
constexpr int kDQBM = 256;     // query rows per workgroup
constexpr int kDQBN = 32;      // keys per tile

template <int D>
struct DQShape {
  static constexpr int ROWB = D * 2;
  static constexpr int TILE = kDQBN * ROWB;
  // Three buffers each, so that the buffer of step i (i % 3) is the same for
  // K and V and the main loop can be compiled per buffer.
  static constexpr int NKBUF = 3, NVBUF = 3;
  static constexpr int LDS = (NKBUF + NVBUF) * TILE;
  static constexpr int NQK = D / 16;                     // MFMAs over the head dim
  static constexpr int NDT = D / 32;                     // head-dim blocks of dQ
  static constexpr int UNITS = D / 8;                    // 16-byte units per row
  static constexpr int NLD = kDQBN * UNITS / kDQGroup;   // loads per thread per tile
  static_assert(NLD * kDQGroup == kDQBN * UNITS, "even split");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  // Block-sparse: the list of key blocks and the compaction scratch.
  static constexpr int OFF_TL = LDS;
  static constexpr int LDS_SPARSE = OFF_TL + 2 * kMaxMaskBlocks + 4 * 8;
};

// Workgroup `bid` of `nblk` of the dQ grid (the XCD of bid is bid % 8).
template <typename T, int D, bool CAUSAL, bool SPARSE>
__device__ __forceinline__ void dq16_body(const BwdArgs& a, char* lds, int bid, int nblk) {
  using S = DQShape<D>;
  using E = Elem<T>;
  using Raw = u32x4;
  constexpr int ROWB = S::ROWB;
  static_assert(kMaskBlock == 2 * kDQBN && kDQBM == 4 * kMaskBlock, "mask blocks of two key tiles");

  char* const kbuf = lds;
  char* const vbuf = lds + S::NKBUF * S::TILE;

  const int N = a.N;
  const int nqt = (N + kDQBM - 1) / kDQBM;
  const int lin = CAUSAL ? xcd_remap_ranked(bid, nblk, nqt, 1) : xcd_remap(bid, nblk);
  const int bh = lin / nqt;
  const int qtile = CAUSAL ? nqt - 1 - lin % nqt : lin % nqt;
  const int q0 = qtile * kDQBM;

  const size_t qhead = (size_t)bh * N;
  // Query head h reads K/V head h / (H / Hkv).
  const size_t kvhead = (size_t)((bh / a.H) * a.Hkv + (bh % a.H) / (a.H / a.Hkv)) * N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const HeadBuf Q(reinterpret_cast<const T*>(a.q) + qhead * D, head_bytes);
  const HeadBuf G(reinterpret_cast<const T*>(a.dout) + qhead * D, head_bytes);
  const HeadBuf K(reinterpret_cast<const T*>(a.k) + kvhead, head_bytes);
  const HeadBuf V(reinterpret_cast<const T*>(a.v) + kvhead, head_bytes);
  T* dQ = reinterpret_cast<T*>(a.dq) + qhead * D;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;  // 0: A, 1: B (one phase behind)
  const int gtid = tid & (kDQGroup - 1);
  const int col = lane & 31, half = lane >> 5;
  const int qw0 = q0 + wave * 32;  // first query row of this wave
  const int qrow = qw0 + col;      // the query row this lane serves

  // Key tiles t0 .. t0+nkv-1 hold a key some of the workgroup's rows see;
  // this wave's rows see tiles [w_lo, w_end) of them (none if past N).
  const int qlast = min(q0 + kDQBM, N) - 1;
  const int t0 = first_visible_key(q0, a.wl) / kDQBN;
  int nkv = last_visible_key(qlast, N, CAUSAL, a.wr) / kDQBN - t0 + 1;
  // Block-sparse: the tiles are those of the key blocks in that range that
  // one of the workgroup's four 64-row query blocks keeps (an LDS list,
  // entries flagging which); every wave takes all of them, and a wave whose
  // block drops a tile's block hides all its scores there.
  const uint16_t* klist = nullptr;
  const int b0 = t0 / 2;
  if constexpr (SPARSE) {
    uint16_t* sl = reinterpret_cast<uint16_t*>(lds + S::OFF_TL);
    int* sw = reinterpret_cast<int*>(lds + S::OFF_TL + 2 * kMaxMaskBlocks);
    const int qb0 = q0 / kMaskBlock;
    const int nb = (t0 + nkv - 1) / 2 - b0 + 1;
    nkv = 2 * compact_blocks<kDQThreads, 4>(a.block_mask, (long long)qb0 * a.nmb + b0, 1, a.nmb,
                                            min(kDQBM / kMaskBlock, a.nmb - qb0), nb, sl, sw);
    klist = sl;
  }
  // Key tile of step i, and whether this wave's query block keeps it.
  auto ktile = [&](int i) -> int {
    if constexpr (SPARSE) return 2 * (b0 + (__builtin_amdgcn_readfirstlane(klist[i >> 1]) >> 4)) + (i & 1);
    return t0 + i;
  };
  auto kept = [&](int i) -> bool {
    if constexpr (SPARSE) return (__builtin_amdgcn_readfirstlane(klist[i >> 1]) >> (wave >> 1)) & 1;
    return true;
  };
  int w_lo = nkv + 1, w_end = -1;
  if (qw0 < N) {
    if (SPARSE) {
      w_lo = 0;
      w_end = nkv;
    } else {
      w_lo = first_visible_key(qw0, a.wl) / kDQBN - t0;
      w_end = last_visible_key(min(qw0 + 31, N - 1), N, CAUSAL, a.wr) / kDQBN - t0 + 1;
    }
  }

  // This row's LSE (log2 units) and D; rows past N get LSE = +inf, so their
  // probabilities (and dS) are exactly 0 (as do rows that see no key, whose
  // LSE is -inf).
  const float lr = qrow < N && (!SPARSE || a.lse[qhead + qrow] > -INFINITY) ? a.lse[qhead + qrow] * kLog2e : INFINITY;
  const float dr = qrow < N ? a.dsum[qhead + qrow] : 0.f;
  // -D in every register of this lane's column: the dP^T products start
  // from it, so the accumulator holds dP - D and dS = P * (dP - D) takes
  // one multiply per score.
  const f32x16 negd = f32x16{} - dr;

  // Q^T and dO^T as MFMA B operands: lane half h holds head-dim elements
  // [h*D/2, h*D/2 + D/2) of its row, 8 per MFMA.
  Raw qf[S::NQK], gf[S::NQK];
#pragma unroll
  for (int i = 0; i < S::NQK; ++i) {
    const int off = (qrow * D + half * (D / 2) + i * 8) * 2;
    qf[i] = Q.ld16(off);
    gf[i] = G.ld16(off);
  }
  // This lane's 16-byte A-operand reads of a K or V tile: row `col` (+32
  // for the second key block), elements half*D/2 + 8i, i.e. 16-byte unit
  // half*D/16 + i of the row, XOR-swizzled by the row (mod 16, so the same
  // for both key blocks).
  const int arow = col * ROWB;
  const int aswz = row_swz<ROWB>(col);
  auto aoff = [&](int i) { return arow + (((half * (D / 16) + i) ^ aswz) << 4); };

  const float c = a.scale_log2;
  f32x16 dq[S::NDT];
#pragma unroll
  for (int dt = 0; dt < S::NDT; ++dt) dq[dt] = f32x16{};
  // Scores of the current tile, then its dS packed as the two dS^T B
  // operands into words 0-7 of s (operand k in words [4k, 4k+4)); dP
  // alongside.
  f32x16 s = f32x16{}, dp = f32x16{};

  // Matrix phase: dQ^T += K^T dS^T for the previous tile (DQ, from the
  // packed words of s), then S^T = K Q^T and dP^T = V dO^T for the current
  // one (SP). The MFMAs run in chunks of four; the LDS operands of chunk
  // c + 1 are read while chunk c computes. DQ chunk cc covers head-dim
  // blocks 2cc and 2cc + 1 (two operands each); SP chunk j covers product
  // j / QKH (0: S from K, 1: dP from V) and head-dim operands 4h .. 4h + 3
  // with h = j % QKH.
  auto mphase = [&](const char* kprev, const char* kcur, const char* vcur, auto dq_c, auto sp_c) {
    constexpr bool DQ = decltype(dq_c)::value, SP = decltype(sp_c)::value;
    constexpr int QKH = S::NQK / 4;  // chunks per product
    constexpr int NDQC = DQ ? S::NDT / 2 : 0;
    constexpr int NC = NDQC + (SP ? 2 * QKH : 0);
    const f32x16 x = s;
    const Raw dsf[2] = {__builtin_bit_cast(Raw, __builtin_shufflevector(x, x, 0, 1, 2, 3)),
                        __builtin_bit_cast(Raw, __builtin_shufflevector(x, x, 4, 5, 6, 7))};
    Raw op[2][4];
    auto fetch = [&](int cc, Raw(&dst)[4]) {
      if (cc < NDQC) {
#pragma unroll
        for (int u = 0; u < 4; ++u) dst[u] = tr_operand<ROWB, false>(kprev, 16 * (u & 1), 32 * (2 * cc + (u >> 1)), lane);
      } else {
        const int j = cc - NDQC, pr = j / QKH, h = j % QKH;
        const char* tp = pr == 0 ? kcur : vcur;
#pragma unroll
        for (int u = 0; u < 4; ++u) dst[u] = ld<Raw>(tp + aoff(4 * h + u));
      }
    };
    auto compute = [&](int cc, const Raw(&src)[4]) {
      if (cc < NDQC) {
#pragma unroll
        for (int u = 0; u < 4; ++u) dq[2 * cc + (u >> 1)] = E::mma(src[u], dsf[u & 1], dq[2 * cc + (u >> 1)]);
      } else {
        const int j = cc - NDQC, pr = j / QKH, h = j % QKH;
        f32x16& acc = pr == 0 ? s : dp;
        if (h == 0) acc = pr == 0 ? f32x16{} : negd;
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = E::mma(src[u], pr == 0 ? qf[4 * h + u] : gf[4 * h + u], acc);
      }
    };
    __builtin_amdgcn_s_setprio(1);
    fetch(0, op[0]);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      if (cc + 1 < NC) fetch(cc + 1, op[(cc + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      compute(cc, op[cc & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Vector phase: dS = P * (dP - D) for the current tile (dp already holds
  // dP - D), packed into s
  // (word w of operand u pairs registers 8u + 2w, 8u + 2w + 1; every word is
  // written after the scores it overwrites were read). Hidden keys get
  // S = -inf, so P = 0 and dS = 0.
  auto vphase = [&](int k0, bool keep) {
    if (SPARSE && !keep) {
      s = f32x16{} - INFINITY;
    } else if (!block_all_visible(qw0, qw0 + 31, k0, k0 + kDQBN - 1, N, CAUSAL, a.wl, a.wr)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (!key_visible(key, qrow, N, CAUSAL, a.wl, a.wr)) s[r] = -INFINITY;
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float d[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[8 * u + e], c, -lr));
        d[e] = p * dp[8 * u + e];
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) s[4 * u + w] = __builtin_bit_cast(float, E::pack_pair(d[2 * w], d[2 * w + 1]));
    }
  };

  // Global -> LDS staging of one group's tile (rows past N read as zeros).
  u32x4 stg[S::NLD];
  auto gload = [&](const HeadBuf& X, int tile) {
#pragma unroll
    for (int j = 0; j < S::NLD; ++j) {
      const int idx = gtid + kDQGroup * j, row = idx / S::UNITS, u = idx % S::UNITS;
      stg[j] = X.ld16((ktile(tile) * kDQBN * D + row * D + u * 8) * 2);
    }
  };
  auto lstore = [&](char* tile) {
#pragma unroll
    for (int j = 0; j < S::NLD; ++j) {
      const int idx = gtid + kDQGroup * j, row = idx / S::UNITS, u = idx % S::UNITS;
      st<u32x4>(tile + tile_off<ROWB>(row, u * 16), stg[j]);
    }
  };
  auto kt = [&](int i) -> char* { return kbuf + (i % S::NKBUF) * S::TILE; };
  auto vt = [&](int i) -> char* { return vbuf + (i % S::NVBUF) * S::TILE; };
  // The same with the buffer a compile-time constant.
  auto kts = [&](auto bc) -> char* { return kbuf + decltype(bc)::value * S::TILE; };
  auto vts = [&](auto bc) -> char* { return vbuf + decltype(bc)::value * S::TILE; };

  // Epilogue: dQ = scale * accumulator; lane = query row, registers =
  // head-dim rows of dQ^T.
  auto epilogue = [&]() {
    if (w_end <= 0 && !SPARSE) return;
    if (qrow >= N) return;
    T* qrow_p = dQ + (size_t)qrow * D;
    const float sc = a.scale;
#pragma unroll
    for (int dt = 0; dt < S::NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = dt * 32 + 8 * g + 4 * half;
        const f32x16& v = dq[dt];
        st<u32x2>(qrow_p + d0, u32x2{E::bits(v[4 * g] * sc) | ((uint32_t)E::bits(v[4 * g + 1] * sc) << 16),
                                     E::bits(v[4 * g + 2] * sc) | ((uint32_t)E::bits(v[4 * g + 3] * sc) << 16)});
      }
  };
  if (SPARSE && nkv == 0) {  // no key block is kept: dQ = 0
    epilogue();
    return;
  }

  // Prologue: K tile 0 (group A), V tiles 0 and 1 (group B).
  const bool kgrp = group == 0;  // group A streams K, group B V
  gload(kgrp ? K : V, 0);
  lstore(kgrp ? kt(0) : vt(0));
  if (!kgrp && nkv > 1) {
    gload(V, 1);
    lstore(vt(1));
  }
#pragma unroll
  for (int i = 0; i < S::NQK; ++i) {
    settle(qf[i]);
    settle(gf[i]);
  }
  __syncthreads();

  // Step i is a matrix phase M(i) (dQ of tile i-1; S and dP of tile i) then
  // a vector phase V(i) (dS of tile i), each ending at a barrier; group B
  // runs one phase behind group A (one extra barrier first, A one extra at
  // the end). Group A loads K tile i + 1 in M(i) and stores it in V(i);
  // group B loads V tile i + 2 in M(i) and stores it in V(i). K tile j and
  // V tile j live in buffer j % 3; each store lands in a buffer whose last
  // readers passed an earlier barrier. At step w_lo (> 0) the dQ half adds
  // the zero initial dS; at step w_end (< nkv) the S, dP half is unused.
  const HeadBuf& X = kgrp ? K : V;
  if (!kgrp) __syncthreads();
  {
    const int lt = kgrp ? 1 : 2;
    if (lt < nkv) gload(X, lt);
    if (w_lo == 0 && w_end > 0) mphase(kt(0), kt(0), vt(0), BoolC<false>{}, BoolC<true>{});
    __syncthreads();
    if (w_lo == 0 && w_end > 0) vphase(ktile(0) * kDQBN, kept(0));
    if (lt < nkv) lstore(kgrp ? kt(lt) : vt(lt));
    __syncthreads();
  }
  // Step i with its buffer b = i % 3 a compile-time constant, so that every
  // LDS operand address is a loop-invariant base plus an immediate offset
  // (with a runtime buffer index each matrix phase re-added the buffer
  // offsets to every operand address).
  auto step = [&](int i, auto bc) {
    constexpr int b = decltype(bc)::value;
    const int lt = kgrp ? i + 1 : i + 2;
    if (lt < nkv) gload(X, lt);
    if (w_lo <= i && i <= w_end)
      mphase(kts(IntC<(b + 2) % 3>{}), kts(bc), vts(bc), BoolC<true>{}, BoolC<true>{});
    __syncthreads();
    if (w_lo <= i && i < w_end) vphase(ktile(i) * kDQBN, kept(i));
    if (lt < nkv) lstore(kgrp ? kts(IntC<(b + 1) % 3>{}) : vts(IntC<(b + 2) % 3>{}));
    __syncthreads();
  };
  // Unrolled by the three buffers, straight-line (no register copies where
  // differently compiled steps would meet).
  int i = 1;
  for (; i + 2 < nkv; i += 3) {
    step(i, IntC<1>{});
    step(i + 1, IntC<2>{});
    step(i + 2, IntC<0>{});
  }
  if (i < nkv) step(i++, IntC<1>{});
  if (i < nkv) step(i++, IntC<2>{});
  // Final matrix phase: dQ of the last tile.
  if (w_end == nkv) {
    const int b = (nkv - 1) % 3;
    if (b == 0)
      mphase(kts(IntC<0>{}), kts(IntC<0>{}), vts(IntC<0>{}), BoolC<true>{}, BoolC<false>{});
    else if (b == 1)
      mphase(kts(IntC<1>{}), kts(IntC<1>{}), vts(IntC<0>{}), BoolC<true>{}, BoolC<false>{});
    else
      mphase(kts(IntC<2>{}), kts(IntC<2>{}), vts(IntC<0>{}), BoolC<true>{}, BoolC<false>{});
  }
  __syncthreads();
  if (kgrp) __syncthreads();
  epilogue();
}

template <typename T, int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(kDQThreads, 1) void bwd_dq16_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[SPARSE ? DQShape<D>::LDS_SPARSE : DQShape<D>::LDS];
  dq16_body<T, D, CAUSAL, SPARSE>(a, lds, blockIdx.x, gridDim.x);
}

// The dK/dV and dQ grids in one launch: workgroups [0, n_dq) are the dQ
// grid, [kv0, kv0 + n_kv) the dK/dV grid (kv0 = n_dq rounded up to a
// multiple of 8, so that both keep the XCD of each of their workgroups;
// the workgroups in between return at once). The two kernels read the same
// inputs and write disjoint outputs, so running them side by side changes
// no result. What it gains: when one grid ends in a partial round -- the
// causal dQ grid of a short sequence is a single round whose longest
// workgroup sees every key tile and whose shortest only those up to its own
// rows -- the other grid's workgroups fill the compute units that would
// otherwise idle.
template <int D, bool SPARSE>
constexpr int fused_lds() {
  constexpr int kv = SPARSE ? KVShape<D>::LDS_SPARSE : KVShape<D>::LDS;
  constexpr int dq = SPARSE ? DQShape<D>::LDS_SPARSE : DQShape<D>::LDS;
  return kv > dq ? kv : dq;
}

// Grids of at most this many workgroups (four rounds of one per compute
// unit) are launched fused; larger ones run the two kernels one after the
// other, where the fused launch measured the same.
constexpr long long kFuseMaxWorkgroups = 4 * kCUs;

template <typename T, int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(kKVThreads, 1) void bwd_fused16_kernel(BwdArgs a, int n_dq, int kv0,
                                                                   int n_kv) {
  static_assert(kKVThreads == kDQThreads, "one workgroup size");
  __shared__ __attribute__((aligned(16))) char lds[fused_lds<D, SPARSE>()];
  const int b = blockIdx.x;
  if (b < n_dq)
    dq16_body<T, D, CAUSAL, SPARSE>(a, lds, b, n_dq);
  else if (b >= kv0)
    kv16_body<T, D, CAUSAL, SPARSE>(a, lds, b - kv0, n_kv);
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
    if constexpr (sizeof(T) == 4) {  // 16-bit types write dQ without an accumulator
      float* z = a.dq_acc + off;
#pragma unroll
      for (int e = 0; e < EPV; e += 4) st<f32x4>(z + e, f32x4{0.f, 0.f, 0.f, 0.f});
    }
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
  // Grouped K/V heads with few K/V heads: split each group's query heads
  // over up to grp workgroups per key tile until the grid covers the
  // compute units (16-bit types; the parts' dK/dV are summed afterwards).
  const int nkt = (a.N + kBN - 1) / kBN;
  if constexpr (sizeof(T) == 2) {
    const int grp = a.H / a.Hkv;
    int parts = 1;
    while (parts * 2 <= grp && grp % (parts * 2) == 0 &&
           (long long)a.B * a.Hkv * nkt * parts < kCUs)
      parts *= 2;
    args.kv_parts = parts;
  }
  if constexpr (sizeof(T) == 2) {
    const int nqt = (a.N + kDQBM - 1) / kDQBM;
    int n_dq = (int)((long long)a.B * a.H * nqt);
    int kv0 = (n_dq + 7) / 8 * 8;
    int n_kv = (int)((long long)a.B * a.Hkv * nkt * args.kv_parts);
    const bool causal = a.causal, sparse = a.block_mask != nullptr;
    hipError_t e;
    if ((long long)kv0 + n_kv <= kFuseMaxWorkgroups) {
      // Short grids: dQ and dK/dV in one launch (bwd_fused16_kernel).
      void* kargs[] = {&args, &n_dq, &kv0, &n_kv};
      const void* fn =
          sparse ? (causal ? reinterpret_cast<const void*>(&bwd_fused16_kernel<T, D, true, true>)
                           : reinterpret_cast<const void*>(&bwd_fused16_kernel<T, D, false, true>))
                 : (causal ? reinterpret_cast<const void*>(&bwd_fused16_kernel<T, D, true, false>)
                           : reinterpret_cast<const void*>(&bwd_fused16_kernel<T, D, false, false>));
      e = hipLaunchKernel(fn, dim3((unsigned)((long long)kv0 + n_kv)), dim3(kKVThreads), kargs, 0,
                          stream);
    } else {
      // dK/dV grid, then the dQ grid (after the part sums, when there are
      // parts; both orders give the same results).
      void* kargs[] = {&args};
      const void* fn =
          sparse ? (causal ? reinterpret_cast<const void*>(&bwd_kv16_kernel<T, D, true, true>)
                           : reinterpret_cast<const void*>(&bwd_kv16_kernel<T, D, false, true>))
                 : (causal ? reinterpret_cast<const void*>(&bwd_kv16_kernel<T, D, true, false>)
                           : reinterpret_cast<const void*>(&bwd_kv16_kernel<T, D, false, false>));
      e = hipLaunchKernel(fn, dim3((unsigned)n_kv), dim3(kKVThreads), kargs, 0, stream);
      if (e != hipSuccess) return e;
      fn = sparse ? (causal ? reinterpret_cast<const void*>(&bwd_dq16_kernel<T, D, true, true>)
                            : reinterpret_cast<const void*>(&bwd_dq16_kernel<T, D, false, true>))
                  : (causal ? reinterpret_cast<const void*>(&bwd_dq16_kernel<T, D, true, false>)
                            : reinterpret_cast<const void*>(&bwd_dq16_kernel<T, D, false, false>));
      e = hipLaunchKernel(fn, dim3((unsigned)n_dq), dim3(kDQThreads), kargs, 0, stream);
    }
    if (e != hipSuccess || args.kv_parts == 1) return e;
    long long n4 = (long long)a.B * a.Hkv * a.N * D / 4;
    void* sargs[] = {&args, &n4};
    const dim3 grid((unsigned)((2 * n4 + kThreads - 1) / kThreads));
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_kvsum_kernel<T>), grid,
                           dim3(kThreads), sargs, 0, stream);
  } else {
    {
      void* kargs[] = {&args};
      const dim3 grid((unsigned)((long long)a.B * a.Hkv * nkt));
      const void* fn = a.causal ? reinterpret_cast<const void*>(&bwd_main_kernel<T, D, true>)
                                : reinterpret_cast<const void*>(&bwd_main_kernel<T, D, false>);
      hipError_t e = hipLaunchKernel(fn, grid, dim3(kThreads), kargs, 0, stream);
      if (e != hipSuccess) return e;
    }
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

// The library's own scratch for fa_bwd_noalloc (callers that cannot
// allocate): a file-scope device array, one copy per GPU, held until the
// process ends. Host code never passes its name to a kernel (in host code
// the name is a host-side stand-in); it passes the device address that
// hipGetSymbolAddress returns for the current GPU.
static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;

}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  switch (a.dtype) {
    case 0: return dispatch_d<float>(a, stream);
    case 1: return dispatch_d<_Float16>(a, stream);
    default: return dispatch_d<__bf16>(a, stream);
  }
}

}  // namespace fa
