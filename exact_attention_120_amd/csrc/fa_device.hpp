// fa_device.hpp -- gfx950 (CDNA4) device helpers shared by the attention
// kernels: vector types, matrix-core (MFMA) operand traits per element type,
// packing of float32 probabilities into MFMA operands, the workgroup-to-XCD
// remap, and raw LDS/global vector accesses.
//
// MFMA operand conventions used throughout (wave64, 32x32 output tiles):
//   A (32 x K)  : lane l holds row (l & 31), K-elements [h*KH, h*KH + KH)
//                 with h = l >> 5;
//   B (K x 32)  : lane l holds column (l & 31), the same K-elements;
//   C (32 x 32) : lane l, register r holds column (l & 31) and row
//                 8*(r >> 2) + 4*h + (r & 3).
// Only the pairing of A and B matters for the contraction, so any mapping of
// the K index onto data is legal as long as both operands use it; the
// kernels exploit that freedom to keep every operand a contiguous read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;

// Element traits. KH = operand elements one lane contributes to one MFMA
// (half of the instruction's K depth); Raw = those elements as bits.
template <typename T>
struct Elem;

template <>
struct Elem<__bf16> {
  static constexpr int KH = 8;
  using Raw = u32x4;
  __device__ static inline f32x16 mma(Raw a, Raw b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // Round 8 floats to bf16 (nearest-even), pack them as one operand, and add
  // the 8 *unrounded* values to acc: bf16's 2^-9 relative rounding would not
  // average out in rows that see only a few keys, so the normalizer is kept
  // in float32. Each pair is converted once (one v_cvt_pk_bf16_f32) and kept
  // as its own 32-bit word: extracting pairs back out of a packed 8-element
  // vector mis-compiles (every pair read as the first one).
  __device__ static inline Raw pack_sum(const float* p, float& acc) {
    Raw r;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const bf16x2 pr = {(__bf16)p[2 * w], (__bf16)p[2 * w + 1]};
      acc += p[2 * w] + p[2 * w + 1];
      r[w] = __builtin_bit_cast(uint32_t, pr);
    }
    return r;
  }
  // One pair of pack_sum: the packed word of (a, b); acc += a + b.
  __device__ static inline uint32_t pack2(float a, float b, float& acc) {
    const bf16x2 pr = {(__bf16)a, (__bf16)b};
    acc += a + b;
    return __builtin_bit_cast(uint32_t, pr);
  }
  // The packed word of (a, b) alone.
  __device__ static inline uint32_t pack_pair(float a, float b) {
    const bf16x2 pr = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, pr);
  }
  // The two values of a packed word (exact).
  __device__ static inline void unpack_pair(uint32_t w, float& a, float& b) {
    a = __builtin_bit_cast(float, w << 16);
    b = __builtin_bit_cast(float, w & 0xffff0000u);
  }
  __device__ static inline uint16_t bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  }
};

template <>
struct Elem<_Float16> {
  static constexpr int KH = 8;
  using Raw = u32x4;
  __device__ static inline f32x16 mma(Raw a, Raw b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // As for bf16, but the sum is taken over the rounded values with one
  // dot product per pair: fp16 keeps 11 significant bits, so the rounded
  // normalizer is accurate to 2^-12 relative, and it costs half the adds.
  __device__ static inline Raw pack_sum(const float* p, float& acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    Raw r;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f16x2 pr = {(_Float16)p[2 * w], (_Float16)p[2 * w + 1]};
      acc = __builtin_amdgcn_fdot2(pr, one, acc, false);
      r[w] = __builtin_bit_cast(uint32_t, pr);
    }
    return r;
  }
  __device__ static inline uint32_t pack2(float a, float b, float& acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    const f16x2 pr = {(_Float16)a, (_Float16)b};
    acc = __builtin_amdgcn_fdot2(pr, one, acc, false);
    return __builtin_bit_cast(uint32_t, pr);
  }
  __device__ static inline uint32_t pack_pair(float a, float b) {
    const f16x2 pr = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, pr);
  }
  __device__ static inline void unpack_pair(uint32_t w, float& a, float& b) {
    const f16x2 pr = __builtin_bit_cast(f16x2, w);
    a = (float)pr[0];
    b = (float)pr[1];
  }
  __device__ static inline uint16_t bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
};

template <>
struct Elem<float> {
  static constexpr int KH = 1;
  using Raw = uint32_t;
  __device__ static inline f32x16 mma(Raw a, Raw b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(float, a),
                                               __builtin_bit_cast(float, b), c, 0, 0, 0);
  }
  __device__ static inline Raw pack_sum(const float* p, float& acc) {
    acc += p[0];
    return __builtin_bit_cast(Raw, p[0]);
  }
};

// Raw loads/stores of KH elements (16 bytes for 16-bit types, 4 for f32).
template <typename Raw>
__device__ inline Raw ld(const void* p) {
  return *reinterpret_cast<const Raw*>(p);
}
template <typename Raw>
__device__ inline void st(void* p, Raw x) {
  *reinterpret_cast<Raw*>(p) = x;
}

// When a 32x32 C tile (scores, or score gradients) becomes the B operand of
// the next product, register r of lane half h holds row 8*(r>>2) + 4*h + (r&3)
// of each 32-row block, and MFMA number u takes registers [u*KH, u*KH+KH).
// vt_pos gives, for row `idx` of a tile, the position at which the matching
// A operand must store it (in a transposed LDS copy) so that both operands
// walk the contraction in the same order and every A read is contiguous.
template <int KH>
__device__ constexpr int vt_pos(int idx) {
  const int blk = idx >> 5, kb = idx & 31;
  const int h = (kb >> 2) & 1;
  const int r = 4 * (kb >> 3) + (kb & 3);
  return blk * 32 + (r / KH) * (2 * KH) + h * KH + (r % KH);
}

// Raw buffer access to one head's [N, D] slab: loads at byte offsets at or
// past `bytes` return zeros (the hardware range check), so tail rows need
// no branches. The descriptor lives in scalar registers (uniform base).
struct HeadBuf {
  __amdgpu_buffer_rsrc_t r;
  __device__ HeadBuf(const void* base, uint32_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000)) {}
  __device__ inline u32x4 ld16(int byte_off) const {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
  }
  // Per-lane offset plus a wave-uniform one (kept in a scalar register).
  __device__ inline u32x4 ld16(int byte_off, int uniform_off) const {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, uniform_off, 0);
  }
  __device__ inline uint32_t ld4(int byte_off) const {
    return __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0);
  }
};

// Transposing LDS read (ds_read_b64_tr_b16, gfx950). Within each group of 16
// lanes, output lane i receives, as its element r (r = 0..3), element (i % 4)
// of the 8-byte chunk addressed by lane 4*r + i/4 of the group. So when lane
// 4*r + q addresses row R_r, columns [c + 4q, c + 4q + 4) of a row-major
// 16-bit tile, lane i ends up holding column c + i of rows R_0..R_3: a
// column-major (transposed) operand read straight from a row-major tile.
__device__ inline u32x2 lds_read_tr16(const void* p) {
  typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// max(x, x of lane ^ 32) in every lane, without LDS: permlane32_swap with
// both operands x leaves [x_lo, x_lo] in the first result and [x_hi, x_hi]
// in the second.
__device__ inline float max_with_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                  __builtin_bit_cast(uint32_t, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

// An empty asm statement that reads `x`: the compiler must complete any load
// into `x` before this point. Used after a kernel's prologue so that no load
// is still pending when its main loop starts; otherwise the wait-count
// insertion, which merges loop-entry and back-edge states, waits on that
// load inside every iteration, and thereby also on the next tile's
// prefetch loads issued after it.
template <typename X>
__device__ inline void settle(const X& x) {
  asm volatile("" ::"v"(x));
}

__device__ inline bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// Visibility of keys to queries: the causal rule (key <= query) and a local
// window (query - wl <= key <= query + wr; a negative bound is unbounded),
// plus keys past the sequence end.
__device__ inline bool key_visible(int key, int q, int N, bool causal, int wl, int wr) {
  return key < N && (!causal || key <= q) && (wr < 0 || key <= q + wr) && (wl < 0 || key >= q - wl);
}

// First and last key (inclusive, within [0, N)) visible to any of the query
// rows r0..r1 (r0 <= r1 < N).
__device__ inline int first_visible_key(int r0, int wl) { return wl >= 0 ? max(0, r0 - wl) : 0; }
__device__ inline int last_visible_key(int r1, int N, bool causal, int wr) {
  int hi = N - 1;
  if (causal) hi = min(hi, r1);
  if (wr >= 0) hi = min(hi, r1 + wr);
  return hi;
}

// Every key k0..k1 visible to every query r0..r1 (no masking needed).
__device__ inline bool block_all_visible(int r0, int r1, int k0, int k1, int N, bool causal,
                                         int wl, int wr) {
  return k1 < N && (!causal || k1 <= r0) && (wr < 0 || k1 <= r0 + wr) && (wl < 0 || k0 >= r1 - wl);
}

// The query rows that see at least one key of k0..k1 (k0 <= k1 < N) form the
// range [first_query_seeing(k0), last_query_seeing(k1)]: key j is visible
// from query i iff i >= j - r (r = 0 if causal, else window_right when
// bounded) and i <= j + window_left (when bounded).
__device__ inline int first_query_seeing(int k0, bool causal, int wr) {
  const int r = causal ? 0 : wr;
  return r >= 0 ? max(0, k0 - r) : 0;
}
__device__ inline int last_query_seeing(int k1, int N, int wl) {
  return wl >= 0 ? min(N - 1, k1 + wl) : N - 1;
}

// MI355X: 8 XCDs (chiplets, each with its own L2) of 32 compute units.
constexpr int kXCDs = 8, kCUsPerXCD = 32;

// Workgroups are dispatched round-robin over the 8 XCDs (bid % 8). Remap so
// that consecutive logical tiles (the query tiles of one head, which read the
// same K/V) land on the same XCD and share its L2. A bijection on [0, total).
__device__ inline int xcd_remap(int bid, int total) {
  constexpr int X = kXCDs;
  const int per = total / X, rem = total % X;
  const int x = bid % X, idx = bid / X;
  return x * per + (x < rem ? x : rem) + idx;
}

// Causal grids: the work of a unit (a query tile in the forward and the dQ
// kernel, a key tile in the dK/dV kernel) falls with its rank r (r = 0 the
// longest), and a head has per_head = R * inner units, unit (r, i) at
// r * inner + i (i: a split slice or a grouped-head part, equal work). Where
// every XCD holds whole heads (total = 8 * hpx * per_head), each XCD takes
// its heads in groups of G and each group rank by rank across its heads
// (the group's rank-0 units first), so that the longest units start first
// and the short ones fill the end. G is the fewest heads (at least two)
// whose units cover an XCD's 32 compute units, rounded up to a divisor of
// hpx: enough for the balance, while few heads share the XCD's L2 at a time
// (measured: interleaving every head of the XCD lost up to 11% at N = 1024
// with 32 heads per XCD; one head at a time lost 1-4% at N = 8192-16384).
// Otherwise the plain remap. A bijection on [0, total) either way.
__device__ inline int xcd_remap_ranked(int bid, int total, int per_head, int inner) {
  constexpr int X = kXCDs;
  if (total % (X * per_head) != 0) return xcd_remap(bid, total);
  const int hpx = total / (X * per_head);  // heads per XCD
  int G = (kCUsPerXCD * inner + per_head - 1) / per_head;
  if (G < 2) G = 2;
  if (G >= hpx) G = hpx;
  while (hpx % G != 0) ++G;
  const int x = bid % X, idx = bid / X;
  const int grp = idx / (G * per_head), gi = idx % (G * per_head);
  const int rank = gi / (G * inner), rem = gi % (G * inner);
  const int hl = grp * G + rem / inner, in = rem % inner;
  return (x * hpx + hl) * per_head + rank * inner + in;
}

// Block-sparse tile lists. All threads of the workgroup (NT of them) call
// this together. For x = 0 .. n-1 it ORs the ny mask bytes
// mask[base + x*sx + y*sy] (y = 0 .. ny-1) into a bit field and, for every x
// with a nonzero field, appends (x << SHIFT) | field to list in increasing x.
// Returns the count (the same in every thread). wsum is LDS scratch of NT/64
// ints; list is LDS with room for n entries.
template <int NT, int SHIFT>
__device__ inline int compact_blocks(const uint8_t* mask, long long base, int sx, int sy, int ny,
                                     int n, uint16_t* list, int* wsum) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int total = 0;
  for (int c0 = 0; c0 < n; c0 += NT) {
    const int x = c0 + tid;
    int bits = 0;
    if (x < n)
      for (int y = 0; y < ny; ++y) bits |= (mask[base + (long long)x * sx + (long long)y * sy] != 0) << y;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(bits != 0);
    const int pre = __builtin_popcountll(bal & ((1ull << lane) - 1));
    if (lane == 0) wsum[wave] = __builtin_popcountll(bal);
    __syncthreads();
    int off = total, chunk = 0;
    for (int w = 0; w < NW; ++w) {
      if (w < wave) off += wsum[w];
      chunk += wsum[w];
    }
    if (bits != 0) list[off + pre] = (uint16_t)((x << SHIFT) | bits);
    total += chunk;
    __syncthreads();
  }
  return total;
}

}  // namespace fa
