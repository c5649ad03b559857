// fp8_mfma_probe.hip -- test-only measurement of how the gfx950 FP8 matrix
// instruction (v_mfma_f32_32x32x64_f8f6f4, E4M3 x E4M3, float32 result)
// accumulates its 64 products. Not part of libfa.so: the FP8 parity test
// bounds the kernels' score error with a constant derived from this
// measurement, and tests/test_hw_fp8_mfma.py checks the constant against
// it on the GPU.
//
// One wave per tile t. Operands are byte matrices, E4M3 codes:
//   a [t][32 rows][64 k], b [t][32 cols][64 k]   (both k-contiguous)
//   c [t][32 rows][32 cols] float32 = a[t] * b[t]^T from one instruction
// with a zero accumulator input. Lane l supplies row/column (l & 31) and
// k-bytes [32 h, 32 h + 32) with h = l >> 5 for both operands; the result
// register r of lane l is row 8 (r >> 2) + 4 h + (r & 3), column (l & 31).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

__global__ __launch_bounds__(64) void fp8_mfma_probe_kernel(const uint8_t* a, const uint8_t* b,
                                                             float* c) {
  const int t = blockIdx.x, l = threadIdx.x, row = l & 31, h = l >> 5;
  const size_t off = (size_t)t * 2048 + row * 64 + 32 * h;
  const i32x4 a0 = *reinterpret_cast<const i32x4*>(a + off);
  const i32x4 a1 = *reinterpret_cast<const i32x4*>(a + off + 16);
  const i32x4 b0 = *reinterpret_cast<const i32x4*>(b + off);
  const i32x4 b1 = *reinterpret_cast<const i32x4*>(b + off + 16);
  const i32x8 av = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
  const i32x8 bv = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
  const f32x16 r = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, f32x16{}, 0, 0, 0, 0,
                                                                    0, 0);
  float* ct = c + (size_t)t * 1024;
#pragma unroll
  for (int i = 0; i < 16; ++i) ct[(8 * (i >> 2) + 4 * h + (i & 3)) * 32 + row] = r[i];
}

// a, b: n_tiles * 2048 bytes each; c: n_tiles * 1024 floats (device
// pointers, 16-byte aligned). Returns 0, or -1 for bad arguments, or the
// HIP error code of the launch.
extern "C" int fa_probe_fp8_mfma(const void* a, const void* b, float* c, int n_tiles,
                                 void* stream) {
  if (!a || !b || !c || n_tiles < 1 || n_tiles > (1 << 20)) return -1;
  if (((uintptr_t)a | (uintptr_t)b | (uintptr_t)c) & 15) return -1;
  hipLaunchKernelGGL(fp8_mfma_probe_kernel, dim3(n_tiles), dim3(64), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const uint8_t*>(a),
                     static_cast<const uint8_t*>(b), c);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}
