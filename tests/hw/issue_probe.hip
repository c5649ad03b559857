// issue_probe.hip -- test-only measurement of instruction issue rates on one
// gfx950 compute unit: how fast one wave, or two waves sharing a SIMD, issue
// 32x32x16 bf16 MFMAs, float32 FMAs and exponentials, alone and side by
// side. Not part of libfa.so. It backs the issue-rate figures the kernel
// designs rest on (one wave issues vector instructions at about half a
// SIMD's rate; a second wave on the SIMD doubles it; vector work beside an
// MFMA stream slows that stream little).
//
// One workgroup of 4 or 8 waves on one compute unit; waves 0-3 run on four
// different SIMDs and wave w + 4 on the SIMD of wave w (the test checks
// this from the recorded SIMD ids), so with 8 waves each SIMD holds two.
// Each wave runs
// `iters` iterations of its role's loop and records the shader-clock cycles
// (s_memtime) between its start and end in cycles[w], and the SIMD it ran
// on (HW_REG_HW_ID bits 5:4) in cycles[n_waves + w]:
//   role 0: 8 MFMAs (v_mfma_f32_32x32x16_bf16, 4 independent accumulators)
//   role 1: 32 FMAs (v_fma_f32, 8 independent chains)
//   role 2: 16 exponentials (v_exp_f32, 8 independent chains)
//   role 3: idle (returns at once)
// roles[w] gives each wave's role. The loops' instructions are written in
// inline assembly (plain vector ALU work, no memory access) so that their
// count is exact; the MFMAs use the compiler's builtin.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

__global__ __launch_bounds__(512) void issue_probe_kernel(const int* roles, int iters,
                                                          long long* cycles, float* sink) {
  const int wave = threadIdx.x >> 6;
  const int role = roles[wave];
  const int hw_id = __builtin_amdgcn_s_getreg(4 | (0 << 6) | (31 << 11));  // hwreg(HW_ID)
  if ((threadIdx.x & 63) == 0) cycles[(blockDim.x >> 6) + wave] = (hw_id >> 4) & 3;
  if (role == 3) return;
  const float seed = (float)(threadIdx.x & 63) * 1e-3f;
  const long long t0 = __builtin_amdgcn_s_memtime();
  float keep = 0.f;
  if (role == 0) {
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) a[i] = b[i] = (__bf16)(seed + i);
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    keep = c0[0] + c1[1] + c2[2] + c3[3];
  } else {
    float x0 = seed, x1 = seed + 1, x2 = seed + 2, x3 = seed + 3;
    float x4 = seed + 4, x5 = seed + 5, x6 = seed + 6, x7 = seed + 7;
    const float m = 0.999f;
    for (int it = 0; it < iters; ++it) {
      if (role == 1) {
#define FA_FMA8                                                                      \
  "v_fma_f32 %0, %0, %8, %8\n\tv_fma_f32 %1, %1, %8, %8\n\tv_fma_f32 %2, %2, %8, %8\n\t" \
  "v_fma_f32 %3, %3, %8, %8\n\tv_fma_f32 %4, %4, %8, %8\n\tv_fma_f32 %5, %5, %8, %8\n\t" \
  "v_fma_f32 %6, %6, %8, %8\n\tv_fma_f32 %7, %7, %8, %8\n\t"
        asm volatile(FA_FMA8 FA_FMA8 FA_FMA8 FA_FMA8
                     : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3), "+v"(x4), "+v"(x5), "+v"(x6),
                       "+v"(x7)
                     : "v"(m));
#undef FA_FMA8
      } else {
#define FA_EXP8                                                                             \
  "v_exp_f32 %0, %0\n\tv_exp_f32 %1, %1\n\tv_exp_f32 %2, %2\n\tv_exp_f32 %3, %3\n\t" \
  "v_exp_f32 %4, %4\n\tv_exp_f32 %5, %5\n\tv_exp_f32 %6, %6\n\tv_exp_f32 %7, %7\n\t"
        asm volatile(FA_EXP8 FA_EXP8
                     : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3), "+v"(x4), "+v"(x5), "+v"(x6),
                       "+v"(x7));
#undef FA_EXP8
      }
    }
    keep = x0 + x1 + x2 + x3 + x4 + x5 + x6 + x7;
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  if ((threadIdx.x & 63) == 0) cycles[wave] = t1 - t0;
  sink[threadIdx.x] = keep;
}

// roles: n_waves ints (host), cycles: 2 * n_waves long longs (device), sink:
// 64 * n_waves floats (device). n_waves 4 or 8. Returns 0, -1 for bad
// arguments, or a HIP error code.
extern "C" int fa_probe_issue(const int* roles_host, int n_waves, int iters, long long* cycles,
                              float* sink, void* stream) {
  if (!roles_host || !cycles || !sink || (n_waves != 4 && n_waves != 8) || iters < 1 ||
      iters > (1 << 20))
    return -1;
  for (int w = 0; w < n_waves; ++w)
    if (roles_host[w] < 0 || roles_host[w] > 3) return -1;
  int* roles = nullptr;
  hipError_t e = hipMalloc(&roles, sizeof(int) * n_waves);
  if (e != hipSuccess) return (int)e;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  e = hipMemcpyAsync(roles, roles_host, sizeof(int) * n_waves, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(issue_probe_kernel, dim3(1), dim3(64 * n_waves), 0, s, roles, iters, cycles,
                       sink);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  (void)hipFree(roles);
  return e == hipSuccess ? 0 : (int)e;
}
