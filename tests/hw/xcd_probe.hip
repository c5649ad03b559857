// xcd_probe.hip -- test-only check of the workgroup-to-XCD assignment that
// the attention kernels' grid remaps assume (block b runs on XCD b mod 8 of
// the MI355X's 8 XCDs, each with its own L2). Not part of libfa.so.
//
// Each workgroup (512 threads, as the 16-bit attention kernels use) reads
// HW_REG_XCC_ID (bits 3:0: the XCD it runs on) and lane 0 writes it to
// out[blockIdx.x].
#include <hip/hip_runtime.h>
#include <stdint.h>

__global__ __launch_bounds__(512) void xcd_probe_kernel(int* out) {
  const int xcc = __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11));  // hwreg(XCC_ID, 0, 4)
  if (threadIdx.x == 0) out[blockIdx.x] = xcc;
}

// out: n_workgroups ints (device). Returns 0, -1 for bad arguments, or the
// HIP error code of the launch.
extern "C" int fa_probe_xcd_ids(int* out, int n_workgroups, void* stream) {
  if (!out || n_workgroups < 1 || n_workgroups > (1 << 20)) return -1;
  hipLaunchKernelGGL(xcd_probe_kernel, dim3(n_workgroups), dim3(512), 0,
                     reinterpret_cast<hipStream_t>(stream), out);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}
