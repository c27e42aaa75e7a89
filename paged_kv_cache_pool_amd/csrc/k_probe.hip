// Placement probe (diagnostic): records where the GPU dispatches the
// workgroups of launches shaped like the library's own.  The planners rely on
// placements that HIP does not promise and that affect only speed:
//  * the matrix-core decode kernel's paired form holds one wave per SIMD
//    (over 256 registers per lane), and its 4 x CUs one-wave workgroups are
//    sized to put exactly one wave on every SIMD;
//  * its two-wave form (eight one-wave workgroups per compute unit) assumes
//    workgroups u and u + 4 x CUs share a SIMD;
//  * the extend and shared-prefix passes assume workgroup b runs on XCD b % 8
//    (each (request, kv head) pinned to one XCD's L2).
// Each probe workgroup records its HW_ID and XCC_ID hardware registers, then
// stays resident for a fixed number of sleeps, so that the whole launch is
// resident at once, as the real launches are.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

// s_getreg operand: size - 1 in bits 15:11, offset 0, register id in 5:0
constexpr int kHwRegHwId = (31 << 11) | 4;
constexpr int kHwRegXccId = (31 << 11) | 20;
constexpr int kSleeps = 64;                      // about 0.2 ms resident

__device__ __forceinline__ void record(uint32_t *ids) {
  const uint32_t hw = __builtin_amdgcn_s_getreg(kHwRegHwId);
  const uint32_t xcc = __builtin_amdgcn_s_getreg(kHwRegXccId);
  if (threadIdx.x == 0) {
    ids[2 * blockIdx.x] = hw;
    ids[2 * blockIdx.x + 1] = xcc;
  }
}

// Bounded residency: a fixed number of sleeps, so every wave ends.
__device__ __forceinline__ void stay() {
  for (int i = 0; i < kSleeps; ++i) __builtin_amdgcn_s_sleep(127);
}

}  // namespace

// One-wave workgroups holding 256 VGPRs + 152 AGPRs (one wave per SIMD).
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_probe_one_wave(uint32_t *ids) {
  record(ids);
  asm volatile("" ::: "v255", "a151");
  stay();
}

// One-wave workgroups holding 218 VGPRs (two waves per SIMD).
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_probe_two_wave(uint32_t *ids) {
  record(ids);
  asm volatile("" ::: "v217");
  stay();
}

// 512-thread workgroups holding 160 KB of LDS (one per compute unit).
__global__ __launch_bounds__(512) void k_probe_wide(uint32_t *ids) {
  extern __shared__ uint32_t lds[];
  record(ids);
  if (threadIdx.x == 0) lds[0] = 0;
  asm volatile("" ::: "v209");                 // the extend kernels' 210 VGPRs
  stay();
}

hipError_t launch_placement_probe(int cus, uint32_t *one_ids, uint32_t *two_ids, uint32_t *wide_ids,
                                  hipStream_t s) {
  constexpr int kLds = 160 * 1024;
  hipError_t e = hipFuncSetAttribute((const void *)k_probe_wide, hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_probe_one_wave, dim3(4 * cus), dim3(64), 0, s, one_ids);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_probe_two_wave, dim3(8 * cus), dim3(64), 0, s, two_ids);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_probe_wide, dim3(2 * cus), dim3(512), kLds, s, wide_ids);
  return hipGetLastError();
}

}  // namespace pa
