// Test-only kernels: one matrix-core instruction per wave on host-made
// tiles, so a test can compare the hardware's sums with exact ones.  Used to
// check the FP8 MFMA accumulation model that the fused prefill's error bound
// rests on (indexer.hip, FP8 scoring pass) and the f16 MFMA's sums.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// Tile i: A [16][128] and B^T [16][128] E4M3 bytes (row c of B^T is column c
// of B); D[i][r][c] = sum_k A[r][k] B[k][c] by one 16x16x128 FP8 MFMA.
__global__ __launch_bounds__(64) void fp8_tiles_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ bt,
                                                       float* __restrict__ d, int ntiles) {
  const int tile = blockIdx.x;
  if (tile >= ntiles) return;
  const int lane = threadIdx.x, row = lane & 15, grp = lane >> 4;
  const v8i av = *(const v8i*)(a + (size_t)tile * 2048 + row * 128 + 32 * grp);
  const v8i bv = *(const v8i*)(bt + (size_t)tile * 2048 + row * 128 + 32 * grp);
  const v4f acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127,
                                                                   0, 127);
  for (int i = 0; i < 4; ++i) d[(size_t)tile * 256 + (4 * grp + i) * 16 + row] = acc[i];
}

// Tile i: A [16][32] and B^T [16][32] f16; one 16x16x32 f16 MFMA.
__global__ __launch_bounds__(64) void f16_tiles_kernel(const _Float16* __restrict__ a, const _Float16* __restrict__ bt,
                                                       float* __restrict__ d, int ntiles) {
  const int tile = blockIdx.x;
  if (tile >= ntiles) return;
  const int lane = threadIdx.x, row = lane & 15, grp = lane >> 4;
  const v8h av = *(const v8h*)(a + (size_t)tile * 512 + row * 32 + 8 * grp);
  const v8h bv = *(const v8h*)(bt + (size_t)tile * 512 + row * 32 + 8 * grp);
  const v4f acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  for (int i = 0; i < 4; ++i) d[(size_t)tile * 256 + (4 * grp + i) * 16 + row] = acc[i];
}

extern "C" int mfma_probe_fp8(const void* a, const void* bt, void* d, int ntiles, void* stream) {
  if (ntiles <= 0) return 0;
  hipLaunchKernelGGL(fp8_tiles_kernel, dim3(ntiles), dim3(64), 0, (hipStream_t)stream, (const uint8_t*)a,
                     (const uint8_t*)bt, (float*)d, ntiles);
  return (int)hipGetLastError();
}

extern "C" int mfma_probe_f16(const void* a, const void* bt, void* d, int ntiles, void* stream) {
  if (ntiles <= 0) return 0;
  hipLaunchKernelGGL(f16_tiles_kernel, dim3(ntiles), dim3(64), 0, (hipStream_t)stream, (const _Float16*)a,
                     (const _Float16*)bt, (float*)d, ntiles);
  return (int)hipGetLastError();
}
