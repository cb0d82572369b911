// Seeded, counter-based synthetic input generator (device side).
//
// Implements, for the GPU, the same definition as gen.py in this directory:
// SplitMix64 output function as a counter-based hash, Irwin-Hall(12) normals
// from 16-bit fields, 24-bit uniforms, fp32 -> bf16 and fp32 -> E4M3FN
// round-to-nearest-even.  Test and bench infrastructure only; it holds none of
// the sparse-attention arithmetic.  Built with -ffp-contract=off so no fused
// multiply-add changes a rounding.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t draw(uint64_t key, uint64_t c) {
  return mix64(key + (c + 1ull) * 0x9E3779B97F4A7C15ull);
}

__device__ __forceinline__ float normal_f32(uint64_t key, uint64_t i) {
  int64_t s = 0;
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    uint64_t h = draw(key, i * 3ull + (uint64_t)r);
#pragma unroll
    for (int f = 0; f < 4; ++f) s += (int64_t)((h >> (16 * f)) & 0xFFFFull);
  }
  return (float)(s - 393210) * (1.0f / 65536.0f);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint8_t f32_to_e4m3_bits(float x) {
  uint32_t u = __float_as_uint(x);
  uint8_t sign = (uint8_t)((u >> 31) << 7);
  uint32_t a = u & 0x7FFFFFFFu;
  uint32_t exp32 = a >> 23;
  uint32_t code;
  if (exp32 < 121u) {
    float q = __uint_as_float(a) * 512.0f;
    // round to nearest even via the 2^23 magic number (IEEE adds, not folded
    // without fast-math)
    float r = (q + 8388608.0f) - 8388608.0f;
    code = (uint32_t)r;
  } else {
    int e = (int)exp32 - 127;
    uint32_t m23 = a & 0x7FFFFFu;
    uint32_t keep = m23 >> 20, rem = m23 & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) keep += 1;
    if (keep == 8u) { keep = 0; e += 1; }
    code = ((uint32_t)(e + 7) << 3) | keep;
    if (a >= 0x43E80000u || code > 0x7Eu) code = 0x7Eu;
  }
  return (uint8_t)(code | sign);
}

enum Recipe : int32_t {
  E4M3_NORMAL = 0,
  E4M3_INT = 1,
  F32_UNIFORM = 2,
  F32_POW2Q = 3,
  BF16_NORMAL = 4,
};

__global__ void fill_kernel(void* out, int64_t rows, int32_t dim, const int64_t* rowmap,
                            int32_t recipe, uint64_t key, float div, int32_t lo, int32_t hi) {
  int64_t n = rows * (int64_t)dim;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = e / dim, c = e - r * dim;
    int64_t lr = rowmap ? rowmap[r] : r;
    uint64_t i = (uint64_t)(lr * dim + c);
    switch (recipe) {
      case E4M3_NORMAL:
        ((uint8_t*)out)[e] = f32_to_e4m3_bits(normal_f32(key, i));
        break;
      case E4M3_INT: {
        uint64_t h = draw(key, i);
        int64_t v = (int64_t)(h % (uint64_t)(hi - lo + 1)) + lo;
        ((uint8_t*)out)[e] = f32_to_e4m3_bits((float)v);
        break;
      }
      case F32_UNIFORM:
        ((float*)out)[e] = (float)(draw(key, i) >> 40) * (1.0f / 16777216.0f);
        break;
      case F32_POW2Q: {
        int ex = (int)(draw(key, i) & 3ull) - 2;
        ((float*)out)[e] = ldexpf(1.0f, ex);
        break;
      }
      case BF16_NORMAL: {
        float x = normal_f32(key, i);
        if (div != 1.0f) x = __fdiv_rn(x, div);
        ((uint16_t*)out)[e] = f32_to_bf16_bits(x);
        break;
      }
      default:
        break;
    }
  }
}

uint64_t host_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace

extern "C" {

// Fills out[r, c] (r < rows, c < dim) with the recipe's value of logical
// element (rowmap ? rowmap[r] : r) * dim + c of stream `stream`.
// Returns 0 on success, otherwise the hipError_t of the launch.
int dsagen_fill(void* out, int64_t rows, int32_t dim, const int64_t* rowmap, int32_t recipe,
                uint64_t seed, uint32_t stream, float div, int32_t lo, int32_t hi, void* hip_stream) {
  if (rows <= 0 || dim <= 0) return 0;
  uint64_t key = host_mix64((seed << 32) ^ (uint64_t)stream);
  int64_t n = rows * (int64_t)dim;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536 * 8) blocks = 65536 * 8;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)hip_stream, out,
                     rows, dim, rowmap, recipe, key, div, lo, hi);
  return (int)hipGetLastError();
}

}
