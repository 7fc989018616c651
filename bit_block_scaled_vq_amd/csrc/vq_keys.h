// Device helpers shared by the GEMM and sampling kernels: the monotone 64-bit
// candidate key of a logit.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vq {

// Monotone 64-bit argmax key: (orderable fp32 << 32) | (~index). Larger key =
// larger value, and on equal values the lower index. NaN -> 0 (never wins);
// -0 is treated as +0. 0 also means "no candidate".
__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t idx) {
  if (v != v) return 0ull;
  if (v == 0.0f) v = 0.0f;
  uint32_t u = __float_as_uint(v);
  uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)k << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ float key_value(unsigned long long key) {
  uint32_t k = (uint32_t)(key >> 32);
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return key ? __uint_as_float(u) : __builtin_nanf("");
}
// Token id carried by a non-zero key.
__device__ __forceinline__ int key_index(unsigned long long key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

}  // namespace vq
