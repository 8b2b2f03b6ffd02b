// Eight consecutive elements of a row in 16-byte accesses (one for bf16, two
// for fp32), as fp32 values; the address must be aligned to 8 elements.
#pragma once
#include "common.h"

namespace hy {

typedef __bf16 bf16v8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void ld8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void ld8(const bf16* p, float (&v)[8]) {
  const bf16v8 a = *reinterpret_cast<const bf16v8*>(p);
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = (float)a[k];
}
__device__ __forceinline__ void st8(float* p, const float (&v)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void st8(bf16* p, const float (&v)[8]) {
  bf16v8 a;
#pragma unroll
  for (int k = 0; k < 8; ++k) a[k] = (bf16)v[k];
  *reinterpret_cast<bf16v8*>(p) = a;
}

}  // namespace hy
