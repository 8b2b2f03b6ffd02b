// Elementwise parts of the 1D backward pass in the four-step regime
// (2L >= 16384). The long convolutions themselves run on the forward's
// four-step passes: with R the time reversal t -> L - 1 - t on [0, L), the
// transpose of the convolution with h is R conv_h R, and the filter gradient
// dh(tau) = sum_t dc(t) z(t - tau) is conv(R dc, z)(L - 1 - tau) for tau in
// [0, L), a causal convolution of R dc with z taken as the filter (the negative
// lags of two-sided filters: dh(-tau) = conv(R z, dc)(L - 1 - tau)). The
// kernels here stage the inputs of those convolutions (reversed where needed),
// apply gates and skips, and read the results back reversed. Rows are L
// positions long (a multiple of 8); every thread takes 8 consecutive positions
// of a row per step in 16-byte accesses (a reversed run of 8 is the aligned run
// of 8 that ends where the forward one starts, read or written backwards).
#include "common.h"
#include "kernels_bwd.h"
#include "vec8.h"

namespace hy {
namespace {

// grid for n elements taken 8 at a time
int grid_of(size_t n) {
  const size_t g = (n / 8 + 255) / 256;
  return (int)(g < 8192 ? (g > 0 ? g : 1) : 8192);
}

// grid-stride loop over the 8-element chunks of n elements
#define FOR_CHUNKS(i, n) \
  for (size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8; i < (n); i += (size_t)gridDim.x * 256 * 8)

__device__ __forceinline__ void rev8(const float (&a)[8], float (&b)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) b[7 - k] = a[k];
}

// i runs over [B][D][L]; r = d L + t is the offset inside a sample's D rows
template <typename T>
__global__ __launch_bounds__(256) void bwd4_z_init_kernel(const T* __restrict__ sp, float* __restrict__ zf,
                                                          T* __restrict__ tmp, int B, int D, int L, int NO) {
  const size_t DL = (size_t)D * L, JL = (size_t)(NO + 1) * DL;
  FOR_CHUNKS(i, (size_t)B * DL) {
    const size_t b = i / DL, r = i - b * DL;
    float v[8];
    ld8(sp + b * JL + r, v);
    st8(zf + i, v);
    st8(tmp + b * 2 * DL + r, v);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void bwd4_z_next_kernel(const T* __restrict__ sp, const T* __restrict__ c,
                                                          const float* __restrict__ zf,
                                                          const float* __restrict__ dskip_n, float* __restrict__ zfn,
                                                          T* __restrict__ tmp, T* __restrict__ zfin, int B, int D,
                                                          int L, int NO, int n) {
  const size_t DL = (size_t)D * L, JL = (size_t)(NO + 1) * DL;
  FOR_CHUNKS(i, (size_t)B * DL) {
    const size_t b = i / DL, r = i - b * DL;
    const float dd = dskip_n[r / L];
    float x[8], cv[8], z[8];
    ld8(sp + b * JL + (size_t)(n + 1) * DL + r, x);
    ld8(c + i, cv);
    ld8(zf + i, z);
#pragma unroll
    for (int k = 0; k < 8; ++k) z[k] = x[k] * cv[k] + dd * z[k];
    if (zfn != nullptr) {
      st8(zfn + i, z);
      st8(tmp + b * 2 * DL + r, z);
    } else {
      st8(zfin + i, z);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void bwd4_to_f32_kernel(const T* __restrict__ in, float* __restrict__ out,
                                                          size_t n) {
  FOR_CHUNKS(i, n) {
    float v[8];
    ld8(in + i, v);
    st8(out + i, v);
  }
}

// One workgroup per row (b, d) of g = dz^{n+1}: dx^n = g c^n into ds block n+1,
// R(g x^n) into tmp block 0 (and g x^n into dcf, fp32, unless null), and
// sum_t g z^n (a fixed-order tree sum).
template <typename T>
__global__ __launch_bounds__(256) void bwd4_rev_prep_kernel(const float* __restrict__ g, const T* __restrict__ sp,
                                                            const T* __restrict__ c, const float* __restrict__ zf,
                                                            float* __restrict__ sbar, T* __restrict__ tmp,
                                                            float* __restrict__ dcf, float* __restrict__ dd_part,
                                                            int D, int L, int NO, int n) {
  __shared__ float sh[256];
  const int row = blockIdx.x, b = row / D, d = row - b * D;
  const size_t J = (size_t)(NO + 1) * D;
  const size_t xrow = ((size_t)b * J + (size_t)(n + 1) * D + d) * L;
  const float* gr = g + (size_t)row * L;
  const T* xr = sp + xrow;
  const T* cr = c + (size_t)row * L;
  const float* zr = zf + (size_t)row * L;
  float* dxr = sbar + xrow;
  T* vr = tmp + ((size_t)b * 2 * D + d) * L;
  float acc = 0.f;
  float* dcr = dcf != nullptr ? dcf + (size_t)row * L : nullptr;
  // 8 consecutive positions per thread and step; their reversed images
  // L - 1 - t are the 8 consecutive positions from L - 8 - t0, in reverse order
  for (int t0 = 8 * (int)threadIdx.x; t0 < L; t0 += 8 * 256) {
    float gv[8], xv[8], cv[8], zv[8], dx[8], dc[8], rv[8];
    ld8(gr + t0, gv);
    ld8(xr + t0, xv);
    ld8(cr + t0, cv);
    ld8(zr + t0, zv);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      dx[k] = gv[k] * cv[k];
      dc[k] = gv[k] * xv[k];
      rv[7 - k] = dc[k];
      acc += gv[k] * zv[k];
    }
    st8(dxr + t0, dx);
    st8(vr + (L - 8 - t0), rv);
    if (dcr != nullptr) st8(dcr + t0, dc);
  }
  sh[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) dd_part[((size_t)b * NO + n) * D + d] = sh[0];
}

template <typename T>
__global__ __launch_bounds__(256) void bwd4_rev_finish_kernel(const float* __restrict__ g, const T* __restrict__ conv,
                                                              const float* __restrict__ dskip_n,
                                                              float* __restrict__ out, size_t ostride, int B, int D,
                                                              int L) {
  FOR_CHUNKS(i, (size_t)B * D * L) {
    const size_t row = i / L, t = i - row * L;
    const size_t b = row / D, d = row - b * D;
    const float dd = dskip_n[d];
    float gv[8], cr[8], cv[8], o[8];
    ld8(g + i, gv);
    ld8(conv + row * L + (L - 8 - t), cr);
    rev8(cr, cv);
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = dd * gv[k] + cv[k];
    st8(out + b * ostride + d * L + t, o);
  }
}

// Lags tau in [0, L) of rows of length HL: dh[d][tau] = conv[d][L - 1 - tau].
template <typename T>
__global__ __launch_bounds__(256) void bwd4_dh_store_kernel(const T* __restrict__ conv, float* __restrict__ dh, int D,
                                                            int L, int HL) {
  FOR_CHUNKS(i, (size_t)D * L) {
    const size_t row = i / L, tau = i - row * L;
    float cr[8], o[8];
    ld8(conv + row * L + (L - 8 - tau), cr);
    rev8(cr, o);
    st8(dh + row * HL + tau, o);
  }
}

// Lags -(L-1) .. -1 of wrapped two-sided rows [2L] (lag -tau at 2L - tau), from
// conv = conv(R z, dc): dh[d][j] = conv[d][j - L - 1] for j in (L, 2L), and the
// entry L, no tap, zero.
template <typename T>
__global__ __launch_bounds__(256) void bwd4_dh_store_neg_kernel(const T* __restrict__ conv, float* __restrict__ dh,
                                                                int D, int L) {
  FOR_CHUNKS(i, (size_t)D * L) {
    const size_t row = i / L, k = i - row * L;  // j = L + k
    const T* cr = conv + row * L;
    float cv[8], o[8];
    ld8(cr + k, cv);
    o[0] = k == 0 ? 0.f : ldf(cr + (k - 1));
#pragma unroll
    for (int q = 1; q < 8; ++q) o[q] = cv[q - 1];
    st8(dh + row * 2 * L + L + k, o);
  }
}

// tmp block 0 of one sample = R z (z fp32 [D][L])
template <typename T>
__global__ __launch_bounds__(256) void bwd4_stage_rev_kernel(const float* __restrict__ zf, T* __restrict__ tmp, int D,
                                                             int L) {
  FOR_CHUNKS(i, (size_t)D * L) {
    const size_t row = i / L, t = i - row * L;
    float z[8], o[8];
    ld8(zf + i, z);
    rev8(z, o);
    st8(tmp + row * L + (L - 8 - t), o);
  }
}

}  // namespace

hipError_t bwd4_z_init(const void* sp, float* zf, void* tmp, int B, int D, int L, int NO, bool bf16, hipStream_t s) {
  const size_t n = (size_t)B * D * L;
  if (bf16)
    hipLaunchKernelGGL(bwd4_z_init_kernel<hy::bf16>, dim3(grid_of(n)), dim3(256), 0, s, (const hy::bf16*)sp, zf,
                       (hy::bf16*)tmp, B, D, L, NO);
  else
    hipLaunchKernelGGL(bwd4_z_init_kernel<float>, dim3(grid_of(n)), dim3(256), 0, s, (const float*)sp, zf,
                       (float*)tmp, B, D, L, NO);
  return hipGetLastError();
}

hipError_t bwd4_z_next(const void* sp, const void* c, const float* zf, const float* dskip_n, float* zf_next,
                       void* tmp, void* zfin, int B, int D, int L, int NO, int n, bool bf16, hipStream_t s) {
  const size_t m = (size_t)B * D * L;
  if (bf16)
    hipLaunchKernelGGL(bwd4_z_next_kernel<hy::bf16>, dim3(grid_of(m)), dim3(256), 0, s, (const hy::bf16*)sp,
                       (const hy::bf16*)c, zf, dskip_n, zf_next, (hy::bf16*)tmp, (hy::bf16*)zfin, B, D, L, NO, n);
  else
    hipLaunchKernelGGL(bwd4_z_next_kernel<float>, dim3(grid_of(m)), dim3(256), 0, s, (const float*)sp,
                       (const float*)c, zf, dskip_n, zf_next, (float*)tmp, (float*)zfin, B, D, L, NO, n);
  return hipGetLastError();
}

hipError_t bwd4_to_f32(const void* in, float* out, size_t n, bool bf16, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(bwd4_to_f32_kernel<hy::bf16>, dim3(grid_of(n)), dim3(256), 0, s, (const hy::bf16*)in, out, n);
  else
    hipLaunchKernelGGL(bwd4_to_f32_kernel<float>, dim3(grid_of(n)), dim3(256), 0, s, (const float*)in, out, n);
  return hipGetLastError();
}

hipError_t bwd4_rev_prep(const float* g, const void* sp, const void* c, const float* zf, float* sbar, void* tmp,
                         float* dcf, float* dd_part, int B, int D, int L, int NO, int n, bool bf16, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(bwd4_rev_prep_kernel<hy::bf16>, dim3(B * D), dim3(256), 0, s, g, (const hy::bf16*)sp,
                       (const hy::bf16*)c, zf, sbar, (hy::bf16*)tmp, dcf, dd_part, D, L, NO, n);
  else
    hipLaunchKernelGGL(bwd4_rev_prep_kernel<float>, dim3(B * D), dim3(256), 0, s, g, (const float*)sp,
                       (const float*)c, zf, sbar, (float*)tmp, dcf, dd_part, D, L, NO, n);
  return hipGetLastError();
}

hipError_t bwd4_rev_finish(const float* g, const void* conv, const float* dskip_n, float* out, size_t ostride, int B,
                           int D, int L, bool bf16, hipStream_t s) {
  const size_t n = (size_t)B * D * L;
  if (bf16)
    hipLaunchKernelGGL(bwd4_rev_finish_kernel<hy::bf16>, dim3(grid_of(n)), dim3(256), 0, s, g,
                       (const hy::bf16*)conv, dskip_n, out, ostride, B, D, L);
  else
    hipLaunchKernelGGL(bwd4_rev_finish_kernel<float>, dim3(grid_of(n)), dim3(256), 0, s, g, (const float*)conv,
                       dskip_n, out, ostride, B, D, L);
  return hipGetLastError();
}

hipError_t bwd4_dh_store(const void* conv, float* dh, int D, int L, int HL, bool bf16, hipStream_t s) {
  const size_t n = (size_t)D * L;
  if (bf16)
    hipLaunchKernelGGL(bwd4_dh_store_kernel<hy::bf16>, dim3(grid_of(n)), dim3(256), 0, s, (const hy::bf16*)conv, dh,
                       D, L, HL);
  else
    hipLaunchKernelGGL(bwd4_dh_store_kernel<float>, dim3(grid_of(n)), dim3(256), 0, s, (const float*)conv, dh, D, L,
                       HL);
  return hipGetLastError();
}

hipError_t bwd4_dh_store_neg(const void* conv, float* dh, int D, int L, bool bf16, hipStream_t s) {
  const size_t n = (size_t)D * L;
  if (bf16)
    hipLaunchKernelGGL(bwd4_dh_store_neg_kernel<hy::bf16>, dim3(grid_of(n)), dim3(256), 0, s, (const hy::bf16*)conv,
                       dh, D, L);
  else
    hipLaunchKernelGGL(bwd4_dh_store_neg_kernel<float>, dim3(grid_of(n)), dim3(256), 0, s, (const float*)conv, dh, D,
                       L);
  return hipGetLastError();
}

hipError_t bwd4_stage_rev(const float* zf, void* tmp, int D, int L, bool bf16, hipStream_t s) {
  const size_t n = (size_t)D * L;
  if (bf16)
    hipLaunchKernelGGL(bwd4_stage_rev_kernel<hy::bf16>, dim3(grid_of(n)), dim3(256), 0, s, zf, (hy::bf16*)tmp, D, L);
  else
    hipLaunchKernelGGL(bwd4_stage_rev_kernel<float>, dim3(grid_of(n)), dim3(256), 0, s, zf, (float*)tmp, D, L);
  return hipGetLastError();
}

}  // namespace hy
