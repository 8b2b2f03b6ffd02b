// Implicit filter generation of the 1D Hyena operator (gfx950).
//
// An MLP of the position parameterises each long filter (TWIML #690 podcast,
// 4:29) and the filter is as long as the input (TWIML #690, 5:48):
//   e_t = [tau, cos(2 pi k tau)_{k=1..K}, sin(2 pi k tau)_{k=1..K}],  tau = t / L
//   o_t = W3^T sin(W2^T sin(W1^T e_t + b1) + b2) + b3
//   h^n_c(t) = exp(-decay_c tau) o_t[n D + c]
// One workgroup evaluates a tile of 64 positions: features and both hidden
// layers go to LDS, then every thread produces one output column for the 64
// positions (the W x N*D output layer dominates the work).
#include "common.h"
#include "kernels.h"

namespace hy {

constexpr int kFT = 64;     // positions per workgroup
constexpr int kMaxW = 128;  // FFN width limit
constexpr int kMaxF = 65;   // 1 + 2K, K <= 32

__global__ __launch_bounds__(256) void filter1d_mlp_kernel(Filter1DArgs a) {
  __shared__ float e_s[kFT][kMaxF + 1];
  __shared__ float h1[kFT][kMaxW + 1];
  __shared__ float h2[kFT][kMaxW + 1];
  const int t0 = blockIdx.x * kFT;
  const int F = 1 + 2 * a.K, W = a.W, L = a.L;
  const int tid = threadIdx.x;
  for (int idx = tid; idx < kFT * F; idx += 256) {
    const int tl = idx / F, f = idx % F;
    const int t = t0 + tl;
    float v = 0.f;
    if (t < L) {
      if (f == 0) {
        v = (float)t / (float)L;
      } else {
        const int k = (f <= a.K) ? f : f - a.K;
        // angle 2 pi k t / L reduced exactly: 2 pi m / L with m = (k t) mod L
        const long long m = ((long long)k * t) % L;
        float sv, cv;
        sincospif(2.0f * (float)m / (float)L, &sv, &cv);
        v = (f <= a.K) ? cv : sv;
      }
    }
    e_s[tl][f] = v;
  }
  __syncthreads();
  for (int idx = tid; idx < kFT * W; idx += 256) {
    const int tl = idx / W, j = idx % W;
    float s = a.b1[j];
    for (int f = 0; f < F; ++f) s += e_s[tl][f] * a.w1[f * W + j];
    h1[tl][j] = sinf(s);
  }
  __syncthreads();
  for (int idx = tid; idx < kFT * W; idx += 256) {
    const int tl = idx / W, j = idx % W;
    float s = a.b2[j];
    for (int f = 0; f < W; ++f) s += h1[tl][f] * a.w2[f * W + j];
    h2[tl][j] = sinf(s);
  }
  __syncthreads();
  const int ND = a.NO * a.D;
  const float invL = 1.0f / (float)L;
  for (int col = tid; col < ND; col += 256) {
    float acc[kFT];
    const float bias = a.b3[col];
#pragma unroll
    for (int tl = 0; tl < kFT; ++tl) acc[tl] = bias;
    for (int j = 0; j < W; ++j) {
      const float wv = a.w3[(size_t)j * ND + col];
#pragma unroll
      for (int tl = 0; tl < kFT; ++tl) acc[tl] += h2[tl][j] * wv;
    }
    const int c = col % a.D;
    const float dc = a.decay[c];
    float* dst = a.h + (size_t)col * L + t0;   // h[n][c][t] with col = n D + c
#pragma unroll
    for (int tl = 0; tl < kFT; ++tl) {
      if (t0 + tl < L) dst[tl] = acc[tl] * expf(-dc * (float)(t0 + tl) * invL);
    }
  }
}

hipError_t filter1d_mlp(const Filter1DArgs& a, hipStream_t s) {
  dim3 grid((a.L + kFT - 1) / kFT), block(256);
  hipLaunchKernelGGL(filter1d_mlp_kernel, grid, block, 0, s, a);
  return hipGetLastError();
}

__global__ void twiddle_kernel(float2* tw, int n, int count) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= count) return;
  double sv, cv;
  sincospi(2.0 * (double)m / (double)n, &sv, &cv);
  tw[m] = make_float2((float)cv, (float)-sv);
}

hipError_t twiddles(float2* tw, int n, int count, hipStream_t s) {
  hipLaunchKernelGGL(twiddle_kernel, dim3((count + 255) / 256), dim3(256), 0, s, tw, n, count);
  return hipGetLastError();
}

}  // namespace hy
