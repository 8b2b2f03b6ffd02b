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
//
// Non-causal layers evaluate the same generator at the signed lags of a
// two-sided filter, written wrapped for the 2L-point transform: position
// m in [0, 2L) holds lag m (m < L) or m - 2L (m > L), and m = L is zero. The
// features at lag tau are [tau / L, cos, sin of 2 pi k tau / L] (the angles
// equal those at m, the cosines and sines having period L) and the window is
// exp(-decay |tau| / L).
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
  const int P = a.noncausal ? 2 * L : L;  // positions evaluated
  const int tid = threadIdx.x;
  for (int idx = tid; idx < kFT * F; idx += 256) {
    const int tl = idx / F, f = idx % F;
    const int t = t0 + tl;
    float v = 0.f;
    if (t < P) {
      if (f == 0) {
        v = (float)(t > L ? t - 2 * L : t) / (float)L;
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
    float* dst = a.h + (size_t)col * P + t0;   // h[n][c][t] with col = n D + c
#pragma unroll
    for (int tl = 0; tl < kFT; ++tl) {
      const int t = t0 + tl;
      const int lag = t > L ? 2 * L - t : t;   // |tau|
      if (t < P) dst[tl] = (t == L && P > L) ? 0.f : acc[tl] * expf(-dc * (float)lag * invL);
    }
  }
}

// The same MLP on the fp32 matrix cores (v_mfma_f32_32x32x2_f32, full fp32
// products and sums), for FFN widths of 64 or 128. A workgroup (four waves)
// takes 64 positions: the features, then each layer's activations, go to LDS
// (two buffers: features then second layer in one, first layer in the other);
// every layer is a [64 x K] x [K x cols] product in 32 x 32 blocks with the A
// operand read from LDS. In the output layer a wave takes one 32-column block
// (columns n D + c) for both 32-position halves at a time, with the whole
// K x 32 slice of W3 in registers and the next block's slice in flight; the
// block is windowed and written as 16-byte runs of positions.
typedef __attribute__((ext_vector_type(16))) float f32x16;

template <int WW>
__global__ __launch_bounds__(256) void filter1d_mfma_kernel(Filter1DArgs a) {
  constexpr int LDH = WW + 1;   // activation row stride (floats)
  constexpr int KW = WW / 2;    // K steps of the hidden and output layers
  __shared__ float buf0[kFT * (kMaxF + 2 > LDH ? kMaxF + 2 : LDH)];  // features, then layer 2
  __shared__ float buf1[kFT * LDH];                                  // layer 1
  const int t0 = blockIdx.x * kFT;
  const int F = 1 + 2 * a.K, Fp = (F + 1) & ~1, L = a.L;
  const int P = a.noncausal ? 2 * L : L;  // positions evaluated
  const int LDE = Fp + 1;  // feature row stride
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, k2 = lane >> 5;
  for (int idx = tid; idx < kFT * Fp; idx += 256) {
    const int tl = idx / Fp, f = idx % Fp;
    const int t = t0 + tl;
    float v = 0.f;
    if (t < P && f < F) {
      if (f == 0) {
        v = (float)(t > L ? t - 2 * L : t) / (float)L;
      } else {
        const int k = (f <= a.K) ? f : f - a.K;
        // angle 2 pi k t / L reduced exactly: 2 pi m / L with m = (k t) mod L
        const long long m = ((long long)k * t) % L;
        float sv, cv;
        sincospif(2.0f * (float)m / (float)L, &sv, &cv);
        v = (f <= a.K) ? cv : sv;
      }
    }
    buf0[tl * LDE + f] = v;
  }
  __syncthreads();
  auto zero = [](f32x16& c) {
#pragma unroll
    for (int e = 0; e < 16; ++e) c[e] = 0.f;
  };
  // hidden layers: 2 x (WW / 32) blocks of 32 x 32 over the four waves
  constexpr int NB = 2 * (WW / 32);
  for (int blk = wave; blk < NB; blk += 4) {
    const int rb = blk & 1, j = (blk >> 1) * 32 + r32;
    f32x16 acc;
    zero(acc);
    // feature Fp - 1 (when F is odd) is zero; it meets weight row F - 1 again
#pragma unroll 8
    for (int k = 0; k < Fp; k += 2) {
      const int f = k + k2;
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(buf0[(rb * 32 + r32) * LDE + f],
                                                 a.w1[(size_t)(f < F ? f : F - 1) * WW + j], acc, 0, 0, 0);
    }
    const float bj = a.b1[j];
#pragma unroll
    for (int e = 0; e < 16; ++e) buf1[(rb * 32 + (e >> 2) * 8 + k2 * 4 + (e & 3)) * LDH + j] = sinf(acc[e] + bj);
  }
  __syncthreads();
  for (int blk = wave; blk < NB; blk += 4) {
    const int rb = blk & 1, j = (blk >> 1) * 32 + r32;
    f32x16 acc;
    zero(acc);
#pragma unroll
    for (int k = 0; k < WW; k += 2)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(buf1[(rb * 32 + r32) * LDH + k + k2],
                                                 a.w2[(size_t)(k + k2) * WW + j], acc, 0, 0, 0);
    const float bj = a.b2[j];
#pragma unroll
    for (int e = 0; e < 16; ++e) buf0[(rb * 32 + (e >> 2) * 8 + k2 * 4 + (e & 3)) * LDH + j] = sinf(acc[e] + bj);
  }
  __syncthreads();
  // output layer
  const int ND = a.NO * a.D;
  const int ncb = (ND + 31) / 32;
  const float invL = 1.0f / (float)L;
  float wv[KW];  // W3 rows k2, k2 + 2, ... of this lane's column
  auto load_w3 = [&](int cb) {
    const int col = cb * 32 + r32;
    const float* w = a.w3 + (col < ND ? col : ND - 1) + (size_t)k2 * ND;
#pragma unroll
    for (int k = 0; k < KW; ++k) wv[k] = w[(size_t)(2 * k) * ND];
  };
  int cb = wave;
  if (cb >= ncb) return;
  load_w3(cb);
  while (true) {
    const int col = cb * 32 + r32;
    const int colc = col < ND ? col : ND - 1;  // ragged last block: valid loads, no stores
    f32x16 acc0, acc1;
    zero(acc0);
    zero(acc1);
#pragma unroll
    for (int k = 0; k < KW; ++k) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(buf0[r32 * LDH + 2 * k + k2], wv[k], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(buf0[(32 + r32) * LDH + 2 * k + k2], wv[k], acc1, 0, 0, 0);
    }
    const int nxt = cb + 4;
    const bool more = nxt < ncb;
    load_w3(more ? nxt : cb);  // the next block's slice (this one's again after the last: unused)
    const float bias = a.b3[colc];
    const float dc = a.decay[colc % a.D];
    float* dst = a.h + (size_t)colc * P;  // h[n][c][t] with col = n D + c
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int t = t0 + rb * 32 + g * 8 + k2 * 4;  // four consecutive positions
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int lag = t + i > L ? 2 * L - (t + i) : t + i;  // |tau|
          o[i] = ((rb ? acc1[4 * g + i] : acc0[4 * g + i]) + bias) * expf(-dc * (float)lag * invL);
          if (t + i == L && P > L) o[i] = 0.f;
        }
        if (col < ND) {
          if (t + 3 < P && (P & 3) == 0) {
            *reinterpret_cast<float4*>(dst + t) = make_float4(o[0], o[1], o[2], o[3]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (t + i < P) dst[t + i] = o[i];
          }
        }
      }
    }
    if (!more) break;
    cb = nxt;
  }
}

hipError_t filter1d_mlp(const Filter1DArgs& a, hipStream_t s) {
  const int P = a.noncausal ? 2 * a.L : a.L;
  dim3 grid((P + kFT - 1) / kFT), block(256);
  if (a.W == 64 && 1 + 2 * a.K <= kMaxF)
    hipLaunchKernelGGL(filter1d_mfma_kernel<64>, grid, block, 0, s, a);
  else if (a.W == 128 && 1 + 2 * a.K <= kMaxF)
    hipLaunchKernelGGL(filter1d_mfma_kernel<128>, grid, block, 0, s, a);
  else
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
