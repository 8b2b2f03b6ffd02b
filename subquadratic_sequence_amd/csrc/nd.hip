// 3D (HyenaND) path on gfx950: coordinate-MLP kernel, channel-mean gate and the
// 3D FFT convolution with gating, zero padded (non-circular) or periodic
// (circular) (HyenaND explainer, gist.science, "Methodology: HyenaND": Native ND
// Convolution, Input-Dependent Kernels, Kernel Synthesis, Handling Boundaries).
//
// Layouts: activations channel-major [B][C][X][Y][Z] (z contiguous); transform
// size (MX, MY, MZ) = (2X, 2Y, 2Z) zero padded or (X, Y, Z) circular; the
// three axes are independent (MY x MZ planes; MX = 1 for 2D grids, X = 1).
// The kernel lives on the matching offset grid, offset d at index d + M/2 per
// axis (M the axis' transform length), at coordinates d / (M/2).
//
// The gate g_{b,c} is one scalar per sample and channel, so it commutes with
// the convolution and is applied to the convolution output in the spatial
// domain. The same channel of two samples then travels as one complex field
// z_{b0,c} + i z_{b1,c}: both halves are filtered by the same real kernel K_c,
// so the spectrum product is a plain pointwise multiply by K^_c and the inverse
// transform returns (K_c * z_{b0,c}) + i (K_c * z_{b1,c}). Each channel's
// spectrum is read once for both samples.
//
// Per order: a plane pass (2D DFT over (y, z) of the X non-zero x-planes, with
// the Y x Z non-zero block zero padded), a pencil pass (DFT over x, X non-zero
// inputs, times K^_c, inverse DFT over x keeping x < X) and the inverse plane
// pass (inverse 2D DFT, crop to Y x Z, gate, skip), which also starts the next
// order's forward plane DFT from the same LDS plane. With the circular boundary
// the same passes run with no zero padding and no crop (M = G).
#include "common.h"
#include "kernels_nd.h"

namespace hy {

// ======================================================= coordinate MLP
constexpr int kNP = 64;       // offset points per workgroup
constexpr int kNdMaxW = 128;

// FILM: the register-conditioned SIREN (each hidden pre-activation times the
// sample's gamma, plus its beta; omega0 folded into the first layer's gamma) with
// a Gaussian window exp(-a_c |c|^2); otherwise sin(W^T h + b) with the window
// exp(-a_c |c|).
template <bool FILM>
__global__ __launch_bounds__(256) void nd_mlp_kernel(NdFilterArgs a) {
  __shared__ float cs[kNP][3];
  __shared__ float rad[kNP];
  __shared__ float h1[kNP][kNdMaxW + 1];
  __shared__ float h2[kNP][kNdMaxW + 1];
  const int MX = a.MX, MY = a.MY, MZ = a.MZ;
  const int P = MX * MY * MZ;
  const int p0 = blockIdx.x * kNP;
  const int W = a.W, tid = threadIdx.x;
  for (int t = tid; t < kNP; t += 256) {
    const int pt = p0 + t;
    const int k = pt % MZ, j = (pt / MZ) % MY, i = pt / (MZ * MY);
    const float cx = MX > 1 ? (float)(i - MX / 2) / (float)(MX / 2) : 0.f;  // 2D grids: dx = 0
    const float cy = (float)(j - MY / 2) / (float)(MY / 2);
    const float cz = (float)(k - MZ / 2) / (float)(MZ / 2);
    cs[t][0] = cx;
    cs[t][1] = cy;
    cs[t][2] = cz;
    const float r2 = cx * cx + cy * cy + cz * cz;
    rad[t] = FILM ? r2 : sqrtf(r2);
  }
  __syncthreads();
  for (int idx = tid; idx < kNP * W; idx += 256) {
    const int t = idx / W, j = idx % W;
    const float s = a.b1[j] + cs[t][0] * a.w1[j] + cs[t][1] * a.w1[W + j] + cs[t][2] * a.w1[2 * W + j];
    h1[t][j] = FILM ? sinf(a.film[j] * s + a.film[W + j]) : sinf(s);
  }
  __syncthreads();
  for (int idx = tid; idx < kNP * W; idx += 256) {
    const int t = idx / W, j = idx % W;
    float s = a.b2[j];
    for (int f = 0; f < W; ++f) s += h1[t][f] * a.w2[f * W + j];
    h2[t][j] = FILM ? sinf(a.film[2 * W + j] * s + a.film[3 * W + j]) : sinf(s);
  }
  __syncthreads();
  const int NC = a.N * a.C;
  for (int col = tid; col < NC; col += 256) {
    float acc[kNP];
    const float bias = a.b3[col];
#pragma unroll
    for (int t = 0; t < kNP; ++t) acc[t] = bias;
    for (int j = 0; j < W; ++j) {
      const float wv = a.w3[(size_t)j * NC + col];
#pragma unroll
      for (int t = 0; t < kNP; ++t) acc[t] += h2[t][j] * wv;
    }
    const float dc = a.decay[col % a.C];
    float* dst = a.k + (size_t)col * P + p0;  // K[n][c][i][j][k], col = n C + c
#pragma unroll
    for (int t = 0; t < kNP; ++t) dst[t] = acc[t] * expf(-dc * rad[t]);
  }
}

// The same MLP on the fp32 matrix cores (v_mfma_f32_32x32x2_f32, full fp32
// products and sums), for widths 64 and 128: 64 offset points per workgroup of
// four waves; each layer is a [64 x K] x [K x cols] product in 32 x 32 blocks
// with the activations in LDS; in the output layer a wave takes one 32-column
// block (columns n C + c) for both 32-point halves with the K x 32 slice of
// W3 in registers and the next block's slice in flight.
typedef __attribute__((ext_vector_type(16))) float f32x16;

// sin(x) for the sine layers: x = k pi + r with k = rint(x / pi) and |r| <= pi/2
// (Cody-Waite reduction, pi split into 3.140625, a 12-bit middle part and the
// fp32 rest, so that k times the first two parts is exact for |x| < 12000),
// sin(x) = (-1)^k sin(r), sin(r) by its Taylor series through r^13 (truncation
// below 7e-9 for |r| <= pi/2). Measured against sin in fp64 on 6 million
// arguments in |x| <= 3000: absolute error at most 1.1e-7. Larger arguments
// take sinf.
__device__ __forceinline__ float sin_layer(float x) {
  if (!(fabsf(x) < 12000.f)) return sinf(x);
  const float k = rintf(x * 0.318309886183790672f);
  float r = fmaf(-k, 3.140625f, x);
  r = fmaf(-k, 9.677410125732422e-4f, r);
  r = fmaf(-k, -8.742278e-8f, r);
  const float r2 = r * r;
  float p = 1.6059043836821614e-10f;        // 1/13!
  p = fmaf(p, r2, -2.5052108385441720e-8f);  // -1/11!
  p = fmaf(p, r2, 2.7557319223985893e-6f);   // 1/9!
  p = fmaf(p, r2, -1.9841269841269841e-4f);  // -1/7!
  p = fmaf(p, r2, 8.3333333333333333e-3f);   // 1/5!
  p = fmaf(p, r2, -1.6666666666666667e-1f);  // -1/3!
  const float sr = fmaf(r * r2, p, r);
  return ((int)k & 1) ? -sr : sr;
}

// DIRECT: the output goes to the transform's wrapped channel-pair fields
// a.fdirect[pair][w] = (K_{2 pair}, K_{2 pair + 1}) at w = (offset + M/2) mod M
// per axis, the layout nd_pack_kernel produces; lanes holding columns 2 pair and
// 2 pair + 1 are neighbours and swap halves of their four points.
template <int WW, bool FILM, bool DIRECT>
__global__ __launch_bounds__(256) void nd_mlp_mfma_kernel(NdFilterArgs a) {
  constexpr int LDH = WW + 1;
  constexpr int KW = WW / 2;
  __shared__ float cs[kNP][5];  // the three coordinates, a zero pad column, the radius (FILM: its square)
  __shared__ int fidx[kNP];     // DIRECT: index of the point in the wrapped transform field
  __shared__ float buf0[kNP * LDH];  // layer 2
  __shared__ float buf1[kNP * LDH];  // layer 1
  const int MX = a.MX, MY = a.MY, MZ = a.MZ;
  const int P = MX * MY * MZ;
  const int p0 = blockIdx.x * kNP;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, k2 = lane >> 5;
  for (int t = tid; t < kNP; t += 256) {
    const int pt = p0 + t;
    const int k = pt % MZ, j = (pt / MZ) % MY, i = pt / (MZ * MY);
    const float cx = MX > 1 ? (float)(i - MX / 2) / (float)(MX / 2) : 0.f;  // 2D grids: dx = 0
    const float cy = (float)(j - MY / 2) / (float)(MY / 2);
    const float cz = (float)(k - MZ / 2) / (float)(MZ / 2);
    cs[t][0] = cx;
    cs[t][1] = cy;
    cs[t][2] = cz;
    cs[t][3] = 0.f;
    const float r2 = cx * cx + cy * cy + cz * cz;
    cs[t][4] = FILM ? r2 : sqrtf(r2);
    if (DIRECT) fidx[t] = (((i + MX / 2) % MX) * MY + (j + MY / 2) % MY) * MZ + (k + MZ / 2) % MZ;
  }
  __syncthreads();
  auto zero = [](f32x16& c) {
#pragma unroll
    for (int e = 0; e < 16; ++e) c[e] = 0.f;
  };
  constexpr int NB = 2 * (WW / 32);
  for (int blk = wave; blk < NB; blk += 4) {
    const int rb = blk & 1, j = (blk >> 1) * 32 + r32;
    f32x16 acc;
    zero(acc);
#pragma unroll
    for (int k = 0; k < 4; k += 2) {
      const int f = k + k2;  // feature 3 is the zero pad; it meets weight row 2 again
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(cs[rb * 32 + r32][f], a.w1[(size_t)(f < 3 ? f : 2) * WW + j], acc,
                                                 0, 0, 0);
    }
    const float bj = a.b1[j];
    const float gj = FILM ? a.film[j] : 1.f, ej = FILM ? a.film[WW + j] : 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      buf1[(rb * 32 + (e >> 2) * 8 + k2 * 4 + (e & 3)) * LDH + j] =
          FILM ? sin_layer(gj * (acc[e] + bj) + ej) : sin_layer(acc[e] + bj);
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
    const float gj = FILM ? a.film[2 * WW + j] : 1.f, ej = FILM ? a.film[3 * WW + j] : 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      buf0[(rb * 32 + (e >> 2) * 8 + k2 * 4 + (e & 3)) * LDH + j] =
          FILM ? sin_layer(gj * (acc[e] + bj) + ej) : sin_layer(acc[e] + bj);
  }
  __syncthreads();
  const int NC = a.N * a.C;  // a multiple of 64
  const int ncb = NC / 32;
  float wv[KW];
  auto load_w3 = [&](int cb) {
    const float* w = a.w3 + cb * 32 + r32 + (size_t)k2 * NC;
#pragma unroll
    for (int k = 0; k < KW; ++k) wv[k] = w[(size_t)(2 * k) * NC];
  };
  int cb = wave;
  if (cb >= ncb) return;
  load_w3(cb);
  while (true) {
    const int col = cb * 32 + r32;
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
    const float bias = a.b3[col];
    // window exp(-decay x) as 2^(-decay log2(e) x) on the hardware exp2: the
    // rounding of the scaled argument changes the window by a relative
    // 2^-23 |decay x|, i.e. by at most about 5e-8 of the window's maximum
    // (x e^-x <= 1/e), far inside the kernel's fp32 tolerance
    const float dcl = a.decay[col % a.C] * 1.44269504088896341f;
    float* dst = a.k + (size_t)col * P + p0;  // K[n][c][i][j][k], col = n C + c
    const bool odd = col & 1;
    float* fdst = reinterpret_cast<float*>(a.fdirect + (size_t)(col >> 1) * P);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int t = rb * 32 + g * 8 + k2 * 4;  // four consecutive points
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o[i] = ((rb ? acc1[4 * g + i] : acc0[4 * g + i]) + bias) * __builtin_amdgcn_exp2f(-dcl * cs[t + i][4]);
        if (DIRECT) {
          // the four points sit at consecutive field indices (M/2 is a multiple
          // of 4); the even column's lane stores points 0-1, the odd one's 2-3
          float pv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) pv[i] = __shfl_xor(o[i], 1);
          const float4 v = odd ? make_float4(pv[2], o[2], pv[3], o[3]) : make_float4(o[0], pv[0], o[1], pv[1]);
          *reinterpret_cast<float4*>(fdst + 2 * (size_t)fidx[t] + (odd ? 4 : 0)) = v;
        } else {
          *reinterpret_cast<float4*>(dst + t) = make_float4(o[0], o[1], o[2], o[3]);
        }
      }
    }
    if (!more) break;
    cb = nxt;
  }
}

// ======================================================= register conditioning
// One workgroup per sample: scores s_r = reg_r . q (a wave per register, lanes
// over channels), softmax weights over the registers, the control vector
// z = sum_r w_r reg_r, then the four FiLM vectors film_b[k] + film_w[k]^T z
// (k = gamma_1, beta_1, gamma_2, beta_2), gamma_1 times omega0.
// LDS: z [C], scores [R], weights [R].
__global__ __launch_bounds__(256) void nd_film_mod_kernel(const float* __restrict__ reg, const float* __restrict__ q,
                                                          const float* __restrict__ fw, const float* __restrict__ fb,
                                                          const float* __restrict__ om, float* __restrict__ mod,
                                                          int R, int C, int W) {
  extern __shared__ float sm[];
  float* z = sm;
  float* sc = sm + C;
  float* wt = sc + R;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* rb = reg + (size_t)b * R * C;
  for (int r = wave; r < R; r += 4) {
    float acc = 0.f;
    for (int c = lane; c < C; c += 64) acc += rb[(size_t)r * C + c] * q[c];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) sc[r] = acc;
  }
  __syncthreads();
  float mx = sc[0];
  for (int r = 1; r < R; ++r) mx = fmaxf(mx, sc[r]);
  float sum = 0.f;
  for (int r = 0; r < R; ++r) sum += expf(sc[r] - mx);
  for (int r = tid; r < R; r += 256) wt[r] = expf(sc[r] - mx) / sum;
  __syncthreads();
  for (int c = tid; c < C; c += 256) {
    float acc = 0.f;
    for (int r = 0; r < R; ++r) acc += wt[r] * rb[(size_t)r * C + c];
    z[c] = acc;
  }
  __syncthreads();
  for (int o = tid; o < 4 * W; o += 256) {
    const int k = o / W, j = o - k * W;
    const float* w = fw + (size_t)k * C * W + j;
    float acc = fb[o];
    for (int c = 0; c < C; ++c) acc += z[c] * w[(size_t)c * W];
    mod[(size_t)b * 4 * W + o] = k == 0 ? om[j] * acc : acc;
  }
}

hipError_t nd_film_mod(const float* reg, const float* q, const float* film_w, const float* film_b,
                       const float* omega0, float* mod, int B, int R, int C, int W, hipStream_t s) {
  const size_t lds = (size_t)(C + 2 * R) * sizeof(float);
  hipLaunchKernelGGL(nd_film_mod_kernel, dim3(B), dim3(256), lds, s, reg, q, film_w, film_b, omega0, mod, R, C, W);
  return hipGetLastError();
}

__global__ void fill_kernel(float* __restrict__ p, size_t n, float v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

hipError_t fill(float* p, size_t n, float v, hipStream_t s) {
  const unsigned g = (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  hipLaunchKernelGGL(fill_kernel, dim3(g ? g : 1), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

// Two channels of the offset-indexed kernel, wrapped (offset d stored at d mod M),
// as one complex field per channel pair: F = K_{2cp} + i K_{2cp+1}.
__global__ void nd_pack_kernel(const float* __restrict__ k, float2* __restrict__ F, int MX, int MY, int MZ,
                               int npairs) {
  const size_t P = (size_t)MX * MY * MZ;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= P * npairs) return;
  const size_t pr = idx / P, w = idx % P;
  const int wz = (int)(w % MZ), wy = (int)((w / MZ) % MY), wx = (int)(w / ((size_t)MZ * MY));
  const size_t o = ((size_t)((wx + MX / 2) % MX) * MY + (wy + MY / 2) % MY) * MZ + (wz + MZ / 2) % MZ;
  F[idx] = make_float2(k[(2 * pr) * P + o], k[(2 * pr + 1) * P + o]);
}

// Per-channel half spectra (kz in [0, MZ/2]) from the spectra of the packed pairs:
// Ha(k) = (F(k) + conj F(-k)) / 2, Hb(k) = (F(k) - conj F(-k)) / 2i, scaled by
// 1 / (MX MY MZ) (the inverse transforms are unnormalised).
__global__ void nd_split_kernel(const float2* __restrict__ F, float2* __restrict__ Kh, int MX, int MY, int MZ,
                                int npairs) {
  const int ZH = MZ / 2 + 1;
  const size_t PH = (size_t)MX * MY * ZH, P = (size_t)MX * MY * MZ;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= PH * npairs) return;
  const size_t pr = idx / PH, w = idx % PH;
  const int kz = (int)(w % ZH), ky = (int)((w / ZH) % MY), kx = (int)(w / ((size_t)ZH * MY));
  const float2* Fp = F + pr * P;
  const float2 fk = Fp[((size_t)kx * MY + ky) * MZ + kz];
  const float2 fm = conjf2(Fp[((size_t)((MX - kx) % MX) * MY + (MY - ky) % MY) * MZ + (MZ - kz) % MZ]);
  const float s = 0.5f / (float)P;
  const float2 ha = cadd(fk, fm), d = csub(fk, fm);
  Kh[(2 * pr) * PH + w] = make_float2(s * ha.x, s * ha.y);
  Kh[(2 * pr + 1) * PH + w] = make_float2(s * d.y, -s * d.x);
}

// ================================================ FFT along LDS lines
// M-point Stockham FFT of the line buf[base + i*stride], i in [0, M), by M/E
// threads (lt); every thread of the workgroup calls it (barriers), `active`
// selects the ones that own a line. tw128[m] = W_128^m, a copy in LDS (a table
// lookup from global memory inside a stage would make the stage wait for every
// load issued before it).
template <int M, int E, int Ns, bool INV>
__device__ __forceinline__ void line_stage(float2* buf, int base, int stride, int lt, bool active,
                                           const float2* __restrict__ tw128) {
  constexpr int R = (E < M / Ns) ? E : M / Ns;
  constexpr int NB = E / R;
  constexpr int T = M / E;
  float2 v[NB][R];
  if (active) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int j = lt + b * T;
#pragma unroll
      for (int r = 0; r < R; ++r) v[b][r] = buf[base + (j + r * (M / R)) * stride];
      if (Ns > 1) {
        const int k = j % Ns;
#pragma unroll
        for (int r = 1; r < R; ++r) v[b][r] = twmul<INV>(v[b][r], tw128[r * k * (128 / (Ns * R))]);
      }
      Dft<R, INV>::run(v[b]);
    }
  }
  __syncthreads();
  if (active) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int j = lt + b * T;
      const int base_o = (j / Ns) * Ns * R + j % Ns;
#pragma unroll
      for (int r = 0; r < R; ++r) buf[base + (base_o + r * Ns) * stride] = v[b][r];
    }
  }
  __syncthreads();
}

template <int M, int E, int Ns, bool INV> struct LineFrom {
  static __device__ __forceinline__ void run(float2* buf, int base, int stride, int lt, bool active,
                                             const float2* tw) {
    constexpr int R = (E < M / Ns) ? E : M / Ns;
    line_stage<M, E, Ns, INV>(buf, base, stride, lt, active, tw);
    LineFrom<M, E, Ns * R, INV>::run(buf, base, stride, lt, active, tw);
  }
};
template <int M, int E, bool INV> struct LineFrom<M, E, M, INV> {
  static __device__ __forceinline__ void run(float2*, int, int, int, bool, const float2*) {}
};

// ======================================================== plane pass
// One workgroup per (sample pair or filter pair, channel, x-plane). The plane
// (MY x MZ complex) lives in LDS at [y][z] with row stride MZ + 1. Thread t
// works on line t % nlines (one of the lines of a direction) as its
// (t / nlines)-th FFT thread, so the 64 lanes of a wave sit on 64 lines.
enum { PL_FWD_V = 0, PL_FWD_FULL = 1, PL_INV = 2, PL_INV_FWD = 3 };

template <int MY, int MZ = MY> struct PlaneCfg {
  static constexpr int EZ = MZ >= 16 ? 16 : MZ;  // values per thread along a row (z)
  static constexpr int TZ = MZ / EZ;             // threads per row
  static constexpr int EY = MY >= 16 ? 16 : MY;  // along a column (y)
  static constexpr int TY = MY / EY;
  static constexpr int E = EZ, T = TZ;           // the square planes' names
  static constexpr int RS = MZ + 1;              // LDS row stride
  // every thread owns part of a line in the line stages (at least one wave)
  static constexpr int LT = MY * TZ > MZ * TY ? MY * TZ : MZ * TY;
  static constexpr int THREADS = LT < 64 ? 64 : LT;
  static constexpr int PER = MY * MZ / THREADS;  // plane elements per thread
  static constexpr size_t LDS = (size_t)MY * RS * 8 + 128 * 8;  // plane + W_128 table
};

// rows (lines along z, MZ points), the first nrows of them
template <int MY, int MZ, bool INV>
__device__ __forceinline__ void plane_rows_r(float2* P, int nrows, const float2* tw) {
  using C = PlaneCfg<MY, MZ>;
  const int line = threadIdx.x % MY, lt = threadIdx.x / MY;
  const bool active = line < nrows && lt < C::TZ;
  LineFrom<MZ, C::EZ, 1, INV>::run(P, line * C::RS, 1, lt, active, tw);
}

// columns (lines along y, MY points), all MZ of them
template <int MY, int MZ, bool INV>
__device__ __forceinline__ void plane_cols_r(float2* P, const float2* tw) {
  using C = PlaneCfg<MY, MZ>;
  const int line = threadIdx.x % MZ, lt = threadIdx.x / MZ;
  const bool active = lt < C::TY;
  LineFrom<MY, C::EY, 1, INV>::run(P, line, C::RS, lt, active, tw);
}

template <int M, bool INV>
__device__ __forceinline__ void plane_rows(float2* P, int nrows, const float2* tw) {
  plane_rows_r<M, M, INV>(P, nrows, tw);
}

template <int M, bool INV>
__device__ __forceinline__ void plane_cols(float2* P, const float2* tw) {
  plane_cols_r<M, M, INV>(P, tw);
}

// Plane element loops run a fixed count per thread (element tid + k THREADS),
// unrolled, so that all of a thread's loads are in flight together.
template <int MY, int MZ, int MODE>
__global__ __launch_bounds__((PlaneCfg<MY, MZ>::THREADS)) void nd_plane_kernel(NdConvArgs a) {
  using C = PlaneCfg<MY, MZ>;
  constexpr int PER = C::PER;
  extern __shared__ float4 smem4[];
  float2* P = reinterpret_cast<float2*>(smem4);
  float2* tw = P + MY * C::RS;  // W_128^m, m < 128
  const int X = a.X, Y = a.Y, Z = a.Z;
  const size_t V = (size_t)X * Y * Z;
  const size_t plane = (size_t)MY * MZ;
  const int x = blockIdx.x;          // plane index
  const int c = blockIdx.y;          // channel (or filter pair)
  const int bp = blockIdx.z;         // sample pair (or order of the filter)
  const int tid = threadIdx.x;
  for (int i = tid; i < 128; i += C::THREADS) tw[i] = a.tw128[i];  // visible after the next barrier
  auto el = [&](int k) { return tid + k * C::THREADS; };           // this thread's k-th element
  auto lds = [&](int i) { return (i / MZ) * C::RS + i % MZ; };

  if constexpr (MODE == PL_FWD_FULL) {
    // filter: full M x M complex plane, all MX planes
    float2* Fp = a.F + (((size_t)bp * a.npairs + c) * a.MX + x) * plane;
    float2 t[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) t[k] = Fp[el(k)];
#pragma unroll
    for (int k = 0; k < PER; ++k) P[lds(el(k))] = t[k];
    __syncthreads();
    plane_rows_r<MY, MZ, false>(P, MY, tw);
    plane_cols_r<MY, MZ, false>(P, tw);
#pragma unroll
    for (int k = 0; k < PER; ++k) Fp[el(k)] = P[lds(el(k))];
    return;
  }

  const int b0 = 2 * bp, b1 = b0 + 1;
  const bool has_b1 = b1 < a.B;
  const int CC = a.C;
  float2* Yp = a.Yint + (((size_t)bp * CC + c) * X + x) * plane;
  const size_t J = (size_t)(a.NO + 1) * CC;
  const float* s0 = a.p + (size_t)b0 * J * V;
  const float* s1 = a.p + (size_t)(has_b1 ? b1 : b0) * J * V;
  const size_t xoff = (size_t)x * Y * Z;

  if constexpr (MODE == PL_FWD_V) {
    const float* v0 = s0 + (size_t)c * V + xoff;
    const float* v1 = s1 + (size_t)c * V + xoff;
    float2 t[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int y = el(k) / MZ, z = el(k) % MZ;
      t[k] = make_float2(0.f, 0.f);
      if (y < Y && z < Z) t[k] = make_float2(v0[y * Z + z], has_b1 ? v1[y * Z + z] : 0.f);
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) P[lds(el(k))] = t[k];
    __syncthreads();
  } else {
    {
      float2 t[PER];
#pragma unroll
      for (int k = 0; k < PER; ++k) t[k] = Yp[el(k)];
#pragma unroll
      for (int k = 0; k < PER; ++k) P[lds(el(k))] = t[k];
    }
    __syncthreads();
    plane_cols_r<MY, MZ, true>(P, tw);
    plane_rows_r<MY, MZ, true>(P, Y, tw);
    // gate and skip on the kept Y x Z block
    const int n = a.n;
    const float* x0 = s0 + (size_t)((n + 1) * CC + c) * V + xoff;
    const float* x1 = s1 + (size_t)((n + 1) * CC + c) * V + xoff;
    const float* z0 = (n == 0) ? s0 + (size_t)c * V + xoff : a.zin + ((size_t)b0 * CC + c) * V + xoff;
    const float* z1 = (n == 0) ? s1 + (size_t)c * V + xoff
                               : a.zin + ((size_t)(has_b1 ? b1 : b0) * CC + c) * V + xoff;
    float* o0 = a.zout + ((size_t)b0 * CC + c) * V + xoff;
    float* o1 = a.zout + ((size_t)(has_b1 ? b1 : b0) * CC + c) * V + xoff;
    const float g0 = a.gate[((size_t)b0 * a.NO + n) * CC + c];
    const float g1 = has_b1 ? a.gate[((size_t)b1 * a.NO + n) * CC + c] : 0.f;
    const float dk = a.dskip[n * CC + c];
    // gate and skip inputs of this thread's kept elements: all loads first
    // where the registers allow it (up to 256 threads: 256 registers each),
    // else element by element
    constexpr bool BATCH = C::THREADS <= 256;
    constexpr int NB = BATCH ? PER : 1;
    float gx0[NB], gx1[NB], gz0[NB], gz1[NB];
    auto gate_in = [&](int k, int j) {
      const int y = el(k) / MZ, z = el(k) % MZ;
      const int q = (y < Y && z < Z) ? y * Z + z : 0;
      gx0[j] = x0[q];
      gz0[j] = z0[q];
      gx1[j] = x1[q];
      gz1[j] = z1[q];
    };
    if constexpr (BATCH) {
#pragma unroll
      for (int k = 0; k < PER; ++k) gate_in(k, k);
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int y = el(k) / MZ, z = el(k) % MZ;
      const int j = BATCH ? k : 0;
      if (!BATCH) gate_in(k, 0);
      float2 nv = make_float2(0.f, 0.f);
      if (y < Y && z < Z) {
        const int q = y * Z + z;
        const float2 cv = P[y * C::RS + z];
        const float a0 = gx0[j] * g0 * cv.x + dk * gz0[j];
        o0[q] = a0;
        float a1 = 0.f;
        if (has_b1) {
          a1 = gx1[j] * g1 * cv.y + dk * gz1[j];
          o1[q] = a1;
        }
        nv = make_float2(a0, a1);
      }
      if (MODE == PL_INV_FWD) P[y * C::RS + z] = nv;
    }
    if (MODE == PL_INV) return;
    __syncthreads();
  }
  // forward plane DFT of the (zero padded) Y x Z block
  plane_rows_r<MY, MZ, false>(P, Y, tw);
  plane_cols_r<MY, MZ, false>(P, tw);
#pragma unroll
  for (int k = 0; k < PER; ++k) Yp[el(k)] = P[lds(el(k))];
}

// Persistent plane pass for M = 128 (the 64^3 grids): items (sample pair,
// channel, x-plane) walked with a stride of gridDim.x, one 1024-thread
// workgroup per CU (the padded plane takes 133 KB of LDS). In the first forward
// the next item's v block is fetched into registers while the current one is
// transformed; the inverse passes fetch their plane when the item starts and
// the gate and skip inputs during (or, fused with the next forward, after) the
// inverse row stage.
template <int MODE>
__global__ __launch_bounds__(1024) void nd_plane128_kernel(NdConvArgs a, int nitems) {
  constexpr int M = 128;
  using C = PlaneCfg<M>;
  constexpr int PER = M * M / C::THREADS;          // plane elements per thread (16)
  constexpr int KEPT = M * M / 4 / C::THREADS;     // kept (y < Y, z < Z) positions per thread (4)
  constexpr bool INV = MODE != PL_FWD_V;
  // The first forward fetches the next item's v block during the current item.
  // The inverse modes fetch their intermediate plane when the item starts:
  // holding 16 complex values of prefetch through the transforms spills at 128
  // registers, and the spill traffic (about 0.8 GB per pass at 64^3) costs more
  // than the exposed load.
  constexpr bool PREF = MODE == PL_FWD_V;
  extern __shared__ float4 smem4[];
  float2* P = reinterpret_cast<float2*>(smem4);
  float2* tw = P + M * C::RS;
  const int X = a.X, Y = a.Y, Z = a.Z;  // Y = Z = 64
  const size_t V = (size_t)X * Y * Z;
  const size_t plane = (size_t)M * M;
  const int tid = threadIdx.x;
  if (tid < 128) tw[tid] = a.tw128[tid];
  const int CC = a.C;
  const size_t J = (size_t)(a.NO + 1) * CC;
  struct Item {
    int x, c, bp, b0, b1;
    bool has_b1;
  };
  auto item_of = [&](int item) {
    Item it;
    it.x = item % X;
    const int pc = item / X;
    it.c = pc % CC;
    it.bp = pc / CC;
    it.b0 = 2 * it.bp;
    it.has_b1 = it.b0 + 1 < a.B;
    it.b1 = it.has_b1 ? it.b0 + 1 : it.b0;
    return it;
  };
  // kept position q of this thread: i = tid + k * 1024 over the Y x Z block
  auto kept = [&](int k) { return tid + k * C::THREADS; };
  struct In {
    float2 y[INV ? PER : 1];            // intermediate plane, element tid + k * 1024
    float va[INV ? 1 : KEPT], vb[INV ? 1 : KEPT];  // v block of both samples (first forward)
  };
  auto load_in = [&](const Item& it, In& in) {
    if constexpr (INV) {
      const float2* Yp = a.Yint + (((size_t)it.bp * CC + it.c) * X + it.x) * plane;
#pragma unroll
      for (int k = 0; k < PER; ++k) in.y[k] = Yp[tid + k * C::THREADS];
    } else {
      const size_t xoff = (size_t)it.x * Y * Z;
      const float* v0 = a.p + (size_t)it.b0 * J * V + (size_t)it.c * V + xoff;
      const float* v1 = a.p + (size_t)it.b1 * J * V + (size_t)it.c * V + xoff;
#pragma unroll
      for (int k = 0; k < KEPT; ++k) {
        in.va[k] = v0[kept(k)];
        in.vb[k] = v1[kept(k)];
      }
    }
  };

  int item = blockIdx.x;
  if (item >= nitems) return;
  In in;
  if (PREF) load_in(item_of(item), in);
  while (true) {
    const int next = item + gridDim.x;
    const bool more = next < nitems;
    const Item it = item_of(item);
    float2* Yp = a.Yint + (((size_t)it.bp * CC + it.c) * X + it.x) * plane;
    const size_t xoff = (size_t)it.x * Y * Z;
    if (!PREF) load_in(it, in);
    if constexpr (INV) {
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int i = tid + k * C::THREADS;
        P[(i / M) * C::RS + i % M] = in.y[k];
      }
    } else {
      for (int i = tid; i < M * M; i += C::THREADS) P[(i / M) * C::RS + i % M] = make_float2(0.f, 0.f);
      __syncthreads();
#pragma unroll
      for (int k = 0; k < KEPT; ++k) {
        const int q = kept(k), y = q / Z, z = q % Z;
        P[y * C::RS + z] = make_float2(in.va[k], it.has_b1 ? in.vb[k] : 0.f);
      }
    }
    // the next item's v block (the last item fetches itself again)
    if (PREF) load_in(item_of(more ? next : item), in);
    if constexpr (INV) {
      // gate and skip inputs of the kept block, needed after the inverse transform
      const int n = a.n;
      const float* x0 = a.p + (size_t)it.b0 * J * V + (size_t)((n + 1) * CC + it.c) * V + xoff;
      const float* x1 = a.p + (size_t)it.b1 * J * V + (size_t)((n + 1) * CC + it.c) * V + xoff;
      const float* z0 = (n == 0) ? a.p + (size_t)it.b0 * J * V + (size_t)it.c * V + xoff
                                 : a.zin + ((size_t)it.b0 * CC + it.c) * V + xoff;
      const float* z1 = (n == 0) ? a.p + (size_t)it.b1 * J * V + (size_t)it.c * V + xoff
                                 : a.zin + ((size_t)it.b1 * CC + it.c) * V + xoff;
      __syncthreads();
      plane_cols<M, true>(P, tw);
      // gate inputs: fetched during the inverse row stage, or, in the fused
      // inverse + forward mode (more live registers), after it
      constexpr bool GLATE = MODE == PL_INV_FWD;
      float gx0[KEPT], gx1[KEPT], gz0[KEPT], gz1[KEPT];
      auto load_gate = [&]() {
#pragma unroll
        for (int k = 0; k < KEPT; ++k) {
          gx0[k] = x0[kept(k)];
          gx1[k] = x1[kept(k)];
          gz0[k] = z0[kept(k)];
          gz1[k] = z1[kept(k)];
        }
      };
      if (!GLATE) load_gate();
      plane_rows<M, true>(P, Y, tw);
      if (GLATE) load_gate();
      float* o0 = a.zout + ((size_t)it.b0 * CC + it.c) * V + xoff;
      float* o1 = a.zout + ((size_t)it.b1 * CC + it.c) * V + xoff;
      const float g0 = a.gate[((size_t)it.b0 * a.NO + n) * CC + it.c];
      const float g1 = it.has_b1 ? a.gate[((size_t)it.b1 * a.NO + n) * CC + it.c] : 0.f;
      const float dk = a.dskip[n * CC + it.c];
      // rows y >= Y of the plane must be zero for the forward transform
      if (MODE == PL_INV_FWD) {
        for (int i = tid; i < (M - Y) * M; i += C::THREADS) P[(Y + i / M) * C::RS + i % M] = make_float2(0.f, 0.f);
      }
#pragma unroll
      for (int k = 0; k < KEPT; ++k) {
        const int q = kept(k), y = q / Z, z = q % Z;
        const float2 cv = P[y * C::RS + z];
        const float a0 = gx0[k] * g0 * cv.x + dk * gz0[k];
        o0[q] = a0;
        float a1 = 0.f;
        if (it.has_b1) {
          a1 = gx1[k] * g1 * cv.y + dk * gz1[k];
          o1[q] = a1;
        }
        if (MODE == PL_INV_FWD) P[y * C::RS + z] = make_float2(a0, a1);
      }
      if (MODE == PL_INV_FWD) {
        // columns z >= Z of the kept rows must be zero too
        for (int i = tid; i < Y * (M - Z); i += C::THREADS) P[(i / (M - Z)) * C::RS + Z + i % (M - Z)] = make_float2(0.f, 0.f);
      }
    }
    if (MODE != PL_INV) {
      __syncthreads();
      // forward plane DFT of the (zero padded) Y x Z block
      plane_rows<M, false>(P, Y, tw);
      plane_cols<M, false>(P, tw);
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int i = tid + k * C::THREADS;
        Yp[i] = P[(i / M) * C::RS + i % M];
      }
    }
    if (!more) break;
    item = next;
    __syncthreads();  // P fully read before the next item writes it
  }
}

// ======================================================= pencil pass
// DFT over x of 64 consecutive (ky, kz) pencils; N1 = MX = RA * RB points,
// n1 = j + RA r, k1 = ka + RB kb. Forward: threads (lane, j < RA) hold
// x[j + RA r]; stage 2 threads (lane, ka < RB) end with X[ka + RB kb]. PAD = 2
// (zero padded: x < X = N1 / 2 non-zero and kept) or 1 (circular: all N1).
enum { PN_CONV = 0, PN_FWD_FULL = 1 };

template <int RA, int RB, int MODE, int PAD>
__global__ __launch_bounds__(64 * RA) void nd_pencil_kernel(NdConvArgs a) {
  constexpr int N1 = RA * RB;
  extern __shared__ float4 smem4[];
  float2* S = reinterpret_cast<float2*>(smem4);  // [RA][RB][64] / [RB][RA][64]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int X = a.X;
  const int MY = a.MY, MZ = a.MZ, ZH = MZ / 2 + 1;
  const size_t plane = (size_t)MY * MZ;
  const int f = blockIdx.x * 64 + lane;  // flattened (ky, kz)
  const int c = blockIdx.y, bp = blockIdx.z;
  constexpr int nin = (MODE == PN_FWD_FULL) ? RB : RB / PAD;  // non-zero r per thread
  float2* base = (MODE == PN_FWD_FULL) ? a.F + (((size_t)bp * a.npairs + c) * N1) * plane
                                       : a.Yint + (((size_t)bp * a.C + c) * X) * plane;
  // forward stage 1: threads (lane, j)
  float2 v[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) v[r] = (r < nin) ? base[(size_t)(w + RA * r) * plane + f] : make_float2(0.f, 0.f);
  Dft<RB, false>::run(v);
#pragma unroll
  for (int ka = 0; ka < RB; ++ka) {
    if (ka) v[ka] = cmul(v[ka], a.tw128[(w * ka * (128 / N1)) & 127]);
    S[(w * RB + ka) * 64 + lane] = v[ka];
  }
  __syncthreads();
  float2 u[RA];
  const bool act2 = w < RB;  // stage-2 threads (lane, ka = w)
  if (act2) {
#pragma unroll
    for (int j = 0; j < RA; ++j) u[j] = S[(j * RB + w) * 64 + lane];
    Dft<RA, false>::run(u);
  }
  if constexpr (MODE == PN_FWD_FULL) {
    if (act2) {
#pragma unroll
      for (int kb = 0; kb < RA; ++kb) base[(size_t)(w + RB * kb) * plane + f] = u[kb];
    }
    return;
  }
  if (act2) {
    // times K^_c(kx, ky, kz); kz > Z from the conjugate symmetric half spectrum
    const int ky = f / MZ, kz = f % MZ;
    const float2* Kc = a.kh + (size_t)(a.n * a.C + c) * N1 * MY * ZH;
    const bool lower = kz <= MZ / 2;
    const int ky2 = lower ? ky : (MY - ky) % MY;
    const int kz2 = lower ? kz : MZ - kz;
#pragma unroll
    for (int kb = 0; kb < RA; ++kb) {
      const int kx = w + RB * kb;
      const int kx2 = lower ? kx : (N1 - kx) % N1;
      float2 kv = Kc[((size_t)kx2 * MY + ky2) * ZH + kz2];
      if (!lower) kv = conjf2(kv);
      u[kb] = cmul(u[kb], kv);
    }
    // inverse stage 1 on the same threads: IDFT over kb -> B[na]
    Dft<RA, true>::run(u);
#pragma unroll
    for (int na = 0; na < RA; ++na) {
      if (na) u[na] = cmulc(u[na], a.tw128[(w * na * (128 / N1)) & 127]);
    }
  }
  __syncthreads();  // everyone finished reading S
  if (act2) {
#pragma unroll
    for (int na = 0; na < RA; ++na) S[(w * RA + na) * 64 + lane] = u[na];
  }
  __syncthreads();
  // inverse stage 2: threads (lane, na = w < RA), IDFT over ka -> x = na + RA nb
  float2 q[RB];
#pragma unroll
  for (int ka = 0; ka < RB; ++ka) q[ka] = S[(ka * RA + w) * 64 + lane];
  Dft<RB, true>::run(q);
#pragma unroll
  for (int nb = 0; nb < RB / PAD; ++nb) base[(size_t)(w + RA * nb) * plane + f] = q[nb];
}

// Persistent pencil pass for 2X = 128 (the 64^3 grids), conv mode: items are
// (sample pair, channel, block of 64 pencils) walked with a stride of
// gridDim.x by 512-thread workgroups (8 waves, two workgroups per CU). Same
// decomposition as nd_pencil_kernel (n1 = j + 16 r, k1 = ka + 8 kb), with every
// wave busy in both stages: stage 1 (x -> r) runs the DFT-8s of j = w and
// j = w + 8, stage 2 the DFT-16 of ka = w. Each item's input column and
// kernel spectrum entries are in registers when it starts: the next item's are
// fetched as soon as the current one has used them (the last item fetches
// itself again, so that the loads stay unconditional).
__global__ __launch_bounds__(512) void nd_pencil128_kernel(NdConvArgs a, int nitems) {
  constexpr int N1 = 128, RA = 16, RB = 8;
  extern __shared__ float4 smem4[];
  float2* S = reinterpret_cast<float2*>(smem4);  // [RA][RB][64] forward, [RB][RA][64] inverse
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int X = a.X, Y = a.Y, Z = a.Z;
  const int MY = 2 * Y, MZ = 2 * Z, ZH = Z + 1;
  const size_t plane = (size_t)MY * MZ;
  const int nfb = MY * MZ / 64;  // pencil blocks per channel
  struct Item {
    float2* base;        // Yint of (pair, channel), plane 0
    const float2* Kc;    // half spectrum of (order, channel)
    int f;               // this lane's pencil (ky, kz) = (f / MZ, f % MZ)
  };
  auto item_of = [&](int item) {
    Item it;
    const int fb = item % nfb, pc = item / nfb;  // pc = bp * C + c
    const int c = pc % a.C;
    it.base = a.Yint + (size_t)pc * X * plane;
    it.Kc = a.kh + (size_t)(a.n * a.C + c) * N1 * MY * ZH;
    it.f = fb * 64 + lane;
    return it;
  };
  struct In {
    float2 y[2][RB / 2];  // x = j + 16 r, j in {w, w + 8}, r < 4 (x < X = 64)
    float2 k[RA];         // K^(kx = w + 8 kb, ky, kz), conjugated where taken from -k
  };
  auto load_y = [&](const Item& it, In& in) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int r = 0; r < RB / 2; ++r) in.y[jj][r] = it.base[(size_t)(w + 8 * jj + RA * r) * plane + it.f];
  };
  auto load_k = [&](const Item& it, In& in) {
    const int ky = it.f / MZ, kz = it.f % MZ;
    const bool lower = kz <= Z;
    const int ky2 = lower ? ky : (MY - ky) % MY;
    const int kz2 = lower ? kz : MZ - kz;
#pragma unroll
    for (int kb = 0; kb < RA; ++kb) {
      const int kx = w + RB * kb;
      const int kx2 = lower ? kx : (N1 - kx) % N1;
      const float2 kv = it.Kc[((size_t)kx2 * MY + ky2) * ZH + kz2];
      in.k[kb] = lower ? kv : conjf2(kv);
    }
  };

  int item = blockIdx.x;
  if (item >= nitems) return;
  In in;
  {
    const Item it = item_of(item);
    load_y(it, in);
    load_k(it, in);
  }
  while (true) {
    const int next = item + gridDim.x;
    const bool more = next < nitems;
    const Item it = item_of(item), nt = item_of(more ? next : item);
    // forward stage 1: DFT-8 over r of j = w and w + 8, inner twiddles W_128^(j ka)
    float2 v[2][RB];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int r = 0; r < RB; ++r) v[jj][r] = r < RB / 2 ? in.y[jj][r] : make_float2(0.f, 0.f);
    load_y(nt, in);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = w + 8 * jj;
      Dft<RB, false>::run(v[jj]);
#pragma unroll
      for (int ka = 0; ka < RB; ++ka) {
        if (ka) v[jj][ka] = cmul(v[jj][ka], a.tw128[(j * ka) & 127]);
        S[(j * RB + ka) * 64 + lane] = v[jj][ka];
      }
    }
    __syncthreads();
    // stage 2: DFT-16 over j for ka = w: X[w + 8 kb]
    float2 u[RA];
#pragma unroll
    for (int j = 0; j < RA; ++j) u[j] = S[(j * RB + w) * 64 + lane];
    Dft<RA, false>::run(u);
#pragma unroll
    for (int kb = 0; kb < RA; ++kb) u[kb] = cmul(u[kb], in.k[kb]);
    load_k(nt, in);
    // inverse stage 2 on the same threads, then the inner twiddles
    Dft<RA, true>::run(u);
#pragma unroll
    for (int na = 1; na < RA; ++na) u[na] = cmulc(u[na], a.tw128[(w * na) & 127]);
    __syncthreads();  // everyone finished reading S
#pragma unroll
    for (int na = 0; na < RA; ++na) S[(w * RA + na) * 64 + lane] = u[na];
    __syncthreads();
    // inverse stage 1: DFT-8 over ka for na = w and w + 8 -> x = na + 16 nb, nb < 4
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int na = w + 8 * jj;
      float2 q[RB];
#pragma unroll
      for (int ka = 0; ka < RB; ++ka) q[ka] = S[(ka * RA + na) * 64 + lane];
      Dft<RB, true>::run(q);
#pragma unroll
      for (int nb = 0; nb < RB / 2; ++nb) it.base[(size_t)(na + RA * nb) * plane + it.f] = q[nb];
    }
    if (!more) break;
    item = next;
    __syncthreads();  // S of this item fully read before the next one writes it
  }
}

// Persistent pencil pass for 2X = 2Z = 128 with mirrored pencil blocks in one
// item. The kernel spectrum is kept for kz <= Z only; a pencil with kz > Z
// uses the conjugates of the entries of its mirror image (-ky, MZ - kz). An
// item is the block pair A = (ky, kz < 64) and B = (MY - ky, kz >= 64) of one
// (sample pair, channel): pencil kz in [1, 63] of A and pencil 128 - kz of B
// are mirror images, so A reads their spectrum entries once and leaves them in
// LDS for B (B's entry at kx is A's at -kx, conjugated; B's kz = 64 pencil,
// which lies on the kept plane, reads its own). The workgroup runs A, then B,
// each with the decomposition of nd_pencil128_kernel; every block's inputs are
// fetched while the block before it runs.
__global__ __launch_bounds__(512) void nd_pencil128p_kernel(NdConvArgs a, int nitems) {
  constexpr int N1 = 128, RA = 16, RB = 8;
  extern __shared__ float4 smem4[];
  float2* S = reinterpret_cast<float2*>(smem4);  // [RA][RB][64] forward, [RB][RA][64] inverse
  float2* KA = S + RA * RB * 64;                  // A's spectrum entries [kx][lane], read by B
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int X = a.X, MY = a.MY;
  constexpr int MZ = 128, ZH = 65;
  const size_t plane = (size_t)MY * MZ;
  struct Blk {
    float2* base;      // Yint of (pair, channel), plane 0
    const float2* Kr;  // kept entries read by this lane: row (kx = 0, ky or B's row, kz)
    int f;             // this lane's pencil (ky, kz) = (f / MZ, f % MZ)
  };
  // block q of this workgroup's sequence: item blockIdx.x + (q / 2) gridDim.x, A for even q
  auto blk_of = [&](int item, bool isB) {
    Blk bk;
    const int ky = item % MY, pc = item / MY;  // pc = bp * C + c
    const int c = pc % a.C;
    const int kyb = (MY - ky) % MY;
    bk.base = a.Yint + (size_t)pc * X * plane;
    // every lane of B reads the kz = 64 column (only its lane 0 uses it), so
    // that the loads stay unconditional
    bk.Kr = a.kh + (size_t)(a.n * a.C + c) * N1 * MY * ZH + (size_t)(isB ? kyb : ky) * ZH + (isB ? 64 : lane);
    bk.f = isB ? kyb * MZ + 64 + lane : ky * MZ + lane;
    return bk;
  };
  struct In {
    float2 y[2][RB / 2];  // x = j + 16 r, j in {w, w + 8}, r < 4 (x < X = 64)
    float2 k[RA];         // kept entries at kx = w + 8 kb
  };
  auto load_y = [&](const Blk& bk, In& in) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int r = 0; r < RB / 2; ++r) in.y[jj][r] = bk.base[(size_t)(w + 8 * jj + RA * r) * plane + bk.f];
  };
  auto load_k = [&](const Blk& bk, In& in) {
#pragma unroll
    for (int kb = 0; kb < RA; ++kb) in.k[kb] = bk.Kr[(size_t)(w + RB * kb) * MY * ZH];
  };

  // one block; nb: the block after it (itself for the last one)
  auto run = [&](auto isBc, const Blk& bk, const Blk& nb, In& in) {
    constexpr bool isB = decltype(isBc)::value;
    // forward stage 1: DFT-8 over r of j = w and w + 8, inner twiddles W_128^(j ka)
    float2 v[2][RB];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int r = 0; r < RB; ++r) v[jj][r] = r < RB / 2 ? in.y[jj][r] : make_float2(0.f, 0.f);
    load_y(nb, in);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = w + 8 * jj;
      Dft<RB, false>::run(v[jj]);
#pragma unroll
      for (int ka = 0; ka < RB; ++ka) {
        if (ka) v[jj][ka] = cmul(v[jj][ka], a.tw128[(j * ka) & 127]);
        S[(j * RB + ka) * 64 + lane] = v[jj][ka];
      }
    }
    __syncthreads();
    // stage 2: DFT-16 over j for ka = w: X[w + 8 kb]
    float2 u[RA];
#pragma unroll
    for (int j = 0; j < RA; ++j) u[j] = S[(j * RB + w) * 64 + lane];
    Dft<RA, false>::run(u);
    if constexpr (!isB) {
#pragma unroll
      for (int kb = 0; kb < RA; ++kb) {
        KA[(w + RB * kb) * 64 + lane] = in.k[kb];
        u[kb] = cmul(u[kb], in.k[kb]);
      }
    } else {
      // pencil 64 + lane of B mirrors pencil 64 - lane of A
#pragma unroll
      for (int kb = 0; kb < RA; ++kb) {
        const int kxm = (N1 - (w + RB * kb)) & (N1 - 1);
        const float2 km = conjf2(KA[kxm * 64 + ((64 - lane) & 63)]);
        u[kb] = cmul(u[kb], lane ? km : in.k[kb]);
      }
    }
    load_k(nb, in);
    // inverse stage 2 on the same threads, then the inner twiddles
    Dft<RA, true>::run(u);
#pragma unroll
    for (int na = 1; na < RA; ++na) u[na] = cmulc(u[na], a.tw128[(w * na) & 127]);
    __syncthreads();  // everyone finished reading S (and, after B, KA)
#pragma unroll
    for (int na = 0; na < RA; ++na) S[(w * RA + na) * 64 + lane] = u[na];
    __syncthreads();
    // inverse stage 1: DFT-8 over ka for na = w and w + 8 -> x = na + 16 nb, nb < 4
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int na = w + 8 * jj;
      float2 q[RB];
#pragma unroll
      for (int ka = 0; ka < RB; ++ka) q[ka] = S[(ka * RA + na) * 64 + lane];
      Dft<RB, true>::run(q);
#pragma unroll
      for (int nb2 = 0; nb2 < RB / 2; ++nb2) bk.base[(size_t)(na + RA * nb2) * plane + bk.f] = q[nb2];
    }
    __syncthreads();  // S fully read before the next block writes it
  };

  using TA = std::integral_constant<bool, false>;
  using TB = std::integral_constant<bool, true>;
  int item = blockIdx.x;
  if (item >= nitems) return;
  In in;
  {
    const Blk bk = blk_of(item, false);
    load_y(bk, in);
    load_k(bk, in);
  }
  while (true) {
    const int next = item + gridDim.x;
    const bool more = next < nitems;
    const Blk ba = blk_of(item, false), bb = blk_of(item, true);
    run(TA{}, ba, bb, in);
    run(TB{}, bb, blk_of(more ? next : item, !more), in);
    if (!more) break;
    item = next;
  }
}

// ========================================================= channel mean
__global__ __launch_bounds__(256) void nd_mean_partial_kernel(const float* __restrict__ u, float* __restrict__ part,
                                                              int C, int V, int chunk) {
  const int ch = blockIdx.x, b = blockIdx.y;
  const float* ub = u + ((size_t)b * V + (size_t)ch * chunk) * C;
  for (int c = threadIdx.x; c < C; c += 256) {
    float s = 0.f;
    for (int v = 0; v < chunk; ++v) s += ub[(size_t)v * C + c];
    part[((size_t)b * gridDim.x + ch) * C + c] = s;
  }
}

// Means and gates for any C (a multiple of 64): one workgroup per (sample,
// block of 64 channels); four groups of 64 threads sum interleaved partial rows
// with independent accumulators, combined in LDS.
__global__ __launch_bounds__(256) void nd_gate_kernel(const float* __restrict__ part, const float* __restrict__ ga,
                                                      const float* __restrict__ gb, float* __restrict__ gate, int NO,
                                                      int C, int nch, int V) {
  __shared__ float red[256];
  const int t = threadIdx.x, b = blockIdx.y;
  const int c = blockIdx.x * 64 + (t & 63), g = t >> 6;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  int k = g;
  for (; k + 12 < nch; k += 16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] += part[((size_t)b * nch + k + 4 * j) * C + c];
  }
  for (; k < nch; k += 4) acc[0] += part[((size_t)b * nch + k) * C + c];
  red[t] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  if (t < 64) {
    const float m = ((red[t] + red[t + 64]) + (red[t + 128] + red[t + 192])) / (float)V;
    for (int n = 0; n < NO; ++n) {
      const float arg = ga[n * C + c] * m + gb[n * C + c];
      gate[((size_t)b * NO + n) * C + c] = 1.f / (1.f + expf(-arg));
    }
  }
}

// Faster forms for C dividing 256 (C = 64, 128, 256): a voxel chunk of the
// channels-last input is one contiguous run of chunk * C floats, read 256 at a
// time with independent partial sums; thread t always meets channel t % C, and
// the 256 / C threads of a channel are combined in LDS.
__global__ __launch_bounds__(256) void nd_mean_partial256_kernel(const float* __restrict__ u, float* __restrict__ part,
                                                                 int C, int V, int chunk) {
  __shared__ float red[256];
  const int ch = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const float* ub = u + ((size_t)b * V + (size_t)ch * chunk) * C;
  const int n = chunk * C;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  int i = t;
  for (; i + 3 * 256 < n; i += 4 * 256) {
    s0 += ub[i];
    s1 += ub[i + 256];
    s2 += ub[i + 2 * 256];
    s3 += ub[i + 3 * 256];
  }
  for (; i < n; i += 256) s0 += ub[i];
  red[t] = (s0 + s1) + (s2 + s3);
  __syncthreads();
  if (t < C) {
    float s = 0.f;
    for (int r = t; r < 256; r += C) s += red[r];
    part[((size_t)b * gridDim.x + ch) * C + t] = s;
  }
}

__global__ __launch_bounds__(256) void nd_gate256_kernel(const float* __restrict__ part, const float* __restrict__ ga,
                                                         const float* __restrict__ gb, float* __restrict__ gate,
                                                         int NO, int C, int nch, int V) {
  __shared__ float red[256];
  const int b = blockIdx.x, t = threadIdx.x;
  const int c = t % C, R = 256 / C;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int k = t / C;
  for (; k + 7 * R < nch; k += 8 * R) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += part[((size_t)b * nch + k + j * R) * C + c];
  }
  for (; k < nch; k += R) acc[0] += part[((size_t)b * nch + k) * C + c];
  red[t] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  __syncthreads();
  if (t < C) {
    float s = 0.f;
    for (int r = t; r < 256; r += C) s += red[r];
    const float m = s / (float)V;
    for (int n = 0; n < NO; ++n) {
      const float arg = ga[n * C + c] * m + gb[n * C + c];
      gate[((size_t)b * NO + n) * C + c] = 1.f / (1.f + expf(-arg));
    }
  }
}

// ================================================= 2D grids (X = 1)
// A 2D grid (Y x Z, a single x-plane) has dx = 0 for every offset: the
// transform over x is the identity, and each (sample pair, channel) plane runs
// all orders in LDS: forward 2D DFT of the (zero padded) block, product with
// the channel's half spectrum, inverse 2D DFT, crop, gate and skip, and the
// next order from the same plane. HBM sees v, x^n, the spectra and z^{N+1}
// only. Items (channel, sample pair), pair index fastest, are dealt so that the
// workgroups of one XCD (blockIdx mod 8) take consecutive items: the pairs of
// a channel read its spectrum through that XCD's L2. The plane is MY x MZ
// (transform lengths along y and z), each side on its own.
//
// PQ: a kernel per sample (a.kh_stride != 0), the (P, Q) spectral product.
template <int MY, int MZ, bool CIRC, bool PQ>
__global__ __launch_bounds__((PlaneCfg<MY, MZ>::THREADS)) void nd_plane2d_kernel(NdConvArgs a, int per_xcd) {
  using C = PlaneCfg<MY, MZ>;
  constexpr int NT = C::THREADS;
  constexpr int PER = C::PER;                       // plane elements per thread
  constexpr int KEPT = CIRC ? PER : (PER + 3) / 4;  // kept positions per thread (a quarter when padded)
  constexpr int ZH = MZ / 2 + 1;
  // Smaller planes fetch the spectrum entries before the forward transform and
  // the gate inputs before the inverse; 1024-thread planes (128 x 128, 128
  // registers per thread) fetch them where they are used.
  constexpr bool EARLY = NT < 1024;
  static_assert(PER * NT == MY * MZ, "plane split");
  extern __shared__ float4 smem4[];
  float2* P = reinterpret_cast<float2*>(smem4);
  float2* tw = P + MY * C::RS;
  const int tid = threadIdx.x;
  const int BP = (a.B + 1) / 2, CC = a.C;
  const int item = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (item >= BP * CC) return;  // the whole workgroup, before any barrier
  for (int i = tid; i < 128; i += NT) tw[i] = a.tw128[i];
  const int c = item / BP, bp = item % BP;
  const int b0 = 2 * bp;
  const bool has_b1 = b0 + 1 < a.B;
  const int b1 = has_b1 ? b0 + 1 : b0;
  const int Y = a.Y, Z = a.Z, V = Y * Z;
  const size_t J = (size_t)(a.NO + 1) * CC;
  const float* s0 = a.p + (size_t)b0 * J * V;
  const float* s1 = a.p + (size_t)b1 * J * V;
  // z^n of both samples at the kept positions q = tid + k NT (q < V), in registers
  float z0[KEPT], z1[KEPT];
#pragma unroll
  for (int k = 0; k < KEPT; ++k) {
    const int q = tid + k * NT;
    z0[k] = q < V ? s0[(size_t)c * V + q] : 0.f;
    z1[k] = (q < V && has_b1) ? s1[(size_t)c * V + q] : 0.f;
  }
  for (int n = 0; n < a.NO; ++n) {
    // spectrum entries of this thread's bins i = tid + e NT; bins with kz > MZ/2
    // come from the conjugate of bin -k
    const float2* Kc = a.kh + (size_t)(n * CC + c) * MY * ZH;
    float2 kk[PER];
    auto load_k = [&]() {
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int i = tid + e * NT;
        const int ky = i / MZ, kz = i % MZ;
        const bool lower = kz <= MZ / 2;
        const int ky2 = lower ? ky : (MY - ky) % MY;
        const int kz2 = lower ? kz : MZ - kz;
        const float2 kv = Kc[ky2 * ZH + kz2];
        kk[e] = lower ? kv : conjf2(kv);
      }
    };
    if (EARLY && !PQ) load_k();
    if (!CIRC) {
      for (int i = tid; i < MY * MZ; i += NT) P[(i / MZ) * C::RS + i % MZ] = make_float2(0.f, 0.f);
      __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < KEPT; ++k) {
      const int q = tid + k * NT;
      if (q < V) P[(q / Z) * C::RS + q % Z] = make_float2(z0[k], z1[k]);
    }
    __syncthreads();
    plane_rows_r<MY, MZ, false>(P, Y, tw);
    plane_cols_r<MY, MZ, false>(P, tw);
    if constexpr (!PQ) {
      if (!EARLY) load_k();
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int i = tid + e * NT;
        float2* pe = P + (i / MZ) * C::RS + i % MZ;
        *pe = cmul(*pe, kk[e]);
      }
    } else {
      // a kernel per sample: Y(k) = P F(k) + Q conj F(-k), P, Q the half sum and
      // difference of the two samples' spectra (P(-k) = conj P(k), Q likewise).
      // A thread takes whole bin pairs {k, -k} of the canonical half (rows 1 ..
      // MY/2 - 1, and kz <= MZ/2 on rows 0 and MY/2, their own mirrors): it reads
      // both bins and writes both, so every bin has one reader and one writer.
      const float2* K0 = a.kh + (size_t)b0 * a.kh_stride + (size_t)(n * CC + c) * MY * ZH;
      const float2* K1 = a.kh + (size_t)b1 * a.kh_stride + (size_t)(n * CC + c) * MY * ZH;
      constexpr int INNER = (MY / 2 - 1) * MZ, NPAIR = INNER + 2 * (MZ / 2 + 1);
      for (int pr = tid; pr < NPAIR; pr += NT) {
        int ky, kz;
        if (pr < INNER) {
          ky = 1 + pr / MZ;
          kz = pr % MZ;
        } else {
          const int e2 = pr - INNER;
          ky = e2 < MZ / 2 + 1 ? 0 : MY / 2;
          kz = e2 % (MZ / 2 + 1);
        }
        const int kym = (MY - ky) % MY, kzm = (MZ - kz) % MZ;
        // half-spectrum entry at k (kz <= MZ/2) or the conjugate of the one at -k
        const bool lower = kz <= MZ / 2;
        const int o = lower ? ky * ZH + kz : kym * ZH + kzm;
        float2 k0 = K0[o], k1 = K1[o];
        if (!lower) {
          k0 = conjf2(k0);
          k1 = conjf2(k1);
        }
        const float2 Pk = make_float2(0.5f * (k0.x + k1.x), 0.5f * (k0.y + k1.y));
        const float2 Qk = make_float2(0.5f * (k0.x - k1.x), 0.5f * (k0.y - k1.y));
        float2* pa = P + ky * C::RS + kz;
        float2* pb = P + kym * C::RS + kzm;
        const float2 A = *pa, Bm = *pb;
        *pa = cadd(cmul(A, Pk), cmul(conjf2(Bm), Qk));
        if (pb != pa) *pb = cadd(cmul(Bm, conjf2(Pk)), cmul(conjf2(A), conjf2(Qk)));
      }
    }
    // gate inputs, used after the inverse transform
    const float* x0 = s0 + (size_t)((n + 1) * CC + c) * V;
    const float* x1 = s1 + (size_t)((n + 1) * CC + c) * V;
    float xa[KEPT], xb[KEPT];
    auto load_x = [&]() {
#pragma unroll
      for (int k = 0; k < KEPT; ++k) {
        const int q = tid + k * NT;
        xa[k] = q < V ? x0[q] : 0.f;
        xb[k] = q < V ? x1[q] : 0.f;
      }
    };
    if (EARLY) load_x();
    __syncthreads();
    plane_cols_r<MY, MZ, true>(P, tw);
    plane_rows_r<MY, MZ, true>(P, Y, tw);
    if (!EARLY) load_x();
    const float g0 = a.gate[((size_t)b0 * a.NO + n) * CC + c];
    const float g1 = has_b1 ? a.gate[((size_t)b1 * a.NO + n) * CC + c] : 0.f;
    const float dk = a.dskip[n * CC + c];
#pragma unroll
    for (int k = 0; k < KEPT; ++k) {
      const int q = tid + k * NT;
      if (q < V) {
        const float2 cv = P[(q / Z) * C::RS + q % Z];
        z0[k] = xa[k] * g0 * cv.x + dk * z0[k];
        z1[k] = xb[k] * g1 * cv.y + dk * z1[k];
      }
    }
    __syncthreads();  // the plane is refilled by the next order
  }
  float* o0 = a.zfinal + ((size_t)b0 * CC + c) * V;
  float* o1 = a.zfinal + ((size_t)b1 * CC + c) * V;
#pragma unroll
  for (int k = 0; k < KEPT; ++k) {
    const int q = tid + k * NT;
    if (q < V) {
      o0[q] = z0[k];
      if (has_b1) o1[q] = z1[k];
    }
  }
}

// ============================================================ launchers

static hipError_t nd_allow_lds(const void* fn, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int MY, int MZ, int MODE>
static hipError_t launch_plane_t(const NdConvArgs& a, dim3 grid, hipStream_t s) {
  using C = PlaneCfg<MY, MZ>;
  auto fn = nd_plane_kernel<MY, MZ, MODE>;
  hipError_t e = nd_allow_lds((const void*)fn, C::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, grid, dim3(C::THREADS), C::LDS, s, a);
  return hipGetLastError();
}

template <int MY, int MODE>
static hipError_t launch_plane_z(const NdConvArgs& a, dim3 grid, hipStream_t s) {
  switch (a.MZ) {
    case 8: return launch_plane_t<MY, 8, MODE>(a, grid, s);
    case 16: return launch_plane_t<MY, 16, MODE>(a, grid, s);
    case 32: return launch_plane_t<MY, 32, MODE>(a, grid, s);
    case 64: return launch_plane_t<MY, 64, MODE>(a, grid, s);
    case 128: return launch_plane_t<MY, 128, MODE>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int MODE>
static hipError_t launch_plane(const NdConvArgs& a, dim3 grid, hipStream_t s) {
  switch (a.MY) {
    case 8: return launch_plane_z<8, MODE>(a, grid, s);
    case 16: return launch_plane_z<16, MODE>(a, grid, s);
    case 32: return launch_plane_z<32, MODE>(a, grid, s);
    case 64: return launch_plane_z<64, MODE>(a, grid, s);
    case 128: return launch_plane_z<128, MODE>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

// Pencil pass with a kernel per sample. The packed field F = Z_b0 + i Z_b1
// holds two samples whose real kernels differ, so the product is
//   Y(k) = P(k) F(k) + Q(k) conj(F(-k)),  P = (K_b0 + K_b1) / 2,  Q = (K_b0 - K_b1) / 2,
// whose inverse transform is (K_b0 * z_b0) + i (K_b1 * z_b1). F(-k) of pencil
// (ky, kz) lies on the mirror pencil (-ky, -kz) at -kx, so each lane takes a
// pencil and its mirror: both forward DFTs over x land in two [N1][64] LDS
// buffers; the thread owning kx reads A(kx) and B(-kx), which are exactly the
// inputs of pencil A's product at kx and pencil B's at -kx, and writes both
// back in place (no other thread reads those two slots); then both inverse DFTs.
// Each pair is taken once: lanes cover rows ky in [0, MY/2]; on rows 0 and MY/2
// (their own mirrors) only kz <= MZ/2 is active, the other lanes compute on
// pencil 0 and store nothing. Grid (ceil((MY/2 + 1) MZ / 64), C, sample pairs).
// SPLIT: the kernel-spectrum pass instead. F = K_a + i K_b is a channel pair's
// full field (all N1 x inputs); after the forward DFTs the thread owning kx
// forms both channels' half spectra, Ka = (F(k) + conj F(-k)) / 2 and
// Kb = (F(k) - conj F(-k)) / 2i scaled by 1 / (MX MY MZ), for pencil A at kx and
// pencil B at -kx wherever kz <= MZ/2, into a.kh; no inverse. Grid
// (ceil((MY/2 + 1) MZ / 64), channel pairs).
template <int RA, int RB, int PAD, bool SPLIT>
__global__ __launch_bounds__(64 * RA) void nd_pencil_pq_kernel(NdConvArgs a) {
  constexpr int N1 = RA * RB;
  extern __shared__ float4 smem4[];
  float2* SA = reinterpret_cast<float2*>(smem4);  // [N1][64]: stage buffer, then pencil A's spectrum
  float2* SB = SA + N1 * 64;                      // the same for the mirror pencil B
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int X = a.X, MY = a.MY, MZ = a.MZ, ZH = MZ / 2 + 1;
  const size_t plane = (size_t)MY * MZ;
  const int c = blockIdx.y, bp = blockIdx.z;
  const int fl = blockIdx.x * 64 + lane;
  const int kyl = fl / MZ, kzl = fl % MZ;
  const bool active = fl < (MY / 2 + 1) * MZ && !((kyl == 0 || kyl == MY / 2) && kzl > MZ / 2);
  const int f = active ? fl : 0;
  const int ky = f / MZ, kz = f % MZ;
  const int kyb = (MY - ky) % MY, kzb = (MZ - kz) % MZ;
  const int fb = kyb * MZ + kzb;
  float2* base = SPLIT ? a.F + (size_t)c * N1 * plane : a.Yint + (((size_t)bp * a.C + c) * X) * plane;
  const int b0 = 2 * bp, b1 = b0 + 1 < a.B ? b0 + 1 : b0;
  const size_t kofs = (size_t)(a.n * a.C + c) * N1 * MY * ZH;
  const float2* K0 = a.kh + (size_t)b0 * a.kh_stride + kofs;
  const float2* K1 = a.kh + (size_t)b1 * a.kh_stride + kofs;
  // K^(kx, y, z) from the conjugate-symmetric half spectrum
  auto kval = [&](const float2* K, int kx, int y, int z) {
    const bool lower = z <= MZ / 2;
    const int x2 = lower ? kx : (N1 - kx) % N1, y2 = lower ? y : (MY - y) % MY, z2 = lower ? z : MZ - z;
    const float2 v = K[((size_t)x2 * MY + y2) * ZH + z2];
    return lower ? v : conjf2(v);
  };
  // Waves [0, RB) work on pencil A and, when there are enough waves (RA >= 2 RB),
  // waves [RB, 2 RB) on pencil B at the same time in the 16-point stages and the
  // products; otherwise the same waves take B after A. All RA waves run the
  // 8-point stages, A then B.
  constexpr bool PAR = RA >= 2 * RB;
  constexpr int NW = PAR ? 2 * RB : RB;  // waves of the product loop
  const bool onB = PAR && w >= RB && w < 2 * RB;
  const bool on16 = w < RB || onB;       // this wave runs a 16-point stage
  const int ka = onB ? w - RB : w;
  float2* D = onB ? SB : SA;

  // forward stage 1 (x = w + RA r, r < RB / PAD non-zero) into the stage layout
  auto stage1 = [&](int g, float2* E) {
    float2 v[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) v[r] = (r < RB / PAD) ? base[(size_t)(w + RA * r) * plane + g] : make_float2(0.f, 0.f);
    Dft<RB, false>::run(v);
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      if (k) v[k] = cmul(v[k], a.tw128[(w * k * (128 / N1)) & 127]);
      E[(w * RB + k) * 64 + lane] = v[k];
    }
  };
  // forward stage 2 of buffer E for column k (DFT over j), result to E[kx][lane]
  auto stage2 = [&](float2* E, int k, bool run) {
    float2 u[RA];
    if (run) {
#pragma unroll
      for (int j = 0; j < RA; ++j) u[j] = E[(j * RB + k) * 64 + lane];
      Dft<RA, false>::run(u);
    }
    __syncthreads();
    if (run) {
#pragma unroll
      for (int kb = 0; kb < RA; ++kb) E[(k + RB * kb) * 64 + lane] = u[kb];
    }
  };
  // inverse stage 1 of buffer E for column k: spectrum E[kx] -> stage layout
  auto istage1 = [&](float2* E, int k, bool run) {
    float2 y[RA];
    if (run) {
#pragma unroll
      for (int kb = 0; kb < RA; ++kb) y[kb] = E[(k + RB * kb) * 64 + lane];
    }
    __syncthreads();
    if (run) {
      Dft<RA, true>::run(y);
#pragma unroll
      for (int na = 1; na < RA; ++na) y[na] = cmulc(y[na], a.tw128[(k * na * (128 / N1)) & 127]);
#pragma unroll
      for (int na = 0; na < RA; ++na) E[(k * RA + na) * 64 + lane] = y[na];
    }
  };
  // inverse stage 2 (all waves): stage layout of E -> pencil g, x < X
  auto istage2 = [&](const float2* E, int g) {
    float2 q[RB];
#pragma unroll
    for (int k = 0; k < RB; ++k) q[k] = E[(k * RA + w) * 64 + lane];
    Dft<RB, true>::run(q);
    if (active) {
#pragma unroll
      for (int nb = 0; nb < RB / PAD; ++nb) base[(size_t)(w + RA * nb) * plane + g] = q[nb];
    }
  };

  stage1(f, SA);
  stage1(fb, SB);
  __syncthreads();
  stage2(D, ka, on16);
  if (!PAR) {
    __syncthreads();
    stage2(SB, w, w < RB);
  }
  __syncthreads();
  if constexpr (SPLIT) {
    if (w < NW && active) {
      const size_t PH = (size_t)N1 * MY * ZH;
      float2* Ka = const_cast<float2*>(a.kh) + (size_t)(2 * c) * PH;
      float2* Kb = Ka + PH;
      const float sc = 0.5f / (float)((size_t)N1 * plane);
      const int kc = w % RB, h = w / RB;
      constexpr int KBN = RA * RB / NW;  // kb per wave
#pragma unroll
      for (int i = 0; i < KBN; ++i) {
        const int kx = kc + RB * (h * KBN + i), km = (N1 - kx) % N1;
        const float2 A = SA[kx * 64 + lane], Bm = SB[km * 64 + lane];
        if (kz <= MZ / 2) {  // pencil A at (kx, ky, kz): partner conj(B(-kx))
          const float2 fm = conjf2(Bm), hs = cadd(A, fm), d = csub(A, fm);
          const size_t o = ((size_t)kx * MY + ky) * ZH + kz;
          Ka[o] = make_float2(sc * hs.x, sc * hs.y);
          Kb[o] = make_float2(sc * d.y, -sc * d.x);
        }
        // pencil B at (-kx, -ky, -kz): partner conj(A(kx)); a pencil that is its
        // own mirror has all its entries written as pencil A already (one
        // writer per entry: the two copies' DFTs need not agree to the last bit)
        if (kzb <= MZ / 2 && fb != f) {
          const float2 fm = conjf2(A), hs = cadd(Bm, fm), d = csub(Bm, fm);
          const size_t o = ((size_t)km * MY + kyb) * ZH + kzb;
          Ka[o] = make_float2(sc * hs.x, sc * hs.y);
          Kb[o] = make_float2(sc * d.y, -sc * d.x);
        }
      }
    }
    return;
  }
  if (w < NW) {
    const int kc = w % RB, h = w / RB;
    constexpr int KBN = RA * RB / NW;  // kb per wave
#pragma unroll
    for (int i = 0; i < KBN; ++i) {
      const int kx = kc + RB * (h * KBN + i), km = (N1 - kx) % N1;
      const float2 A = SA[kx * 64 + lane], Bm = SB[km * 64 + lane];
      // pencil A at k = (kx, ky, kz)
      const float2 p0 = kval(K0, kx, ky, kz), p1 = kval(K1, kx, ky, kz);
      const float2 P = make_float2(0.5f * (p0.x + p1.x), 0.5f * (p0.y + p1.y));
      const float2 Q = make_float2(0.5f * (p0.x - p1.x), 0.5f * (p0.y - p1.y));
      // pencil B at -k: its own value B(-kx), partner A(kx); the kernels are
      // real, so P(-k) = conj P(k) and Q(-k) = conj Q(k)
      SA[kx * 64 + lane] = cadd(cmul(A, P), cmul(conjf2(Bm), Q));
      SB[km * 64 + lane] = cadd(cmul(Bm, conjf2(P)), cmul(conjf2(A), conjf2(Q)));
    }
  }
  __syncthreads();
  istage1(D, ka, on16);
  if (!PAR) {
    __syncthreads();
    istage1(SB, w, w < RB);
  }
  __syncthreads();
  // a self-mirrored pencil (f == fb) is stored twice by the same thread, A then
  // B: the last store in program order stands
  istage2(SA, f);
  istage2(SB, fb);
}

template <int RA, int RB, int PAD, bool SPLIT>
static hipError_t launch_pencil_pq_t(const NdConvArgs& a, hipStream_t s) {
  const size_t lds = (size_t)2 * RA * RB * 64 * 8;
  auto fn = nd_pencil_pq_kernel<RA, RB, PAD, SPLIT>;
  hipError_t e = nd_allow_lds((const void*)fn, lds);
  if (e != hipSuccess) return e;
  const unsigned nb = (unsigned)(((a.MY / 2 + 1) * a.MZ + 63) / 64);
  const dim3 grid = SPLIT ? dim3(nb, a.npairs, 1) : dim3(nb, a.C, (a.B + 1) / 2);
  hipLaunchKernelGGL(fn, grid, dim3(64 * RA), lds, s, a);
  return hipGetLastError();
}

template <int PAD, bool SPLIT = false>
static hipError_t launch_pencil_pq_p(const NdConvArgs& a, hipStream_t s) {
  switch (a.MX) {
    case 8: return launch_pencil_pq_t<4, 2, PAD, SPLIT>(a, s);
    case 16: return launch_pencil_pq_t<4, 4, PAD, SPLIT>(a, s);
    case 32: return launch_pencil_pq_t<8, 4, PAD, SPLIT>(a, s);
    case 64: return launch_pencil_pq_t<8, 8, PAD, SPLIT>(a, s);
    case 128: return launch_pencil_pq_t<16, 8, PAD, SPLIT>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int RA, int RB, int MODE, int PAD>
static hipError_t launch_pencil_t(const NdConvArgs& a, dim3 grid, hipStream_t s) {
  const size_t lds = (size_t)RA * RB * 64 * 8;
  auto fn = nd_pencil_kernel<RA, RB, MODE, PAD>;
  hipError_t e = nd_allow_lds((const void*)fn, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, grid, dim3(64 * RA), lds, s, a);
  return hipGetLastError();
}

template <int MODE, int PAD>
static hipError_t launch_pencil_p(const NdConvArgs& a, dim3 grid, hipStream_t s) {
  switch (a.MX) {
    case 8: return launch_pencil_t<4, 2, MODE, PAD>(a, grid, s);
    case 16: return launch_pencil_t<4, 4, MODE, PAD>(a, grid, s);
    case 32: return launch_pencil_t<8, 4, MODE, PAD>(a, grid, s);
    case 64: return launch_pencil_t<8, 8, MODE, PAD>(a, grid, s);
    case 128: return launch_pencil_t<16, 8, MODE, PAD>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int MODE>
static hipError_t launch_pencil(const NdConvArgs& a, dim3 grid, hipStream_t s) {
  // the filter transform has no zero half; the conv pass has one unless circular
  if (MODE == PN_FWD_FULL || a.MX == a.X) return launch_pencil_p<MODE, 1>(a, grid, s);
  return launch_pencil_p<MODE, 2>(a, grid, s);
}

hipError_t nd_filter(const NdFilterArgs& fin, float2* F, float2* kh, const float2* tw128, hipStream_t s,
                     bool keep_k) {
  NdFilterArgs f = fin;
  const int MX = f.MX, MY = f.MY, MZ = f.MZ;
  const size_t P = (size_t)MX * MY * MZ;
  const dim3 g((unsigned)(P / kNP));
  const bool film = f.film != nullptr;
  const bool direct = !keep_k && (f.W == 64 || f.W == 128);
  f.fdirect = direct ? F : nullptr;
  using MlpFn = void (*)(NdFilterArgs);
  MlpFn fn;
  if (f.W == 64)
    fn = direct ? (film ? nd_mlp_mfma_kernel<64, true, true> : nd_mlp_mfma_kernel<64, false, true>)
                : (film ? nd_mlp_mfma_kernel<64, true, false> : nd_mlp_mfma_kernel<64, false, false>);
  else if (f.W == 128)
    fn = direct ? (film ? nd_mlp_mfma_kernel<128, true, true> : nd_mlp_mfma_kernel<128, false, true>)
                : (film ? nd_mlp_mfma_kernel<128, true, false> : nd_mlp_mfma_kernel<128, false, false>);
  else
    fn = film ? nd_mlp_kernel<true> : nd_mlp_kernel<false>;
  hipLaunchKernelGGL(fn, g, dim3(256), 0, s, f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int npairs = f.N * f.C / 2;
  const size_t tot = P * npairs;
  if (!direct) {
    hipLaunchKernelGGL(nd_pack_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, (const float*)f.k, F,
                       MX, MY, MZ, npairs);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  NdConvArgs a{};
  a.X = f.X;
  a.Y = f.Y;
  a.Z = f.Z;
  a.MX = MX;
  a.MY = MY;
  a.MZ = MZ;
  a.F = F;
  a.npairs = npairs;
  a.tw128 = tw128;
  if ((e = launch_plane<PL_FWD_FULL>(a, dim3(MX, npairs, 1), s)) != hipSuccess) return e;
  if (MX > 1) {
    // transform over x and the split into the channels' half spectra in one pass
    a.kh = kh;
    return launch_pencil_pq_p<1, true>(a, s);
  }
  // 2D grids (MX = 1): the transform over x is the identity
  const size_t th = (size_t)MX * MY * (MZ / 2 + 1) * npairs;
  hipLaunchKernelGGL(nd_split_kernel, dim3((unsigned)((th + 255) / 256)), dim3(256), 0, s, (const float2*)F, kh,
                     MX, MY, MZ, npairs);
  return hipGetLastError();
}

hipError_t nd_gate(const float* u, float* part, const float* ga, const float* gb, float* gate, int B, int NO, int C,
                   int V, hipStream_t s) {
  const int nch = V < 512 ? V : 512;
  if (256 % C == 0) {
    hipLaunchKernelGGL(nd_mean_partial256_kernel, dim3(nch, B), dim3(256), 0, s, u, part, C, V, V / nch);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(nd_gate256_kernel, dim3(B), dim3(256), 0, s, (const float*)part, ga, gb, gate, NO, C, nch, V);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(nd_mean_partial_kernel, dim3(nch, B), dim3(256), 0, s, u, part, C, V, V / nch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(nd_gate_kernel, dim3(C / 64, B), dim3(256), 0, s, (const float*)part, ga, gb, gate, NO, C, nch,
                     V);
  return hipGetLastError();
}

size_t nd_gate_partial_floats(int B, int C, int V) { return (size_t)B * (V < 512 ? V : 512) * C; }

template <int MODE>
static hipError_t launch_plane128(const NdConvArgs& a, int nitems, hipStream_t s) {
  using C = PlaneCfg<128>;
  auto fn = nd_plane128_kernel<MODE>;
  hipError_t e = nd_allow_lds((const void*)fn, C::LDS);
  if (e != hipSuccess) return e;
  static DeviceCache grid_cache;
  const int grid = grid_cache.get([] {
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    return cus;  // one 1024-thread workgroup per CU (LDS)
  });
  hipLaunchKernelGGL(fn, dim3(grid < nitems ? grid : nitems), dim3(C::THREADS), C::LDS, s, a, nitems);
  return hipGetLastError();
}

static hipError_t launch_pencil128p(const NdConvArgs& a, int nitems, hipStream_t s) {
  const size_t lds = (size_t)2 * 16 * 8 * 64 * 8;  // exchange buffer + A's spectrum entries
  auto fn = nd_pencil128p_kernel;
  hipError_t e = nd_allow_lds((const void*)fn, lds);
  if (e != hipSuccess) return e;
  static DeviceCache grid_cache;
  const int grid = grid_cache.get([&] {
    int cus = 0, dev = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)fn, 512, lds) != hipSuccess || per_cu <= 0)
      per_cu = 1;
    return cus * per_cu;
  });
  hipLaunchKernelGGL(fn, dim3(grid < nitems ? grid : nitems), dim3(512), lds, s, a, nitems);
  return hipGetLastError();
}

static hipError_t launch_pencil128(const NdConvArgs& a, int nitems, hipStream_t s) {
  const size_t lds = (size_t)16 * 8 * 64 * 8;
  auto fn = nd_pencil128_kernel;
  hipError_t e = nd_allow_lds((const void*)fn, lds);
  if (e != hipSuccess) return e;
  static DeviceCache grid_cache;
  const int grid = grid_cache.get([&] {
    int cus = 0, dev = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)fn, 512, lds) != hipSuccess || per_cu <= 0)
      per_cu = 1;
    return cus * per_cu;
  });
  hipLaunchKernelGGL(fn, dim3(grid < nitems ? grid : nitems), dim3(512), lds, s, a, nitems);
  return hipGetLastError();
}

template <int MY, int MZ, bool CIRC>
static hipError_t launch_plane2d_t(const NdConvArgs& a, hipStream_t s) {
  using C = PlaneCfg<MY, MZ>;
  auto fn = a.kh_stride != 0 ? nd_plane2d_kernel<MY, MZ, CIRC, true> : nd_plane2d_kernel<MY, MZ, CIRC, false>;
  hipError_t e = nd_allow_lds((const void*)fn, C::LDS);
  if (e != hipSuccess) return e;
  const int items = (a.B + 1) / 2 * a.C;
  const int per_xcd = (items + 7) / 8;
  hipLaunchKernelGGL(fn, dim3(8 * per_xcd), dim3(C::THREADS), C::LDS, s, a, per_xcd);
  return hipGetLastError();
}

template <int MY, bool CIRC>
static hipError_t launch_plane2d_z(const NdConvArgs& a, hipStream_t s) {
  switch (a.MZ) {
    case 8: return launch_plane2d_t<MY, 8, CIRC>(a, s);
    case 16: return launch_plane2d_t<MY, 16, CIRC>(a, s);
    case 32: return launch_plane2d_t<MY, 32, CIRC>(a, s);
    case 64: return launch_plane2d_t<MY, 64, CIRC>(a, s);
    case 128: return launch_plane2d_t<MY, 128, CIRC>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool CIRC>
static hipError_t launch_plane2d(const NdConvArgs& a, hipStream_t s) {
  switch (a.MY) {
    case 8: return launch_plane2d_z<8, CIRC>(a, s);
    case 16: return launch_plane2d_z<16, CIRC>(a, s);
    case 32: return launch_plane2d_z<32, CIRC>(a, s);
    case 64: return launch_plane2d_z<64, CIRC>(a, s);
    case 128: return launch_plane2d_z<128, CIRC>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t nd_conv(const NdConvArgs& in, hipStream_t s) {
  NdConvArgs a = in;
  if (a.X == 1) {
    // 2D grid: all orders in one launch; the result goes to zfinal
    a.zfinal = in.zfinal;
    return a.MY == a.Y ? launch_plane2d<true>(a, s) : launch_plane2d<false>(a, s);
  }
  const int BP = (a.B + 1) / 2;
  const unsigned nf = (unsigned)(a.MY * a.MZ / 64);
  // persistent kernels: the zero-padded 64^3 case (128-point axes, half of each kept)
  const bool p128 = a.MY == 128 && a.MY == 2 * a.Y && a.Y == a.Z;
  const int nplanes = a.X * a.C * BP;
  hipError_t e = p128 ? launch_plane128<PL_FWD_V>(a, nplanes, s) : launch_plane<PL_FWD_V>(a, dim3(a.X, a.C, BP), s);
  if (e != hipSuccess) return e;
  for (int n = 0; n < a.NO; ++n) {
    a.n = n;
    if (a.kh_stride != 0) {
      e = a.MX == a.X ? launch_pencil_pq_p<1>(a, s) : launch_pencil_pq_p<2>(a, s);
    } else if (a.MX == 128 && a.MX == 2 * a.X && a.MZ == 128 && a.MZ == 2 * a.Z) {
      e = launch_pencil128p(a, a.MY * a.C * BP, s);
    } else if (a.MX == 128 && a.MX == 2 * a.X) {
      e = launch_pencil128(a, (int)(nf * a.C * BP), s);
    } else {
      e = launch_pencil<PN_CONV>(a, dim3(nf, a.C, BP), s);
    }
    if (e != hipSuccess) return e;
    a.zin = (n == 0) ? nullptr : in.zbuf[(n - 1) & 1];
    a.zout = (n == a.NO - 1) ? in.zfinal : in.zbuf[n & 1];
    if (n == a.NO - 1)
      e = p128 ? launch_plane128<PL_INV>(a, nplanes, s) : launch_plane<PL_INV>(a, dim3(a.X, a.C, BP), s);
    else
      e = p128 ? launch_plane128<PL_INV_FWD>(a, nplanes, s) : launch_plane<PL_INV_FWD>(a, dim3(a.X, a.C, BP), s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace hy
