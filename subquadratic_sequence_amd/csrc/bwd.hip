// Backward pass (vector-Jacobian product) of the 1D Hyena operator on gfx950,
// and of its implicit filter generator.
//
// The operator is trained (Hyena Hierarchy abstract: training compute at
// sequence length 2K; HyenaDNA abstract: training speed at long contexts), so
// its gradients are computed here from the chain rule of the forward steps:
//   dz^{N+1} = dy W_out^T; for n = N .. 1 with g = dz^{n+1}:
//     dx^n = g c^n,  dc = g x^n,  dD^n = sum g z^n,
//     dz^n = D^n g + (h^n correlated with dc),  dh^n = sum_b (dc cross-correlated with z^n)
// The correlation with a filter is the transpose of the causal convolution; in
// the 2L-point transform it is a product with the conjugate filter spectrum,
// and with the two channels of a pair packed as one complex signal
// X = DFT(dc_a + i dc_b) its spectrum is
//     Y_k = X_k conj(P_k) + conj(X_{-k}) conj(Q_k)
// with the same (P, Q) the forward reads from the layer cache. The filter
// gradient of each channel is the inverse DFT of C_k conj(Z_k) (C, Z the two
// channels' spectra separated from the packed transforms), summed over the
// batch. Zero padding to 2L keeps every circular result equal to the linear
// one on the kept outputs, causal and two-sided alike.
//
// This file holds the on-chip regime (2L <= 8192): one group of threads keeps
// a channel pair's transforms in LDS, as the forward kernel does.
#include "common.h"
#include "kernels.h"
#include "kernels_bwd.h"
#include "vec8.h"

namespace hy {

template <int N> struct BwdCfg {
  static constexpr int E = (N >= 256) ? 16 : N / 16;  // values per thread in a transform
  static constexpr int TG = N / E;                    // threads per transform
  static constexpr int WG = TG > 256 ? TG : 256;      // threads per workgroup
  static constexpr int G = WG / TG;                   // channel pairs per workgroup
  static constexpr int FB = padded_len(N);            // float2 per transform buffer
  static constexpr int NT = E / 2;                    // positions t < L per thread: t = lt + i TG
};

// ------------------------------------------------- forward recompute

// The forward orders of one channel pair, keeping every order's input z^n and
// convolution c^n (fp32, [NO][B][D][L]) and writing z^{NO+1} in the storage type.
template <typename T, int N>
__global__ __launch_bounds__(BwdCfg<N>::WG) void bwd_fwd_save_kernel(
    const T* __restrict__ sp, const float* __restrict__ dskip, const float4* __restrict__ pq,
    const float2* __restrict__ tw, float* __restrict__ zsave, float* __restrict__ csave, T* __restrict__ zfin,
    int B, int D, int NO) {
  using C = BwdCfg<N>;
  constexpr int L = N / 2;
  extern __shared__ float4 smem4[];
  float2* fb = reinterpret_cast<float2*>(smem4) + (threadIdx.x / C::TG) * C::FB;
  const int lt = threadIdx.x % C::TG;
  const int pr = blockIdx.x * C::G + threadIdx.x / C::TG;
  const int half = D / 2;
  const int b = pr / half, cp = pr % half;
  const int ca = 2 * cp, cb = ca + 1;
  const size_t J = (size_t)(NO + 1) * D;
  const T* sb = sp + (size_t)b * J * L;
  float za[C::NT], zb[C::NT];
#pragma unroll
  for (int i = 0; i < C::NT; ++i) {
    const int t = lt + i * C::TG;
    za[i] = ldf(sb + (size_t)ca * L + t);
    zb[i] = ldf(sb + (size_t)cb * L + t);
  }
  for (int n = 0; n < NO; ++n) {
    float* zs = zsave + ((size_t)n * B + b) * D * L;
    float* cs = csave + ((size_t)n * B + b) * D * L;
#pragma unroll
    for (int i = 0; i < C::NT; ++i) {
      const int t = lt + i * C::TG;
      zs[(size_t)ca * L + t] = za[i];
      zs[(size_t)cb * L + t] = zb[i];
      fb[pad16(t)] = make_float2(za[i], zb[i]);
      fb[pad16(t + L)] = make_float2(0.f, 0.f);
    }
    __syncthreads();
    fft_lds<N, C::E, false>(fb, lt, tw);
    const float4* pqn = pq + ((size_t)n * half + cp) * (L + 1);
    for (int k = lt; k <= L; k += C::TG) {
      const float4 w = pqn[k];
      const float2 P = make_float2(w.x, w.y), Q = make_float2(w.z, w.w);
      const int m = (N - k) & (N - 1);
      const float2 xk = fb[pad16(k)], xm = fb[pad16(m)];
      const float2 yk = cadd(cmul(xk, P), cmul(conjf2(xm), Q));
      if (m != k) fb[pad16(m)] = cadd(cmulc(xm, P), cmulc(conjf2(xk), Q));
      fb[pad16(k)] = yk;
    }
    __syncthreads();
    fft_lds<N, C::E, true>(fb, lt, tw);
    const int jx = (n + 1) * D;
    const float da = dskip[n * D + ca], db = dskip[n * D + cb];
#pragma unroll
    for (int i = 0; i < C::NT; ++i) {
      const int t = lt + i * C::TG;
      const float2 y = fb[pad16(t)];
      cs[(size_t)ca * L + t] = y.x;
      cs[(size_t)cb * L + t] = y.y;
      const float xa = ldf(sb + (size_t)(jx + ca) * L + t);
      const float xb = ldf(sb + (size_t)(jx + cb) * L + t);
      za[i] = xa * y.x + da * za[i];
      zb[i] = xb * y.y + db * zb[i];
    }
  }
#pragma unroll
  for (int i = 0; i < C::NT; ++i) {
    const int t = lt + i * C::TG;
    stf(zfin + ((size_t)b * D + ca) * L + t, za[i]);
    stf(zfin + ((size_t)b * D + cb) * L + t, zb[i]);
  }
}

// ------------------------------------------------- reverse orders

__device__ __forceinline__ float2 mul_negi(float2 a) { return make_float2(a.y, -a.x); }  // -i a

// Orders N .. 1 of one channel pair in reverse. Reads dz^{N+1} (gz, storage
// type), the saved z^n and c^n and the gates x^n; writes ds = (dz^1, dx^1, ..,
// dx^N) (fp32 [B][(NO+1)D][L], the block order of W_in's columns), this
// sample's filter gradients (fp32 [B][NO][D][HL], HL = L causal or 2L for the
// wrapped two-sided filters) and skip gradients (fp32 [B][NO][D]).
template <typename T, int N>
__global__ __launch_bounds__(BwdCfg<N>::WG) void bwd_conv_kernel(
    const T* __restrict__ sp, const T* __restrict__ gz, const float* __restrict__ zsave,
    const float* __restrict__ csave, const float* __restrict__ dskip, const float4* __restrict__ pq,
    const float2* __restrict__ tw, float* __restrict__ sbar, float* __restrict__ dh_part,
    float* __restrict__ dd_part, int B, int D, int NO, int HL) {
  using C = BwdCfg<N>;
  constexpr int L = N / 2;
  extern __shared__ float4 smem4[];
  const int grp = threadIdx.x / C::TG, lt = threadIdx.x % C::TG;
  float2* f1 = reinterpret_cast<float2*>(smem4) + (size_t)grp * 2 * C::FB;
  float2* f2 = f1 + C::FB;
  float2* red = reinterpret_cast<float2*>(smem4) + (size_t)C::G * 2 * C::FB + (size_t)grp * C::TG;
  const int pr = blockIdx.x * C::G + grp;
  const int half = D / 2;
  const int b = pr / half, cp = pr % half;
  const int ca = 2 * cp, cb = ca + 1;
  const size_t J = (size_t)(NO + 1) * D;
  const T* sb = sp + (size_t)b * J * L;
  float* sbb = sbar + (size_t)b * J * L;
  const float inv_n = 1.f / (float)N;
  float ga[C::NT], gb[C::NT];
#pragma unroll
  for (int i = 0; i < C::NT; ++i) {
    const int t = lt + i * C::TG;
    ga[i] = ldf(gz + ((size_t)b * D + ca) * L + t);
    gb[i] = ldf(gz + ((size_t)b * D + cb) * L + t);
  }
  for (int n = NO - 1; n >= 0; --n) {
    const float* zs = zsave + ((size_t)n * B + b) * D * L;
    const float* cs = csave + ((size_t)n * B + b) * D * L;
    const int jx = (n + 1) * D;
    float acc_a = 0.f, acc_b = 0.f;
#pragma unroll
    for (int i = 0; i < C::NT; ++i) {
      const int t = lt + i * C::TG;
      const float xa = ldf(sb + (size_t)(jx + ca) * L + t), xb = ldf(sb + (size_t)(jx + cb) * L + t);
      const float za = zs[(size_t)ca * L + t], zb = zs[(size_t)cb * L + t];
      sbb[(size_t)(jx + ca) * L + t] = ga[i] * cs[(size_t)ca * L + t];
      sbb[(size_t)(jx + cb) * L + t] = gb[i] * cs[(size_t)cb * L + t];
      f1[pad16(t)] = make_float2(ga[i] * xa, gb[i] * xb);
      f1[pad16(t + L)] = make_float2(0.f, 0.f);
      f2[pad16(t)] = make_float2(za, zb);
      f2[pad16(t + L)] = make_float2(0.f, 0.f);
      acc_a += ga[i] * za;
      acc_b += gb[i] * zb;
    }
    red[lt] = make_float2(acc_a, acc_b);
    __syncthreads();
    if (lt == 0) {
      float sa = 0.f, sbv = 0.f;
      for (int r = 0; r < C::TG; ++r) {
        sa += red[r].x;
        sbv += red[r].y;
      }
      dd_part[((size_t)b * NO + n) * D + ca] = sa;
      dd_part[((size_t)b * NO + n) * D + cb] = sbv;
    }
    fft_lds<N, C::E, false>(f1, lt, tw);
    fft_lds<N, C::E, false>(f2, lt, tw);
    const float4* pqn = pq + ((size_t)n * half + cp) * (L + 1);
    for (int k = lt; k <= L; k += C::TG) {
      const float4 w = pqn[k];
      const float2 P = make_float2(w.x, w.y), Q = make_float2(w.z, w.w);
      const int m = (N - k) & (N - 1);
      const float2 xk = f1[pad16(k)], xm = f1[pad16(m)];
      const float2 sk = f2[pad16(k)], sm = f2[pad16(m)];
      // transposed filter: conj(P), conj(Q) in place of P, Q
      const float2 yk = cadd(cmulc(xk, P), cmulc(conjf2(xm), Q));
      const float2 ym = cadd(cmul(xm, P), cmul(conjf2(xk), Q));
      // the two channels' spectra at bin k (times 2): a from the Hermitian part,
      // b from the anti-Hermitian part divided by i
      const float2 ca2 = cadd(xk, conjf2(xm)), cb2 = mul_negi(csub(xk, conjf2(xm)));
      const float2 za2 = cadd(sk, conjf2(sm)), zb2 = mul_negi(csub(sk, conjf2(sm)));
      const float2 aa = cmulc(ca2, za2), ab = cmulc(cb2, zb2);  // 4 C_a conj(Z_a), 4 C_b conj(Z_b)
      const float s = 0.25f * inv_n;
      const float2 tk = make_float2(s * (aa.x - ab.y), s * (aa.y + ab.x));    // Aa + i Ab
      const float2 tm = make_float2(s * (aa.x + ab.y), s * (-aa.y + ab.x));   // conj(Aa) + i conj(Ab)
      f1[pad16(k)] = yk;
      f2[pad16(k)] = tk;
      if (m != k) {
        f1[pad16(m)] = ym;
        f2[pad16(m)] = tm;
      }
    }
    __syncthreads();
    fft_lds<N, C::E, true>(f1, lt, tw);
    fft_lds<N, C::E, true>(f2, lt, tw);
    const float da = dskip[n * D + ca], db = dskip[n * D + cb];
#pragma unroll
    for (int i = 0; i < C::NT; ++i) {
      const int t = lt + i * C::TG;
      const float2 y = f1[pad16(t)];
      ga[i] = da * ga[i] + y.x;
      gb[i] = db * gb[i] + y.y;
    }
    float* dha = dh_part + (((size_t)b * NO + n) * D + ca) * HL;
    float* dhb = dha + HL;
    for (int t = lt; t < HL; t += C::TG) {
      // entry L of a wrapped two-sided filter (lag +-L) is not a tap
      const float2 hv = (HL == N && t == L) ? make_float2(0.f, 0.f) : f2[pad16(t)];
      dha[t] = hv.x;
      dhb[t] = hv.y;
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < C::NT; ++i) {
    const int t = lt + i * C::TG;
    sbb[(size_t)ca * L + t] = ga[i];
    sbb[(size_t)cb * L + t] = gb[i];
  }
}

// ------------------------------------------------- short convolution

// Deterministic sum of one value per thread of a 256-thread workgroup; the
// result is valid in thread 0.
__device__ __forceinline__ float block_sum256(float v, float* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  const float r = sh[0];
  __syncthreads();
  return r;
}

// s_j(t) = sum_k w[j,k] p_j(t - k): dp_j(t) = sum_k w[j,k] ds_j(t + k) (zero past
// L - 1) and this sample's dw[j,k] = sum_t ds_j(t) p_j(t - k). One workgroup per
// (sample, column j); each thread takes 8 consecutive positions per step in
// 16-byte accesses, the two neighbours past its block from the cache.
template <typename T>
__global__ __launch_bounds__(256) void short_conv_bwd_kernel(const float* __restrict__ sbar, const T* __restrict__ p,
                                                             const float* __restrict__ short_w, T* __restrict__ pbar,
                                                             float* __restrict__ dsw_part, int L, int J) {
  __shared__ float sh[256];
  const int row = blockIdx.x, j = row % J;
  const float* s = sbar + (size_t)row * L;
  const T* pr = p + (size_t)row * L;
  T* o = pbar + (size_t)row * L;
  const float w0 = short_w[j * 3], w1 = short_w[j * 3 + 1], w2 = short_w[j * 3 + 2];
  float a0 = 0.f, a1 = 0.f, a2 = 0.f;
  for (int t0 = 8 * (int)threadIdx.x; t0 < L; t0 += 8 * 256) {
    float sv[8], pv[8], out[8];
    ld8(s + t0, sv);
    ld8(pr + t0, pv);
    const float s8 = t0 + 8 < L ? s[t0 + 8] : 0.f, s9 = t0 + 9 < L ? s[t0 + 9] : 0.f;
    const float pm1 = t0 >= 1 ? ldf(pr + t0 - 1) : 0.f, pm2 = t0 >= 2 ? ldf(pr + t0 - 2) : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float s1 = k + 1 < 8 ? sv[k + 1] : s8;
      const float s2 = k + 2 < 8 ? sv[k + 2] : (k + 2 == 8 ? s8 : s9);
      out[k] = w0 * sv[k] + w1 * s1 + w2 * s2;
      const float p1 = k >= 1 ? pv[k - 1] : pm1;
      const float p2 = k >= 2 ? pv[k - 2] : (k == 1 ? pm1 : pm2);
      a0 += sv[k] * pv[k];
      a1 += sv[k] * p1;
      a2 += sv[k] * p2;
    }
    st8(o + t0, out);
  }
  a0 = block_sum256(a0, sh);
  a1 = block_sum256(a1, sh);
  a2 = block_sum256(a2, sh);
  if (threadIdx.x == 0) {
    dsw_part[(size_t)row * 3] = a0;
    dsw_part[(size_t)row * 3 + 1] = a1;
    dsw_part[(size_t)row * 3 + 2] = a2;
  }
}

// The forward's short convolution from p (channel-major rows of L): s_j(t) =
// w0 p_j(t) + w1 p_j(t-1) + w2 p_j(t-2), zero history; 8 positions per thread
// per step. One workgroup per row.
template <typename T>
__global__ __launch_bounds__(256) void short_conv_rows_kernel(const T* __restrict__ p,
                                                              const float* __restrict__ short_w, T* __restrict__ s,
                                                              int L, int J) {
  const int row = blockIdx.x, j = row % J;
  const T* pr = p + (size_t)row * L;
  T* o = s + (size_t)row * L;
  const float w0 = short_w[j * 3], w1 = short_w[j * 3 + 1], w2 = short_w[j * 3 + 2];
  for (int t0 = 8 * (int)threadIdx.x; t0 < L; t0 += 8 * 256) {
    float pv[8], out[8];
    ld8(pr + t0, pv);
    const float pm1 = t0 >= 1 ? ldf(pr + t0 - 1) : 0.f, pm2 = t0 >= 2 ? ldf(pr + t0 - 2) : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float p1 = k >= 1 ? pv[k - 1] : pm1;
      const float p2 = k >= 2 ? pv[k - 2] : (k == 1 ? pm1 : pm2);
      out[k] = w0 * pv[k] + w1 * p1 + w2 * p2;
    }
    st8(o + t0, out);
  }
}

// out[i] = sum_{r < R} in[r * stride + i], in a fixed order (bit-reproducible).
template <typename T>
__global__ __launch_bounds__(256) void sum_rows_kernel(const T* __restrict__ in, float* __restrict__ out, int R,
                                                       size_t stride, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    float s = 0.f;
    for (int r = 0; r < R; ++r) s += ldf(in + (size_t)r * stride + i);
    out[i] = s;
  }
}

// part[r * S + seg] = sum of in[r * K + k] over segment seg of K / S entries
__global__ __launch_bounds__(256) void row_sum_seg_kernel(const float* __restrict__ in, float* __restrict__ part,
                                                          int K, int S) {
  __shared__ float sh[256];
  const int r = blockIdx.x / S, seg = blockIdx.x - r * S, SK = K / S;
  const float* x = in + (size_t)r * K + (size_t)seg * SK;
  float v = 0.f;
  for (int k = threadIdx.x; k < SK; k += 256) v += x[k];
  v = block_sum256(v, sh);
  if (threadIdx.x == 0) part[blockIdx.x] = v;
}

// Band sums of a tall [R][n] array of partial results, in place: workgroup
// (column block, g) adds rows [g R/G, (g+1) R/G) in order and writes the sum
// into row g R/G (a row of its own band).
__global__ __launch_bounds__(256) void sum_bands_kernel(float* __restrict__ part, int R, int G, size_t n) {
  const size_t col = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (col >= n) return;
  const int RG = R / G, r0 = (int)blockIdx.y * RG;
  float v = 0.f;
  for (int r = r0; r < r0 + RG; ++r) v += part[(size_t)r * n + col];
  part[(size_t)r0 * n + col] = v;
}

// out[r] = sum_k in[r * K + k]; one workgroup per row.
__global__ __launch_bounds__(256) void row_sum_kernel(const float* __restrict__ in, float* __restrict__ out, int K) {
  __shared__ float sh[256];
  const float* x = in + (size_t)blockIdx.x * K;
  float s = 0.f;
  for (int k = threadIdx.x; k < K; k += 256) s += x[k];
  s = block_sum256(s, sh);
  if (threadIdx.x == 0) out[blockIdx.x] = s;
}

// ------------------------------------------------- filter generator

constexpr int kFbT = 64;    // positions per workgroup
constexpr int kFbMaxW = 128;
constexpr int kFbMaxF = 65;

// Features e and both hidden layers of the filter MLP at positions
// [64 blockIdx.x, +64): e [P][F], a1, c1 = cos(q1), a2, c2 = cos(q2) [P][W]
// (row-major, q the pre-activations). Positions as in the forward generator:
// t / L causal, the wrapped signed lags of a two-sided filter otherwise.
__global__ __launch_bounds__(256) void filter_bwd_feat_kernel(FilterBwdArgs a) {
  __shared__ float e_s[kFbT][kFbMaxF + 1];
  __shared__ float h1[kFbT][kFbMaxW + 1];
  const int t0 = blockIdx.x * kFbT;
  const int F = 1 + 2 * a.K, W = a.W, L = a.L;
  const int P = a.noncausal ? 2 * L : L;
  const int tid = threadIdx.x;
  for (int idx = tid; idx < kFbT * F; idx += 256) {
    const int tl = idx / F, f = idx % F;
    const int t = t0 + tl;
    float v = 0.f;
    if (t < P) {
      if (f == 0) {
        v = (float)(t > L ? t - 2 * L : t) / (float)L;
      } else {
        const int k = (f <= a.K) ? f : f - a.K;
        const long long m = ((long long)k * t) % L;  // angle 2 pi k t / L reduced exactly
        float sv, cv;
        sincospif(2.0f * (float)m / (float)L, &sv, &cv);
        v = (f <= a.K) ? cv : sv;
      }
      a.e[(size_t)t * F + f] = v;
    }
    e_s[tl][f] = v;
  }
  __syncthreads();
  for (int idx = tid; idx < kFbT * W; idx += 256) {
    const int tl = idx / W, j = idx % W;
    float s = a.b1[j];
    for (int f = 0; f < F; ++f) s += e_s[tl][f] * a.w1[f * W + j];
    float sv, cv;
    sincosf(s, &sv, &cv);
    h1[tl][j] = sv;
    const int t = t0 + tl;
    if (t < P) {
      a.a1[(size_t)t * W + j] = sv;
      a.c1[(size_t)t * W + j] = cv;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < kFbT * W; idx += 256) {
    const int tl = idx / W, j = idx % W;
    float s = a.b2[j];
    for (int i = 0; i < W; ++i) s += h1[tl][i] * a.w2[i * W + j];
    float sv, cv;
    sincosf(s, &sv, &cv);
    const int t = t0 + tl;
    if (t < P) {
      a.a2[(size_t)t * W + j] = sv;
      a.c2[(size_t)t * W + j] = cv;
    }
  }
}

// Per channel c (one workgroup): do[n D + c][t] = dh[n][c][t] * win_c(t) (zero at
// the non-tap entry L of a wrapped two-sided filter) and
// ddecay[c] = sum_{n,t} dh * o * (-|tau|) * win, win = exp(-decay_c |tau|);
// o = (a2 W3) [N D][P] channel-major, plus b3.
// One workgroup per (channel c, segment of P / S positions): dL/do = dh x window
// and the segment's share of the decay gradient, into part[c][seg] (summed in
// segment order by row_sum_kernel). L is a power of two, so tau = t * (1/L)
// equals t / L exactly.
__global__ __launch_bounds__(256) void filter_bwd_out_kernel(FilterBwdArgs a, float* __restrict__ part, int S) {
  __shared__ float sh[256];
  const int c = blockIdx.x, seg = blockIdx.y, L = a.L, D = a.D;
  const int P = a.noncausal ? 2 * L : L, SL = P / S;
  const float dc = a.decay[c], invL = 1.f / (float)L;
  float acc = 0.f;
  for (int n = 0; n < a.NO; ++n) {
    const size_t row = ((size_t)n * D + c) * P;
    const float ob = a.b3[n * D + c];
    for (int t = seg * SL + threadIdx.x; t < (seg + 1) * SL; t += 256) {
      const bool tap = !(a.noncausal && t == L);
      const float tau = fabsf((float)(t > L ? t - 2 * L : t) * invL);
      const float win = expf(-dc * tau);
      const float g = tap ? a.dh[row + t] : 0.f;
      a.dout[row + t] = g * win;
      acc += g * (a.o[row + t] + ob) * (-tau) * win;
    }
  }
  acc = block_sum256(acc, sh);
  if (threadIdx.x == 0) part[(size_t)c * S + seg] = acc;
}

// x[i] *= y[i]
__global__ __launch_bounds__(256) void mul_inplace_kernel(float* __restrict__ x, const float* __restrict__ y,
                                                          size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) x[i] *= y[i];
}

// ------------------------------------------------- host launchers

static int grid_for(size_t n) {
  const size_t g = (n + 255) / 256;
  return (int)(g < 8192 ? (g > 0 ? g : 1) : 8192);
}

static hipError_t allow_lds_bwd(const void* fn, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename T, int N>
static hipError_t launch_bwd_lds(const BwdConvArgs& a, hipStream_t s) {
  using C = BwdCfg<N>;
  const int pairs = a.B * a.D / 2;
  {
    auto fn = bwd_fwd_save_kernel<T, N>;
    const size_t lds = (size_t)C::G * C::FB * 8;
    hipError_t e = allow_lds_bwd((const void*)fn, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3(pairs / C::G), dim3(C::WG), lds, s, (const T*)a.s, a.dskip, a.pq, a.tw, a.zsave,
                       a.csave, (T*)a.zfin, a.B, a.D, a.NO);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  auto fn = bwd_conv_kernel<T, N>;
  const size_t lds = (size_t)C::G * 2 * C::FB * 8 + (size_t)C::WG * 8;
  hipError_t e = allow_lds_bwd((const void*)fn, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(pairs / C::G), dim3(C::WG), lds, s, (const T*)a.s, (const T*)a.gz, a.zsave, a.csave,
                     a.dskip, a.pq, a.tw, a.sbar, a.dh_part, a.dd_part, a.B, a.D, a.NO, a.HL);
  return hipGetLastError();
}

hipError_t bwd_lds_conv(const BwdConvArgs& a, bool is_bf16, hipStream_t s) {
  hipError_t e = hipSuccess;
  switch (2 * a.L) {
#define HY_BWD_CASE(n)                                                                  \
  case n:                                                                               \
    e = is_bf16 ? launch_bwd_lds<bf16, n>(a, s) : launch_bwd_lds<float, n>(a, s);       \
    break;
    HY_BWD_CASE(32)
    HY_BWD_CASE(64)
    HY_BWD_CASE(128)
    HY_BWD_CASE(256)
    HY_BWD_CASE(512)
    HY_BWD_CASE(1024)
    HY_BWD_CASE(2048)
    HY_BWD_CASE(4096)
    HY_BWD_CASE(8192)
#undef HY_BWD_CASE
    default: return hipErrorInvalidValue;
  }
  return e;
}

hipError_t short_conv_bwd(const float* sbar, const void* p, const float* short_w, void* pbar, float* dsw_part, int rows,
                          int L, int J, bool is_bf16, hipStream_t s) {
  if (is_bf16)
    hipLaunchKernelGGL(short_conv_bwd_kernel<bf16>, dim3(rows), dim3(256), 0, s, sbar, (const bf16*)p, short_w,
                       (bf16*)pbar, dsw_part, L, J);
  else
    hipLaunchKernelGGL(short_conv_bwd_kernel<float>, dim3(rows), dim3(256), 0, s, sbar, (const float*)p, short_w,
                       (float*)pbar, dsw_part, L, J);
  return hipGetLastError();
}

hipError_t short_conv_rows(const void* p, const float* short_w, void* s_out, int rows, int L, int J, bool is_bf16,
                           hipStream_t s) {
  if (is_bf16)
    hipLaunchKernelGGL(short_conv_rows_kernel<bf16>, dim3(rows), dim3(256), 0, s, (const bf16*)p, short_w,
                       (bf16*)s_out, L, J);
  else
    hipLaunchKernelGGL(short_conv_rows_kernel<float>, dim3(rows), dim3(256), 0, s, (const float*)p, short_w,
                       (float*)s_out, L, J);
  return hipGetLastError();
}

hipError_t sum_rows(const void* in, float* out, int R, size_t stride, size_t n, bool in_bf16, hipStream_t s) {
  if (in_bf16)
    hipLaunchKernelGGL(sum_rows_kernel<bf16>, dim3(grid_for(n)), dim3(256), 0, s, (const bf16*)in, out, R, stride, n);
  else
    hipLaunchKernelGGL(sum_rows_kernel<float>, dim3(grid_for(n)), dim3(256), 0, s, (const float*)in, out, R, stride,
                       n);
  return hipGetLastError();
}

hipError_t row_sums(const float* in, float* out, int rows, int K, float* part, hipStream_t s) {
  // few rows: each row in S segments (power of two, at least 1024 entries each),
  // the segment sums then added in order
  int S = 1;
  while (rows * S * 2 <= 1024 && K % (S * 2) == 0 && K / (S * 2) >= 1024) S *= 2;
  if (S == 1 || part == nullptr) {
    hipLaunchKernelGGL(row_sum_kernel, dim3(rows), dim3(256), 0, s, in, out, K);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(row_sum_seg_kernel, dim3(rows * S), dim3(256), 0, s, in, part, K, S);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(row_sum_kernel, dim3(rows), dim3(256), 0, s, part, out, S);
  return hipGetLastError();
}

hipError_t sum_rows_tall(float* part, float* out, int R, size_t n, hipStream_t s) {
  // bands G (a power of two dividing R) so that about 512 workgroups run
  const size_t cb = (n + 255) / 256;
  int G = 1;
  while ((size_t)G * 2 * cb <= 512 && R % (G * 2) == 0 && R / (G * 2) >= 4) G *= 2;
  if (G == 1) return sum_rows(part, out, R, n, n, false, s);
  hipLaunchKernelGGL(sum_bands_kernel, dim3((unsigned)cb, G), dim3(256), 0, s, part, R, G, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the G band sums sit in rows 0, R/G, 2 R/G, ...
  return sum_rows(part, out, G, (size_t)(R / G) * n, n, false, s);
}

hipError_t filter_bwd_feat(const FilterBwdArgs& a, hipStream_t s) {
  const int P = a.noncausal ? 2 * a.L : a.L;
  hipLaunchKernelGGL(filter_bwd_feat_kernel, dim3((P + kFbT - 1) / kFbT), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t filter_bwd_out(const FilterBwdArgs& a, float* part, hipStream_t s) {
  // position segments of at least 2048 (P is a power of two)
  const int P = a.noncausal ? 2 * a.L : a.L;
  int S = 1;
  while (S < 16 && P / (S * 2) >= 2048) S *= 2;
  hipLaunchKernelGGL(filter_bwd_out_kernel, dim3(a.D, S), dim3(256), 0, s, a, part, S);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(row_sum_kernel, dim3(a.D), dim3(256), 0, s, part, a.ddecay, S);
  return hipGetLastError();
}

hipError_t mul_inplace(float* x, const float* y, size_t n, hipStream_t s) {
  hipLaunchKernelGGL(mul_inplace_kernel, dim3(grid_for(n)), dim3(256), 0, s, x, y, n);
  return hipGetLastError();
}

}  // namespace hy
