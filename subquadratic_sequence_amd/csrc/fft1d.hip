// Long causal convolution + gating kernels of the 1D Hyena operator (gfx950).
//
// The convolution of each channel with its filter is taken through the
// convolution theorem (TWIML #690 podcast, 6:27) at size N = 2L, the input zero
// padded so that the circular result equals the causal one on [0, L)
// (HyenaND explainer, Methodology, "Handling Boundaries"). Two real channels
// (a, b) travel together as one complex signal z_a + i z_b; with
// X = DFT(z_a + i z_b) the spectrum of the two filtered outputs is
//     Y_k = X_k P_k + conj(X_{-k}) Q_k,   P = (Ha + Hb) / 2N,  Q = (Ha - Hb) / 2N,
// and the inverse DFT of Y gives c_a + i c_b directly. (P, Q) per channel pair
// is what the filter cache stores.
//
// Two regimes:
//  * 2L <= 8192: one workgroup keeps a channel pair in LDS for all orders
//    (forward FFT, spectrum product, inverse FFT, gate, skip, next order), so
//    only the last z^{N+1} is written to HBM.
//  * 2L >= 16384: four-step FFT with N = 256 x N2 (t = N2 n1 + n2). A column
//    pass does the 256-point DFTs over n1 (128 non-zero inputs) for blocks of 64
//    columns, applies the cross twiddle W_N^{n2 k1} and writes the
//    intermediate; a row pass does the N2-point DFT of rows k1 and 256 - k1
//    together (they hold the bins k and N - k), the spectrum product and the
//    inverse row DFT; the next column pass inverts the columns (keeping the 128
//    outputs t < L), gates, adds the skip, writes z^{n+1} once and, in the same
//    registers, starts the forward column DFT of the next order.
#include "common.h"
#include "kernels.h"

namespace hy {

// ============================================================ LDS regime

template <int N> struct LdsCfg {
  static constexpr int E = (N >= 256) ? 16 : N / 16;  // values per thread
  static constexpr int TG = N / E;                    // threads per FFT
  static constexpr int WG = TG > 256 ? TG : 256;      // threads per workgroup
  static constexpr int G = WG / TG;                   // channel pairs per workgroup
};

// causal length-3 short convolution of one projected channel at time t
template <typename T>
__device__ __forceinline__ float short_conv_at(const T* __restrict__ row, const float* __restrict__ w3, int t) {
  float s = w3[0] * ldf(row + t);
  if (t >= 1) s += w3[1] * ldf(row + t - 1);
  if (t >= 2) s += w3[2] * ldf(row + t - 2);
  return s;
}

template <typename T, int N>
__global__ __launch_bounds__(LdsCfg<N>::WG) void fftconv_lds_kernel(
    const T* __restrict__ p, const float* __restrict__ short_w, const float* __restrict__ dskip,
    const float4* __restrict__ pq, const float2* __restrict__ tw, T* __restrict__ zout, int D, int NO) {
  using C = LdsCfg<N>;
  constexpr int L = N / 2;
  extern __shared__ float4 smem4[];
  float2* fbase = reinterpret_cast<float2*>(smem4);
  float* zbase = reinterpret_cast<float*>(fbase + C::G * N);
  const int g = threadIdx.x / C::TG, lt = threadIdx.x % C::TG;
  float2* fb = fbase + g * N;
  float* za = zbase + g * N;  // z^n of channel a in [0, L), channel b in [L, 2L)
  float* zb = za + L;
  const int pr = blockIdx.x * C::G + g;
  const int half = D / 2;
  const int b = pr / half, cp = pr % half;
  const int ca = 2 * cp, cb = ca + 1;
  const size_t J = (size_t)(NO + 1) * D;
  const T* pb = p + (size_t)b * J * L;

  // z^1 = short conv of the v block
  for (int t = lt; t < L; t += C::TG) {
    float a = short_conv_at(pb + (size_t)ca * L, short_w + 3 * ca, t);
    float c = short_conv_at(pb + (size_t)cb * L, short_w + 3 * cb, t);
    za[t] = a;
    zb[t] = c;
    fb[t] = make_float2(a, c);
    fb[t + L] = make_float2(0.f, 0.f);
  }
  for (int n = 0; n < NO; ++n) {
    __syncthreads();
    fft_lds<N, C::E, false>(fb, lt, tw);
    // spectrum product on the pairs (k, N - k), k in [0, N/2]
    const float4* pqn = pq + ((size_t)n * half + cp) * (L + 1);
    for (int k = lt; k <= L; k += C::TG) {
      float4 w = pqn[k];
      float2 P = make_float2(w.x, w.y), Q = make_float2(w.z, w.w);
      const int m = (N - k) & (N - 1);
      float2 xk = fb[k], xm = fb[m];
      float2 yk = cadd(cmul(xk, P), cmul(conjf2(xm), Q));
      if (m != k) {
        float2 ym = cadd(cmulc(xm, P), cmulc(conjf2(xk), Q));
        fb[m] = ym;
      }
      fb[k] = yk;
    }
    __syncthreads();
    fft_lds<N, C::E, true>(fb, lt, tw);
    // gate + skip
    const int jx = (n + 1) * D;
    const float da = dskip[n * D + ca], db = dskip[n * D + cb];
    const bool last = (n == NO - 1);
    for (int t = lt; t < L; t += C::TG) {
      float2 y = fb[t];
      float xa = short_conv_at(pb + (size_t)(jx + ca) * L, short_w + 3 * (jx + ca), t);
      float xb = short_conv_at(pb + (size_t)(jx + cb) * L, short_w + 3 * (jx + cb), t);
      float na = xa * y.x + da * za[t];
      float nb = xb * y.y + db * zb[t];
      if (last) {
        stf(zout + ((size_t)b * D + ca) * L + t, na);
        stf(zout + ((size_t)b * D + cb) * L + t, nb);
      } else {
        za[t] = na;
        zb[t] = nb;
        fb[t] = make_float2(na, nb);
        fb[t + L] = make_float2(0.f, 0.f);
      }
    }
  }
}

// Filter spectrum in the LDS regime: (h_a + i h_b) zero padded -> DFT -> (P, Q).
template <int N>
__global__ __launch_bounds__(LdsCfg<N>::WG) void filter_spec_lds_kernel(
    const float* __restrict__ h, const float2* __restrict__ tw, float4* __restrict__ pq, int D, int NO) {
  using C = LdsCfg<N>;
  constexpr int L = N / 2;
  extern __shared__ float4 smem4[];
  float2* fb = reinterpret_cast<float2*>(smem4) + (threadIdx.x / C::TG) * N;
  const int lt = threadIdx.x % C::TG;
  const int pr = blockIdx.x * C::G + threadIdx.x / C::TG;  // over NO * D/2
  const int half = D / 2;
  const int n = pr / half, cp = pr % half;
  const float* ha = h + ((size_t)n * D + 2 * cp) * L;
  const float* hb = ha + L;
  for (int t = lt; t < L; t += C::TG) {
    fb[t] = make_float2(ha[t], hb[t]);
    fb[t + L] = make_float2(0.f, 0.f);
  }
  __syncthreads();
  fft_lds<N, C::E, false>(fb, lt, tw);
  const float s = 0.5f / (float)N;
  float4* out = pq + (size_t)pr * (L + 1);
  for (int k = lt; k <= L; k += C::TG) {
    float2 fk = fb[k], fm = conjf2(fb[(N - k) & (N - 1)]);
    float2 ha2 = cadd(fk, fm);                 // 2 Ha
    float2 d = csub(fk, fm);                   // 2i Hb
    float2 hb2 = make_float2(d.y, -d.x);       // 2 Hb
    // P = (Ha + Hb) / 2N, Q = (Ha - Hb) / 2N
    out[k] = make_float4(0.5f * s * (ha2.x + hb2.x), 0.5f * s * (ha2.y + hb2.y),
                         0.5f * s * (ha2.x - hb2.x), 0.5f * s * (ha2.y - hb2.y));
  }
}

// ============================================================ four-step

constexpr int kN1 = 256;  // column DFT length
constexpr int kCW = 64;   // columns per column-pass workgroup

struct ColArgs {
  const void* p;          // projections [B][(NO+1)D][L] (storage type)
  const float* short_w;   // [(NO+1)D][3]
  const float* dskip;     // [NO][D]
  const void* zin;        // z^n [B][D][L] for n >= 1
  void* zout;             // z^{n+1} [B][D][L]
  float2* Y;              // intermediate [pairs][256][N2]
  const float* h;         // filter rows [NO][D][L] (filter mode)
  const float2* w256;     // W_256^m, m in [0, 256)
  const float2* tw_lo;    // W_N^m = tw_lo[m & lo_mask] * tw_hi[m >> lo_bits]
  const float2* tw_hi;
  int lo_bits, L, N2, D, NO, n;
  int pair_off;           // global index of the first channel pair of this launch
};

enum { COL_FWD_V = 0, COL_FWD_H = 1, COL_INV = 2, COL_INV_FWD = 3 };

__device__ __forceinline__ float2 twN(const ColArgs& a, unsigned m) {
  return cmul(a.tw_lo[m & ((1u << a.lo_bits) - 1)], a.tw_hi[m >> a.lo_bits]);
}

// Forward column DFT. Thread (lane c, wave j) holds x[n1 = j + 16 r] in v[r]
// (v[r] = 0 for r >= 8). Writes Y[k1][n2] * W_N^{n2 k1}.
__device__ __forceinline__ void col_forward(const ColArgs& a, float2 (&v)[16], float2* S,
                                            float2* Yp, int c, int w, int n2) {
  const unsigned N = 2u * (unsigned)a.L;
  Dft<16, false>::run(v);
#pragma unroll
  for (int ka = 0; ka < 16; ++ka) {
    if (ka) v[ka] = cmul(v[ka], a.w256[(w * ka) & 255]);
    S[(w * 16 + ka) * kCW + c] = v[ka];
  }
  __syncthreads();
  float2 u[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) u[j] = S[(j * 16 + w) * kCW + c];
  Dft<16, false>::run(u);
  // k1 = w + 16 kb
  float2 wk = twN(a, ((unsigned)n2 * (unsigned)w) & (N - 1));
  const float2 ws = twN(a, ((unsigned)n2 * 16u) & (N - 1));
#pragma unroll
  for (int kb = 0; kb < 16; ++kb) {
    Yp[(size_t)(w + 16 * kb) * a.N2 + n2] = cmul(u[kb], wk);
    wk = cmul(wk, ws);
  }
}

// Inverse column DFT; returns out[n1 = w + 16 nb] in u[nb] for nb < 8.
__device__ __forceinline__ void col_inverse(const ColArgs& a, float2 (&u)[16], float2* S,
                                            const float2* Yp, int c, int w, int n2) {
  const unsigned N = 2u * (unsigned)a.L;
  float2 v[16];
  float2 wk = twN(a, ((unsigned)n2 * (unsigned)w) & (N - 1));
  const float2 ws = twN(a, ((unsigned)n2 * 16u) & (N - 1));
#pragma unroll
  for (int kb = 0; kb < 16; ++kb) {
    v[kb] = cmulc(Yp[(size_t)(w + 16 * kb) * a.N2 + n2], wk);
    wk = cmul(wk, ws);
  }
  Dft<16, true>::run(v);
#pragma unroll
  for (int na = 0; na < 16; ++na) {
    if (na) v[na] = cmulc(v[na], a.w256[(w * na) & 255]);
    S[(w * 16 + na) * kCW + c] = v[na];
  }
  __syncthreads();
#pragma unroll
  for (int ka = 0; ka < 16; ++ka) u[ka] = S[(ka * 16 + w) * kCW + c];
  Dft<16, true>::run(u);
}

template <typename T, int MODE>
__global__ __launch_bounds__(1024) void colpass_kernel(ColArgs a) {
  extern __shared__ float4 smem4[];
  float2* S = reinterpret_cast<float2*>(smem4);
  const int c = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n2 = blockIdx.x * kCW + c;
  const int pr = blockIdx.y + a.pair_off;
  const int L = a.L, N2 = a.N2, D = a.D;
  const int half = D / 2;
  float2* Yp = a.Y + (size_t)blockIdx.y * kN1 * N2;
  float2 v[16];

  if (MODE == COL_FWD_H) {
    const int n = pr / half, cp = pr % half;
    const float* ha = a.h + ((size_t)n * D + 2 * cp) * L;
    const float* hb = ha + L;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (r < 8) {
        const int t = N2 * (w + 16 * r) + n2;
        v[r] = make_float2(ha[t], hb[t]);
      } else {
        v[r] = make_float2(0.f, 0.f);
      }
    }
    col_forward(a, v, S, Yp, c, w, n2);
    return;
  }

  const int b = pr / half, cp = pr % half;
  const int ca = 2 * cp, cb = ca + 1;
  const T* pb = reinterpret_cast<const T*>(a.p) + (size_t)b * (a.NO + 1) * D * L;

  if (MODE == COL_FWD_V) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (r < 8) {
        const int t = N2 * (w + 16 * r) + n2;
        v[r] = make_float2(short_conv_at(pb + (size_t)ca * L, a.short_w + 3 * ca, t),
                           short_conv_at(pb + (size_t)cb * L, a.short_w + 3 * cb, t));
      } else {
        v[r] = make_float2(0.f, 0.f);
      }
    }
    col_forward(a, v, S, Yp, c, w, n2);
    return;
  }

  // inverse, gate, skip
  float2 u[16];
  col_inverse(a, u, S, Yp, c, w, n2);
  const int n = a.n;
  const int jx = (n + 1) * D;
  const float da = a.dskip[n * D + ca], db = a.dskip[n * D + cb];
  const T* zin = reinterpret_cast<const T*>(a.zin) + (size_t)b * D * L;
  T* zo = reinterpret_cast<T*>(a.zout) + (size_t)b * D * L;
#pragma unroll
  for (int nb = 0; nb < 16; ++nb) {
    if (nb < 8) {
      const int t = N2 * (w + 16 * nb) + n2;
      float xa = short_conv_at(pb + (size_t)(jx + ca) * L, a.short_w + 3 * (jx + ca), t);
      float xb = short_conv_at(pb + (size_t)(jx + cb) * L, a.short_w + 3 * (jx + cb), t);
      float zpa, zpb;
      if (n == 0) {
        zpa = short_conv_at(pb + (size_t)ca * L, a.short_w + 3 * ca, t);
        zpb = short_conv_at(pb + (size_t)cb * L, a.short_w + 3 * cb, t);
      } else {
        zpa = ldf(zin + (size_t)ca * L + t);
        zpb = ldf(zin + (size_t)cb * L + t);
      }
      float na = xa * u[nb].x + da * zpa;
      float nbv = xb * u[nb].y + db * zpb;
      stf(zo + (size_t)ca * L + t, na);
      stf(zo + (size_t)cb * L + t, nbv);
      v[nb] = make_float2(na, nbv);
    } else {
      v[nb] = make_float2(0.f, 0.f);
    }
  }
  if (MODE == COL_INV_FWD) {
    __syncthreads();  // S is reused
    col_forward(a, v, S, Yp, c, w, n2);
  }
}

// Row pass: N2-point DFTs of rows k1 and 256 - k1 (rows 0 and 128 for slot 0).
template <int N2> struct RowCfg {
  static constexpr int E = 16;
  static constexpr int TG = N2 / E;                    // threads per row
  static constexpr int SP = N2 >= 4096 ? 1 : 4096 / N2;  // row pairs per workgroup
  static constexpr int WG = SP * 2 * TG;
};

enum { ROW_CONV = 0, ROW_SPEC = 1 };

template <int N2, int MODE>
__global__ __launch_bounds__(RowCfg<N2>::WG) void rowpass_kernel(float2* __restrict__ Y, float4* __restrict__ pq,
                                                                 const float2* __restrict__ tw_row, int pq_off,
                                                                 int pair_off, int pq_mod) {
  using C = RowCfg<N2>;
  extern __shared__ float4 smem4[];
  float2* rows = reinterpret_cast<float2*>(smem4);
  const int r = threadIdx.x / C::TG, lt = threadIdx.x % C::TG;
  const int s = blockIdx.x * C::SP + r / 2;      // slot 0..127
  const int isB = r & 1;
  const int k1 = isB ? (s == 0 ? 128 : 256 - s) : s;
  float2* Yr = Y + ((size_t)blockIdx.y * kN1 + k1) * N2;
  float2* row = rows + r * N2;
  for (int i = lt; i < N2; i += C::TG) row[i] = Yr[i];
  __syncthreads();
  fft_lds<N2, C::E, false>(row, lt, tw_row);
  // (P, Q) rows of this channel pair: 129 rows of N2
  // filters are shared by every batch: pair (b, cp) uses the rows of cp
  float4* pqp = pq + ((size_t)pq_off + (blockIdx.y + pair_off) % pq_mod) * 129 * N2;
  const float nrm = 0.25f / (float)(kN1 * N2);  // (1/2)(1/2N) with 2 Ha, 2 Hb below
  if (s != 0) {
    float2* ra = rows + (r & ~1) * N2;
    float2* rb = ra + N2;
    const float4* pqs = pqp + (size_t)s * N2;
    for (int k2 = isB * C::TG + lt; k2 < N2; k2 += 2 * C::TG) {
      const int m2 = N2 - 1 - k2;
      float2 xk = ra[k2], xm = rb[m2];
      if (MODE == ROW_CONV) {
        float4 q = pqs[k2];
        float2 P = make_float2(q.x, q.y), Q = make_float2(q.z, q.w);
        ra[k2] = cadd(cmul(xk, P), cmul(conjf2(xm), Q));
        rb[m2] = cadd(cmulc(xm, P), cmulc(conjf2(xk), Q));
      } else {
        float2 fm = conjf2(xm);
        float2 ha2 = cadd(xk, fm), d = csub(xk, fm);
        float2 hb2 = make_float2(d.y, -d.x);
        pqp[(size_t)s * N2 + k2] = make_float4(nrm * (ha2.x + hb2.x), nrm * (ha2.y + hb2.y),
                                               nrm * (ha2.x - hb2.x), nrm * (ha2.y - hb2.y));
      }
    }
  } else {
    // row 0 pairs k2 with (N2 - k2) mod N2; row 128 pairs k2 with N2 - 1 - k2
    const int pqrow = isB ? 128 : 0;
    const float4* pqs = pqp + (size_t)pqrow * N2;
    const int kend = (MODE == ROW_CONV) ? (isB ? N2 / 2 - 1 : N2 / 2) : N2 - 1;
    for (int k2 = lt; k2 <= kend; k2 += C::TG) {
      const int m2 = isB ? (N2 - 1 - k2) : ((N2 - k2) & (N2 - 1));
      float2 xk = row[k2], xm = row[m2];
      if (MODE == ROW_CONV) {
        float4 q = pqs[k2];
        float2 P = make_float2(q.x, q.y), Q = make_float2(q.z, q.w);
        float2 yk = cadd(cmul(xk, P), cmul(conjf2(xm), Q));
        if (m2 != k2) row[m2] = cadd(cmulc(xm, P), cmulc(conjf2(xk), Q));
        row[k2] = yk;
      } else {
        float2 fm = conjf2(xm);
        float2 ha2 = cadd(xk, fm), d = csub(xk, fm);
        float2 hb2 = make_float2(d.y, -d.x);
        pqp[(size_t)pqrow * N2 + k2] = make_float4(nrm * (ha2.x + hb2.x), nrm * (ha2.y + hb2.y),
                                                   nrm * (ha2.x - hb2.x), nrm * (ha2.y - hb2.y));
      }
    }
  }
  if (MODE == ROW_SPEC) return;
  __syncthreads();
  fft_lds<N2, C::E, true>(row, lt, tw_row);
  for (int i = lt; i < N2; i += C::TG) Yr[i] = row[i];
}

// ============================================================ launchers

template <typename T, int N>
static hipError_t launch_lds_conv(const LdsConvArgs& a, hipStream_t s) {
  using C = LdsCfg<N>;
  const int pairs = a.B * a.D / 2;
  const size_t lds = (size_t)C::G * N * 12;
  hipLaunchKernelGGL((fftconv_lds_kernel<T, N>), dim3(pairs / C::G), dim3(C::WG), lds, s,
                     (const T*)a.p, a.short_w, a.dskip, a.pq, a.tw, (T*)a.zout, a.D, a.NO);
  return hipGetLastError();
}

template <int N>
static hipError_t launch_lds_spec(const float* h, const float2* tw, float4* pq, int D, int NO, hipStream_t s) {
  using C = LdsCfg<N>;
  const int pairs = NO * D / 2;
  hipLaunchKernelGGL((filter_spec_lds_kernel<N>), dim3(pairs / C::G), dim3(C::WG), (size_t)C::G * N * 8, s,
                     h, tw, pq, D, NO);
  return hipGetLastError();
}

#define HY_LDS_SWITCH(N, CALL) \
  switch (N) {                 \
    case 32: CALL(32); break;  \
    case 64: CALL(64); break;  \
    case 128: CALL(128); break; \
    case 256: CALL(256); break; \
    case 512: CALL(512); break; \
    case 1024: CALL(1024); break; \
    case 2048: CALL(2048); break; \
    case 4096: CALL(4096); break; \
    case 8192: CALL(8192); break; \
    default: return hipErrorInvalidValue; \
  }

hipError_t lds_conv(const LdsConvArgs& a, bool is_bf16, hipStream_t s) {
  const int N = 2 * a.L;
  hipError_t e = hipSuccess;
  if (is_bf16) {
#define CALLB(n) e = launch_lds_conv<bf16, n>(a, s)
    HY_LDS_SWITCH(N, CALLB)
#undef CALLB
  } else {
#define CALLF(n) e = launch_lds_conv<float, n>(a, s)
    HY_LDS_SWITCH(N, CALLF)
#undef CALLF
  }
  return e;
}

hipError_t lds_spec(const float* h, const float2* tw, float4* pq, int L, int D, int NO, hipStream_t s) {
  const int N = 2 * L;
  hipError_t e = hipSuccess;
#define CALLS(n) e = launch_lds_spec<n>(h, tw, pq, D, NO, s)
  HY_LDS_SWITCH(N, CALLS)
#undef CALLS
  return e;
}

size_t lds_conv_smem(int L) {
  const int N = 2 * L;
  int G = 1;
#define CALLG(n) G = LdsCfg<n>::G
  switch (N) {
    case 32: CALLG(32); break;
    case 64: CALLG(64); break;
    case 128: CALLG(128); break;
    case 256: CALLG(256); break;
    case 512: CALLG(512); break;
    case 1024: CALLG(1024); break;
    case 2048: CALLG(2048); break;
    case 4096: CALLG(4096); break;
    case 8192: CALLG(8192); break;
    default: return 0;
  }
#undef CALLG
  return (size_t)G * N * 12;
}

static hipError_t launch_col(const ColArgs& a, int mode, bool is_bf16, int pairs, hipStream_t s) {
  dim3 grid(a.N2 / kCW, pairs), block(1024);
  const size_t lds = 16 * 16 * kCW * sizeof(float2);
#define COLCASE(T, M) hipLaunchKernelGGL((colpass_kernel<T, M>), grid, block, lds, s, a)
  if (is_bf16) {
    switch (mode) {
      case COL_FWD_V: COLCASE(bf16, COL_FWD_V); break;
      case COL_FWD_H: COLCASE(bf16, COL_FWD_H); break;
      case COL_INV: COLCASE(bf16, COL_INV); break;
      default: COLCASE(bf16, COL_INV_FWD); break;
    }
  } else {
    switch (mode) {
      case COL_FWD_V: COLCASE(float, COL_FWD_V); break;
      case COL_FWD_H: COLCASE(float, COL_FWD_H); break;
      case COL_INV: COLCASE(float, COL_INV); break;
      default: COLCASE(float, COL_INV_FWD); break;
    }
  }
#undef COLCASE
  return hipGetLastError();
}

template <int N2>
static hipError_t launch_row_t(float2* Y, float4* pq, const float2* tw_row, int pq_off, int pair_off,
                               int pq_mod, int pairs, int mode, hipStream_t s) {
  using C = RowCfg<N2>;
  dim3 grid(128 / C::SP, pairs), block(C::WG);
  const size_t lds = (size_t)C::SP * 2 * N2 * sizeof(float2);
  if (mode == ROW_CONV)
    hipLaunchKernelGGL((rowpass_kernel<N2, ROW_CONV>), grid, block, lds, s, Y, pq, tw_row, pq_off, pair_off, pq_mod);
  else
    hipLaunchKernelGGL((rowpass_kernel<N2, ROW_SPEC>), grid, block, lds, s, Y, pq, tw_row, pq_off, pair_off, pq_mod);
  return hipGetLastError();
}

static hipError_t launch_row(int N2, float2* Y, float4* pq, const float2* tw_row, int pq_off, int pair_off,
                             int pq_mod, int pairs, int mode, hipStream_t s) {
#define ROWCASE(n) case n: return launch_row_t<n>(Y, pq, tw_row, pq_off, pair_off, pq_mod, pairs, mode, s)
  switch (N2) {
    ROWCASE(64);
    ROWCASE(128);
    ROWCASE(256);
    ROWCASE(512);
    ROWCASE(1024);
    ROWCASE(2048);
    ROWCASE(4096);
    ROWCASE(8192);
    default: return hipErrorInvalidValue;
  }
#undef ROWCASE
}

static ColArgs col_args(const FourStepTables& tb, int L, int D, int NO) {
  ColArgs a{};
  a.w256 = tb.w256;
  a.tw_lo = tb.tw_lo;
  a.tw_hi = tb.tw_hi;
  a.lo_bits = tb.lo_bits;
  a.L = L;
  a.N2 = 2 * L / kN1;
  a.D = D;
  a.NO = NO;
  return a;
}

hipError_t fourstep_spec(const FourStepTables& tb, const float* h, float2* Y, float4* pq, int L, int D, int NO,
                         hipStream_t s) {
  ColArgs a = col_args(tb, L, D, NO);
  a.h = h;
  a.Y = Y;
  const int pairs = NO * D / 2;
  hipError_t e = launch_col(a, COL_FWD_H, false, pairs, s);
  if (e != hipSuccess) return e;
  return launch_row(a.N2, Y, pq, tb.tw_row, 0, 0, pairs, pairs, ROW_SPEC, s);
}

hipError_t fourstep_conv(const FourStepTables& tb, const FourStepConvArgs& c, bool is_bf16, hipStream_t s) {
  ColArgs a = col_args(tb, c.L, c.D, c.NO);
  a.p = c.p;
  a.short_w = c.short_w;
  a.dskip = c.dskip;
  a.Y = c.Y;
  const int half = c.D / 2;
  const int pairs_all = c.B * half;
  // Channel-pair groups bound the intermediate (8 * 2L bytes per pair) so that
  // it can stay in the last-level cache between the passes of one group.
  const int gp = (c.group_pairs > 0 && c.group_pairs < pairs_all) ? c.group_pairs : pairs_all;
  for (int p0 = 0; p0 < pairs_all; p0 += gp) {
    const int np = (pairs_all - p0 < gp) ? pairs_all - p0 : gp;
    ColArgs g = a;
    g.pair_off = p0;
    hipError_t e = launch_col(g, COL_FWD_V, is_bf16, np, s);
    if (e != hipSuccess) return e;
    for (int n = 0; n < c.NO; ++n) {
      e = launch_row(a.N2, c.Y, const_cast<float4*>(c.pq), tb.tw_row, n * half, p0, half, np, ROW_CONV, s);
      if (e != hipSuccess) return e;
      ColArgs gi = g;
      gi.n = n;
      gi.zin = (n == 0) ? nullptr : c.z[(n - 1) & 1];
      gi.zout = (n == c.NO - 1) ? c.zfinal : c.z[n & 1];
      e = launch_col(gi, (n == c.NO - 1) ? COL_INV : COL_INV_FWD, is_bf16, np, s);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace hy
