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
//  * 2L >= 16384: four-step FFT with N = N1 x N2 (t = N2 n1 + n2, N1 = 64 or
//    256). A column pass does the N1-point DFTs over n1 (N1/2 non-zero inputs)
//    for blocks of 64 columns, applies the cross twiddle W_N^{n2 k1} and writes
//    the intermediate; a row pass does the N2-point DFT of rows k1 and N1 - k1
//    together (they hold the bins k and N - k), the spectrum product and the
//    inverse row DFT; the next column pass inverts the columns (keeping the
//    N1/2 outputs t < L), gates, adds the skip, writes z^{n+1} once and, from
//    the same registers, starts the forward column DFT of the next order.
#include <stdlib.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hy {

// ============================================================ LDS regime

template <int N> struct LdsCfg {
  static constexpr int E = (N >= 256) ? 16 : N / 16;  // values per thread
  static constexpr int TG = N / E;                    // threads per FFT
  static constexpr int WG = TG > 256 ? TG : 256;      // threads per workgroup
  static constexpr int G = WG / TG;                   // channel pairs per workgroup
  static constexpr int FB = padded_len(N);            // float2 per FFT buffer
  static constexpr size_t LDS = (size_t)G * (FB * 8 + N * 4);
};

template <typename T, int N>
__global__ __launch_bounds__(LdsCfg<N>::WG) void fftconv_lds_kernel(
    const T* __restrict__ sp, const float* __restrict__ dskip, const float4* __restrict__ pq,
    const float2* __restrict__ tw, T* __restrict__ zout, int D, int NO) {
  using C = LdsCfg<N>;
  constexpr int L = N / 2;
  extern __shared__ float4 smem4[];
  float2* fbase = reinterpret_cast<float2*>(smem4);
  float* zbase = reinterpret_cast<float*>(fbase + C::G * C::FB);
  const int g = threadIdx.x / C::TG, lt = threadIdx.x % C::TG;
  float2* fb = fbase + g * C::FB;
  float* za = zbase + g * N;  // z^n of channel a in [0, L), channel b in [L, 2L)
  float* zb = za + L;
  const int pr = blockIdx.x * C::G + g;
  const int half = D / 2;
  const int b = pr / half, cp = pr % half;
  const int ca = 2 * cp, cb = ca + 1;
  const size_t J = (size_t)(NO + 1) * D;
  const T* sb = sp + (size_t)b * J * L;  // short-convolved blocks (v, x^1, .., x^NO)

  // z^1 = v block
  for (int t = lt; t < L; t += C::TG) {
    float a = ldf(sb + (size_t)ca * L + t);
    float c = ldf(sb + (size_t)cb * L + t);
    za[t] = a;
    zb[t] = c;
    fb[pad16(t)] = make_float2(a, c);
    fb[pad16(t + L)] = make_float2(0.f, 0.f);
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
      float2 xk = fb[pad16(k)], xm = fb[pad16(m)];
      float2 yk = cadd(cmul(xk, P), cmul(conjf2(xm), Q));
      if (m != k) fb[pad16(m)] = cadd(cmulc(xm, P), cmulc(conjf2(xk), Q));
      fb[pad16(k)] = yk;
    }
    __syncthreads();
    fft_lds<N, C::E, true>(fb, lt, tw);
    // gate + skip
    const int jx = (n + 1) * D;
    const float da = dskip[n * D + ca], db = dskip[n * D + cb];
    const bool last = (n == NO - 1);
    for (int t = lt; t < L; t += C::TG) {
      float2 y = fb[pad16(t)];
      float xa = ldf(sb + (size_t)(jx + ca) * L + t);
      float xb = ldf(sb + (size_t)(jx + cb) * L + t);
      float na = xa * y.x + da * za[t];
      float nb = xb * y.y + db * zb[t];
      if (last) {
        stf(zout + ((size_t)b * D + ca) * L + t, na);
        stf(zout + ((size_t)b * D + cb) * L + t, nb);
      } else {
        za[t] = na;
        zb[t] = nb;
        fb[pad16(t)] = make_float2(na, nb);
        fb[pad16(t + L)] = make_float2(0.f, 0.f);
      }
    }
  }
}

// Filter spectrum in the LDS regime: (h_a + i h_b) zero padded -> DFT -> (P, Q).
// WRAP: two-sided filters, rows of 2L already wrapped (no zero half).
template <int N, bool WRAP>
__global__ __launch_bounds__(LdsCfg<N>::WG) void filter_spec_lds_kernel(
    const float* __restrict__ h, const float2* __restrict__ tw, float4* __restrict__ pq, int D, int NO) {
  using C = LdsCfg<N>;
  constexpr int L = N / 2;
  constexpr int RL = WRAP ? N : L;  // row length of h
  extern __shared__ float4 smem4[];
  float2* fb = reinterpret_cast<float2*>(smem4) + (threadIdx.x / C::TG) * C::FB;
  const int lt = threadIdx.x % C::TG;
  const int pr = blockIdx.x * C::G + threadIdx.x / C::TG;  // over NO * D/2
  const int half = D / 2;
  const int n = pr / half, cp = pr % half;
  const float* ha = h + ((size_t)n * D + 2 * cp) * RL;
  const float* hb = ha + RL;
  for (int t = lt; t < L; t += C::TG) {
    fb[pad16(t)] = make_float2(ha[t], hb[t]);
    fb[pad16(t + L)] = WRAP ? make_float2(ha[t + L], hb[t + L]) : make_float2(0.f, 0.f);
  }
  __syncthreads();
  fft_lds<N, C::E, false>(fb, lt, tw);
  const float s = 0.25f / (float)N;  // (1/2) * (1/2N) with 2 Ha, 2 Hb below
  float4* out = pq + (size_t)pr * (L + 1);
  for (int k = lt; k <= L; k += C::TG) {
    float2 fk = fb[pad16(k)], fm = conjf2(fb[pad16((N - k) & (N - 1))]);
    float2 ha2 = cadd(fk, fm);                 // 2 Ha
    float2 d = csub(fk, fm);                   // 2i Hb
    float2 hb2 = make_float2(d.y, -d.x);       // 2 Hb
    // P = (Ha + Hb) / 2N, Q = (Ha - Hb) / 2N
    out[k] = make_float4(s * (ha2.x + hb2.x), s * (ha2.y + hb2.y), s * (ha2.x - hb2.x), s * (ha2.y - hb2.y));
  }
}

// ============================================================ four-step

// Columns per column-pass item: 64 (one per lane, one wave per j) for R = 8;
// 32 for R = 16, two j per wave, so that the workgroup has 512 threads (256
// VGPRs each) instead of 1024.
template <int R> constexpr int col_width() { return R >= 16 ? 32 : 64; }

struct ColArgs {
  const void* s;          // short-convolved projections [B][(NO+1)D][L] (storage type)
  const float* dskip;     // [NO][D]
  const void* zin;        // z^n [B][D][L] for n >= 1
  void* zout;             // z^{n+1} [B][D][L]
  void* Y;                // intermediate [pairs][N1][N2] (complex fp32 or bf16 pairs)
  const float* h;         // filter rows [NO][D][L] (filter mode), [NO][D][2L] wrapped (two-sided)
  const float2* w256;     // W_256^m, m in [0, 256)
  const float2* tw_lo;    // W_N^m = tw_lo[m & lo_mask] * tw_hi[m >> lo_bits]
  const float2* tw_hi;
  int lo_bits, L, N2, D, NO, n;
  int pair_off;           // global index of the first channel pair of this launch
};

// COL_FWD_HW: forward column pass of two-sided filters (wrapped rows of 2L, no zero half);
// COL_INV_PLAIN: inverse only, z^{n+1} = h * z^n with no gate and no skip (the
// backward pass's one-order convolutions)
enum { COL_FWD_V = 0, COL_FWD_H = 1, COL_INV = 2, COL_INV_FWD = 3, COL_FWD_HW = 4, COL_INV_PLAIN = 5 };

__device__ __forceinline__ float2 cvt2(float2 v) { return v; }
__device__ __forceinline__ float2 cvt2(cbf16 v) {
  return make_float2(__uint_as_float(v.v << 16), __uint_as_float(v.v & 0xFFFF0000u));
}
__device__ __forceinline__ float cvt1(float v) { return v; }
__device__ __forceinline__ float cvt1(bf16 v) { return (float)v; }

// Twiddles of one column-pass item (column n2, wave w): W_N^(n2 w) and W_N^(n2 R),
// each the product of two table entries (W_N^m = tw_lo[m & lo_mask] * tw_hi[m >> lo_bits]).
struct ColTw {
  float2 lo0, hi0, lo1, hi1;
};
__device__ __forceinline__ void col_tw_load(const ColArgs& a, ColTw& t, unsigned m0, unsigned m1) {
  const unsigned mask = (1u << a.lo_bits) - 1;
  t.lo0 = a.tw_lo[m0 & mask];
  t.hi0 = a.tw_hi[m0 >> a.lo_bits];
  t.lo1 = a.tw_lo[m1 & mask];
  t.hi1 = a.tw_hi[m1 >> a.lo_bits];
}

// Column DFT of N1 = R*R points, n1 = j + R r, k1 = ka + R kb.
// Forward: thread (lane c, wave j) holds x[j + R r] in v[r] (zero for r >= R/2);
// writes Y[k1][n2] * W_N^{n2 k1} through the resource rY of the pair's
// intermediate (per-lane offset voY of element (w, c), uniform offset soY of
// the item's first column). wr[ka] = W_N1^(w ka), the inner twiddles of this
// wave.
template <int R, typename YT>
__device__ __forceinline__ void col_forward(float2 (&v)[R], float2* S, brsrc rY, int voY, int soY, int N2, int c,
                                            int w, const float2 (&wr)[R], float2 wk, float2 ws) {
  constexpr int kCW = col_width<R>();
  Dft<R, false>::run(v);
#pragma unroll
  for (int ka = 0; ka < R; ++ka) {
    if (ka) v[ka] = cmul(v[ka], wr[ka]);
    S[(w * R + ka) * kCW + c] = v[ka];
  }
  __syncthreads();
  float2 u[R];
#pragma unroll
  for (int j = 0; j < R; ++j) u[j] = S[(j * R + w) * kCW + c];
  Dft<R, false>::run(u);
  // k1 = w + R kb: W_N^(n2 k1) = wk ws^kb
#pragma unroll
  for (int kb = 0; kb < R; ++kb) {
    BufIO<YT>::st(rY, voY, soY + kb * R * N2 * (int)sizeof(YT), cmul(u[kb], wk));
    wk = cmul(wk, ws);
  }
}

// Inverse column DFT of the column v0[kb] = Y[w + R kb][n2] (twiddles W_N^(n2 k1)
// = wk ws^kb removed first); returns out[n1 = w + R nb] in u[nb] (only nb < R/2
// are needed).
template <int R>
__device__ __forceinline__ void col_inverse(float2 (&u)[R], float2* S, const float2 (&v0)[R], int c, int w,
                                            const float2 (&wr)[R], float2 wk, float2 ws) {
  constexpr int kCW = col_width<R>();
  float2 v[R];
#pragma unroll
  for (int kb = 0; kb < R; ++kb) {
    v[kb] = cmulc(v0[kb], wk);
    wk = cmul(wk, ws);
  }
  Dft<R, true>::run(v);
#pragma unroll
  for (int na = 0; na < R; ++na) {
    if (na) v[na] = cmulc(v[na], wr[na]);
    S[(w * R + na) * kCW + c] = v[na];
  }
  __syncthreads();
#pragma unroll
  for (int ka = 0; ka < R; ++ka) u[ka] = S[(ka * R + w) * kCW + c];
  Dft<R, true>::run(u);
}

// Persistent column pass: each workgroup walks items (channel pair, block of 64
// columns) with a stride of gridDim.x. Everything an item reads from memory
// (its column of the intermediate or of the input, the gate and skip inputs,
// its twiddles) is in registers when the item starts: each part of the next
// item's data is loaded into the same registers as soon as the current item
// has used that part, so one set of registers carries a whole item of
// prefetch, and no other vector-memory load comes between a prefetch and its
// use (the in-order load counter never makes the work wait for later loads).
// Memory is reached through buffer resources over the item's channel pair:
// every address is the thread's fixed offset (row w, column c of the item)
// plus a workgroup-uniform offset.
template <typename T, typename YT, int R, int MODE>
__global__ __launch_bounds__(R * col_width<R>()) void colpass_kernel(ColArgs a, int nitems) {
  constexpr int N1 = R * R, H = R / 2;
  constexpr bool INVERSE = (MODE == COL_INV || MODE == COL_INV_FWD || MODE == COL_INV_PLAIN);
  constexpr bool GATE = INVERSE && MODE != COL_INV_PLAIN;
  constexpr bool FILT = (MODE == COL_FWD_H || MODE == COL_FWD_HW);
  constexpr int HF = MODE == COL_FWD_HW ? R : H;  // non-zero filter rows per thread
  constexpr int sT = (int)sizeof(T), sY = (int)sizeof(YT);
  extern __shared__ float4 smem4[];
  float2* S = reinterpret_cast<float2*>(smem4);
  // thread (j, c): row j of the R x R column DFT (w below), column c of the item
  constexpr int kCW = col_width<R>();
  const int c = threadIdx.x % kCW, w = threadIdx.x / kCW;
  const int L = a.L, N2 = a.N2, D = a.D;
  const int half = D / 2, ncb = N2 / kCW;
  const size_t J = (size_t)(a.NO + 1) * D;
  const unsigned N = 2u * (unsigned)L;
  // per-lane offsets of element (w N2 + c): in the time-domain rows and in the intermediate
  const int lane_el = w * N2 + c;
  const int voT = lane_el * sT, voY = lane_el * sY, voH = lane_el * 4;
  // inner twiddles W_N1^(w k) of this wave, fixed for the whole launch
  float2 wr[R];
#pragma unroll
  for (int k = 0; k < R; ++k) wr[k] = a.w256[(w * k * (256 / N1)) & 255];

  struct In {
    YT y[INVERSE ? R : 1];                    // inverse: column of the intermediate
    T xa[GATE ? H : 1], xb[GATE ? H : 1];     // inverse: gates x^n
    T za[H], zb[H];                           // z^n (forward of z^1: the v block)
    float ha[FILT ? HF : 1], hb[FILT ? HF : 1];  // filter modes
    float da, db;                             // inverse: skip weights D^n of the pair
    ColTw tw;
  };
  struct Item {
    int pl, cb, pr;
  };
  auto item_of = [&](int item) {
    Item it;
    it.pl = item / ncb;
    it.cb = item - it.pl * ncb;
    it.pr = it.pl + a.pair_off;
    return it;
  };
  // resource over rows row0 and row0 + 1 (the channel pair) of a [rows][L] array
  auto pair_rows = [&](const void* base, size_t row0, int esize) {
    return make_brsrc(static_cast<const char*>(base) + row0 * L * esize, 2u * (unsigned)L * esize);
  };
  auto inter = [&](const Item& it) {  // the pair's intermediate [N1][N2]
    return make_brsrc(static_cast<const char*>(a.Y) + (size_t)it.pl * N1 * N2 * sY, (unsigned)(N1 * N2 * sY));
  };
  // uniform element offset of row w + R r (w = 0) of the item's columns
  auto col0 = [&](const Item& it, int r) { return R * r * N2 + it.cb * kCW; };
  auto load_tw = [&](const Item& it, In& in) {
    const unsigned n2 = (unsigned)(it.cb * kCW + c);
    col_tw_load(a, in.tw, (n2 * (unsigned)w) & (N - 1), (n2 * (unsigned)R) & (N - 1));
  };
  // first part: what the item's first transform reads
  auto load_head = [&](const Item& it, In& in) {
    if constexpr (FILT) {
      const int n = it.pr / half, cp = it.pr % half;
      const int RL = MODE == COL_FWD_HW ? 2 * L : L;  // filter row length
      const brsrc rh = make_brsrc(a.h + ((size_t)n * D + 2 * cp) * RL, 2u * (unsigned)RL * 4);
#pragma unroll
      for (int r = 0; r < HF; ++r) {
        in.ha[r] = BufIO<float>::ld(rh, voH, col0(it, r) * 4);
        in.hb[r] = BufIO<float>::ld(rh, voH, (col0(it, r) + RL) * 4);
      }
    } else if constexpr (MODE == COL_FWD_V) {
      const int b = it.pr / half, cp = it.pr % half;
      const brsrc rv = pair_rows(a.s, (size_t)b * J + 2 * cp, sT);
#pragma unroll
      for (int r = 0; r < H; ++r) {
        in.za[r] = BufIO<T>::ld(rv, voT, col0(it, r) * sT);
        in.zb[r] = BufIO<T>::ld(rv, voT, (col0(it, r) + L) * sT);
      }
    } else {
      const brsrc rY = inter(it);
#pragma unroll
      for (int kb = 0; kb < R; ++kb) in.y[kb] = BufIO<YT>::ld(rY, voY, col0(it, kb) * sY);
    }
  };
  // second part (inverse modes): gate and skip inputs
  auto load_gate = [&](const Item& it, In& in) {
    if constexpr (GATE) {
      const int b = it.pr / half, cp = it.pr % half;
      const int n = a.n;
      const brsrc rx = pair_rows(a.s, (size_t)b * J + (size_t)(n + 1) * D + 2 * cp, sT);
      const brsrc rz = (n == 0) ? pair_rows(a.s, (size_t)b * J + 2 * cp, sT)
                                : pair_rows(a.zin, (size_t)b * D + 2 * cp, sT);
#pragma unroll
      for (int nb = 0; nb < H; ++nb) {
        const int so = col0(it, nb) * sT, so1 = (col0(it, nb) + L) * sT;
        in.xa[nb] = BufIO<T>::ld(rx, voT, so);
        in.xb[nb] = BufIO<T>::ld(rx, voT, so1);
        in.za[nb] = BufIO<T>::ld(rz, voT, so);
        in.zb[nb] = BufIO<T>::ld(rz, voT, so1);
      }
      in.da = a.dskip[n * D + 2 * cp];
      in.db = a.dskip[n * D + 2 * cp + 1];
    }
  };

  // Processes item `item` from `in`, refilling `in` with item `nxt` part by part.
  auto process = [&](int item, In& in, int nxt) {
    const Item it = item_of(item), nt = item_of(nxt);
    const brsrc rY = inter(it);
    const int soY = it.cb * kCW * sY;
    // twiddles of this item, then fetch the next item's
    const float2 wk = cmul(in.tw.lo0, in.tw.hi0), ws = cmul(in.tw.lo1, in.tw.hi1);
    load_tw(nt, in);
    float2 v[R];
    if constexpr (FILT || MODE == COL_FWD_V) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if constexpr (FILT)
          v[r] = r < HF ? make_float2(in.ha[r], in.hb[r]) : make_float2(0.f, 0.f);
        else
          v[r] = r < H ? make_float2(cvt1(in.za[r]), cvt1(in.zb[r])) : make_float2(0.f, 0.f);
      }
      load_head(nt, in);
      col_forward<R, YT>(v, S, rY, voY, soY, N2, c, w, wr, wk, ws);
    } else {
      const int b = it.pr / half, cp = it.pr % half;
#pragma unroll
      for (int r = 0; r < R; ++r) v[r] = cvt2(in.y[r]);
      load_head(nt, in);
      float2 u[R];
      col_inverse<R>(u, S, v, c, w, wr, wk, ws);
      const brsrc rzo = pair_rows(a.zout, (size_t)b * D + 2 * cp, sT);
      float na[H], nbv[H];
#pragma unroll
      for (int nb = 0; nb < H; ++nb) {
        if constexpr (GATE) {
          na[nb] = cvt1(in.xa[nb]) * u[nb].x + in.da * cvt1(in.za[nb]);
          nbv[nb] = cvt1(in.xb[nb]) * u[nb].y + in.db * cvt1(in.zb[nb]);
        } else {
          na[nb] = u[nb].x;
          nbv[nb] = u[nb].y;
        }
      }
      load_gate(nt, in);
#pragma unroll
      for (int nb = 0; nb < R; ++nb) {
        if (nb < H) {
          BufIO<T>::st(rzo, voT, col0(it, nb) * sT, na[nb]);
          BufIO<T>::st(rzo, voT, (col0(it, nb) + L) * sT, nbv[nb]);
          v[nb] = make_float2(na[nb], nbv[nb]);
        } else {
          v[nb] = make_float2(0.f, 0.f);
        }
      }
      if constexpr (MODE == COL_INV_FWD) {
        __syncthreads();  // S is reused
        col_forward<R, YT>(v, S, rY, voY, soY, N2, c, w, wr, wk, ws);
      }
    }
  };

  // The last item fetches itself again: the loads stay unconditional, which
  // keeps the compiler's count of loads in flight exact.
  int item = blockIdx.x;
  if (item >= nitems) return;
  In in;
  {
    const Item it = item_of(item);
    load_tw(it, in);
    load_head(it, in);
    load_gate(it, in);
  }
  while (true) {
    const int next = item + gridDim.x;
    const bool more = next < nitems;
    process(item, in, more ? next : item);
    if (!more) break;
    item = next;
    __syncthreads();  // S of this item fully read before the next one writes it
  }
}

// Row pass: N2-point DFTs of rows k1 and N1 - k1 (rows 0 and N1/2 for slot 0).
//
// Each row is spread over T = N2/E threads, E elements per thread: the thread
// of role l owns elements l + q*T (q < E), in registers before the first radix
// stage and after the last; the stages in between exchange through the padded
// LDS row. Row a (k1) sits in the lower 32 lanes of a wave, row b in the upper
// 32, and the upper lane of role T - 1 - i pairs with the lower lane of role i:
// bin N2 - 1 - k2 of row b, the partner of bin k2 of row a in the two-for-one
// product, then lives in the lane 32 apart (slot E - 1 - q), one lane swap away.
template <int N2> struct RowCfg {
  static constexpr int E = 16;
  static constexpr int T = N2 / E;                       // threads per row
  static constexpr int SP = N2 >= 2048 ? 1 : 2048 / N2;  // row pairs per workgroup
  static constexpr int WG = SP * 2 * T;
  static constexpr int RB = padded_len(N2);              // float2 per row buffer
  // two LDS buffers per row (one barrier per radix stage) while they fit two
  // workgroups per CU, else one buffer used in place
  static constexpr int NBUF = (size_t)SP * 4 * RB * 8 <= 80 * 1024 ? 2 : 1;
  static_assert(T % 16 == 0 && WG % 64 == 0, "row layout");
};

enum { ROW_CONV = 0, ROW_SPEC = 1 };

// Filter spectrum entry (P, Q) of the four-step row pass: float4 (P.re, P.im,
// Q.re, Q.im) or, next to a bf16 intermediate, the same four values as bf16 in
// 64 bits (two cbf16 words).
struct pq16 {
  unsigned int p, q;
};
template <typename YT> struct PqOf {
  using type = float4;
};
template <> struct PqOf<cbf16> {
  using type = pq16;
};
__device__ __forceinline__ float4 ldpq(const float4& x) { return x; }
__device__ __forceinline__ float4 ldpq(const pq16& x) {
  return make_float4(__uint_as_float(x.p << 16), __uint_as_float(x.p & 0xFFFF0000u), __uint_as_float(x.q << 16),
                     __uint_as_float(x.q & 0xFFFF0000u));
}
__device__ __forceinline__ void stpq(float4* p, float4 x) { *p = x; }
__device__ __forceinline__ void stpq(pq16* p, float4 x) {
  cbf16 a, b;
  stc(&a, make_float2(x.x, x.y));
  stc(&b, make_float2(x.z, x.w));
  *p = pq16{a.v, b.v};
}
// spectrum entry i: into p and, unless pb is null, its bf16 copy into pb
template <typename PT>
__device__ __forceinline__ void stspec(PT* p, pq16* pb, size_t i, float4 x) {
  stpq(p + i, x);
  if (pb != nullptr) stpq(pb + i, x);
}

// value of x held by the lane 32 apart: a backward permute through the LDS
// crossbar (an LDS-pipe instruction, no VALU work); `sw` is the byte address
// 4 * (lane ^ 32)
__device__ __forceinline__ float xhalf(float x, int sw) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(sw, __float_as_int(x)));
}
__device__ __forceinline__ unsigned xhalf(unsigned x, int sw) {
  return (unsigned)__builtin_amdgcn_ds_bpermute(sw, (int)x);
}
// a spectrum entry of the lane 32 apart, exchanged in its stored form
__device__ __forceinline__ float4 xhalf(const float4& x, int sw) {
  return make_float4(xhalf(x.x, sw), xhalf(x.y, sw), xhalf(x.z, sw), xhalf(x.w, sw));
}
__device__ __forceinline__ pq16 xhalf(const pq16& x, int sw) { return pq16{xhalf(x.p, sw), xhalf(x.q, sw)}; }

// Radix of the row DFT stage that starts at span Ns: the first stage takes the
// factor left over by 16s (2048 = 8 * 16 * 16), the later stages, which need
// twiddles, are radix 16.
constexpr int row_radix(int N, int E, int Ns) {
  if (Ns == 1) {
    int r = N;
    while (r > 16) r /= 16;
    return r < E ? r : E;
  }
  return (16 < N / Ns) ? 16 : N / Ns;
}

// number of radix stages of an N-point row DFT
constexpr int row_stages(int N, int E) {
  int n = 0;
  for (int ns = 1; ns < N; ns *= row_radix(N, E, ns)) ++n;
  return n;
}
// largest butterfly count per thread over the stages after the first
constexpr int row_nbmax(int N, int E) {
  int m = 1;
  for (int ns = row_radix(N, E, 1); ns < N; ns *= row_radix(N, E, ns)) {
    const int nb = E / row_radix(N, E, ns);
    m = nb > m ? nb : m;
  }
  return m;
}
// Sized exactly, so that the compiler keeps it in registers (CACHE false: the
// stages read the twiddle table tab instead).
template <int N, int E> struct RowTw {
  static constexpr bool CACHE = true;
  float2 w[CACHE ? row_stages(N, E) - 1 : 1][CACHE ? row_nbmax(N, E) : 1][4];
  const float2* tab;
};

template <int N, int E, int Ns, int SI> struct RowTwLoad {
  static constexpr int R = row_radix(N, E, Ns);
  static constexpr int NB = E / R;
  static constexpr int T = N / E;
  static constexpr bool LAST = Ns * R == N;
  static __device__ __forceinline__ void run(RowTw<N, E>& tw, int l, const float2* __restrict__ tab) {
    tw.tab = tab;
    if constexpr (Ns > 1 && RowTw<N, E>::CACHE) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int k = ((l + b * T) % Ns) * (N / (Ns * R));
#pragma unroll
        for (int p = 0; (1 << p) < R; ++p) tw.w[SI - 1][b][p] = tab[k << p];
      }
    }
    if constexpr (!LAST) RowTwLoad<N, E, Ns * R, SI + 1>::run(tw, l, tab);
  }
};

// One radix stage of the row DFT. Stages write alternately to the two LDS
// buffers of the row (bufs[0], bufs[1]); W is the buffer this stage writes, and
// the next stage reads it. A buffer is written again only two writes later,
// after a barrier that every reader of its previous contents has passed, so one
// barrier per stage suffices. With a single buffer (bufs[0] == bufs[1], ONE)
// the stage also waits for all reads before it writes.
template <int N, int E, int Ns, int SI, int W, bool INV, bool ONE>
__device__ __forceinline__ void row_stage(float2 (&v)[E], float2* const (&bufs)[2], int l, const RowTw<N, E>& tw) {
  constexpr int R = row_radix(N, E, Ns);
  constexpr int NB = E / R;
  constexpr int T = N / E;
  constexpr bool FIRST = Ns == 1, LAST = Ns * R == N;
  const float2* src = bufs[W ^ 1];
  float2* dst = bufs[W];
  // butterfly b, leg r works on element l + b*T + r*(N/R) = l + T*(b + r*NB)
  float2 x[NB][R];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < R; ++r) x[b][r] = FIRST ? v[b + r * NB] : src[pad16(l + b * T + r * (N / R))];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if constexpr (Ns > 1) {
      // W^(k r): powers of two from the base registers, the rest as one product
      float2 w[R];
#pragma unroll
      for (int r = 1; r < R; ++r) {
        if ((r & (r - 1)) == 0) {
          if constexpr (RowTw<N, E>::CACHE)
            w[r] = tw.w[SI - 1][b][__builtin_ctz(r)];
          else
            w[r] = tw.tab[(((l + b * T) % Ns) * (N / (Ns * R))) << __builtin_ctz(r)];
        } else {
          const int hb = 1 << (31 - __builtin_clz(r));
          w[r] = cmul(w[hb], w[r - hb]);
        }
      }
#pragma unroll
      for (int r = 1; r < R; ++r) x[b][r] = twmul<INV>(x[b][r], w[r]);
    }
    Dft<R, INV>::run(x[b]);
  }
  if (LAST) {
    // outputs land on element l + b*T + r*Ns = l + T*(b + r*NB)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int r = 0; r < R; ++r) v[b + r * NB] = x[b][r];
  } else {
    if (ONE) __syncthreads();
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int j = l + b * T;
      const int base = (j / Ns) * Ns * R + j % Ns;
#pragma unroll
      for (int r = 0; r < R; ++r) dst[pad16(base + r * Ns)] = x[b][r];
    }
    __syncthreads();
  }
}

// Runs the stages from Ns (stage number SI) on; W is the buffer the next write goes to.
template <int N, int E, int Ns, int SI, int W, bool INV, bool ONE> struct RowFrom {
  static constexpr int R = row_radix(N, E, Ns);
  static constexpr bool LAST = Ns * R == N;
  using Next = RowFrom<N, E, Ns * R, SI + 1, LAST ? W : (W ^ 1), INV, ONE>;
  static constexpr int WEND = Next::WEND;
  static __device__ __forceinline__ void run(float2 (&v)[E], float2* const (&bufs)[2], int l, const RowTw<N, E>& tw) {
    row_stage<N, E, Ns, SI, W, INV, ONE>(v, bufs, l, tw);
    Next::run(v, bufs, l, tw);
  }
};
template <int N, int E, int SI, int W, bool INV, bool ONE> struct RowFrom<N, E, N, SI, W, INV, ONE> {
  static constexpr int WEND = W;
  static __device__ __forceinline__ void run(float2 (&)[E], float2* const (&)[2], int, const RowTw<N, E>&) {}
};

// Persistent row pass; items are (channel pair, group of SP slots).
// PT: the spectrum entry type, by default the one stored next to YT; the
// spectrum pass may write bf16 entries from an fp32 intermediate.
template <typename YT, int N1, int N2, int MODE, int PF, typename PT = typename PqOf<YT>::type>
__global__ __launch_bounds__(RowCfg<N2>::WG) void rowpass_kernel(YT* __restrict__ Y, PT* __restrict__ pq,
                                                                 const float2* __restrict__ tw_row, int pq_off,
                                                                 int pair_off, int pq_mod, int nitems,
                                                                 pq16* __restrict__ pqb) {
  using C = RowCfg<N2>;
  constexpr int E = C::E, T = C::T;
  constexpr int HALF = N1 / 2;
  constexpr int PQROWS = HALF + 1;
  constexpr int NSG = HALF / C::SP;  // slot groups per channel pair
  __shared__ float2 rowbuf[C::SP * 2 * C::NBUF * C::RB];
  const int g = (threadIdx.x >> 6) * 32 + (threadIdx.x & 31);  // row-pair lane index in the workgroup
  const bool up = (threadIdx.x >> 5) & 1;                       // row b
  const int sw32 = 4 * ((int)(threadIdx.x & 63) ^ 32);            // byte address of the lane 32 apart
  const int slot = g / T, i = g % T;
  const int l = up ? T - 1 - i : i;
  float2* buf = rowbuf + (slot * 2 + (up ? 1 : 0)) * C::RB;
  float2* const bufs[2] = {buf, C::NBUF == 2 ? buf + C::SP * 2 * C::RB : buf};
  constexpr bool ONE = C::NBUF == 1;
  using Fwd = RowFrom<N2, E, 1, 0, 0, false, ONE>;
  using Inv = RowFrom<N2, E, 1, 0, Fwd::WEND, true, ONE>;
  static_assert(ONE || Inv::WEND == 0, "each item starts writing buffer 0");
  RowTw<N2, E> tw;
  RowTwLoad<N2, E, 1, 0>::run(tw, l, tw_row);
  const float nrm = 0.25f / (float)(N1 * N2);  // (1/2)(1/2N) with 2 Ha, 2 Hb below

  // slot s of an item: row a is k1 = s, row b is N1 - s (N1/2 for s = 0)
  auto row_of = [&](int item, int& pl, int& sg, int& s) {
    pl = item / NSG;
    sg = item - pl * NSG;
    s = sg * C::SP + slot;
    return up ? (s == 0 ? HALF : N1 - s) : s;
  };
  // Spectrum entries i + T*e, e < E, of a row pair: slot q of row a uses entry
  // q, slot q of row b entry E - 1 - q. The lower lane fetches entries e < E/2,
  // the upper lane entries E - 1 - e, both as pr[e]; slot q < E/2 then finds
  // its entry in its own pr[q], slot E - 1 - q in the other half's pr[q].
  auto spectrum = [&](int pl, int s) {
    // filters are shared by every batch: pair (b, cp) uses the rows of cp
    return pq + ((size_t)pq_off + (pl + pair_off) % pq_mod) * PQROWS * N2 + (size_t)s * N2;
  };
  struct In {
    YT y[E];
  };
  auto load = [&](int item, In& in) {
    int pl, sg, s;
    const int k1 = row_of(item, pl, sg, s);
    const YT* Yr = Y + ((size_t)pl * N1 + k1) * N2;
#pragma unroll
    for (int q = 0; q < E; ++q) in.y[q] = Yr[l + q * T];
  };
  PT pr[E / 2];
  // in 1024-thread workgroups (128 VGPRs) the spectrum entries are fetched
  // after the forward DFT, so that they do not share registers with it
  constexpr bool LATE_PQ = C::WG > 512 && !(PF & 2);
  auto load_spectrum = [&](int item) {
    if (MODE == ROW_CONV) {
      int pl, sg, s;
      row_of(item, pl, sg, s);
      // slot 0 reads its spectrum rows in the LDS branch; load a valid row anyway
      // so that the number of loads in flight does not depend on the item
      const PT* pqs = spectrum(pl, s == 0 ? 1 : s) + i;
#pragma unroll
      for (int e = 0; e < E / 2; ++e) pr[e] = pqs[(up ? E - 1 - e : e) * T];
    }
  };

  auto process = [&](int item, In& in, int next, bool more) {
    int pl, sg, s;
    const int k1 = row_of(item, pl, sg, s);
    PT* pqp = spectrum(pl, 0);
    pq16* pqbp = pqb == nullptr ? nullptr : pqb + (pqp - pq);  // ROW_SPEC: the bf16 copy
    float2 v[E];
#pragma unroll
    for (int q = 0; q < E; ++q) v[q] = cvt2(in.y[q]);
    // the rows are in v: fetch the next item's into the same registers
    if (PF & 1) load(more ? next : item, in);
    Fwd::run(v, bufs, l, tw);
    if (LATE_PQ) load_spectrum(item);
    if (s != 0) {
      // own bin (slot q) and the partner's (the other half's slot E - 1 - q),
      // taken for q and E - 1 - q together before either is overwritten; row b
      // uses conj(P), conj(Q)
      const float sg_ = up ? -1.f : 1.f;
#pragma unroll
      for (int q = 0; q < E / 2; ++q) {
        const int q2 = E - 1 - q;
        const float2 pm = make_float2(xhalf(v[q2].x, sw32), xhalf(v[q2].y, sw32));
        const float2 pm2 = make_float2(xhalf(v[q].x, sw32), xhalf(v[q].y, sw32));
        if (MODE == ROW_CONV) {
          const float4 o = ldpq(xhalf(pr[q], sw32)), w = ldpq(pr[q]);
          const float2 P = make_float2(w.x, sg_ * w.y), Q = make_float2(w.z, sg_ * w.w);
          const float2 P2 = make_float2(o.x, sg_ * o.y), Q2 = make_float2(o.z, sg_ * o.w);
          v[q] = cadd(cmul(v[q], P), cmul(conjf2(pm), Q));
          v[q2] = cadd(cmul(v[q2], P2), cmul(conjf2(pm2), Q2));
        } else if (!up) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float2 xk = h ? v[q2] : v[q], fm = conjf2(h ? pm2 : pm);
            const float2 ha2 = cadd(xk, fm), d = csub(xk, fm);
            const float2 hb2 = make_float2(d.y, -d.x);
            stspec(pqp, pqbp, (size_t)s * N2 + i + (h ? q2 : q) * T,
                   make_float4(nrm * (ha2.x + hb2.x), nrm * (ha2.y + hb2.y), nrm * (ha2.x - hb2.x),
                               nrm * (ha2.y - hb2.y)));
          }
        }
      }
    }
    // this item's spectrum entries have been used: fetch the next item's
    if (PF & 2) load_spectrum(more ? next : item);
    if (sg == 0) {
      // Workgroup-uniform branch: slot 0 holds rows 0 and N1/2, each paired with
      // itself (row 0: k2 with (N2 - k2) mod N2; row N1/2: k2 with N2 - 1 - k2),
      // so their bins meet in LDS.
      __syncthreads();
      if (s == 0) {
#pragma unroll
        for (int q = 0; q < E; ++q) buf[pad16(l + q * T)] = v[q];
      }
      __syncthreads();
      if (s == 0) {
        const int pqrow = up ? HALF : 0;
        const PT* pqs = pqp + (size_t)pqrow * N2;
        const int kend = (MODE == ROW_CONV) ? (up ? N2 / 2 - 1 : N2 / 2) : N2 - 1;
        // fixed trip count (k2 = i + it*T <= kend), so that the loads in it are
        // straight-line code the compiler can count
        constexpr int KIT = (MODE == ROW_CONV) ? E / 2 + 1 : E;
#pragma unroll
        for (int it = 0; it < KIT; ++it) {
          const int k2 = i + it * T;
          if (k2 > kend) continue;
          const int m2 = up ? (N2 - 1 - k2) : ((N2 - k2) & (N2 - 1));
          const float2 xk = buf[pad16(k2)], xm = buf[pad16(m2)];
          if (MODE == ROW_CONV) {
            const float4 q4 = ldpq(pqs[k2]);
            const float2 P = make_float2(q4.x, q4.y), Q = make_float2(q4.z, q4.w);
            const float2 yk = cadd(cmul(xk, P), cmul(conjf2(xm), Q));
            if (m2 != k2) buf[pad16(m2)] = cadd(cmulc(xm, P), cmulc(conjf2(xk), Q));
            buf[pad16(k2)] = yk;
          } else {
            const float2 fm = conjf2(xm);
            const float2 ha2 = cadd(xk, fm), d = csub(xk, fm);
            const float2 hb2 = make_float2(d.y, -d.x);
            stspec(pqp, pqbp, (size_t)pqrow * N2 + k2,
                   make_float4(nrm * (ha2.x + hb2.x), nrm * (ha2.y + hb2.y), nrm * (ha2.x - hb2.x),
                               nrm * (ha2.y - hb2.y)));
          }
        }
      }
      __syncthreads();
      if (MODE == ROW_CONV) {
        if (s == 0) {
#pragma unroll
          for (int q = 0; q < E; ++q) v[q] = buf[pad16(l + q * T)];
        }
        __syncthreads();  // the inverse DFT writes this buffer next
      }
    }
    if (MODE == ROW_SPEC) {
      __syncthreads();  // the next item's first stage writes the buffer read last
      return;
    }
    Inv::run(v, bufs, l, tw);
    YT* Yr = Y + ((size_t)pl * N1 + k1) * N2;
#pragma unroll
    for (int q = 0; q < E; ++q) stc(Yr + l + q * T, v[q]);
  };

  // With PF each part of the next item's data is fetched into the registers of
  // the current item's as soon as that part has been used (the rows after the
  // first radix stage has taken them, the spectrum entries after the product),
  // so one register set carries a whole item of prefetch. The last item fetches
  // itself again: the loads stay unconditional, which keeps the compiler's
  // count of loads in flight exact.
  int item = blockIdx.x;
  if (item >= nitems) return;
  In in;
  load(item, in);
  if (!LATE_PQ) load_spectrum(item);
  while (true) {
    const int next = item + gridDim.x;
    const bool more = next < nitems;
    process(item, in, next, more);
    if (!more) break;
    item = next;
    if (!(PF & 1)) load(item, in);
    if (!(PF & 2) && !LATE_PQ) load_spectrum(item);
  }
  // Between items: buffer 0, which the next item writes first, was last read
  // before a barrier of this item (with one buffer every write waits for one).
}

// Row pass for 8192-point rows: a row pair in one workgroup would need 1024
// threads (128 VGPRs each, too few), so 512 threads take the two rows one after
// the other: forward DFT of row a into its LDS buffer, then of row b, the
// spectrum product between the buffers, then the two inverse DFTs. Same work
// items, layouts and results as rowpass_kernel.
template <int N2> struct RowSeqCfg {
  static constexpr int E = 16;
  static constexpr int T = N2 / E;  // threads, one row at a time
  static constexpr int RB = padded_len(N2);
};

template <typename YT, int N1, int N2, int MODE, typename PT = typename PqOf<YT>::type>
__global__ __launch_bounds__(RowSeqCfg<N2>::T) void rowpass_seq_kernel(YT* __restrict__ Y, PT* __restrict__ pq,
                                                                       const float2* __restrict__ tw_row, int pq_off,
                                                                       int pair_off, int pq_mod, int nitems,
                                                                       pq16* __restrict__ pqb) {
  using C = RowSeqCfg<N2>;
  constexpr int E = C::E, T = C::T;
  constexpr int HALF = N1 / 2;
  constexpr int PQROWS = HALF + 1;
  __shared__ float2 rowbuf[2 * C::RB];
  float2* A = rowbuf;
  float2* B = rowbuf + C::RB;
  const int l = threadIdx.x;
  using Fwd = RowFrom<N2, E, 1, 0, 0, false, true>;
  using Inv = RowFrom<N2, E, 1, 0, 0, true, true>;
  RowTw<N2, E> tw;
  RowTwLoad<N2, E, 1, 0>::run(tw, l, tw_row);
  const float nrm = 0.25f / (float)(N1 * N2);

  // Each row is fetched one forward transform ahead, into one row's worth of
  // registers: row b while row a is transformed, the next item's row a while
  // row b is (the last item fetches itself again, so that the loads stay
  // unconditional).
  auto row_ptr = [&](int item, int h) {
    const int pl = item / HALF, s = item - pl * HALF;
    const int k1 = h ? (s == 0 ? HALF : N1 - s) : s;
    return Y + ((size_t)pl * N1 + k1) * N2;
  };
  if ((int)blockIdx.x >= nitems) return;
  YT rr[E];
  {
    const YT* Yr = row_ptr(blockIdx.x, 0);
#pragma unroll
    for (int q = 0; q < E; ++q) rr[q] = Yr[l + q * T];
  }
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int pl = item / HALF, s = item - pl * HALF;
    const int next = item + gridDim.x < nitems ? item + gridDim.x : item;
    PT* pqp = pq + ((size_t)pq_off + (pl + pair_off) % pq_mod) * PQROWS * N2;
    pq16* pqbp = pqb == nullptr ? nullptr : pqb + (pqp - pq);  // ROW_SPEC: the bf16 copy
    YT* Ya = row_ptr(item, 0);
    YT* Yb = row_ptr(item, 1);
    // forward DFTs, results to the row buffers in natural order (one row at a
    // time: a rolled loop, so that the two rows' work is not interleaved)
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
      float2* bf = h ? B : A;
      float2* const bufs[2] = {bf, bf};
      float2 v[E];
#pragma unroll
      for (int q = 0; q < E; ++q) v[q] = cvt2(rr[q]);
      const YT* Yn = h ? row_ptr(next, 0) : Yb;
#pragma unroll
      for (int q = 0; q < E; ++q) rr[q] = Yn[l + q * T];
      Fwd::run(v, bufs, l, tw);
      __syncthreads();  // the last stage's reads of bf are done
#pragma unroll
      for (int q = 0; q < E; ++q) bf[pad16(l + q * T)] = v[q];
    }
    __syncthreads();
    // spectrum product: bin k2 of row a with bin N2 - 1 - k2 of row b (s != 0);
    // rows 0 and N1/2 (s = 0) are each paired with themselves
    if (s != 0) {
      const PT* pqs = pqp + (size_t)s * N2;
#pragma unroll
      for (int q = 0; q < E; ++q) {
        const int k2 = l + q * T, m2 = N2 - 1 - k2;
        const float2 xk = A[pad16(k2)], xm = B[pad16(m2)];
        const float4 w4 = ldpq(pqs[k2]);
        if (MODE == ROW_CONV) {
          const float2 P = make_float2(w4.x, w4.y), Q = make_float2(w4.z, w4.w);
          A[pad16(k2)] = cadd(cmul(xk, P), cmul(conjf2(xm), Q));
          B[pad16(m2)] = cadd(cmulc(xm, P), cmulc(conjf2(xk), Q));
        } else {
          const float2 fm = conjf2(xm);
          const float2 ha2 = cadd(xk, fm), d = csub(xk, fm);
          const float2 hb2 = make_float2(d.y, -d.x);
          stspec(pqp, pqbp, (size_t)s * N2 + k2,
                 make_float4(nrm * (ha2.x + hb2.x), nrm * (ha2.y + hb2.y), nrm * (ha2.x - hb2.x),
                             nrm * (ha2.y - hb2.y)));
        }
      }
    } else {
#pragma unroll 1
      for (int h = 0; h < 2; ++h) {
        float2* row = h ? B : A;
        const int pqrow = h ? HALF : 0;
        const PT* pqs = pqp + (size_t)pqrow * N2;
        const int kend = (MODE == ROW_CONV) ? (h ? N2 / 2 - 1 : N2 / 2) : N2 - 1;
        constexpr int KIT = (MODE == ROW_CONV) ? E / 2 + 1 : E;
#pragma unroll
        for (int it = 0; it < KIT; ++it) {
          const int k2 = l + it * T;
          if (k2 > kend) continue;
          const int m2 = h ? (N2 - 1 - k2) : ((N2 - k2) & (N2 - 1));
          const float2 xk = row[pad16(k2)], xm = row[pad16(m2)];
          const float4 w4 = ldpq(pqs[k2]);
          if (MODE == ROW_CONV) {
            const float2 P = make_float2(w4.x, w4.y), Q = make_float2(w4.z, w4.w);
            const float2 yk = cadd(cmul(xk, P), cmul(conjf2(xm), Q));
            if (m2 != k2) row[pad16(m2)] = cadd(cmulc(xm, P), cmulc(conjf2(xk), Q));
            row[pad16(k2)] = yk;
          } else {
            const float2 fm = conjf2(xm);
            const float2 ha2 = cadd(xk, fm), d = csub(xk, fm);
            const float2 hb2 = make_float2(d.y, -d.x);
            stspec(pqp, pqbp, (size_t)pqrow * N2 + k2,
                   make_float4(nrm * (ha2.x + hb2.x), nrm * (ha2.y + hb2.y), nrm * (ha2.x - hb2.x),
                               nrm * (ha2.y - hb2.y)));
          }
        }
      }
    }
    __syncthreads();
    if (MODE == ROW_CONV) {
      // inverse DFTs, each from its row buffer, written back to the intermediate
#pragma unroll 1
      for (int h = 0; h < 2; ++h) {
        float2* bf = h ? B : A;
        YT* Yr = h ? Yb : Ya;
        float2* const bufs[2] = {bf, bf};
        float2 v[E];
#pragma unroll
        for (int q = 0; q < E; ++q) v[q] = bf[pad16(l + q * T)];
        Inv::run(v, bufs, l, tw);  // its first write waits for a barrier
#pragma unroll
        for (int q = 0; q < E; ++q) stc(Yr + l + q * T, v[q]);
      }
    }
    __syncthreads();  // the next item writes both buffers
  }
}

// ============================================================ launchers

// ============================================================ LDS regime, register-resident

// All orders of one channel pair in one thread group, for 1024 <= 2L <= 4096.
// Same computation as fftconv_lds_kernel, laid out like the row pass: thread l
// of a pair owns elements l + q T (q < E) in registers before the first radix
// stage and after the last, the stages in between exchange through the padded
// LDS buffers, and the stage twiddles are cached in registers. z^n at
// t = l + q T (q < E/2, the positions t < L) stays in the registers of the
// thread that feeds it to the forward transform and gates the inverse one.
// Each order's filter spectrum entries are requested before its forward
// transform and its gate inputs after it, so that their latency is covered.
template <int N, int NBUF> struct LdsRegCfg {
  static_assert(N >= 1024 && N <= 4096, "256-thread workgroups, two per CU");
  static constexpr int E = 16;
  static constexpr int T = N / E;                // threads per channel pair
  static constexpr int WG = 256;                 // threads per workgroup
  static constexpr int G = WG / T;               // channel pairs per workgroup
  static constexpr int RB = padded_len(N);       // float2 per buffer
  static constexpr size_t LDS = (size_t)G * NBUF * RB * sizeof(float2);
};

template <typename T, int N, int NBUF>
__global__ __launch_bounds__(256, 2) void fftconv_lds_reg_kernel(
    const T* __restrict__ sp, const float* __restrict__ dskip, const float4* __restrict__ pq,
    const float2* __restrict__ twtab, T* __restrict__ zout, int D, int NO) {
  using C = LdsRegCfg<N, NBUF>;
  constexpr int E = C::E, TT = C::T, L = N / 2, H = E / 2;
  constexpr int KIT = (L + 1 + TT - 1) / TT;  // spectrum entries k = l + i T <= L per thread
  constexpr bool ONE = NBUF == 1;
  extern __shared__ float4 smem4[];
  const int g = threadIdx.x / TT, l = threadIdx.x % TT;
  float2* buf = reinterpret_cast<float2*>(smem4) + (size_t)g * NBUF * C::RB;
  float2* const bufs[2] = {buf, ONE ? buf : buf + C::RB};
  using Fwd = RowFrom<N, E, 1, 0, 0, false, ONE>;
  constexpr int WP = Fwd::WEND;  // buffer of the spectrum product (not read by the last forward stage)
  using Inv = RowFrom<N, E, 1, 0, WP ^ 1, true, ONE>;
  RowTw<N, E> tw;
  RowTwLoad<N, E, 1, 0>::run(tw, l, twtab);

  const int pr = blockIdx.x * C::G + g;
  const int half = D / 2;
  const int b = pr / half, cp = pr % half;
  const int ca = 2 * cp, cb = ca + 1;
  const size_t J = (size_t)(NO + 1) * D;
  const T* sb = sp + (size_t)b * J * L;  // short-convolved blocks (v, x^1, .., x^NO)

  float2 z[H];  // (z_a, z_b) at t = l + q T
#pragma unroll
  for (int q = 0; q < H; ++q) {
    const int t = l + q * TT;
    z[q] = make_float2(ldf(sb + (size_t)ca * L + t), ldf(sb + (size_t)cb * L + t));
  }
  for (int n = 0; n < NO; ++n) {
    // this order's spectrum entries (k clamped to L: the extra entries go unused)
    const float4* pqn = pq + ((size_t)n * half + cp) * (L + 1);
    float4 pk[KIT];
#pragma unroll
    for (int i = 0; i < KIT; ++i) {
      const int k = l + i * TT;
      pk[i] = pqn[k <= L ? k : L];
    }
    const float da = dskip[n * D + ca], db = dskip[n * D + cb];

    float2 v[E];
#pragma unroll
    for (int q = 0; q < E; ++q) v[q] = q < H ? z[q] : make_float2(0.f, 0.f);
    Fwd::run(v, bufs, l, tw);
    // this order's gates, needed after the product and the inverse transform
    T xa[H], xb[H];
    const T* sx = sb + (size_t)((n + 1) * D + ca) * L;
#pragma unroll
    for (int q = 0; q < H; ++q) {
      xa[q] = sx[l + q * TT];
      xb[q] = sx[L + l + q * TT];
    }
    // spectrum product on the bin pairs (k, N - k), k in [0, L], through LDS
    float2* P = bufs[WP];
    if (ONE) __syncthreads();
#pragma unroll
    for (int q = 0; q < E; ++q) P[pad16(l + q * TT)] = v[q];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KIT; ++i) {
      const int k = l + i * TT;
      if (k <= L) {
        const float2 Pk = make_float2(pk[i].x, pk[i].y), Qk = make_float2(pk[i].z, pk[i].w);
        const int m = (N - k) & (N - 1);
        const float2 xk = P[pad16(k)], xm = P[pad16(m)];
        const float2 yk = cadd(cmul(xk, Pk), cmul(conjf2(xm), Qk));
        if (m != k) P[pad16(m)] = cadd(cmulc(xm, Pk), cmulc(conjf2(xk), Qk));
        P[pad16(k)] = yk;
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < E; ++q) v[q] = P[pad16(l + q * TT)];
    Inv::run(v, bufs, l, tw);
    // gate + skip on t = l + q T < L
    const bool last = (n == NO - 1);
#pragma unroll
    for (int q = 0; q < H; ++q) {
      const float na = cvt1(xa[q]) * v[q].x + da * z[q].x;
      const float nb = cvt1(xb[q]) * v[q].y + db * z[q].y;
      if (last) {
        const int t = l + q * TT;
        stf(zout + ((size_t)b * D + ca) * L + t, na);
        stf(zout + ((size_t)b * D + cb) * L + t, nb);
      } else {
        z[q] = make_float2(na, nb);
      }
    }
    __syncthreads();  // the next order's first stage writes buffer 0 again
  }
}

static hipError_t allow_lds(const void* fn, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// LDS buffers per channel pair of the register-resident kernel (HYENA_LDS_NBUF:
// 2 = one barrier per radix stage, 1 = half the LDS, two barriers per stage)
static int lds_nbuf() {
  static const int nb = [] {
    const char* e = getenv("HYENA_LDS_NBUF");
    return e && atoi(e) == 1 ? 1 : 2;
  }();
  return nb;
}

template <typename T, int N>
static hipError_t launch_lds_conv(const LdsConvArgs& a, hipStream_t s) {
  const int pairs = a.B * a.D / 2;
  if constexpr (N >= 1024 && N <= 4096) {
    auto go = [&](auto nbuf) -> hipError_t {
      constexpr int NB = decltype(nbuf)::value;
      using C = LdsRegCfg<N, NB>;
      auto fn = fftconv_lds_reg_kernel<T, N, NB>;
      hipError_t e = allow_lds((const void*)fn, C::LDS);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(fn, dim3(pairs / C::G), dim3(C::WG), C::LDS, s, (const T*)a.s, a.dskip, a.pq, a.tw,
                         (T*)a.zout, a.D, a.NO);
      return hipGetLastError();
    };
    return lds_nbuf() == 1 ? go(std::integral_constant<int, 1>{}) : go(std::integral_constant<int, 2>{});
  } else {
    using C = LdsCfg<N>;
    auto fn = fftconv_lds_kernel<T, N>;
    hipError_t e = allow_lds((const void*)fn, C::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3(pairs / C::G), dim3(C::WG), C::LDS, s, (const T*)a.s, a.dskip, a.pq, a.tw,
                       (T*)a.zout, a.D, a.NO);
    return hipGetLastError();
  }
}

template <int N>
static hipError_t launch_lds_spec(const float* h, const float2* tw, float4* pq, int D, int NO, bool wrapped,
                                  hipStream_t s) {
  using C = LdsCfg<N>;
  const int pairs = NO * D / 2;
  const size_t lds = (size_t)C::G * C::FB * 8;
  auto fn = wrapped ? filter_spec_lds_kernel<N, true> : filter_spec_lds_kernel<N, false>;
  hipError_t e = allow_lds((const void*)fn, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(pairs / C::G), dim3(C::WG), lds, s, h, tw, pq, D, NO);
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

hipError_t lds_spec(const float* h, const float2* tw, float4* pq, int L, int D, int NO, bool wrapped,
                    hipStream_t s) {
  const int N = 2 * L;
  hipError_t e = hipSuccess;
#define CALLS(n) e = launch_lds_spec<n>(h, tw, pq, D, NO, wrapped, s)
  HY_LDS_SWITCH(N, CALLS)
#undef CALLS
  return e;
}

// Workgroups of a persistent launch: as many as are resident at once.
static int resident_grid(const void* fn, int block, size_t lds, int items) {
  static DeviceCache cus_cache;
  const int cus = cus_cache.get([] {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    return n;
  });
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block, lds) != hipSuccess || per_cu <= 0) per_cu = 1;
  const long long g = (long long)cus * per_cu;
  return (int)(g < items ? g : items);
}

template <typename T, typename YT, int R, int M>
static hipError_t launch_col_t(const ColArgs& a, int pairs, hipStream_t s) {
  constexpr int kCW = col_width<R>();
  const size_t lds = (size_t)R * R * kCW * sizeof(float2);
  auto fn = colpass_kernel<T, YT, R, M>;
  hipError_t e = allow_lds((const void*)fn, lds);
  if (e != hipSuccess) return e;
  const int items = pairs * (a.N2 / kCW);
  static DeviceCache grid_cache;
  const int grid = grid_cache.get([&] { return resident_grid((const void*)fn, R * kCW, lds, 1 << 30); });
  hipLaunchKernelGGL(fn, dim3(grid < items ? grid : items), dim3(R * kCW), lds, s, a, items);
  return hipGetLastError();
}

template <typename T, typename YT, int R>
static hipError_t launch_col_r(const ColArgs& a, int mode, int pairs, hipStream_t s) {
  switch (mode) {
    case COL_FWD_V: return launch_col_t<T, YT, R, COL_FWD_V>(a, pairs, s);
    case COL_FWD_H: return launch_col_t<float, float2, R, COL_FWD_H>(a, pairs, s);
    case COL_FWD_HW: return launch_col_t<float, float2, R, COL_FWD_HW>(a, pairs, s);
    case COL_INV: return launch_col_t<T, YT, R, COL_INV>(a, pairs, s);
    case COL_INV_PLAIN: return launch_col_t<T, YT, R, COL_INV_PLAIN>(a, pairs, s);
    default: return launch_col_t<T, YT, R, COL_INV_FWD>(a, pairs, s);
  }
}

// act_bf16: activation storage; ybf: intermediate stored as bf16 pairs
static hipError_t launch_col(const ColArgs& a, int N1, int mode, bool act_bf16, bool ybf, int pairs,
                             hipStream_t s) {
  if (N1 == 64) {
    if (act_bf16) return ybf ? launch_col_r<bf16, cbf16, 8>(a, mode, pairs, s)
                             : launch_col_r<bf16, float2, 8>(a, mode, pairs, s);
    return launch_col_r<float, float2, 8>(a, mode, pairs, s);
  }
  if (N1 == 256) {
    if (act_bf16) return ybf ? launch_col_r<bf16, cbf16, 16>(a, mode, pairs, s)
                             : launch_col_r<bf16, float2, 16>(a, mode, pairs, s);
    return launch_col_r<float, float2, 16>(a, mode, pairs, s);
  }
  return hipErrorInvalidValue;
}

// PT other than the entry type stored next to YT: the spectrum pass only (bf16
// entries written from an fp32 intermediate).
template <typename YT, int N1, int N2, typename PT = typename PqOf<YT>::type>
static hipError_t launch_row_t(void* Y, void* pqv, const float2* tw_row, int pq_off, int pair_off, int pq_mod,
                               int pairs, int mode, hipStream_t s, void* pqb) {
  constexpr bool SPEC_ONLY = !std::is_same<PT, typename PqOf<YT>::type>::value;
  if (SPEC_ONLY && mode != ROW_SPEC) return hipErrorInvalidValue;
  YT* y = static_cast<YT*>(Y);
  PT* pq = static_cast<PT*>(pqv);
  if constexpr (N2 >= 8192) {
    const int items = pairs * (N1 / 2);
    auto fn = SPEC_ONLY || mode != ROW_CONV ? rowpass_seq_kernel<YT, N1, N2, ROW_SPEC, PT>
                                            : rowpass_seq_kernel<YT, N1, N2, ROW_CONV, PT>;
    static DeviceCache grid_cache[2];
    const int g = grid_cache[mode == ROW_CONV ? 0 : 1].get(
        [&] { return resident_grid((const void*)fn, RowSeqCfg<N2>::T, 0, 1 << 30); });
    hipLaunchKernelGGL(fn, dim3(g < items ? g : items), dim3(RowSeqCfg<N2>::T), 0, s, y, pq, tw_row, pq_off,
                       pair_off, pq_mod, items, static_cast<pq16*>(pqb));
    return hipGetLastError();
  } else {
    using C = RowCfg<N2>;
    const int items = pairs * ((N1 / 2) / C::SP);
    // HYENA_ROW_PREFETCH: bit 0 fetches the next item's rows early, bit 1 its
    // spectrum entries; otherwise they are loaded when the item starts. Rows
    // early (1) measures best; fetching the spectrum early is slower.
    static const int pf = [] {
      const char* v = getenv("HYENA_ROW_PREFETCH");
      return v ? atoi(v) & 3 : 1;
    }();
    using Fn = void (*)(YT*, PT*, const float2*, int, int, int, int, pq16*);
    Fn fn;
    if constexpr (SPEC_ONLY) {
      fn = rowpass_kernel<YT, N1, N2, ROW_SPEC, 0, PT>;
    } else {
      if (mode != ROW_CONV) fn = rowpass_kernel<YT, N1, N2, ROW_SPEC, 0>;
      else if (pf == 1) fn = rowpass_kernel<YT, N1, N2, ROW_CONV, 1>;
      else if (pf == 2) fn = rowpass_kernel<YT, N1, N2, ROW_CONV, 2>;
      else if (pf == 3) fn = rowpass_kernel<YT, N1, N2, ROW_CONV, 3>;
      else fn = rowpass_kernel<YT, N1, N2, ROW_CONV, 0>;
    }
    // LDS is static in the kernel
    static DeviceCache grid_cache[2];
    const int g = grid_cache[mode == ROW_CONV ? 0 : 1].get(
        [&] { return resident_grid((const void*)fn, C::WG, 0, 1 << 30); });
    hipLaunchKernelGGL(fn, dim3(g < items ? g : items), dim3(C::WG), 0, s, y, pq, tw_row, pq_off, pair_off,
                       pq_mod, items, static_cast<pq16*>(pqb));
    return hipGetLastError();
  }
}

template <typename YT, typename PT = typename PqOf<YT>::type>
static hipError_t launch_row_y(int N1, int N2, void* Y, void* pq, const float2* tw_row, int pq_off, int pair_off,
                               int pq_mod, int pairs, int mode, hipStream_t s, void* pqb = nullptr) {
#define ROWCASE(n1, n2)                                                                                  \
  if (N1 == n1 && N2 == n2)                                                                              \
    return launch_row_t<YT, n1, n2, PT>(Y, pq, tw_row, pq_off, pair_off, pq_mod, pairs, mode, s, pqb);
  ROWCASE(64, 256)
  ROWCASE(64, 512)
  ROWCASE(64, 1024)
  ROWCASE(64, 2048)
  ROWCASE(256, 1024)
  ROWCASE(256, 2048)
  ROWCASE(256, 4096)
  ROWCASE(256, 8192)
#undef ROWCASE
  return hipErrorInvalidValue;
}

static ColArgs col_args(const FourStepTables& tb, int L, int D, int NO) {
  ColArgs a{};
  a.w256 = tb.w256;
  a.tw_lo = tb.tw_lo;
  a.tw_hi = tb.tw_hi;
  a.lo_bits = tb.lo_bits;
  a.L = L;
  a.N2 = 2 * L / fourstep_n1(L);
  a.D = D;
  a.NO = NO;
  return a;
}

// bf16 copy of the filter spectra (rounded to nearest even), read by the row
// passes of bf16 workloads
hipError_t fourstep_spec(const FourStepTables& tb, const float* h, float2* Y, float4* pq, void* pq_bf16, int L,
                         int D, int NO, bool wrapped, hipStream_t s) {
  ColArgs a = col_args(tb, L, D, NO);
  const int N1 = fourstep_n1(L);
  a.h = h;
  a.Y = Y;
  const int pairs = NO * D / 2;
  if (pq == nullptr && pq_bf16 == nullptr) return hipErrorInvalidValue;
  hipError_t e = launch_col(a, N1, wrapped ? COL_FWD_HW : COL_FWD_H, false, false, pairs, s);
  if (e != hipSuccess) return e;
  if (pq == nullptr)  // bf16 entries only, written by the spectrum pass itself
    return launch_row_y<float2, pq16>(N1, a.N2, Y, pq_bf16, tb.tw_row, 0, 0, pairs, pairs, ROW_SPEC, s);
  // fp32 entries, and the bf16 copy (if asked for) from the same values
  return launch_row_y<float2>(N1, a.N2, Y, pq, tb.tw_row, 0, 0, pairs, pairs, ROW_SPEC, s, pq_bf16);
}

hipError_t fourstep_conv(const FourStepTables& tb, const FourStepConvArgs& c, bool is_bf16, hipStream_t s) {
  ColArgs a = col_args(tb, c.L, c.D, c.NO);
  const int N1 = fourstep_n1(c.L);
  a.s = c.s;
  a.dskip = c.dskip;
  a.Y = c.Y;
  const bool ybf = is_bf16 && c.y_bf16;
  const int half = c.D / 2;
  const int pairs_all = c.B * half;
  // Channel-pair groups bound the intermediate so that it can stay in the
  // last-level cache between the passes of one group.
  const int gp = (c.group_pairs > 0 && c.group_pairs < pairs_all) ? c.group_pairs : pairs_all;
  for (int p0 = 0; p0 < pairs_all; p0 += gp) {
    const int np = (pairs_all - p0 < gp) ? pairs_all - p0 : gp;
    ColArgs g = a;
    g.pair_off = p0;
    hipError_t e = launch_col(g, N1, COL_FWD_V, is_bf16, ybf, np, s);
    if (e != hipSuccess) return e;
    for (int n = 0; n < c.NO; ++n) {
      e = ybf ? launch_row_y<cbf16>(N1, a.N2, c.Y, const_cast<void*>(c.pq_bf16), tb.tw_row, n * half, p0, half,
                                    np, ROW_CONV, s)
              : launch_row_y<float2>(N1, a.N2, c.Y, const_cast<float4*>(c.pq), tb.tw_row, n * half, p0, half, np,
                                     ROW_CONV, s);
      if (e != hipSuccess) return e;
      ColArgs gi = g;
      gi.n = n;
      gi.zin = (n == 0) ? nullptr : c.z[(n - 1) & 1];
      gi.zout = (n == c.NO - 1) ? c.zfinal : c.z[n & 1];
      e = launch_col(gi, N1, (n == c.NO - 1) ? (c.plain ? COL_INV_PLAIN : COL_INV) : COL_INV_FWD, is_bf16, ybf,
                     np, s);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace hy
