// Shared device/host helpers of libhyena (gfx950). Internal header.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>
#include <stddef.h>

namespace hy {

typedef __bf16 bf16;

// ------------------------------------------------------------- storage types

template <typename T> __device__ __forceinline__ float ldf(const T* p);
template <> __device__ __forceinline__ float ldf<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ldf<bf16>(const bf16* p) { return (float)(*p); }

template <typename T> __device__ __forceinline__ void stf(T* p, float v);
template <> __device__ __forceinline__ void stf<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void stf<bf16>(bf16* p, float v) { *p = (bf16)v; }

// ------------------------------------------------------------ complex floats

__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
// a * conj(b)
__device__ __forceinline__ float2 cmulc(float2 a, float2 b) {
  return make_float2(a.x * b.x + a.y * b.y, a.y * b.x - a.x * b.y);
}
__device__ __forceinline__ float2 conjf2(float2 a) { return make_float2(a.x, -a.y); }
// multiply by W (forward) or conj(W) (inverse)
template <bool INV> __device__ __forceinline__ float2 twmul(float2 a, float2 w) {
  return INV ? cmulc(a, w) : cmul(a, w);
}

// ------------------------------------------------- small DFTs in registers
// Forward: X[k] = sum_n x[n] exp(-2 pi i n k / R); inverse uses exp(+...),
// unnormalised. Natural order in and out.

// multiply by W_16^j (forward) or W_16^-j (inverse), j compile-time after unrolling
template <bool INV> __device__ __forceinline__ float2 tw16(int j, float2 a) {
  const float c1 = 0.92387953251128674f, s1 = 0.38268343236508978f, h = 0.70710678118654752f;
  // W_16^j = cos(2 pi j / 16) - i sin(2 pi j / 16)
  float c, s;
  switch (j & 15) {
    case 0: return a;
    case 4: return INV ? make_float2(-a.y, a.x) : make_float2(a.y, -a.x);
    case 8: return make_float2(-a.x, -a.y);
    case 12: return INV ? make_float2(a.y, -a.x) : make_float2(-a.y, a.x);
    case 2: { float2 r = INV ? make_float2(a.x - a.y, a.x + a.y) : make_float2(a.x + a.y, a.y - a.x);
              return make_float2(r.x * h, r.y * h); }
    case 6: { float2 r = INV ? make_float2(-a.x - a.y, a.x - a.y) : make_float2(a.y - a.x, -a.x - a.y);
              return make_float2(r.x * h, r.y * h); }
    case 10: { float2 r = INV ? make_float2(a.y - a.x, -a.x - a.y) : make_float2(-a.x - a.y, a.x - a.y);
               return make_float2(r.x * h, r.y * h); }
    case 14: { float2 r = INV ? make_float2(a.x + a.y, a.y - a.x) : make_float2(a.x - a.y, a.x + a.y);
               return make_float2(r.x * h, r.y * h); }
    case 1: c = c1; s = s1; break;
    case 3: c = s1; s = c1; break;
    case 5: c = -s1; s = c1; break;
    case 7: c = -c1; s = s1; break;
    case 9: c = -c1; s = -s1; break;
    case 11: c = -s1; s = -c1; break;
    case 13: c = s1; s = -c1; break;
    default: c = c1; s = -s1; break;  // 15
  }
  // forward: (c - i s); inverse: (c + i s)
  if (INV) s = -s;
  return make_float2(a.x * c + a.y * s, a.y * c - a.x * s);
}

template <int R, bool INV> struct Dft;

template <bool INV> struct Dft<1, INV> {
  static __device__ __forceinline__ void run(float2*) {}
};
template <bool INV> struct Dft<2, INV> {
  static __device__ __forceinline__ void run(float2* v) {
    float2 a = v[0];
    v[0] = cadd(a, v[1]);
    v[1] = csub(a, v[1]);
  }
};
template <bool INV> struct Dft<4, INV> {
  static __device__ __forceinline__ void run(float2* v) {
    float2 a0 = cadd(v[0], v[2]), a1 = csub(v[0], v[2]);
    float2 a2 = cadd(v[1], v[3]), a3 = csub(v[1], v[3]);
    // forward: -i * a3 ; inverse: +i * a3
    float2 r = INV ? make_float2(-a3.y, a3.x) : make_float2(a3.y, -a3.x);
    v[0] = cadd(a0, a2);
    v[2] = csub(a0, a2);
    v[1] = cadd(a1, r);
    v[3] = csub(a1, r);
  }
};
// radix-2 decimation in time on top of the half-size DFT
template <int R, bool INV> struct Dft {
  static __device__ __forceinline__ void run(float2* v) {
    float2 e[R / 2], o[R / 2];
#pragma unroll
    for (int i = 0; i < R / 2; ++i) { e[i] = v[2 * i]; o[i] = v[2 * i + 1]; }
    Dft<R / 2, INV>::run(e);
    Dft<R / 2, INV>::run(o);
#pragma unroll
    for (int k = 0; k < R / 2; ++k) {
      float2 t = tw16<INV>(k * (16 / R), o[k]);
      v[k] = cadd(e[k], t);
      v[k + R / 2] = csub(e[k], t);
    }
  }
};

// ----------------------------------------------------- Stockham FFT in LDS
// LDS buffers holding FFT data use a padded layout: element i lives at
// pad16(i) = i + i/16. Every 16 consecutive lanes of a stage then touch 16
// distinct 8-byte slots modulo 16, i.e. all 32 banks, for both the strided
// reads and the autosort writes of every radix-16 stage.
__device__ __forceinline__ int pad16(int i) { return i + (i >> 4); }
__host__ __device__ constexpr int padded_len(int n) { return n + n / 16; }

// One workgroup-level N-point complex FFT (several independent ones when the
// caller gives each group its own `buf`). `lt` is the thread index inside the
// group (N/E threads per FFT, E values per thread). Stage with radix R and
// current sub-length Ns:
//   butterfly j in [0, N/R): inputs x[j + r N/R]; twiddle W_{Ns R}^{r (j mod Ns)};
//   R-point DFT; outputs x[(j / Ns) Ns R + (j mod Ns) + r Ns]   (autosort).
// tw[m] = W_N^m for m in [0, N). All group threads must call it (barriers).

// twiddle powers w^r, r in [1, R): powers of two from the table, others as
// one product of two of them (at most two roundings deep)
template <int R>
__device__ __forceinline__ void twiddle_powers(float2 (&w)[R], const float2* __restrict__ tw, int step) {
#pragma unroll
  for (int r = 1; r < R; ++r) {
    if ((r & (r - 1)) == 0) {
      w[r] = tw[r * step];
    } else {
      const int hb = 1 << (31 - __builtin_clz(r));
      w[r] = cmul(w[hb], w[r - hb]);
    }
  }
}

template <int N, int E, int Ns, bool INV>
__device__ __forceinline__ void stockham_stage(float2* buf, int lt, const float2* __restrict__ tw) {
  constexpr int R = (E < N / Ns) ? E : N / Ns;
  constexpr int NB = E / R;     // butterflies per thread
  constexpr int T = N / E;      // threads per FFT
  float2 v[NB][R];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int j = lt + b * T;
#pragma unroll
    for (int r = 0; r < R; ++r) v[b][r] = buf[pad16(j + r * (N / R))];
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int j = lt + b * T;
    if (Ns > 1) {
      const int k = j % Ns;
      float2 w[R];
      twiddle_powers<R>(w, tw, k * (N / (Ns * R)));
#pragma unroll
      for (int r = 1; r < R; ++r) v[b][r] = twmul<INV>(v[b][r], w[r]);
    }
    Dft<R, INV>::run(v[b]);
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int j = lt + b * T;
    const int k = j % Ns;
    const int base = (j / Ns) * Ns * R + k;
#pragma unroll
    for (int r = 0; r < R; ++r) buf[pad16(base + r * Ns)] = v[b][r];
  }
  __syncthreads();
}

template <int N, int E, int Ns, bool INV> struct StockhamFrom {
  static __device__ __forceinline__ void run(float2* buf, int lt, const float2* tw) {
    constexpr int R = (E < N / Ns) ? E : N / Ns;
    stockham_stage<N, E, Ns, INV>(buf, lt, tw);
    StockhamFrom<N, E, Ns * R, INV>::run(buf, lt, tw);
  }
};
template <int N, int E, bool INV> struct StockhamFrom<N, E, N, INV> {
  static __device__ __forceinline__ void run(float2*, int, const float2*) {}
};

// In-place N-point FFT of the padded LDS buffer buf (element i at pad16(i)),
// natural order in and out. Needs a __syncthreads() between the last write to
// buf and the call; ends with one.
template <int N, int E, bool INV>
__device__ __forceinline__ void fft_lds(float2* buf, int lt, const float2* __restrict__ tw) {
  StockhamFrom<N, E, 1, INV>::run(buf, lt, tw);
}

// ------------------------------------------------ spectrum storage types
// The four-step intermediate is stored as complex fp32 or, for bf16
// workloads, as a pair of bf16 (real, imag) packed in 32 bits.
struct cbf16 {
  unsigned int v;
};
__device__ __forceinline__ float2 ldc(const float2* p) { return *p; }
__device__ __forceinline__ void stc(float2* p, float2 x) { *p = x; }
__device__ __forceinline__ float2 ldc(const cbf16* p) {
  const unsigned int u = p->v;
  return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xFFFF0000u));
}
__device__ __forceinline__ void stc(cbf16* p, float2 x) {
  const unsigned short lo = __builtin_bit_cast(unsigned short, (bf16)x.x);
  const unsigned short hi = __builtin_bit_cast(unsigned short, (bf16)x.y);
  p->v = (unsigned int)lo | ((unsigned int)hi << 16);
}

// ------------------------------------------------ buffer-resource access
// Raw buffer loads and stores: address = resource base + a 32-bit per-lane
// offset + a 32-bit workgroup-uniform offset (held in a scalar register), so
// that accesses whose addresses differ only by uniform amounts share one
// per-lane offset and cost no per-access vector address arithmetic. Accesses
// at or beyond `bytes` from the base read zero and write nothing.
typedef __amdgpu_buffer_rsrc_t brsrc;
__device__ __forceinline__ brsrc make_brsrc(const void* base, unsigned bytes) {
  // word 3: 32-bit data format, the value used for untyped access on gfx9
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
template <typename V> struct BufIO;
template <> struct BufIO<float> {
  static __device__ __forceinline__ float ld(brsrc r, int vo, int so) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0));
  }
  static __device__ __forceinline__ void st(brsrc r, int vo, int so, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, vo, so, 0);
  }
};
template <> struct BufIO<bf16> {
  static __device__ __forceinline__ bf16 ld(brsrc r, int vo, int so) {
    return __builtin_bit_cast(bf16, __builtin_amdgcn_raw_buffer_load_b16(r, vo, so, 0));
  }
  static __device__ __forceinline__ void st(brsrc r, int vo, int so, float x) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (bf16)x), r, vo, so, 0);
  }
};
template <> struct BufIO<cbf16> {
  static __device__ __forceinline__ cbf16 ld(brsrc r, int vo, int so) {
    return cbf16{__builtin_amdgcn_raw_buffer_load_b32(r, vo, so, 0)};
  }
  static __device__ __forceinline__ void st(brsrc r, int vo, int so, float2 x) {
    const unsigned short lo = __builtin_bit_cast(unsigned short, (bf16)x.x);
    const unsigned short hi = __builtin_bit_cast(unsigned short, (bf16)x.y);
    __builtin_amdgcn_raw_buffer_store_b32((unsigned int)lo | ((unsigned int)hi << 16), r, vo, so, 0);
  }
};
template <> struct BufIO<float2> {
  static __device__ __forceinline__ float2 ld(brsrc r, int vo, int so) {
    const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, 0);
    return make_float2(__uint_as_float(u[0]), __uint_as_float(u[1]));
  }
  static __device__ __forceinline__ void st(brsrc r, int vo, int so, float2 x) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(x.x), __float_as_uint(x.y)}, r, vo, so, 0);
  }
};

// ---------------------------------------------------------------- host side

// Launch-configuration values (resident workgroups of a persistent launch,
// compute-unit counts) cached per device: each entry is written once per
// device with the value computed for that device; concurrent first calls may
// both compute it and store the same value.
constexpr int kMaxDevices = 64;
struct DeviceCache {
  std::atomic<int> v[kMaxDevices];
  template <typename F> int get(F compute) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return compute();
    int x = v[dev].load(std::memory_order_relaxed);
    if (x == 0) {
      x = compute();
      v[dev].store(x, std::memory_order_relaxed);
    }
    return x;
  }
};

#define HY_CHECK_HIP(expr)                         \
  do {                                             \
    hipError_t _e = (expr);                        \
    if (_e != hipSuccess) return HYENA_ERR_HIP;    \
  } while (0)

static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace hy
