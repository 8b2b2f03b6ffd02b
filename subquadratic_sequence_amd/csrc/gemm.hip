// Dense projections of the Hyena operator on the MFMA units of gfx950.
//
// The in-projection (u [B*L][D] times W_in) and the out-projection
// (z [B][D][L] times W_out) are the only dense contractions of the operator.
// C = A * B with B supplied transposed (Bt [N][K], K contiguous) so that both
// MFMA operands are read from LDS as K-contiguous 16-byte fragments.
//  * A_CM: A is channel-major [Bsz][K][Lseq] (the layout the long convolution
//    produces); tiles are loaded along M and transposed while stored to LDS.
//  * C_CM: C is written channel-major [Bsz][N][Lseq] (the layout the long
//    convolution consumes), staged through LDS for 16-byte stores.
//  * SC (with C_CM): the causal length-3 depthwise short convolution along the
//    sequence is applied in the epilogue, s_t = w0 p_t + w1 p_{t-1} + w2 p_{t-2}
//    (zero history at the start of every sequence). M-tiles then overlap by 8
//    rows: a tile computes rows [m0 - 8, m0 + 120) and writes [m0, m0 + 120), so
//    the two previous rows of every written row are on chip.
// bf16 storage uses v_mfma_f32_32x32x16_bf16, fp32 uses v_mfma_f32_32x32x2_f32;
// accumulation is fp32 in both cases.
#include "common.h"
#include "kernels.h"

namespace hy {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int GBM = 128, GBN = 128;

template <typename T> struct GemmCfg {
  static constexpr int VEC = 16 / sizeof(T);    // elements per 16-byte chunk
  static constexpr int BK = 64 / sizeof(T);     // K elements per tile row (64 bytes)
  static constexpr int LDK = BK + VEC;          // padded LDS row (80 bytes)
};

constexpr int kCsLd = GBM + 4;  // staging row (floats) for channel-major output

constexpr int kScRows = 120;  // rows written per M-tile with the short-conv epilogue

template <typename T, bool A_CM, bool C_CM, bool SC>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const T* __restrict__ A, const T* __restrict__ Bt,
                                                      T* __restrict__ C, int M, int N, int K, int Lseq,
                                                      const float* __restrict__ short_w) {
  using Cfg = GemmCfg<T>;
  constexpr int BK = Cfg::BK, LDK = Cfg::LDK, VEC = Cfg::VEC;
  constexpr int TILE_BYTES = 2 * GBM * LDK * (int)sizeof(T);
  constexpr int STAGE_BYTES = 64 * kCsLd * 4;
  __shared__ __attribute__((aligned(16))) char smem[TILE_BYTES > STAGE_BYTES ? TILE_BYTES : STAGE_BYTES];
  T* As = reinterpret_cast<T*>(smem);
  T* Bs = As + GBM * LDK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * GBN;
  const int m0 = SC ? (int)blockIdx.y * kScRows - 8 : (int)blockIdx.y * GBM;  // first A row of the tile

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  uint4 ra[2], rb[2];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256;
      if (!A_CM) {
        const int row = c >> 2, kc = (c & 3) * VEC;
        const int m = m0 + row;
        ra[i] = (m >= 0 && m < M) ? *reinterpret_cast<const uint4*>(A + (size_t)m * K + k0 + kc)
                                  : make_uint4(0, 0, 0, 0);
      } else {
        constexpr int CPR = GBM / VEC;  // chunks per k-row
        const int k = c / CPR, mc = (c % CPR) * VEC;
        const int m = m0 + mc;
        if (m < M) {
          const int b = m / Lseq, t = m - b * Lseq;
          ra[i] = *reinterpret_cast<const uint4*>(A + ((size_t)b * K + k0 + k) * Lseq + t);
        } else {
          ra[i] = make_uint4(0, 0, 0, 0);
        }
      }
      const int row = c >> 2, kc = (c & 3) * VEC;
      const int n = n0 + row;
      rb[i] = (n < N) ? *reinterpret_cast<const uint4*>(Bt + (size_t)n * K + k0 + kc) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256;
      if (!A_CM) {
        const int row = c >> 2, kc = (c & 3) * VEC;
        *reinterpret_cast<uint4*>(As + row * LDK + kc) = ra[i];
      } else {
        constexpr int CPR = GBM / VEC;
        const int k = c / CPR, mc = (c % CPR) * VEC;
        const T* v = reinterpret_cast<const T*>(&ra[i]);
#pragma unroll
        for (int q = 0; q < VEC; ++q) As[(mc + q) * LDK + k] = v[q];
      }
      const int row = c >> 2, kc = (c & 3) * VEC;
      *reinterpret_cast<uint4*>(Bs + row * LDK + kc) = rb[i];
    }
  };

  const int ktiles = K / BK;
  load_tile(0);
  store_tile();
  __syncthreads();
  for (int kt = 0; kt < ktiles; ++kt) {
    if (kt + 1 < ktiles) load_tile((kt + 1) * BK);
    const int ar = wm * 64 + (lane & 31), br = wn * 64 + (lane & 31);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int kk = 0; kk < BK; kk += 16) {
        bf16x8 af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          af[i] = *reinterpret_cast<const bf16x8*>(As + (ar + i * 32) * LDK + kk + (lane >> 5) * 8);
          bfr[i] = *reinterpret_cast<const bf16x8*>(Bs + (br + i * 32) * LDK + kk + (lane >> 5) * 8);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < BK; kk += 2) {
        float af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          af[i] = As[(ar + i * 32) * LDK + kk + (lane >> 5)];
          bfr[i] = Bs[(br + i * 32) * LDK + kk + (lane >> 5)];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
    if (kt + 1 < ktiles) {
      store_tile();
      __syncthreads();
    }
  }

  // Epilogue. Accumulator element e of lane l in block (i, j):
  //   row = i*32 + (e/4)*8 + (l/32)*4 + e%4, col = j*32 + l%32 (within the wave tile).
  if (!C_CM) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = m0 + wm * 64 + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
          const int n = n0 + wn * 64 + j * 32 + (lane & 31);
          if (m < M && n < N) stf(C + (size_t)m * N + n, acc[i][j][e]);
        }
    return;
  }
  float* Cs = reinterpret_cast<float*>(smem);  // [64 n][kCsLd] for one half of the n range
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (wn == h) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int ml = wm * 64 + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
            const int nl = j * 32 + (lane & 31);
            Cs[nl * kCsLd + ml] = acc[i][j][e];
          }
    }
    __syncthreads();
    // 64 rows (n) x 128 (m) in chunks of 8 consecutive m; with SC the first
    // chunk of every row (the 8 overlap rows) is not written
    for (int c = tid; c < 64 * 16; c += 256) {
      const int nl = c >> 4, mc = (c & 15) * 8;
      const int n = n0 + h * 64 + nl, m = m0 + mc;
      if (n < N && m < M && (!SC || mc >= 8)) {
        const int b = m / Lseq, t = m - b * Lseq;
        T* dst = C + ((size_t)b * N + n) * Lseq + t;
        const float* src = Cs + nl * kCsLd + mc;
        float o[8];
        if (SC) {
          const float w0 = short_w[3 * n], w1 = short_w[3 * n + 1], w2 = short_w[3 * n + 2];
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            float s = w0 * src[v];
            if (t + v >= 1) s += w1 * src[v - 1];
            if (t + v >= 2) s += w2 * src[v - 2];
            o[v] = s;
          }
        } else {
#pragma unroll
          for (int v = 0; v < 8; ++v) o[v] = src[v];
        }
        if constexpr (sizeof(T) == 2) {
          bf16x8 ob;
#pragma unroll
          for (int v = 0; v < 8; ++v) ob[v] = (__bf16)o[v];
          *reinterpret_cast<bf16x8*>(dst) = ob;
        } else {
          *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
          *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
        }
      }
    }
    __syncthreads();
  }
}

template <typename T>
static hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  const bool sc = g.short_w != nullptr;
  const int mtiles = sc ? (g.M + kScRows - 1) / kScRows : (g.M + GBM - 1) / GBM;
  dim3 grid((g.N + GBN - 1) / GBN, mtiles), block(256);
  const T* A = static_cast<const T*>(g.A);
  const T* B = static_cast<const T*>(g.Bt);
  T* C = static_cast<T*>(g.C);
#define GEMM_LAUNCH(acm, ccm, scv) \
  hipLaunchKernelGGL((gemm_kernel<T, acm, ccm, scv>), grid, block, 0, s, A, B, C, g.M, g.N, g.K, g.Lseq, g.short_w)
  if (sc) {
    if (!g.c_cm || g.a_cm) return hipErrorInvalidValue;
    GEMM_LAUNCH(false, true, true);
  } else if (g.a_cm && g.c_cm) {
    GEMM_LAUNCH(true, true, false);
  } else if (g.a_cm) {
    GEMM_LAUNCH(true, false, false);
  } else if (g.c_cm) {
    GEMM_LAUNCH(false, true, false);
  } else {
    GEMM_LAUNCH(false, false, false);
  }
#undef GEMM_LAUNCH
  return hipGetLastError();
}

hipError_t gemm(const GemmArgs& g, bool bf16, hipStream_t s) {
  return bf16 ? launch_gemm<__bf16>(g, s) : launch_gemm<float>(g, s);
}

// ------------------------------------------------------------- transpose

template <typename U>
__global__ __launch_bounds__(256) void transpose_kernel(const U* __restrict__ src, U* __restrict__ dst, int rows,
                                                        int cols) {
  __shared__ U tile[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const int r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) tile[i][tx] = src[(size_t)r * cols + c];
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int c = c0 + i, r = r0 + tx;
    if (r < rows && c < cols) dst[(size_t)c * rows + r] = tile[tx][i];
  }
}

hipError_t transpose2d(const void* src, void* dst, int rows, int cols, bool bf16, hipStream_t s) {
  dim3 grid((cols + 31) / 32, (rows + 31) / 32), block(256);
  if (bf16)
    hipLaunchKernelGGL(transpose_kernel<unsigned short>, grid, block, 0, s, (const unsigned short*)src,
                       (unsigned short*)dst, rows, cols);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, block, 0, s, (const float*)src, (float*)dst, rows, cols);
  return hipGetLastError();
}

}  // namespace hy
