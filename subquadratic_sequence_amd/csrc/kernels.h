// Internal launcher interface between the C ABI (api.cpp, nd_api.cpp) and the
// kernels: the projections, shared tables and the 1D path (the 3D path is in
// kernels_nd.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace hy {

// ---------------------------------------------------------------- GEMM
// C = A * B with A [M][K], B given transposed as Bt [N][K], fp32 accumulation.
// A_CM: A is channel-major [Bsz][K][Lseq] (element (m, k) at ((m / Lseq) K + k) Lseq + m % Lseq).
// C_CM: C is written channel-major [Bsz][N][Lseq].
// short_w (optional, with C_CM): [N][3] causal short-convolution taps applied
// along the sequence in the epilogue.
struct GemmArgs {
  const void* A;
  const void* Bt;
  void* C;
  int M, N, K, Lseq;
  bool a_cm, c_cm;
  const float* short_w;
};
hipError_t gemm(const GemmArgs& g, bool bf16, hipStream_t s);
// dst [cols][rows] = transpose of src [rows][cols] (storage type of the dtype)
hipError_t transpose2d(const void* src, void* dst, int rows, int cols, bool bf16, hipStream_t s);

// ---------------------------------------------------------- filter (1D)
struct Filter1DArgs {
  int L, D, NO, K, W;
  const float *w1, *b1, *w2, *b2, *w3, *b3, *decay;
  float* h;       // [NO][D][L], or [NO][D][2L] wrapped when noncausal
  int noncausal;  // two-sided filter: position m holds lag m (m < L) or m - 2L (m > L); m = L is zero
};
hipError_t filter1d_mlp(const Filter1DArgs& a, hipStream_t s);
// tw[m] = exp(-2 pi i m / n) for m in [0, count), computed in double
hipError_t twiddles(float2* tw, int n, int count, hipStream_t s);

// ------------------------------------------------------ LDS regime conv
struct LdsConvArgs {
  const void* s;          // short-convolved projections [B][(NO+1)D][L]
  const float* dskip;
  const float4* pq;       // [NO][D/2][L+1]
  const float2* tw;       // [2L]
  void* zout;             // [B][D][L]
  int B, L, D, NO;
};
hipError_t lds_conv(const LdsConvArgs& a, bool bf16, hipStream_t s);
// h [NO][D][L] (zero padded to 2L here) or, wrapped, [NO][D][2L] (two-sided filters)
hipError_t lds_spec(const float* h, const float2* tw, float4* pq, int L, int D, int NO, bool wrapped,
                    hipStream_t s);
size_t lds_conv_smem(int L);

// --------------------------------------------------------- four-step
// Column DFT length of the four-step decomposition 2L = N1 x N2.
inline int fourstep_n1(int L) { return L <= 65536 ? 64 : 256; }

struct FourStepTables {
  const float2* w256;    // [256]
  const float2* tw_lo;   // [1 << lo_bits]
  const float2* tw_hi;   // [2L >> lo_bits]
  const float2* tw_row;  // [N2]
  int lo_bits;
};
struct FourStepConvArgs {
  const void* s;         // short-convolved projections [B][(NO+1)D][L]
  const float* dskip;
  const float4* pq;      // [NO][D/2][N1/2 + 1][N2]
  const void* pq_bf16;   // the same entries as four bf16 (read with the bf16 intermediate)
  void* z[2];            // ping-pong z^{n+1} buffers [B][D][L]
  void* zfinal;          // z^{NO+1} [B][D][L]
  void* Y;               // intermediate [group_pairs][N1][N2]
  int B, L, D, NO;
  int group_pairs;       // channel pairs per group (0: all)
  bool y_bf16;           // bf16 workloads: keep the intermediate as bf16 pairs
};
hipError_t fourstep_conv(const FourStepTables& tb, const FourStepConvArgs& c, bool bf16, hipStream_t s);
// filter spectra into pq (fp32) and pq_bf16 (the same entries as four bf16)
hipError_t fourstep_spec(const FourStepTables& tb, const float* h, float2* Y, float4* pq, void* pq_bf16, int L,
                         int D, int NO, bool wrapped, hipStream_t s);

}  // namespace hy
