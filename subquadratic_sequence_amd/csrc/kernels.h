// Internal launcher interface between the C ABI (api.cpp, nd_api.cpp) and the
// kernels: shared tables and the 1D path (the projections are in gemm.h, the
// 3D path in kernels_nd.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "gemm.h"

namespace hy {

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
  // one order with no gate and no skip (NO = 1): z^2 = h * z^1; gates and
  // dskip are not read
  bool plain = false;
};
hipError_t fourstep_conv(const FourStepTables& tb, const FourStepConvArgs& c, bool bf16, hipStream_t s);
// filter spectra into pq (fp32) and pq_bf16 (the same entries as four bf16);
// either may be null (not both): with pq null the spectrum pass writes the bf16
// entries itself
hipError_t fourstep_spec(const FourStepTables& tb, const float* h, float2* Y, float4* pq, void* pq_bf16, int L,
                         int D, int NO, bool wrapped, hipStream_t s);

// --------------------------------------------------------- backward (2L <= 8192)
struct BwdConvArgs {
  const void* s;         // short-convolved projections [B][(NO+1)D][L] (storage type)
  const void* gz;        // dz^{NO+1} [B][D][L] (storage type)
  float* zsave;          // z^1 .. z^NO [NO][B][D][L]
  float* csave;          // c^1 .. c^NO [NO][B][D][L]
  void* zfin;            // z^{NO+1} [B][D][L] (storage type)
  const float* dskip;    // [NO][D]
  const float4* pq;      // [NO][D/2][L+1]
  const float2* tw;      // [2L]
  float* sbar;           // ds = (dz^1, dx^1 .. dx^NO) [B][(NO+1)D][L]
  float* dh_part;        // per-sample filter gradients [B][NO][D][HL]
  float* dd_part;        // per-sample skip gradients [B][NO][D]
  int B, L, D, NO, HL;   // HL = L causal, 2L wrapped two-sided
};
hipError_t bwd_lds_conv(const BwdConvArgs& a, bool bf16, hipStream_t s);
// dp and per-row short-conv tap gradients from ds (rows = B (NO+1) D of length L)
hipError_t short_conv_bwd(const float* sbar, const void* p, const float* short_w, void* pbar, float* dsw_part, int rows,
                          int L, int J, bool bf16, hipStream_t s);
// out[i] = sum_{r < R} in[r stride + i], i < n (in: fp32 or bf16)
hipError_t sum_rows(const void* in, float* out, int R, size_t stride, size_t n, bool in_bf16, hipStream_t s);
// out[r] = sum_k in[r K + k]
// out[r] = sum over row r of in [rows][K], in a fixed order; with few rows the
// rows are summed in segments through part (rows * 1024 floats at most)
hipError_t row_sums(const float* in, float* out, int rows, int K, float* part, hipStream_t s);
// out[i] = sum_r part[r][i] over R rows of n, in a fixed order; part is
// overwritten (a tall array of partial results, R a power of two)
hipError_t sum_rows_tall(float* part, float* out, int R, size_t n, hipStream_t s);

struct FilterBwdArgs {
  int L, D, NO, K, W, noncausal;
  const float *w1, *b1, *w2, *b2, *b3, *decay;
  const float* dh;       // [NO][D][P], P = L or 2L (wrapped two-sided)
  const float* o;        // MLP output, channel-major [NO D][P]
  float* e;              // features [P][1 + 2K]
  float *a1, *c1, *a2, *c2;  // hidden activations and cosines of their pre-activations [P][W]
  float* dout;           // dL/do [NO D][P]
  float* ddecay;         // [D]
};
hipError_t filter_bwd_feat(const FilterBwdArgs& a, hipStream_t s);
// dL/do and the decay gradient; part: scratch of D * 16 floats
hipError_t filter_bwd_out(const FilterBwdArgs& a, float* part, hipStream_t s);
hipError_t mul_inplace(float* x, const float* y, size_t n, hipStream_t s);

}  // namespace hy
