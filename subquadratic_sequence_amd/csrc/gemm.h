// Launcher interface of the dense projections (gemm.hip): the MFMA GEMM and
// the weight transposes.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace hy {

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
  // Several products in one launch (grid row y = b * nsplit + s): product b of
  // a batch reads A + b sa and Bt + b sb, its K split s starts at + s ka and
  // + s kb (K elements each), and writes C + y sc (the splits' partial results,
  // summed by the caller). lda: row stride of a row-major A, or the channel
  // count of a channel-major A; ldb: row stride of Bt; 0 means K.
  int batch = 1, nsplit = 1;
  size_t sa = 0, sb = 0, sc = 0, ka = 0, kb = 0;
  int lda = 0, ldb = 0;
};
hipError_t gemm(const GemmArgs& g, bool bf16, hipStream_t s);
// dst [cols][rows] = transpose of src [rows][cols] (storage type of the dtype), for
// each of `batch` matrices stored back to back
hipError_t transpose2d(const void* src, void* dst, int rows, int cols, bool bf16, hipStream_t s, int batch = 1);
// the transposes of two matrices (rows0 x cols0 and rows1 x cols1) in one launch;
// every dimension a multiple of 64
hipError_t transpose2d_pair(const void* src0, void* dst0, int rows0, int cols0, const void* src1, void* dst1,
                            int rows1, int cols1, bool bf16, hipStream_t s);

}  // namespace hy
