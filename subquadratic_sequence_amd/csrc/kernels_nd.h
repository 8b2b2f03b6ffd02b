// Internal launcher interface of the 3D (HyenaND) path between nd_api.cpp and
// nd.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace hy {

// --------------------------------------------------------------- 3D path
// Transform sizes (MX, MY, MZ): (2X, 2Y, 2Z) for the zero-padded boundary,
// (X, Y, Z) for the circular one; the kernel's offset grid has the same shape,
// offset d at index d + M/2 per axis.
struct NdFilterArgs {
  int X, Y, Z, C, N, W;
  int MX, MY, MZ;
  const float *w1, *b1, *w2, *b2, *w3, *b3, *decay;
  float* k;  // kernel on the offset grid [N][C][MX][MY][MZ]
  // register conditioning (null: the plain kernel with an exponential window):
  // [4][W] = omega0 * gamma_1, beta_1, gamma_2, beta_2 of one sample; `decay`
  // then holds the Gaussian window rates
  const float* film = nullptr;
  // set by nd_filter: the matrix-core MLP writes the wrapped channel-pair fields
  // of the transform here (F = K_{2cp} + i K_{2cp+1}) instead of `k`
  float2* fdirect = nullptr;
};
// control vector and FiLM vectors of every sample: mod [B][4][W]
hipError_t nd_film_mod(const float* reg, const float* q, const float* film_w, const float* film_b,
                       const float* omega0, float* mod, int B, int R, int C, int W, hipStream_t s);
hipError_t fill(float* p, size_t n, float v, hipStream_t s);
struct NdConvArgs {
  int X, Y, Z, C, NO, B, n, npairs;
  int MX, MY, MZ;
  const float* p;        // projections [B][(NO+1)C][X*Y*Z] (channel-major)
  const float* dskip;    // [NO][C]
  const float* gate;     // [B][NO][C]
  const float* zin;
  float* zout;
  float* zbuf[2];        // z^{n+1} ping-pong [B][C][V]
  float* zfinal;         // z^{NO+1} [B][C][V]
  float2* Yint;          // [ceil(B/2)][C][X][MY][MZ]
  float2* F;             // filter pairs [N*C/2][MX][MY][MZ]
  const float2* kh;      // half spectra [N*C][MX][MY][MZ/2+1]
  // float2 elements between consecutive samples' spectra in kh; 0: one set of
  // spectra shared by every sample. Non-zero (per-sample kernels, 3D grids):
  // the pencil pass filters the two samples of a packed field with their own
  // kernels through the (P, Q) form.
  size_t kh_stride;
  const float2* tw128;   // W_128^m
};
// Kernel spectra kh from the MLP. F: the transform buffer (N C / 2 pair fields).
// keep_k: also leave the offset-indexed kernel in f.k (otherwise f.k may be
// unused: the 64- and 128-wide MLPs write F directly).
hipError_t nd_filter(const NdFilterArgs& f, float2* F, float2* kh, const float2* tw128, hipStream_t s,
                     bool keep_k = true);
hipError_t nd_gate(const float* u, float* part, const float* ga, const float* gb, float* gate, int B, int NO, int C,
                   int V, hipStream_t s);
size_t nd_gate_partial_floats(int B, int C, int V);
hipError_t nd_conv(const NdConvArgs& a, hipStream_t s);

}  // namespace hy
