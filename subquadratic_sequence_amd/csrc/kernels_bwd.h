// Launchers of elementwise kernels of the backward pass (bwd4.hip: the
// four-step regime; short_conv_rows: bwd.hip).
// Layouts: rows of L positions; s [B][(NO+1)D][L] and ds [B][(NO+1)D][L] in the
// block order (v, x^1 .. x^NO); the staging buffer tmp [B][2D][L] holds a
// convolution input in block 0 (block 1 is not read). T is the storage type.
#pragma once
#include <hip/hip_runtime.h>

namespace hy {

// The forward's causal length-3 short convolution of channel-major rows p
// [rows][L] (row r is column j = r mod J of W_in's blocks): s = w0 p_t + w1
// p_{t-1} + w2 p_{t-2}, zero history (bwd.hip)
hipError_t short_conv_rows(const void* p, const float* short_w, void* s_out, int rows, int L, int J, bool bf16,
                           hipStream_t s);
// z^1 = v block of s: zf [B][D][L] fp32 and tmp block 0 (storage type)
hipError_t bwd4_z_init(const void* sp, float* zf, void* tmp, int B, int D, int L, int NO, bool bf16, hipStream_t s);
// z^{n+1} = x^n c^n + D^n z^n from s block n+1, c (storage) and zf (fp32 z^n):
// into zf_next (fp32) and tmp block 0 (storage), or, for the last order, into
// zfin (storage) when zf_next is null
hipError_t bwd4_z_next(const void* sp, const void* c, const float* zf, const float* dskip_n, float* zf_next,
                       void* tmp, void* zfin, int B, int D, int L, int NO, int n, bool bf16, hipStream_t s);
// storage -> fp32 copy of n elements
hipError_t bwd4_to_f32(const void* in, float* out, size_t n, bool bf16, hipStream_t s);
// with g = dz^{n+1} (fp32 [B][D][L]): ds block n+1 = g c^n, tmp block 0 =
// R(g x^n) (storage, R the reversal t -> L - 1 - t), dcf = g x^n (fp32, unless
// null), dd_part[b][n][d] = sum_t g z^n
hipError_t bwd4_rev_prep(const float* g, const void* sp, const void* c, const float* zf, float* sbar, void* tmp,
                         float* dcf, float* dd_part, int B, int D, int L, int NO, int n, bool bf16, hipStream_t s);
// out[b][d][t] (row stride ostride) = D^n_d g[b][d][t] + conv[b][d][L - 1 - t]
hipError_t bwd4_rev_finish(const float* g, const void* conv, const float* dskip_n, float* out, size_t ostride, int B,
                           int D, int L, bool bf16, hipStream_t s);
// dh[d][tau] = conv[d][L - 1 - tau], tau < L, rows of HL (one sample, fp32 out)
hipError_t bwd4_dh_store(const void* conv, float* dh, int D, int L, int HL, bool bf16, hipStream_t s);
// negative lags of wrapped two-sided rows [2L]: dh[d][j] = conv[d][j - L - 1],
// L < j < 2L, dh[d][L] = 0
hipError_t bwd4_dh_store_neg(const void* conv, float* dh, int D, int L, bool bf16, hipStream_t s);
// one sample's tmp block 0 = R z (z fp32 [D][L])
hipError_t bwd4_stage_rev(const float* zf, void* tmp, int D, int L, bool bf16, hipStream_t s);

}  // namespace hy
