// C ABI of the 3D (HyenaND) path: validation, memory layouts and the launch
// sequence. Every check runs on the host before the first HIP call.
#include "../../include/hyena.h"

#include <stdint.h>

#include "common.h"
#include "kernels.h"
#include "kernels_nd.h"

using hy::align_up;

namespace {

constexpr size_t kAlign = 256;

bool pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }
bool aligned16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }
// B * X * Y * Z * (N+1) * C < 2^31 (element offsets fit int32), for B >= 1 and a
// valid shape, tested by division: the product itself can exceed 64 bits
bool fits_i32(int B, int X, int Y, int Z, int C, int N) {
  return (long long)B <= ((1LL << 31) - 1) / ((long long)X * Y * Z * (N + 1) * C);
}

bool boundary_ok(int bd) { return bd == HYENA_ND_ZERO_PAD || bd == HYENA_ND_CIRCULAR; }
// transform length per grid length: 2 (zero padded) or 1 (circular)
int pad_of(int bd) { return bd == HYENA_ND_CIRCULAR ? 1 : 2; }

// Transform lengths up to 128 (the twiddle table W_128); at least 8 points per
// axis, except X = 1: a 2D grid (one x-plane, every offset with dx = 0). Y and Z
// (and X for 3D grids) are independent.
bool nd_shape_ok(int X, int Y, int Z, int C, int N, int bd) {
  if (!boundary_ok(bd)) return false;
  const int lo = 8 / pad_of(bd), hi = 128 / pad_of(bd);
  return (X == 1 || pow2_in(X, lo, hi)) && pow2_in(Y, lo, hi) && pow2_in(Z, lo, hi) && C >= 64 && C <= 4096 &&
         C % 64 == 0 && N >= 1 && N <= 4;
}

// transform length along x: no padding of a one-point axis
int mx_of(int X, int bd) { return X == 1 ? 1 : pad_of(bd) * X; }

// transform points (MX)(MY)(MZ)
size_t pts(int X, int Y, int Z, int bd) {
  const size_t p = pad_of(bd);
  return (size_t)mx_of(X, bd) * p * p * Y * Z;
}

struct NdCache {
  size_t tw, kh, total;
};
NdCache nd_cache(int X, int Y, int Z, int C, int N, int bd) {
  const int p = pad_of(bd);
  NdCache c{};
  size_t off = 0;
  c.tw = off;
  off = align_up(off + 128 * 8, kAlign);
  c.kh = off;
  off = align_up(off + (size_t)N * C * mx_of(X, bd) * (p * Y) * (p * Z / 2 + 1) * 8, kAlign);
  c.total = off;
  return c;
}

struct NdFws {
  size_t k, F, total;
};
NdFws nd_fws(int X, int Y, int Z, int C, int N, int bd) {
  NdFws w{};
  size_t off = 0;
  w.k = off;
  off = align_up(off + (size_t)N * C * pts(X, Y, Z, bd) * 4, kAlign);
  w.F = off;
  off = align_up(off + (size_t)N * (C / 2) * pts(X, Y, Z, bd) * 8, kAlign);
  w.total = off;
  return w;
}

struct NdWs {
  size_t wt_in, wt_out, p, zfinal, z0, z1, Y, part, gate, total;
};
NdWs nd_ws(int B, int X, int Y, int Z, int C, int N, int bd) {
  const int pd = pad_of(bd);
  NdWs w{};
  const size_t V = (size_t)X * Y * Z;
  const size_t J = (size_t)(N + 1) * C;
  size_t off = 0;
  w.wt_in = off;
  off = align_up(off + J * C * 4, kAlign);
  w.wt_out = off;
  off = align_up(off + (size_t)C * C * 4, kAlign);
  w.p = off;
  off = align_up(off + (size_t)B * J * V * 4, kAlign);
  w.zfinal = off;
  off = align_up(off + (size_t)B * C * V * 4, kAlign);
  w.z0 = off;
  off = align_up(off + (size_t)B * C * V * 4, kAlign);
  w.z1 = off;
  off = align_up(off + (size_t)B * C * V * 4, kAlign);
  w.Y = off;
  off = align_up(off + (size_t)((B + 1) / 2) * C * X * ((size_t)pd * Y * pd * Z) * 8, kAlign);
  w.part = off;
  off = align_up(off + hy::nd_gate_partial_floats(B, C, (int)V) * 4, kAlign);
  w.gate = off;
  off = align_up(off + (size_t)B * N * C * 4, kAlign);
  w.total = off;
  return w;
}

int device_ok() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return HYENA_ERR_HIP;
  return HYENA_OK;
}

}  // namespace

extern "C" {

size_t hyena_nd_cache_bytes_ex(int X, int Y, int Z, int C, int N, int boundary) {
  if (!nd_shape_ok(X, Y, Z, C, N, boundary)) return 0;
  return nd_cache(X, Y, Z, C, N, boundary).total;
}

size_t hyena_nd_filter_workspace_bytes_ex(int X, int Y, int Z, int C, int N, int boundary) {
  if (!nd_shape_ok(X, Y, Z, C, N, boundary)) return 0;
  return nd_fws(X, Y, Z, C, N, boundary).total;
}

size_t hyena_nd_workspace_bytes_ex(int B, int X, int Y, int Z, int C, int N, int boundary) {
  if (!nd_shape_ok(X, Y, Z, C, N, boundary) || B < 1) return 0;
  if (!fits_i32(B, X, Y, Z, C, N)) return 0;
  return nd_ws(B, X, Y, Z, C, N, boundary).total;
}

size_t hyena_nd_cache_bytes(int X, int Y, int Z, int C, int N) {
  return hyena_nd_cache_bytes_ex(X, Y, Z, C, N, HYENA_ND_ZERO_PAD);
}

size_t hyena_nd_filter_workspace_bytes(int X, int Y, int Z, int C, int N) {
  return hyena_nd_filter_workspace_bytes_ex(X, Y, Z, C, N, HYENA_ND_ZERO_PAD);
}

size_t hyena_nd_workspace_bytes(int B, int X, int Y, int Z, int C, int N) {
  return hyena_nd_workspace_bytes_ex(B, X, Y, Z, C, N, HYENA_ND_ZERO_PAD);
}

int hyena_nd_layer_init_ex(hyena_nd_layer* layer, int X, int Y, int Z, int C, int N, int boundary, void* cache,
                           size_t cache_bytes) {
  if (layer == nullptr) return HYENA_ERR_INVALID_ARG;
  if (!nd_shape_ok(X, Y, Z, C, N, boundary)) return HYENA_ERR_UNSUPPORTED;
  if (!aligned16(cache)) return HYENA_ERR_INVALID_ARG;
  if (cache_bytes < nd_cache(X, Y, Z, C, N, boundary).total) return HYENA_ERR_WORKSPACE;
  layer->X = X;
  layer->Y = Y;
  layer->Z = Z;
  layer->C = C;
  layer->N = N;
  layer->built = 0;
  layer->cache = cache;
  layer->cache_bytes = cache_bytes;
  layer->boundary = boundary;
  return HYENA_OK;
}

int hyena_nd_layer_init(hyena_nd_layer* layer, int X, int Y, int Z, int C, int N, void* cache, size_t cache_bytes) {
  return hyena_nd_layer_init_ex(layer, X, Y, Z, C, N, HYENA_ND_ZERO_PAD, cache, cache_bytes);
}

int hyena_nd_filter_gen(hyena_nd_layer* layer, const hyena_nd_filter_params* p, float* k_out, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  if (layer == nullptr || p == nullptr) return HYENA_ERR_INVALID_ARG;
  const int X = layer->X, Y = layer->Y, Z = layer->Z, C = layer->C, N = layer->N, bd = layer->boundary;
  if (!nd_shape_ok(X, Y, Z, C, N, bd)) return HYENA_ERR_UNSUPPORTED;
  if (!aligned16(layer->cache)) return HYENA_ERR_INVALID_ARG;
  const NdCache cl = nd_cache(X, Y, Z, C, N, bd);
  if (layer->cache_bytes < cl.total) return HYENA_ERR_WORKSPACE;
  if (p->width < 1 || p->width > 128) return HYENA_ERR_UNSUPPORTED;
  const void* ptrs[] = {p->w1, p->b1, p->w2, p->b2, p->w3, p->b3, p->decay, ws};
  for (const void* q : ptrs)
    if (!aligned16(q)) return HYENA_ERR_INVALID_ARG;
  if (k_out != nullptr && !aligned16(k_out)) return HYENA_ERR_INVALID_ARG;
  const NdFws fw = nd_fws(X, Y, Z, C, N, bd);
  if (ws_bytes < fw.total) return HYENA_ERR_WORKSPACE;
  if (device_ok() != HYENA_OK) return HYENA_ERR_HIP;

  char* wsb = static_cast<char*>(ws);
  char* cb = static_cast<char*>(layer->cache);
  layer->built = 0;
  float2* tw = reinterpret_cast<float2*>(cb + cl.tw);
  HY_CHECK_HIP(hy::twiddles(tw, 128, 128, stream));
  const int pd = pad_of(bd);
  hy::NdFilterArgs f{X,     Y,     Z,     C,     N,     p->width, mx_of(X, bd), pd * Y,
                     pd * Z, p->w1, p->b1, p->w2, p->b2, p->w3,    p->b3,    p->decay,
                     k_out ? k_out : reinterpret_cast<float*>(wsb + fw.k)};
  HY_CHECK_HIP(hy::nd_filter(f, reinterpret_cast<float2*>(wsb + fw.F), reinterpret_cast<float2*>(cb + cl.kh), tw,
                             stream, k_out != nullptr));
  layer->built = 1;
  return HYENA_OK;
}

}  // extern "C"

namespace {

int nd_fwd_impl(const hyena_nd_layer* layer, const float* u, const float* w_in, const float* dskip,
                const float* gate_a, const float* gate_b, const float* w_out, int B, float* y, void* ws,
                size_t ws_bytes, hipStream_t stream, const hipEvent_t* ev) {
  if (layer == nullptr) return HYENA_ERR_INVALID_ARG;
  const void* ptrs[] = {u, w_in, dskip, gate_a, gate_b, w_out, y, ws};
  for (const void* q : ptrs)
    if (!aligned16(q)) return HYENA_ERR_INVALID_ARG;
  if (B < 1) return HYENA_ERR_INVALID_ARG;
  const int X = layer->X, Y = layer->Y, Z = layer->Z, C = layer->C, N = layer->N, bd = layer->boundary;
  if (!nd_shape_ok(X, Y, Z, C, N, bd)) return HYENA_ERR_UNSUPPORTED;
  if (!layer->built || !aligned16(layer->cache)) return HYENA_ERR_LAYER_MISMATCH;
  const NdCache cl = nd_cache(X, Y, Z, C, N, bd);
  if (layer->cache_bytes < cl.total) return HYENA_ERR_LAYER_MISMATCH;
  if (!fits_i32(B, X, Y, Z, C, N)) return HYENA_ERR_UNSUPPORTED;
  const NdWs w = nd_ws(B, X, Y, Z, C, N, bd);
  if (ws_bytes < w.total) return HYENA_ERR_WORKSPACE;
  if (device_ok() != HYENA_OK) return HYENA_ERR_HIP;

  char* wsb = static_cast<char*>(ws);
  char* cb = static_cast<char*>(layer->cache);
  const int V = X * Y * Z, J = (N + 1) * C;
  float* wt_in = reinterpret_cast<float*>(wsb + w.wt_in);
  float* wt_out = reinterpret_cast<float*>(wsb + w.wt_out);
  float* pbuf = reinterpret_cast<float*>(wsb + w.p);
  float* zfin = reinterpret_cast<float*>(wsb + w.zfinal);
  float* gate = reinterpret_cast<float*>(wsb + w.gate);

  if (ev) HY_CHECK_HIP(hipEventRecord(ev[0], stream));
  HY_CHECK_HIP(hy::nd_gate(u, reinterpret_cast<float*>(wsb + w.part), gate_a, gate_b, gate, B, N, C, V, stream));
  HY_CHECK_HIP(hy::transpose2d_pair(w_in, wt_in, C, J, w_out, wt_out, C, C, false, stream));
  hy::GemmArgs gi{u, wt_in, pbuf, B * V, J, C, V, false, true, nullptr};
  HY_CHECK_HIP(hy::gemm(gi, false, stream));
  if (ev) HY_CHECK_HIP(hipEventRecord(ev[1], stream));
  hy::NdConvArgs a{};
  a.X = X;
  a.Y = Y;
  a.Z = Z;
  a.MX = mx_of(X, bd);
  a.MY = pad_of(bd) * Y;
  a.MZ = pad_of(bd) * Z;
  a.C = C;
  a.NO = N;
  a.B = B;
  a.p = pbuf;
  a.dskip = dskip;
  a.gate = gate;
  a.zbuf[0] = reinterpret_cast<float*>(wsb + w.z0);
  a.zbuf[1] = reinterpret_cast<float*>(wsb + w.z1);
  a.zfinal = zfin;
  a.Yint = reinterpret_cast<float2*>(wsb + w.Y);
  a.kh = reinterpret_cast<const float2*>(cb + cl.kh);
  a.tw128 = reinterpret_cast<const float2*>(cb + cl.tw);
  HY_CHECK_HIP(hy::nd_conv(a, stream));
  if (ev) HY_CHECK_HIP(hipEventRecord(ev[2], stream));
  hy::GemmArgs go{zfin, wt_out, y, B * V, C, C, V, true, false, nullptr};
  HY_CHECK_HIP(hy::gemm(go, false, stream));
  if (ev) HY_CHECK_HIP(hipEventRecord(ev[3], stream));
  return HYENA_OK;
}

}  // namespace

extern "C" {

int hyena_nd_fwd(const hyena_nd_layer* layer, const float* u, const float* w_in, const float* dskip,
                 const float* gate_a, const float* gate_b, const float* w_out, int B, float* y, void* ws,
                 size_t ws_bytes, hipStream_t stream) {
  return nd_fwd_impl(layer, u, w_in, dskip, gate_a, gate_b, w_out, B, y, ws, ws_bytes, stream, nullptr);
}

int hyena_nd_fwd_profiled(const hyena_nd_layer* layer, const float* u, const float* w_in, const float* dskip,
                          const float* gate_a, const float* gate_b, const float* w_out, int B, float* y, void* ws,
                          size_t ws_bytes, hipStream_t stream, const hipEvent_t* events) {
  if (events == nullptr) return HYENA_ERR_INVALID_ARG;
  return nd_fwd_impl(layer, u, w_in, dskip, gate_a, gate_b, w_out, B, y, ws, ws_bytes, stream, events);
}

}  // extern "C"

// ------------------------------------------------- register-conditioned layer
namespace {

// one sample's kernel spectra: N C MX MY (MZ/2 + 1) complex fp32
size_t film_kh_bytes(int X, int Y, int Z, int C, int N, int bd) {
  const int p = pad_of(bd);
  return align_up((size_t)N * C * mx_of(X, bd) * (p * Y) * (p * Z / 2 + 1) * 8, kAlign);
}

struct NdFilmWs {
  size_t base, tw, mod, kh, fws, total;
};
NdFilmWs nd_film_ws(int B, int X, int Y, int Z, int C, int N, int W, int bd) {
  NdFilmWs w{};
  size_t off = 0;
  w.base = off;
  off = align_up(off + nd_ws(B, X, Y, Z, C, N, bd).total, kAlign);
  w.tw = off;
  off = align_up(off + 128 * 8, kAlign);
  w.mod = off;
  off = align_up(off + (size_t)B * 4 * W * 4, kAlign);
  w.kh = off;
  off = align_up(off + (size_t)B * film_kh_bytes(X, Y, Z, C, N, bd), kAlign);
  w.fws = off;
  off = align_up(off + nd_fws(X, Y, Z, C, N, bd).total, kAlign);
  w.total = off;
  return w;
}

bool film_shape_ok(int B, int X, int Y, int Z, int C, int N, int W, int bd) {
  return nd_shape_ok(X, Y, Z, C, N, bd) && B >= 1 && W >= 1 && W <= 128 &&
         fits_i32(B, X, Y, Z, C, N);
}

int film_fwd_impl(int X, int Y, int Z, int C, int N, int bd, const hyena_nd_filter_params* p,
                  const hyena_nd_film_params* fp, const float* u, const float* reg, const float* w_in,
                  const float* dskip, const float* w_out, int B, float* y, float* k_out, void* ws, size_t ws_bytes,
                  hipStream_t stream, const hipEvent_t* ev) {
  if (p == nullptr || fp == nullptr) return HYENA_ERR_INVALID_ARG;
  if (!boundary_ok(bd) || B < 1) return B < 1 ? HYENA_ERR_INVALID_ARG : HYENA_ERR_UNSUPPORTED;
  const int W = p->width, R = fp->registers;
  if (!film_shape_ok(B, X, Y, Z, C, N, W, bd) || R < 1 || R > 1024) return HYENA_ERR_UNSUPPORTED;
  const void* ptrs[] = {p->w1, p->b1, p->w2, p->b2, p->w3, p->b3, p->decay, fp->q, fp->film_w, fp->film_b,
                        fp->omega0, u, reg, w_in, dskip, w_out, y, ws};
  for (const void* q : ptrs)
    if (!aligned16(q)) return HYENA_ERR_INVALID_ARG;
  if (k_out != nullptr && !aligned16(k_out)) return HYENA_ERR_INVALID_ARG;
  const NdFilmWs fw = nd_film_ws(B, X, Y, Z, C, N, W, bd);
  if (ws_bytes < fw.total) return HYENA_ERR_WORKSPACE;
  if (device_ok() != HYENA_OK) return HYENA_ERR_HIP;

  char* wsb = static_cast<char*>(ws);
  const NdWs w = nd_ws(B, X, Y, Z, C, N, bd);
  char* base = wsb + fw.base;
  const NdFws fl = nd_fws(X, Y, Z, C, N, bd);
  char* fbase = wsb + fw.fws;
  const int pd = pad_of(bd), MX = mx_of(X, bd), MY = pd * Y, MZ = pd * Z;
  const size_t P = (size_t)MX * MY * MZ;
  const size_t khs = film_kh_bytes(X, Y, Z, C, N, bd);
  float2* tw = reinterpret_cast<float2*>(wsb + fw.tw);
  float* mod = reinterpret_cast<float*>(wsb + fw.mod);

  // kernel synthesis: FiLM vectors of every sample, then each sample's kernels
  // and their spectra (the synthesis buffers are reused in stream order)
  if (ev) HY_CHECK_HIP(hipEventRecord(ev[0], stream));
  HY_CHECK_HIP(hy::twiddles(tw, 128, 128, stream));
  HY_CHECK_HIP(hy::nd_film_mod(reg, fp->q, fp->film_w, fp->film_b, fp->omega0, mod, B, R, C, W, stream));
  for (int b = 0; b < B; ++b) {
    hy::NdFilterArgs f{X, Y, Z, C, N, W, MX, MY, MZ, p->w1, p->b1, p->w2, p->b2, p->w3, p->b3, p->decay,
                       k_out ? k_out + (size_t)b * N * C * P : reinterpret_cast<float*>(fbase + fl.k)};
    f.film = mod + (size_t)b * 4 * W;
    HY_CHECK_HIP(hy::nd_filter(f, reinterpret_cast<float2*>(fbase + fl.F),
                               reinterpret_cast<float2*>(wsb + fw.kh + b * khs), tw, stream, k_out != nullptr));
  }
  if (ev) HY_CHECK_HIP(hipEventRecord(ev[1], stream));

  const int V = X * Y * Z, J = (N + 1) * C;
  float* wt_in = reinterpret_cast<float*>(base + w.wt_in);
  float* wt_out = reinterpret_cast<float*>(base + w.wt_out);
  float* pbuf = reinterpret_cast<float*>(base + w.p);
  float* zfin = reinterpret_cast<float*>(base + w.zfinal);
  float* ones = reinterpret_cast<float*>(base + w.gate);
  HY_CHECK_HIP(hy::transpose2d_pair(w_in, wt_in, C, J, w_out, wt_out, C, C, false, stream));
  hy::GemmArgs gi{u, wt_in, pbuf, B * V, J, C, V, false, true, nullptr};
  HY_CHECK_HIP(hy::gemm(gi, false, stream));
  if (ev) HY_CHECK_HIP(hipEventRecord(ev[2], stream));

  // unit gates; two samples per packed complex field as in hyena_nd_fwd, the
  // spectral product filtering each half with its own sample's spectra ((P, Q)
  // form: the pencil pass on 3D grids, the fused plane kernel on 2D grids)
  HY_CHECK_HIP(hy::fill(ones, (size_t)B * N * C, 1.f, stream));
  hy::NdConvArgs a{};
  a.X = X;
  a.Y = Y;
  a.Z = Z;
  a.MX = MX;
  a.MY = MY;
  a.MZ = MZ;
  a.C = C;
  a.NO = N;
  a.B = B;
  a.p = pbuf;
  a.dskip = dskip;
  a.gate = ones;
  a.zbuf[0] = reinterpret_cast<float*>(base + w.z0);
  a.zbuf[1] = reinterpret_cast<float*>(base + w.z1);
  a.zfinal = zfin;
  a.Yint = reinterpret_cast<float2*>(base + w.Y);
  a.kh = reinterpret_cast<const float2*>(wsb + fw.kh);
  a.kh_stride = khs / sizeof(float2);
  a.tw128 = tw;
  HY_CHECK_HIP(hy::nd_conv(a, stream));
  if (ev) HY_CHECK_HIP(hipEventRecord(ev[3], stream));
  hy::GemmArgs go{zfin, wt_out, y, B * V, C, C, V, true, false, nullptr};
  HY_CHECK_HIP(hy::gemm(go, false, stream));
  if (ev) HY_CHECK_HIP(hipEventRecord(ev[4], stream));
  return HYENA_OK;
}

}  // namespace

extern "C" {

size_t hyena_nd_film_workspace_bytes(int B, int X, int Y, int Z, int C, int N, int width, int boundary) {
  if (!film_shape_ok(B, X, Y, Z, C, N, width, boundary)) return 0;
  return nd_film_ws(B, X, Y, Z, C, N, width, boundary).total;
}

int hyena_nd_film_fwd(int X, int Y, int Z, int C, int N, int boundary, const hyena_nd_filter_params* p,
                      const hyena_nd_film_params* fp, const float* u, const float* reg, const float* w_in,
                      const float* dskip, const float* w_out, int B, float* y, float* k_out, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
  return film_fwd_impl(X, Y, Z, C, N, boundary, p, fp, u, reg, w_in, dskip, w_out, B, y, k_out, ws, ws_bytes,
                       stream, nullptr);
}

int hyena_nd_film_fwd_profiled(int X, int Y, int Z, int C, int N, int boundary, const hyena_nd_filter_params* p,
                               const hyena_nd_film_params* fp, const float* u, const float* reg,
                               const float* w_in, const float* dskip, const float* w_out, int B, float* y,
                               float* k_out, void* ws, size_t ws_bytes, hipStream_t stream,
                               const hipEvent_t* events) {
  if (events == nullptr) return HYENA_ERR_INVALID_ARG;
  return film_fwd_impl(X, Y, Z, C, N, boundary, p, fp, u, reg, w_in, dskip, w_out, B, y, k_out, ws, ws_bytes,
                       stream, events);
}

}  // extern "C"
