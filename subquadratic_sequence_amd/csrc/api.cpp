// C ABI of libhyena: argument validation, memory layout of the layer cache and
// workspace, and the launch sequence of the forward path. Every check runs on
// the host before the first HIP call.
#include "../../include/hyena.h"

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "kernels.h"

using hy::align_up;

namespace {

// Default bound on the four-step intermediate of one channel-pair group, MB.
constexpr int kGroupMB = 0;

constexpr size_t kAlign = 256;
constexpr int kLdsMaxL = 4096;  // 2L <= 8192 runs fully in LDS

bool is_pow2(long long x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(long long x) {
  int r = 0;
  while ((1LL << r) < x) ++r;
  return r;
}
bool aligned16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }

bool shape_ok(int L, int D, int N) {
  return is_pow2(L) && L >= 16 && L <= (1 << 20) && D >= 64 && D <= 8192 && D % 64 == 0 && N >= 1 && N <= 4;
}

// ---------------------------------------------------------------- cache layout
struct CacheLayout {
  bool lds;
  int N2, lo_bits;
  size_t tw, w256, tw_lo, tw_hi, tw_row, pq, pq_bf16, total;
};

CacheLayout cache_layout(int L, int D, int N) {
  CacheLayout c{};
  const size_t n = 2 * (size_t)L;
  size_t off = 0;
  c.lds = L <= kLdsMaxL;
  if (c.lds) {
    c.tw = off;
    off = align_up(off + n * 8, kAlign);
    c.pq = off;
    off = align_up(off + (size_t)N * (D / 2) * (L + 1) * 16, kAlign);
  } else {
    c.N2 = (int)(n / hy::fourstep_n1(L));
    c.lo_bits = (ilog2((long long)n) + 1) / 2;
    c.w256 = off;
    off = align_up(off + 256 * 8, kAlign);
    c.tw_lo = off;
    off = align_up(off + ((size_t)1 << c.lo_bits) * 8, kAlign);
    c.tw_hi = off;
    off = align_up(off + (n >> c.lo_bits) * 8, kAlign);
    c.tw_row = off;
    off = align_up(off + (size_t)c.N2 * 8, kAlign);
    // filter spectra: fp32 (P, Q) entries, then a bf16 copy for the bf16 row passes
    const size_t entries = (size_t)N * (D / 2) * (hy::fourstep_n1(L) / 2 + 1) * c.N2;
    c.pq = off;
    off = align_up(off + entries * 16, kAlign);
    c.pq_bf16 = off;
    off = align_up(off + entries * 8, kAlign);
  }
  c.total = off;
  return c;
}

hy::FourStepTables tables(const CacheLayout& c, void* cache) {
  char* base = static_cast<char*>(cache);
  hy::FourStepTables t{};
  t.w256 = reinterpret_cast<const float2*>(base + c.w256);
  t.tw_lo = reinterpret_cast<const float2*>(base + c.tw_lo);
  t.tw_hi = reinterpret_cast<const float2*>(base + c.tw_hi);
  t.tw_row = reinterpret_cast<const float2*>(base + c.tw_row);
  t.lo_bits = c.lo_bits;
  return t;
}

// ------------------------------------------------------------ workspace layouts
bool direction_ok(int dir) { return dir == HYENA_CAUSAL || dir == HYENA_NONCAUSAL; }

struct FilterWs {
  size_t h, Y, total;
};
// h: [N][D][L] causal, [N][D][2L] (wrapped two-sided filter) non-causal
FilterWs filter_ws(int L, int D, int N, int dir) {
  FilterWs w{};
  size_t off = 0;
  w.h = off;
  off = align_up(off + (size_t)N * D * L * 4 * (dir == HYENA_NONCAUSAL ? 2 : 1), kAlign);
  w.Y = off;
  if (L > kLdsMaxL) off = align_up(off + (size_t)N * (D / 2) * 2 * (size_t)L * 8, kAlign);
  w.total = off;
  return w;
}

struct FwdWs {
  size_t wt_in, wt_out, p, zfinal, z0, z1, Y, total;
};
FwdWs fwd_ws(int B, int L, int D, int N, int dtype) {
  FwdWs w{};
  const size_t es = dtype == HYENA_BF16 ? 2 : 4;
  const size_t J = (size_t)(N + 1) * D;
  size_t off = 0;
  w.wt_in = off;
  off = align_up(off + J * D * es, kAlign);
  w.wt_out = off;
  off = align_up(off + (size_t)D * D * es, kAlign);
  w.p = off;
  off = align_up(off + (size_t)B * J * L * es, kAlign);
  w.zfinal = off;
  off = align_up(off + (size_t)B * D * L * es, kAlign);
  if (L > kLdsMaxL) {
    w.z0 = off;
    off = align_up(off + (size_t)B * D * L * es, kAlign);
    w.z1 = off;
    off = align_up(off + (size_t)B * D * L * es, kAlign);
    w.Y = off;
    off = align_up(off + (size_t)B * (D / 2) * 2 * (size_t)L * 8, kAlign);
  }
  w.total = off;
  return w;
}

int device_ok() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return HYENA_ERR_HIP;
  return HYENA_OK;
}

// Tuning knobs (read once): HYENA_GROUP_PAIRS = channel pairs per four-step
// group (overrides HYENA_GROUP_MB); HYENA_GROUP_MB = bound on the four-step
// intermediate of one group, in MB (0: all pairs in one group); 
// HYENA_SPECTRUM_FP32 = 1 keeps the four-step intermediate, and the filter
// spectra the row passes read, in fp32 for bf16 workloads.
struct Tuning {
  int group_pairs = 0;
  int group_mb = kGroupMB;
  bool y_bf16 = true;
};
const Tuning& tuning() {
  static const Tuning t = [] {
    Tuning r;
    if (const char* s = getenv("HYENA_GROUP_PAIRS")) r.group_pairs = atoi(s);
    if (const char* s = getenv("HYENA_GROUP_MB")) r.group_mb = atoi(s);
    if (const char* s = getenv("HYENA_SPECTRUM_FP32")) r.y_bf16 = atoi(s) == 0;
    return r;
  }();
  return t;
}

// Channel pairs per four-step group: the passes of one group run back to back,
// so a group whose intermediate fits the 256 MB last-level cache with room to
// spare reads it back from there rather than from HBM. Groups are balanced.
int group_pairs(int pairs_all, size_t y_bytes_per_pair) {
  const Tuning& t = tuning();
  if (t.group_pairs > 0) return t.group_pairs;
  if (t.group_mb <= 0) return pairs_all;
  const size_t cap = (size_t)t.group_mb << 20;
  long long per = (long long)(cap / y_bytes_per_pair);
  if (per < 1) per = 1;
  const long long ng = (pairs_all + per - 1) / per;
  return (int)((pairs_all + ng - 1) / ng);
}

}  // namespace

extern "C" {

const char* hyena_status_str(int status) {
  switch (status) {
    case HYENA_OK: return "ok";
    case HYENA_ERR_INVALID_ARG: return "invalid argument";
    case HYENA_ERR_UNSUPPORTED: return "unsupported shape";
    case HYENA_ERR_WORKSPACE: return "workspace or cache too small";
    case HYENA_ERR_LAYER_MISMATCH: return "layer not built for these sizes";
    case HYENA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

size_t hyena_cache_bytes(int L, int D, int N) {
  if (!shape_ok(L, D, N)) return 0;
  return cache_layout(L, D, N).total;
}

size_t hyena_filter_workspace_bytes_ex(int L, int D, int N, int direction) {
  if (!shape_ok(L, D, N) || !direction_ok(direction)) return 0;
  return filter_ws(L, D, N, direction).total;
}

size_t hyena_filter_workspace_bytes(int L, int D, int N) {
  return hyena_filter_workspace_bytes_ex(L, D, N, HYENA_CAUSAL);
}

size_t hyena_workspace_bytes(int B, int L, int D, int N, int dtype) {
  if (!shape_ok(L, D, N) || B < 1 || (dtype != HYENA_F32 && dtype != HYENA_BF16)) return 0;
  if ((long long)B * L * (N + 1) * D >= (1LL << 31)) return 0;
  return fwd_ws(B, L, D, N, dtype).total;
}

int hyena_layer_init_ex(hyena_layer* layer, int L, int D, int N, int direction, void* cache, size_t cache_bytes) {
  if (layer == nullptr) return HYENA_ERR_INVALID_ARG;
  if (!shape_ok(L, D, N) || !direction_ok(direction)) return HYENA_ERR_UNSUPPORTED;
  if (!aligned16(cache)) return HYENA_ERR_INVALID_ARG;
  if (cache_bytes < cache_layout(L, D, N).total) return HYENA_ERR_WORKSPACE;
  layer->L = L;
  layer->D = D;
  layer->N = N;
  layer->built = 0;
  layer->cache = cache;
  layer->cache_bytes = cache_bytes;
  layer->direction = direction;
  return HYENA_OK;
}

int hyena_layer_init(hyena_layer* layer, int L, int D, int N, void* cache, size_t cache_bytes) {
  return hyena_layer_init_ex(layer, L, D, N, HYENA_CAUSAL, cache, cache_bytes);
}

int hyena_filter_gen(hyena_layer* layer, const hyena_filter_params* p, float* h_out, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  if (layer == nullptr || p == nullptr) return HYENA_ERR_INVALID_ARG;
  const int L = layer->L, D = layer->D, N = layer->N, dir = layer->direction;
  if (!shape_ok(L, D, N) || !direction_ok(dir)) return HYENA_ERR_UNSUPPORTED;
  if (!aligned16(layer->cache)) return HYENA_ERR_INVALID_ARG;
  const CacheLayout cl = cache_layout(L, D, N);
  if (layer->cache_bytes < cl.total) return HYENA_ERR_WORKSPACE;
  if (p->pe_freqs < 1 || p->pe_freqs > 32 || p->width < 1 || p->width > 128) return HYENA_ERR_UNSUPPORTED;
  const void* ptrs[] = {p->w1, p->b1, p->w2, p->b2, p->w3, p->b3, p->decay, ws};
  for (const void* q : ptrs)
    if (!aligned16(q)) return HYENA_ERR_INVALID_ARG;
  if (h_out != nullptr && !aligned16(h_out)) return HYENA_ERR_INVALID_ARG;
  const FilterWs fw = filter_ws(L, D, N, dir);
  if (ws_bytes < fw.total) return HYENA_ERR_WORKSPACE;
  if (device_ok() != HYENA_OK) return HYENA_ERR_HIP;

  char* wsb = static_cast<char*>(ws);
  char* cb = static_cast<char*>(layer->cache);
  float* h = h_out ? h_out : reinterpret_cast<float*>(wsb + fw.h);
  const bool two_sided = dir == HYENA_NONCAUSAL;
  hy::Filter1DArgs fa{L,     D,     N,     p->pe_freqs, p->width, p->w1,    p->b1,
                      p->w2, p->b2, p->w3, p->b3,       p->decay, h,        two_sided ? 1 : 0};
  layer->built = 0;
  HY_CHECK_HIP(hy::filter1d_mlp(fa, stream));
  const int n = 2 * L;
  if (cl.lds) {
    float2* tw = reinterpret_cast<float2*>(cb + cl.tw);
    HY_CHECK_HIP(hy::twiddles(tw, n, n, stream));
    HY_CHECK_HIP(hy::lds_spec(h, tw, reinterpret_cast<float4*>(cb + cl.pq), L, D, N, two_sided, stream));
  } else {
    HY_CHECK_HIP(hy::twiddles(reinterpret_cast<float2*>(cb + cl.w256), 256, 256, stream));
    HY_CHECK_HIP(hy::twiddles(reinterpret_cast<float2*>(cb + cl.tw_lo), n, 1 << cl.lo_bits, stream));
    // tw_hi[i] = W_N^(i << lo_bits): twiddles of size n >> lo_bits
    HY_CHECK_HIP(hy::twiddles(reinterpret_cast<float2*>(cb + cl.tw_hi), n >> cl.lo_bits, n >> cl.lo_bits, stream));
    HY_CHECK_HIP(hy::twiddles(reinterpret_cast<float2*>(cb + cl.tw_row), cl.N2, cl.N2, stream));
    HY_CHECK_HIP(hy::fourstep_spec(tables(cl, layer->cache), h, reinterpret_cast<float2*>(wsb + fw.Y),
                                   reinterpret_cast<float4*>(cb + cl.pq), cb + cl.pq_bf16, L, D, N, two_sided,
                                   stream));
  }
  layer->built = 1;
  return HYENA_OK;
}

static int fwd_impl(const hyena_layer* layer, const void* u, const void* w_in, const float* short_w,
                    const float* dskip, const void* w_out, int B, int dtype, void* y, void* ws, size_t ws_bytes,
                    hipStream_t stream, const hipEvent_t* ev) {
  if (layer == nullptr) return HYENA_ERR_INVALID_ARG;
  if (dtype != HYENA_F32 && dtype != HYENA_BF16) return HYENA_ERR_INVALID_ARG;
  const void* ptrs[] = {u, w_in, short_w, dskip, w_out, y, ws};
  for (const void* q : ptrs)
    if (!aligned16(q)) return HYENA_ERR_INVALID_ARG;
  if (B < 1) return HYENA_ERR_INVALID_ARG;
  const int L = layer->L, D = layer->D, N = layer->N;
  if (!shape_ok(L, D, N)) return HYENA_ERR_UNSUPPORTED;
  if (!layer->built || !aligned16(layer->cache)) return HYENA_ERR_LAYER_MISMATCH;
  const CacheLayout cl = cache_layout(L, D, N);
  if (layer->cache_bytes < cl.total) return HYENA_ERR_LAYER_MISMATCH;
  if ((long long)B * L * (N + 1) * D >= (1LL << 31)) return HYENA_ERR_UNSUPPORTED;
  const FwdWs fw = fwd_ws(B, L, D, N, dtype);
  if (ws_bytes < fw.total) return HYENA_ERR_WORKSPACE;
  if (device_ok() != HYENA_OK) return HYENA_ERR_HIP;

  const bool bf = dtype == HYENA_BF16;
  char* wsb = static_cast<char*>(ws);
  char* cb = static_cast<char*>(layer->cache);
  const int J = (N + 1) * D;
  void* wt_in = wsb + fw.wt_in;
  void* wt_out = wsb + fw.wt_out;
  void* pbuf = wsb + fw.p;
  void* zfin = wsb + fw.zfinal;

  if (ev) HY_CHECK_HIP(hipEventRecord(ev[0], stream));
  HY_CHECK_HIP(hy::transpose2d(w_in, wt_in, D, J, bf, stream));
  HY_CHECK_HIP(hy::transpose2d(w_out, wt_out, D, D, bf, stream));
  // in-projection with the short convolution in the epilogue: pbuf holds s
  hy::GemmArgs gi{u, wt_in, pbuf, B * L, J, D, L, false, true, short_w};
  HY_CHECK_HIP(hy::gemm(gi, bf, stream));
  if (ev) HY_CHECK_HIP(hipEventRecord(ev[1], stream));
  if (cl.lds) {
    hy::LdsConvArgs a{pbuf, dskip, reinterpret_cast<const float4*>(cb + cl.pq),
                      reinterpret_cast<const float2*>(cb + cl.tw), zfin, B, L, D, N};
    HY_CHECK_HIP(hy::lds_conv(a, bf, stream));
  } else {
    hy::FourStepConvArgs a{};
    a.s = pbuf;
    a.dskip = dskip;
    a.pq = reinterpret_cast<const float4*>(cb + cl.pq);
    a.pq_bf16 = cb + cl.pq_bf16;
    a.z[0] = wsb + fw.z0;
    a.z[1] = wsb + fw.z1;
    a.zfinal = zfin;
    a.Y = wsb + fw.Y;
    a.B = B;
    a.L = L;
    a.D = D;
    a.NO = N;
    a.y_bf16 = tuning().y_bf16;
    a.group_pairs = group_pairs(B * (D / 2), (size_t)2 * L * (bf && a.y_bf16 ? 4 : 8));
    HY_CHECK_HIP(hy::fourstep_conv(tables(cl, layer->cache), a, bf, stream));
  }
  if (ev) HY_CHECK_HIP(hipEventRecord(ev[2], stream));
  hy::GemmArgs go{zfin, wt_out, y, B * L, D, D, L, true, false, nullptr};
  HY_CHECK_HIP(hy::gemm(go, bf, stream));
  if (ev) HY_CHECK_HIP(hipEventRecord(ev[3], stream));
  return HYENA_OK;
}

int hyena_fwd(const hyena_layer* layer, const void* u, const void* w_in, const float* short_w, const float* dskip,
              const void* w_out, int B, int dtype, void* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  return fwd_impl(layer, u, w_in, short_w, dskip, w_out, B, dtype, y, ws, ws_bytes, stream, nullptr);
}

int hyena_fwd_profiled(const hyena_layer* layer, const void* u, const void* w_in, const float* short_w,
                       const float* dskip, const void* w_out, int B, int dtype, void* y, void* ws, size_t ws_bytes,
                       hipStream_t stream, const hipEvent_t* events) {
  if (events == nullptr) return HYENA_ERR_INVALID_ARG;
  return fwd_impl(layer, u, w_in, short_w, dskip, w_out, B, dtype, y, ws, ws_bytes, stream, events);
}

}  // extern "C"
