// C ABI of libhyena: argument validation, memory layout of the layer cache and
// workspace, and the launch sequence of the forward path. Every check runs on
// the host before the first HIP call.
#include "../../include/hyena.h"

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "kernels.h"
#include "kernels_bwd.h"

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
// B * L * (N+1) * D < 2^31 (element offsets fit int32), for B >= 1 and a valid
// shape, tested by division: the product itself can exceed 64 bits
bool fits_i32(int B, int L, int D, int N) {
  return (long long)B <= ((1LL << 31) - 1) / ((long long)L * (N + 1) * D);
}

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

// ---------------------------------------------------------------- backward
constexpr int kBwdMinL = 32;  // the weight-gradient products take K = L in whole bf16 K tiles

bool bwd_shape_ok(int L, int D, int N, int dir) { return shape_ok(L, D, N) && L >= kBwdMinL && direction_ok(dir); }

// K splits of a reduction product (weight gradients: K runs over positions)
// so that about 512 workgroups share it: powers of two that keep whole K
// tiles of kt elements and at least 128 elements per split.
int ksplit(int K, int kt, long long tiles) {
  int s = 1;
  while (tiles * s < 512 && K % (2 * s * kt) == 0 && K / (2 * s) >= 128) s *= 2;
  return s;
}
long long tiles_of(int M, int N) { return (long long)((M + 255) / 256) * ((N + 127) / 128); }
int bwd_split_out(int B, int L, int D, int dtype) { return ksplit(L, dtype == HYENA_BF16 ? 32 : 16, tiles_of(D, D) * B); }
int bwd_split_in(int B, int L, int D, int N, int dtype) {
  return ksplit(L, dtype == HYENA_BF16 ? 32 : 16, tiles_of(D, (N + 1) * D) * B);
}

struct BwdWs {
  size_t wt_in, s, p, gz, zsave, csave, zfin, sbar, pbar, dh_part, dd_part, dsw_part, dwo_part, dwi_part;
  // four-step regime: convolution staging and output, the passes' intermediate,
  // dz ping-pong (fp32), one sample's z (or dc) spectrum (fp32 and bf16);
  // two-sided filters: g x^n in fp32
  size_t tmp, cout, Y, g0, g1, pq_tmp, pqb_tmp, dcf;
  size_t total;
};
BwdWs bwd_ws(int B, int L, int D, int N, int dtype, int dir) {
  BwdWs w{};
  const size_t es = dtype == HYENA_BF16 ? 2 : 4;
  const size_t J = (size_t)(N + 1) * D, HL = dir == HYENA_NONCAUSAL ? 2 * (size_t)L : L;
  const size_t BDL = (size_t)B * D * L, BJL = (size_t)B * J * L;
  size_t off = 0;
  auto take = [&](size_t& at, size_t bytes) {
    at = off;
    off = align_up(off + bytes, kAlign);
  };
  take(w.wt_in, J * D * es);
  take(w.s, BJL * es);
  take(w.p, BJL * es);
  take(w.gz, BDL * es);
  take(w.zsave, (size_t)N * BDL * 4);
  take(w.csave, (size_t)N * BDL * 4);
  take(w.zfin, BDL * es);
  take(w.sbar, BJL * 4);
  take(w.pbar, BJL * es);
  // per-sample partial results (with one sample the outputs take them)
  const size_t parts = B == 1 ? 0 : (size_t)B;
  take(w.dh_part, parts * N * D * HL * 4);
  take(w.dd_part, parts * N * D * 4);
  take(w.dsw_part, parts * J * 3 * 4);
  take(w.dwo_part, (size_t)B * bwd_split_out(B, L, D, dtype) * D * D * es);
  take(w.dwi_part, (size_t)B * bwd_split_in(B, L, D, N, dtype) * D * J * es);
  if (L > kLdsMaxL) {
    const int n1 = hy::fourstep_n1(L);
    const size_t entries = (size_t)(D / 2) * (n1 / 2 + 1) * (2 * (size_t)L / n1);
    take(w.tmp, 2 * BDL * es);
    take(w.cout, BDL * es);
    take(w.Y, (size_t)B * (D / 2) * 2 * (size_t)L * 8);
    take(w.g0, BDL * 4);
    take(w.g1, BDL * 4);
    take(w.pq_tmp, entries * 16);
    take(w.pqb_tmp, entries * 8);
    if (dir == HYENA_NONCAUSAL) take(w.dcf, BDL * 4);
  }
  w.total = off;
  return w;
}

struct FilterBwdWs {
  size_t e, a1, c1, a2, c2, w3t, o, dout, g2, g1, a2t, a1t, et, d2t, d1t, part, total;
  int s3, s2, s1, sg;  // K splits of dW3, dW2, dW1 (over positions) and of dL/da2 (over N D)
};
FilterBwdWs filter_bwd_ws(int L, int D, int N, int K, int W, int dir) {
  FilterBwdWs w{};
  const size_t P = dir == HYENA_NONCAUSAL ? 2 * (size_t)L : L, F = 1 + 2 * (size_t)K, ND = (size_t)N * D;
  size_t off = 0;
  auto take = [&](size_t& at, size_t floats) {
    at = off;
    off = align_up(off + floats * 4, kAlign);
  };
  take(w.e, P * F);
  take(w.a1, P * W);
  take(w.c1, P * W);
  take(w.a2, P * W);
  take(w.c2, P * W);
  take(w.w3t, ND * W);
  take(w.o, ND * P);
  take(w.dout, ND * P);
  take(w.g2, P * W);
  take(w.g1, P * W);
  take(w.a2t, P * W);
  take(w.a1t, P * W);
  take(w.et, P * F);
  take(w.d2t, P * W);
  take(w.d1t, P * W);
  w.s3 = ksplit((int)P, 16, tiles_of(W, (int)ND));
  w.s2 = ksplit((int)P, 16, tiles_of(W, W));
  w.s1 = ksplit((int)P, 16, tiles_of((int)F, W));
  w.sg = ksplit((int)ND, 16, tiles_of((int)P, W));
  size_t part = (size_t)w.s3 * W * ND;
  part = part > (size_t)w.s2 * W * W ? part : (size_t)w.s2 * W * W;
  part = part > (size_t)w.s1 * F * W ? part : (size_t)w.s1 * F * W;
  part = part > (size_t)w.sg * P * W ? part : (size_t)w.sg * P * W;
  take(w.part, part);
  w.total = off;
  return w;
}

bool filter_bwd_params_ok(int K, int W) { return K >= 1 && K <= 32 && W >= 16 && W <= 128 && W % 16 == 0; }

// Backward through the orders in the four-step regime, built on the forward's
// four-step convolution: every convolution below is fourstep_conv on one order
// with no gate and no skip (plain: the last column pass writes h * z), its
// input in block 0 of tmp [B][2D][L] (the layout of s with N = 1; block 1 is
// not read). With R the reversal t -> L - 1 - t on [0, L), the
// transposed convolution is R conv_h R (causal and two-sided filters alike: the
// layer's spectra hold either), and the filter gradient
// dh(tau) = sum_t dc(t) z(t - tau) is conv(R dc, z)(L - 1 - tau) for tau >= 0,
// z^n taken as the filter with its spectrum made per sample by the
// filter-spectrum passes; the negative lags of two-sided filters are
// dh(-tau) = conv(R z, dc)(L - 1 - tau), dc taken as the filter. Outputs as
// bwd_lds_conv: z^{N+1}, ds = (dz^1, dx^1 .. dx^N) and the per-sample dh and dD
// partials. Returns a status.
int bwd_fourstep(const hyena_layer* layer, const CacheLayout& cl, const BwdWs& w, char* wb, const float* dskip,
                 float* dh_part, float* dd_part, int B, bool bf, hipStream_t stream) {
  const int L = layer->L, D = layer->D, N = layer->N, half = D / 2, J = (N + 1) * D;
  const size_t es = bf ? 2 : 4, DL = (size_t)D * L, BDL = (size_t)B * DL;
  char* cb = static_cast<char*>(layer->cache);
  const hy::FourStepTables tb = tables(cl, layer->cache);
  const size_t per_order = (size_t)half * (hy::fourstep_n1(L) / 2 + 1) * cl.N2;  // spectrum entries per order
  const float4* pq = reinterpret_cast<const float4*>(cb + cl.pq);
  const char* pqb = cb + cl.pq_bf16;  // 8-byte bf16 entries
  char* tmp = wb + w.tmp;
  void* cout = wb + w.cout;
  float* zs = reinterpret_cast<float*>(wb + w.zsave);  // z^1 .. z^N, fp32
  char* cs = wb + w.csave;                              // c^1 .. c^N, storage type
  float* sbar = reinterpret_cast<float*>(wb + w.sbar);
  const bool two = layer->direction == HYENA_NONCAUSAL;
  const int HL = two ? 2 * L : L;
  float* dcf = two ? reinterpret_cast<float*>(wb + w.dcf) : nullptr;
  const bool ybf = bf && tuning().y_bf16;
  auto conv = [&](const void* in, int Bc, const float4* p, const void* pb, void* out) {
    hy::FourStepConvArgs a{};
    a.s = in;
    a.dskip = nullptr;  // not read by the plain pass
    a.plain = true;
    a.pq = p;
    a.pq_bf16 = pb;
    a.z[0] = a.z[1] = out;  // one order: only zfinal is written
    a.zfinal = out;
    a.Y = wb + w.Y;
    a.B = Bc;
    a.L = L;
    a.D = D;
    a.NO = 1;
    a.y_bf16 = tuning().y_bf16;
    a.group_pairs = group_pairs(Bc * half, (size_t)2 * L * (ybf ? 4 : 8));
    return hy::fourstep_conv(tb, a, bf, stream);
  };
  // forward orders, keeping z^n (fp32) and c^n (storage type)
  HY_CHECK_HIP(hy::bwd4_z_init(wb + w.s, zs, tmp, B, D, L, N, bf, stream));
  for (int n = 0; n < N; ++n) {
    char* cn = cs + (size_t)n * BDL * es;
    HY_CHECK_HIP(conv(tmp, B, pq + n * per_order, pqb + n * per_order * 8, cn));
    float* znext = n == N - 1 ? nullptr : zs + (size_t)(n + 1) * BDL;
    HY_CHECK_HIP(hy::bwd4_z_next(wb + w.s, cn, zs + (size_t)n * BDL, dskip + (size_t)n * D, znext, tmp,
                                 wb + w.zfin, B, D, L, N, n, bf, stream));
  }
  // orders in reverse, g = dz^{n+1} in fp32
  float* g = reinterpret_cast<float*>(wb + w.g0);
  float* gn = reinterpret_cast<float*>(wb + w.g1);
  HY_CHECK_HIP(hy::bwd4_to_f32(wb + w.gz, g, BDL, bf, stream));
  for (int n = N - 1; n >= 0; --n) {
    const float* zn = zs + (size_t)n * BDL;
    // dx^n = g c^n, staging R(g x^n), sum_t g z^n
    HY_CHECK_HIP(hy::bwd4_rev_prep(g, wb + w.s, cs + (size_t)n * BDL * es, zn, sbar, tmp, dcf, dd_part, B, D, L, N,
                                   n, bf, stream));
    // dz^n = D^n g + R conv_h R(g x^n); dz^1 is block 0 of ds
    HY_CHECK_HIP(conv(tmp, B, pq + n * per_order, pqb + n * per_order * 8, cout));
    float* out = n == 0 ? sbar : gn;
    HY_CHECK_HIP(hy::bwd4_rev_finish(g, cout, dskip + (size_t)n * D, out, n == 0 ? (size_t)J * L : DL, B, D, L, bf,
                                     stream));
    // dh^n of each sample: z^n_b as the filter, R(g x^n)_b as the input
    // (then, two-sided, (g x^n)_b as the filter, R z^n_b as the input)
    const float4* pq_t = reinterpret_cast<const float4*>(wb + w.pq_tmp);
    // only the spectrum form the convolution reads (bf16 entries straight from
    // the spectrum pass, or fp32 ones)
    float4* spec32 = ybf ? nullptr : reinterpret_cast<float4*>(wb + w.pq_tmp);
    void* spec16 = ybf ? wb + w.pqb_tmp : nullptr;
    for (int b = 0; b < B; ++b) {
      char* tb_b = tmp + (size_t)b * 2 * DL * es;
      float* dh_b = dh_part + ((size_t)b * N + n) * D * HL;
      HY_CHECK_HIP(hy::fourstep_spec(tb, zn + (size_t)b * DL, reinterpret_cast<float2*>(wb + w.Y), spec32, spec16, L,
                                     D, 1, false, stream));
      HY_CHECK_HIP(conv(tb_b, 1, pq_t, wb + w.pqb_tmp, cout));
      HY_CHECK_HIP(hy::bwd4_dh_store(cout, dh_b, D, L, HL, bf, stream));
      if (two) {
        HY_CHECK_HIP(hy::bwd4_stage_rev(zn + (size_t)b * DL, tb_b, D, L, bf, stream));
        HY_CHECK_HIP(hy::fourstep_spec(tb, dcf + (size_t)b * DL, reinterpret_cast<float2*>(wb + w.Y), spec32,
                                       spec16, L, D, 1, false, stream));
        HY_CHECK_HIP(conv(tb_b, 1, pq_t, wb + w.pqb_tmp, cout));
        HY_CHECK_HIP(hy::bwd4_dh_store_neg(cout, dh_b, D, L, bf, stream));
      }
    }
    float* t = g;
    g = gn;
    gn = t;
  }
  return HYENA_OK;
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
  if (!fits_i32(B, L, D, N)) return 0;
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

}  // extern "C"

namespace hy {

// Every host-side check of a forward call except the workspace pointer (no HIP
// call): hyena_fwd and the allocation-free entry point both run it first.
int fwd_validate(const hyena_layer* layer, const void* u, const void* w_in, const float* short_w,
                 const float* dskip, const void* w_out, int B, int dtype, const void* y, size_t ws_bytes) {
  if (layer == nullptr) return HYENA_ERR_INVALID_ARG;
  if (dtype != HYENA_F32 && dtype != HYENA_BF16) return HYENA_ERR_INVALID_ARG;
  const void* ptrs[] = {u, w_in, short_w, dskip, w_out, y};
  for (const void* q : ptrs)
    if (!aligned16(q)) return HYENA_ERR_INVALID_ARG;
  if (B < 1) return HYENA_ERR_INVALID_ARG;
  const int L = layer->L, D = layer->D, N = layer->N;
  if (!shape_ok(L, D, N)) return HYENA_ERR_UNSUPPORTED;
  if (!layer->built || !aligned16(layer->cache)) return HYENA_ERR_LAYER_MISMATCH;
  if (layer->cache_bytes < cache_layout(L, D, N).total) return HYENA_ERR_LAYER_MISMATCH;
  if (!fits_i32(B, L, D, N)) return HYENA_ERR_UNSUPPORTED;
  if (ws_bytes < fwd_ws(B, L, D, N, dtype).total) return HYENA_ERR_WORKSPACE;
  return HYENA_OK;
}

}  // namespace hy

extern "C" {

static int fwd_impl(const hyena_layer* layer, const void* u, const void* w_in, const float* short_w,
                    const float* dskip, const void* w_out, int B, int dtype, void* y, void* ws, size_t ws_bytes,
                    hipStream_t stream, const hipEvent_t* ev) {
  if (!aligned16(ws)) return HYENA_ERR_INVALID_ARG;
  const int st = hy::fwd_validate(layer, u, w_in, short_w, dskip, w_out, B, dtype, y, ws_bytes);
  if (st != HYENA_OK) return st;
  if (device_ok() != HYENA_OK) return HYENA_ERR_HIP;
  const int L = layer->L, D = layer->D, N = layer->N;
  const CacheLayout cl = cache_layout(L, D, N);
  const FwdWs fw = fwd_ws(B, L, D, N, dtype);

  const bool bf = dtype == HYENA_BF16;
  char* wsb = static_cast<char*>(ws);
  char* cb = static_cast<char*>(layer->cache);
  const int J = (N + 1) * D;
  void* wt_in = wsb + fw.wt_in;
  void* wt_out = wsb + fw.wt_out;
  void* pbuf = wsb + fw.p;
  void* zfin = wsb + fw.zfinal;

  if (ev) HY_CHECK_HIP(hipEventRecord(ev[0], stream));
  HY_CHECK_HIP(hy::transpose2d_pair(w_in, wt_in, D, J, w_out, wt_out, D, D, bf, stream));
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

size_t hyena_bwd_workspace_bytes(int B, int L, int D, int N, int dtype, int direction) {
  if (!bwd_shape_ok(L, D, N, direction) || B < 1 || (dtype != HYENA_F32 && dtype != HYENA_BF16)) return 0;
  if (!fits_i32(B, L, D, N)) return 0;
  return bwd_ws(B, L, D, N, dtype, direction).total;
}

int hyena_bwd(const hyena_layer* layer, const void* u, const void* w_in, const float* short_w, const float* dskip,
              const void* w_out, const void* dy, int B, int dtype, void* du, float* dw_in, float* dshort_w,
              float* ddskip, float* dw_out, float* dh, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (layer == nullptr) return HYENA_ERR_INVALID_ARG;
  if (dtype != HYENA_F32 && dtype != HYENA_BF16) return HYENA_ERR_INVALID_ARG;
  const void* ptrs[] = {u, w_in, short_w, dskip, w_out, dy, du, dw_in, dshort_w, ddskip, dw_out, dh, ws};
  for (const void* q : ptrs)
    if (!aligned16(q)) return HYENA_ERR_INVALID_ARG;
  if (B < 1) return HYENA_ERR_INVALID_ARG;
  const int L = layer->L, D = layer->D, N = layer->N, dir = layer->direction;
  if (!bwd_shape_ok(L, D, N, dir)) return HYENA_ERR_UNSUPPORTED;
  if (!layer->built || !aligned16(layer->cache)) return HYENA_ERR_LAYER_MISMATCH;
  const CacheLayout cl = cache_layout(L, D, N);
  if (layer->cache_bytes < cl.total) return HYENA_ERR_LAYER_MISMATCH;
  if (!fits_i32(B, L, D, N)) return HYENA_ERR_UNSUPPORTED;
  const BwdWs w = bwd_ws(B, L, D, N, dtype, dir);
  if (ws_bytes < w.total) return HYENA_ERR_WORKSPACE;
  if (device_ok() != HYENA_OK) return HYENA_ERR_HIP;

  const bool bf = dtype == HYENA_BF16;
  char* wb = static_cast<char*>(ws);
  char* cb = static_cast<char*>(layer->cache);
  const int J = (N + 1) * D, HL = dir == HYENA_NONCAUSAL ? 2 * L : L;
  // forward projections, channel-major: p = u W_in, and s its short convolution
  HY_CHECK_HIP(hy::transpose2d(w_in, wb + w.wt_in, D, J, bf, stream));
  HY_CHECK_HIP(hy::gemm(hy::GemmArgs{u, wb + w.wt_in, wb + w.p, B * L, J, D, L, false, true, nullptr}, bf, stream));
  HY_CHECK_HIP(hy::short_conv_rows(wb + w.p, short_w, wb + w.s, B * J, L, J, bf, stream));
  // dz^{N+1} = dy W_out^T, channel-major (W_out as stored is the transposed operand)
  HY_CHECK_HIP(hy::gemm(hy::GemmArgs{dy, w_out, wb + w.gz, B * L, D, D, L, false, true, nullptr}, bf, stream));
  // forward recompute and the orders in reverse
  float* sbar = reinterpret_cast<float*>(wb + w.sbar);
  // per-sample partial results, summed over the batch at the end; with one
  // sample they are written to the outputs directly
  const bool one = B == 1;
  float* dh_part = one ? dh : reinterpret_cast<float*>(wb + w.dh_part);
  float* dd_part = one ? ddskip : reinterpret_cast<float*>(wb + w.dd_part);
  float* dsw_part = one ? dshort_w : reinterpret_cast<float*>(wb + w.dsw_part);
  if (!cl.lds) {
    const int st = bwd_fourstep(layer, cl, w, wb, dskip, dh_part, dd_part, B, bf, stream);
    if (st != HYENA_OK) return st;
  } else {
    hy::BwdConvArgs a{};
    a.s = wb + w.s;
    a.gz = wb + w.gz;
    a.zsave = reinterpret_cast<float*>(wb + w.zsave);
    a.csave = reinterpret_cast<float*>(wb + w.csave);
    a.zfin = wb + w.zfin;
    a.dskip = dskip;
    a.pq = reinterpret_cast<const float4*>(cb + cl.pq);
    a.tw = reinterpret_cast<const float2*>(cb + cl.tw);
    a.sbar = sbar;
    a.dh_part = dh_part;
    a.dd_part = dd_part;
    a.B = B;
    a.L = L;
    a.D = D;
    a.NO = N;
    a.HL = HL;
    HY_CHECK_HIP(hy::bwd_lds_conv(a, bf, stream));
  }
  // short convolution transpose: dp, and per-sample tap gradients
  HY_CHECK_HIP(hy::short_conv_bwd(sbar, wb + w.p, short_w, wb + w.pbar, dsw_part, B * J, L, J, bf, stream));
  // du = dp W_in^T (dp channel-major; W_in as stored is the transposed operand)
  HY_CHECK_HIP(hy::gemm(hy::GemmArgs{wb + w.pbar, w_in, du, B * L, D, J, L, true, false, nullptr}, bf, stream));
  // weight gradients dW_out = sum_b z^{N+1}_b dy_b and dW_in = sum_b u_b^T dp_b
  // (K = L): one launch per product over the samples and K splits, the
  // partial results summed below. dy and u are read as stored, [L][D], by the
  // GEMM's channel-major A path (K = positions, M = the D channels of a row):
  // dW_out is formed as dy^T z^{N+1} and written transposed (channel-major
  // output), dW_in as u^T dp with dp channel-major as the transposed operand.
  const int so = bwd_split_out(B, L, D, dtype), si = bwd_split_in(B, L, D, N, dtype);
  hy::GemmArgs go{dy, wb + w.zfin, wb + w.dwo_part, D, D, L / so, D, true, true, nullptr};
  go.batch = B;
  go.nsplit = so;
  go.sa = go.sb = (size_t)D * L;
  go.sc = (size_t)D * D;
  go.ka = (size_t)(L / so) * D;
  go.kb = (size_t)(L / so);
  go.lda = L / so;
  go.ldb = L;
  HY_CHECK_HIP(hy::gemm(go, bf, stream));
  hy::GemmArgs gw{u, wb + w.pbar, wb + w.dwi_part, D, J, L / si, D, true, false, nullptr};
  gw.batch = B;
  gw.nsplit = si;
  gw.sa = (size_t)D * L;
  gw.sb = (size_t)J * L;
  gw.sc = (size_t)D * J;
  gw.ka = (size_t)(L / si) * D;
  gw.kb = (size_t)(L / si);
  gw.lda = L / si;
  gw.ldb = L;
  HY_CHECK_HIP(hy::gemm(gw, bf, stream));
  // sums over the batch, in a fixed order
  HY_CHECK_HIP(hy::sum_rows(wb + w.dwo_part, dw_out, B * so, (size_t)D * D, (size_t)D * D, bf, stream));
  HY_CHECK_HIP(hy::sum_rows(wb + w.dwi_part, dw_in, B * si, (size_t)D * J, (size_t)D * J, bf, stream));
  if (!one) {
    HY_CHECK_HIP(hy::sum_rows(dh_part, dh, B, (size_t)N * D * HL, (size_t)N * D * HL, false, stream));
    HY_CHECK_HIP(hy::sum_rows(dd_part, ddskip, B, (size_t)N * D, (size_t)N * D, false, stream));
    HY_CHECK_HIP(hy::sum_rows(dsw_part, dshort_w, B, (size_t)J * 3, (size_t)J * 3, false, stream));
  }
  return HYENA_OK;
}

size_t hyena_filter_bwd_workspace_bytes(int L, int D, int N, int pe_freqs, int width, int direction) {
  if (!shape_ok(L, D, N) || !direction_ok(direction) || !filter_bwd_params_ok(pe_freqs, width)) return 0;
  return filter_bwd_ws(L, D, N, pe_freqs, width, direction).total;
}

int hyena_filter_bwd(const hyena_layer* layer, const hyena_filter_params* p, const float* dh, float* dw1, float* db1,
                     float* dw2, float* db2, float* dw3, float* db3, float* ddecay, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  if (layer == nullptr || p == nullptr) return HYENA_ERR_INVALID_ARG;
  const int L = layer->L, D = layer->D, N = layer->N, dir = layer->direction;
  if (!shape_ok(L, D, N) || !direction_ok(dir)) return HYENA_ERR_UNSUPPORTED;
  if (!filter_bwd_params_ok(p->pe_freqs, p->width)) return HYENA_ERR_UNSUPPORTED;
  const void* ptrs[] = {p->w1, p->b1, p->w2, p->b2, p->w3, p->b3, p->decay, dh, dw1, db1, dw2, db2, dw3, db3, ddecay,
                        ws};
  for (const void* q : ptrs)
    if (!aligned16(q)) return HYENA_ERR_INVALID_ARG;
  const FilterBwdWs w = filter_bwd_ws(L, D, N, p->pe_freqs, p->width, dir);
  if (ws_bytes < w.total) return HYENA_ERR_WORKSPACE;
  if (device_ok() != HYENA_OK) return HYENA_ERR_HIP;

  char* wb = static_cast<char*>(ws);
  auto f = [&](size_t off) { return reinterpret_cast<float*>(wb + off); };
  const int W = p->width, F = 1 + 2 * p->pe_freqs, ND = N * D;
  const int P = dir == HYENA_NONCAUSAL ? 2 * L : L;
  hy::FilterBwdArgs a{};
  a.L = L;
  a.D = D;
  a.NO = N;
  a.K = p->pe_freqs;
  a.W = W;
  a.noncausal = dir == HYENA_NONCAUSAL ? 1 : 0;
  a.w1 = p->w1;
  a.b1 = p->b1;
  a.w2 = p->w2;
  a.b2 = p->b2;
  a.b3 = p->b3;
  a.decay = p->decay;
  a.dh = dh;
  a.o = f(w.o);
  a.e = f(w.e);
  a.a1 = f(w.a1);
  a.c1 = f(w.c1);
  a.a2 = f(w.a2);
  a.c2 = f(w.c2);
  a.dout = f(w.dout);
  a.ddecay = ddecay;
  // features and hidden layers; output layer o = a2 W3 (channel-major, without b3)
  HY_CHECK_HIP(hy::filter_bwd_feat(a, stream));
  HY_CHECK_HIP(hy::transpose2d(p->w3, f(w.w3t), W, ND, false, stream));
  HY_CHECK_HIP(hy::gemm(hy::GemmArgs{a.a2, f(w.w3t), f(w.o), P, ND, W, P, false, true, nullptr}, false, stream));
  // dL/do = dh * window (and the decay gradient)
  HY_CHECK_HIP(hy::filter_bwd_out(a, f(w.part), stream));
  // back through the hidden layers: dq2 = (do W3^T) cos(q2), dq1 = (dq2 W2^T) cos(q1)
  {
    // dL/da2 = dout^T W3^T over K = N D, split; partial results summed in order
    hy::GemmArgs g{f(w.dout), p->w3, f(w.part), P, W, ND / w.sg, P, true, false, nullptr};
    g.nsplit = w.sg;
    g.ka = (size_t)(ND / w.sg) * P;  // channel-major A: a split is N D / sg channels
    g.kb = (size_t)(ND / w.sg);
    g.sc = (size_t)P * W;
    g.lda = g.ldb = ND;
    HY_CHECK_HIP(hy::gemm(g, false, stream));
    HY_CHECK_HIP(hy::sum_rows(f(w.part), f(w.g2), w.sg, (size_t)P * W, (size_t)P * W, false, stream));
  }
  HY_CHECK_HIP(hy::mul_inplace(f(w.g2), a.c2, (size_t)P * W, stream));
  HY_CHECK_HIP(hy::gemm(hy::GemmArgs{f(w.g2), p->w2, f(w.g1), P, W, W, P, false, false, nullptr}, false, stream));
  HY_CHECK_HIP(hy::mul_inplace(f(w.g1), a.c1, (size_t)P * W, stream));
  // weight gradients as products over the positions (K = P)
  HY_CHECK_HIP(hy::transpose2d(a.a2, f(w.a2t), P, W, false, stream));
  HY_CHECK_HIP(hy::transpose2d(a.a1, f(w.a1t), P, W, false, stream));
  HY_CHECK_HIP(hy::transpose2d(a.e, f(w.et), P, F, false, stream));
  HY_CHECK_HIP(hy::transpose2d(f(w.g2), f(w.d2t), P, W, false, stream));
  HY_CHECK_HIP(hy::transpose2d(f(w.g1), f(w.d1t), P, W, false, stream));
  auto wgrad = [&](const float* A, const float* Bt, float* out, int M, int Nn, int S) -> hipError_t {
    hy::GemmArgs g{A, Bt, f(w.part), M, Nn, P / S, P, false, false, nullptr};
    g.nsplit = S;
    g.ka = g.kb = (size_t)(P / S);
    g.sc = (size_t)M * Nn;
    g.lda = g.ldb = P;
    hipError_t e = hy::gemm(g, false, stream);
    if (e != hipSuccess) return e;
    return hy::sum_rows_tall(f(w.part), out, S, (size_t)M * Nn, stream);
  };
  HY_CHECK_HIP(wgrad(f(w.a2t), f(w.dout), dw3, W, ND, w.s3));
  HY_CHECK_HIP(wgrad(f(w.a1t), f(w.d2t), dw2, W, W, w.s2));
  HY_CHECK_HIP(wgrad(f(w.et), f(w.d1t), dw1, F, W, w.s1));
  HY_CHECK_HIP(hy::row_sums(f(w.dout), db3, ND, P, f(w.part), stream));
  HY_CHECK_HIP(hy::row_sums(f(w.d2t), db2, W, P, f(w.part), stream));
  HY_CHECK_HIP(hy::row_sums(f(w.d1t), db1, W, P, f(w.part), stream));
  return HYENA_OK;
}

}  // extern "C"
