/*
 * hyena.h - C ABI of libhyena.so, the forward hot path of the Hyena operator
 * and of its 3D variant on AMD Instinct MI355X (gfx950).
 *
 * The operator (Hyena Hierarchy abstract, taxoreview.com page; French summary
 * on summarizepaper.com, "Key points") interleaves implicitly parametrised long
 * convolutions with data-controlled gating. This library computes, for order N:
 *
 *   p = u W_in, split into column blocks (v, x^1 .. x^N), each D wide
 *   s = causal depthwise short convolution of length 3 of every column of p
 *   z^1 = s_v;  z^{n+1} = s_{x^n} * (h^n conv z^n) + D^n * z^n   (n = 1..N)
 *   y = z^{N+1} W_out
 *
 * where each h^n is a causal filter as long as the input (TWIML #690 podcast,
 * 5:48) produced by an MLP of the position (TWIML #690, 4:29), applied through
 * the convolution theorem (TWIML #690, 6:27) with zero padding to 2L
 * (HyenaND explainer, gist.science, Methodology, "Handling Boundaries").
 *
 * Conventions used by every entry point
 *  - All tensor arguments are DEVICE pointers, allocated and owned by the
 *    caller (the library never allocates or frees device memory and keeps no
 *    global device state; calls on different streams with different buffers
 *    are independent).
 *  - Row-major layouts; the last listed dimension is contiguous.
 *  - Work is enqueued asynchronously on `stream`; nothing synchronises.
 *  - Every argument is validated on the host before the first HIP call; an
 *    invalid call returns an error code and enqueues nothing. A HIP failure
 *    while enqueuing returns HYENA_ERR_HIP (work enqueued before it may run).
 *  - Pointers must be 16-byte aligned.
 */
#ifndef HYENA_H
#define HYENA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of activations (u, y, intermediates) and projection weights.
 * Arithmetic is always fp32 (accumulation included). */
typedef enum { HYENA_F32 = 0, HYENA_BF16 = 1 } hyena_dtype;

enum {
  HYENA_OK = 0,
  HYENA_ERR_INVALID_ARG = 1,     /* null/misaligned pointer, bad size or dtype */
  HYENA_ERR_UNSUPPORTED = 2,     /* shape outside the supported ranges below */
  HYENA_ERR_WORKSPACE = 3,       /* workspace or cache smaller than required */
  HYENA_ERR_LAYER_MISMATCH = 4,  /* layer not built, or built for other sizes */
  HYENA_ERR_HIP = 5              /* a HIP call failed (no device, launch error) */
};

/* Returns a static string describing a status code. */
const char *hyena_status_str(int status);

/* ------------------------------------------------------------------ 1D ---- */

/* Parameters of the implicit filter (device pointers, fp32, row-major).
 *   PosEnc(t) = [tau, cos(2 pi k tau)_{k=1..K}, sin(2 pi k tau)_{k=1..K}], tau = t/L
 *   o_t = W3^T sin(W2^T sin(W1^T PosEnc(t) + b1) + b2) + b3        in R^{N*D}
 *   h^n_c(t) = exp(-decay_c * tau) * o_t[(n-1)*D + c],  t = 0 .. L-1
 * Shapes: w1 [1+2K][W], b1 [W], w2 [W][W], b2 [W], w3 [W][N*D], b3 [N*D],
 * decay [D]. Supported: 1 <= K <= 32, 1 <= W <= 128. */
typedef struct {
  int pe_freqs;  /* K */
  int width;     /* W */
  const float *w1, *b1, *w2, *b2, *w3, *b3, *decay;
} hyena_filter_params;

/* Direction of the long convolution.
 *   HYENA_CAUSAL     c_t = sum_{s=0..t} h(s) z_{t-s} (the default).
 *   HYENA_NONCAUSAL  two-sided filters: the same generator at the signed lags
 *                    tau in [-(L-1), L-1] (PosEnc at tau/L, window
 *                    exp(-decay_c |tau|/L)) and c_t = sum_tau h(tau) z_{t-tau},
 *                    z zero outside [0, L). The pages name causal use and
 *                    bidirectional comparators only; this is the reading taken.
 *                    The short convolution keeps its causal taps. */
typedef enum { HYENA_CAUSAL = 0, HYENA_NONCAUSAL = 1 } hyena_direction;

/* Host-side handle of one layer's filter cache. The cache is caller-owned
 * device memory of hyena_cache_bytes(L, D, N) bytes holding twiddle tables and
 * the spectra of the zero-padded filters in an internal (opaque) order. It is
 * shared by every batch and every hyena_fwd call of the layer. */
typedef struct {
  int L, D, N;
  int built;            /* set to 1 by hyena_filter_gen */
  void *cache;
  size_t cache_bytes;
  int direction;        /* hyena_direction, set by the init call */
} hyena_layer;

/* Supported shapes: L a power of two in [16, 2^20]; D a multiple of 64 in
 * [64, 8192]; 1 <= N <= 4; B >= 1 with B*L*(N+1)*D < 2^31.
 * The size queries return 0 for unsupported shapes. */
size_t hyena_cache_bytes(int L, int D, int N);
size_t hyena_filter_workspace_bytes(int L, int D, int N);
size_t hyena_workspace_bytes(int B, int L, int D, int N, int dtype);
/* Filter workspace for a direction (twice the filter buffer when non-causal);
 * 0 for an unknown direction. The cache and forward sizes do not depend on it. */
size_t hyena_filter_workspace_bytes_ex(int L, int D, int N, int direction);

/* Fills the host struct (no HIP call). `cache` must hold hyena_cache_bytes.
 * hyena_layer_init is the causal direction; hyena_layer_init_ex takes one
 * (HYENA_ERR_UNSUPPORTED for an unknown direction). */
int hyena_layer_init(hyena_layer *layer, int L, int D, int N, void *cache, size_t cache_bytes);
int hyena_layer_init_ex(hyena_layer *layer, int L, int D, int N, int direction, void *cache,
                        size_t cache_bytes);

/* Evaluates the implicit filters h^n and stores the spectra of their size-2L
 * DFTs in layer->cache: causal, [h^n(0..L-1), 0_L]; non-causal, the two-sided
 * filter wrapped (lag tau at tau mod 2L, entry L zero). If h_out is not NULL the
 * filters are also written there as fp32 [N][D][L] (causal) or in that wrapped
 * form [N][D][2L] (non-causal). `ws` is scratch of at least
 * hyena_filter_workspace_bytes_ex(L, D, N, layer->direction) bytes. Sets
 * layer->built = 1. */
int hyena_filter_gen(hyena_layer *layer, const hyena_filter_params *p, float *h_out,
                     void *ws, size_t ws_bytes, hipStream_t stream);

/* Forward pass of one layer.
 *   u       [B][L][D]        dtype
 *   w_in    [D][(N+1)*D]     dtype, column blocks (v, x^1, .., x^N)
 *   short_w [(N+1)*D][3]     fp32; tap k multiplies p_{t-k}, zero history
 *   dskip   [N][D]           fp32
 *   w_out   [D][D]           dtype
 *   y       [B][L][D]        dtype (output; may not alias the inputs)
 *   ws      scratch of at least hyena_workspace_bytes(B, L, D, N, dtype) bytes
 * The layer must have been built by hyena_filter_gen for the same (L, D, N). */
int hyena_fwd(const hyena_layer *layer, const void *u, const void *w_in,
              const float *short_w, const float *dskip, const void *w_out,
              int B, int dtype, void *y, void *ws, size_t ws_bytes, hipStream_t stream);

/* Same launches as hyena_fwd, plus hipEventRecord(events[i], stream) at the four
 * stage boundaries, for timing the stages on the launch stream:
 *   events[0] before the in-projection,
 *   events[1] after it (weight transposes, GEMM with the short convolutions),
 *   events[2] after the long convolutions with gating (all orders),
 *   events[3] after the out-projection.
 * events: host array of 4 events the caller created (and destroys); nothing here
 * synchronises. A null `events` is HYENA_ERR_INVALID_ARG. */
int hyena_fwd_profiled(const hyena_layer *layer, const void *u, const void *w_in,
                       const float *short_w, const float *dskip, const void *w_out,
                       int B, int dtype, void *y, void *ws, size_t ws_bytes, hipStream_t stream,
                       const hipEvent_t *events);

/* Size of the workspace array inside the library that hyena_fwd_noalloc uses:
 * 128 MiB, which holds hyena_workspace_bytes of B = 8, L = 2048, D = 768, N = 2
 * in bf16 (105 MB) and of every smaller call. */
#define HYENA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): hyena_fwd
 * without the ws argument. The workspace is a file-scope device array of
 * HYENA_NOALLOC_SCRATCH_BYTES bytes inside the library, one copy per GPU,
 * resolved on the first call on that GPU and held until the process ends; no
 * allocation routine is called. The caller still owns every input, the output
 * and the layer cache.
 *  - A call whose hyena_workspace_bytes(B, L, D, N, dtype) exceeds the array
 *    returns HYENA_ERR_WORKSPACE before any HIP call.
 *  - Every call on one GPU uses the same array and leaves its contents behind:
 *    calls that overlap on one GPU (other streams, other threads) race and
 *    must be serialised by the caller.
 *  - Other arguments, layouts and errors as hyena_fwd. */
int hyena_fwd_noalloc(const hyena_layer *layer, const void *u, const void *w_in,
                      const float *short_w, const float *dskip, const void *w_out,
                      int B, int dtype, void *y, hipStream_t stream);

/* ------------------------------------------------------------ 1D backward ---- */
/*
 * Gradients of a scalar loss through the layer (its vector-Jacobian product).
 * The pages' compute and speed claims are about training (Hyena Hierarchy
 * abstract: training compute at sequence length 2K; HyenaDNA abstract: training
 * speed at long contexts); they give no backward formulas, so these are the
 * chain rule of the forward steps in reverse order. With g = dz^{n+1}:
 *   dW_out = sum_b z^{N+1}_b^T dy_b,  dz^{N+1} = dy W_out^T
 *   dx^n = g c^n,  dD^n = sum_{b,t} g z^n,
 *   dz^n = D^n g + sum_{tau} h^n(tau) (g x^n)(t + tau)        (correlation: the
 *          transpose of the convolution; two-sided filters over signed lags)
 *   dh^n(tau) = sum_{b,t} (g x^n)(t) z^n(t - tau)
 *   dp_j(t) = sum_k short_w[j][k] ds_j(t + k),  dshort_w[j][k] = sum_{b,t} ds_j(t) p_j(t - k)
 *   du = dp W_in^T,  dW_in = sum_b u_b^T dp_b,   ds = (dz^1, dx^1 .. dx^N)
 * The correlations run through the layer's cached filter spectra: conjugated
 * in the on-chip regime (L <= 4096); beyond it, through the forward's
 * four-step passes as R conv R with R the time reversal on [0, L), and dh^n as
 * the convolution of R(g x^n) with z^n taken as a filter, transformed per
 * sample (negative lags: R z^n with g x^n as the filter). Supported: L a power
 * of two in [32, 2^20], both directions; D, N and B as hyena_fwd. Every
 * gradient is recomputed from the
 * inputs (nothing is kept from a forward call). The batch sums are taken in a
 * fixed order, so results are bit-reproducible.
 */
size_t hyena_bwd_workspace_bytes(int B, int L, int D, int N, int dtype, int direction);

/* Inputs as hyena_fwd, plus
 *   dy       [B][L][D]      dtype, gradient of the loss with respect to y
 * Outputs (overwritten, not accumulated into):
 *   du       [B][L][D]      dtype
 *   dw_in    [D][(N+1)*D]   fp32
 *   dshort_w [(N+1)*D][3]   fp32
 *   ddskip   [N][D]         fp32
 *   dw_out   [D][D]         fp32
 *   dh       [N][D][L] fp32 (causal) or the wrapped [N][D][2L] of h_out
 *            (non-causal; entry L, no filter tap, is 0): gradient with respect
 *            to the filters h^n; hyena_filter_bwd carries it to the generator's
 *            parameters.
 *   ws       scratch of hyena_bwd_workspace_bytes(B, L, D, N, dtype, layer->direction)
 * The layer must be built (hyena_filter_gen) for the same (L, D, N). */
int hyena_bwd(const hyena_layer *layer, const void *u, const void *w_in, const float *short_w,
              const float *dskip, const void *w_out, const void *dy, int B, int dtype,
              void *du, float *dw_in, float *dshort_w, float *ddskip, float *dw_out, float *dh,
              void *ws, size_t ws_bytes, hipStream_t stream);

/* Scratch for hyena_filter_bwd; 0 for unsupported sizes (those of hyena_cache_bytes;
 * 1 <= pe_freqs <= 32; width a multiple of 16 in [16, 128]) or directions. */
size_t hyena_filter_bwd_workspace_bytes(int L, int D, int N, int pe_freqs, int width, int direction);

/* Gradients of sum(dh * h) with respect to the generator's parameters, h as
 * hyena_filter_gen evaluates it for the layer's direction (dh in h_out's layout):
 *   dw1 [1+2K][W], db1 [W], dw2 [W][W], db2 [W], dw3 [W][N*D], db3 [N*D], ddecay [D]
 * all fp32, overwritten. p: the parameters the filters were generated from. */
int hyena_filter_bwd(const hyena_layer *layer, const hyena_filter_params *p, const float *dh,
                     float *dw1, float *db1, float *dw2, float *db2, float *dw3, float *db3, float *ddecay,
                     void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ 3D ---- */
/*
 * HyenaND on 3D grids (HyenaND explainer, gist.science, "Methodology: HyenaND"):
 * a global convolution on the native grid through a 3D FFT, non-circular by zero
 * padding to twice the grid ("Handling Boundaries"), with a coordinate-MLP kernel
 * times a window ("Kernel Synthesis") whose scale depends on the whole sample
 * ("Input-Dependent Kernels"). Here:
 *   K^n_c(d) = exp(-decay_c |c|_2) * (W3^T sin(W2^T sin(W1^T c + b1) + b2) + b3)[(n-1)C + c]
 *     at coordinates c = (dx/X, dy/Y, dz/Z) of the offsets d in [-X,X)x[-Y,Y)x[-Z,Z);
 *   g^n_{b,c} = sigmoid(gate_a[n][c] * mean_grid(u[b,...,c]) + gate_b[n][c]);
 *   (K conv z)[p] = sum_{q in grid} g * K[p - q] z[q];
 *   the same projection / gating recurrence as 1D, without the short convolution.
 */
typedef struct {
  int width;     /* W, 1 <= W <= 128 */
  const float *w1, *b1, *w2, *b2, *w3, *b3, *decay;  /* [3][W],[W],[W][W],[W],[W][N*C],[N*C],[C] */
} hyena_nd_filter_params;

/* Boundary of the convolution ("Handling Boundaries" names both kinds):
 *   HYENA_ND_ZERO_PAD  non-circular, as above (the default; transform (2X, 2Y, 2Z));
 *   HYENA_ND_CIRCULAR  periodic grids: the kernel covers one period, offsets
 *                      d in [-X/2,X/2)x[-Y/2,Y/2)x[-Z/2,Z/2) at coordinates
 *                      c = (2dx/X, 2dy/Y, 2dz/Z), and
 *                      (K conv z)[p] = sum_{q in grid} g * K[(p - q) mod (X,Y,Z)] z[q]
 *                      for every p, through an unpadded (X, Y, Z) transform.
 * In both modes the coordinates span [-1, 1) over the kernel's support. */
typedef enum { HYENA_ND_ZERO_PAD = 0, HYENA_ND_CIRCULAR = 1 } hyena_nd_boundary;

typedef struct {
  int X, Y, Z, C, N;
  int built;
  void *cache;
  size_t cache_bytes;
  int boundary;  /* hyena_nd_boundary, set by the init call */
} hyena_nd_layer;

/* Supported: X, Y, Z powers of two, each on its own, in [4, 64] (zero padded)
 * or in [8, 128] (circular); C a multiple of 64 in [64, 4096]; 1 <= N <= 4;
 * B >= 1. The size queries return 0 for unsupported shapes or boundaries. The
 * calls without _ex are the zero-padded boundary.
 * X = 1 is a 2D grid (Y x Z; "Native ND Convolution" covers any dimension):
 * every offset has dx = 0 (coordinate 0, so the x row of w1 does not act), the
 * x axis is never padded, and u, y [B][1][Y][Z][C] are the same memory as
 * [B][Y][Z][C]. All orders of a 2D grid run in one launch. */
size_t hyena_nd_cache_bytes(int X, int Y, int Z, int C, int N);
size_t hyena_nd_filter_workspace_bytes(int X, int Y, int Z, int C, int N);
size_t hyena_nd_workspace_bytes(int B, int X, int Y, int Z, int C, int N);
size_t hyena_nd_cache_bytes_ex(int X, int Y, int Z, int C, int N, int boundary);
size_t hyena_nd_filter_workspace_bytes_ex(int X, int Y, int Z, int C, int N, int boundary);
size_t hyena_nd_workspace_bytes_ex(int B, int X, int Y, int Z, int C, int N, int boundary);

int hyena_nd_layer_init(hyena_nd_layer *layer, int X, int Y, int Z, int C, int N,
                        void *cache, size_t cache_bytes);
/* As hyena_nd_layer_init with a boundary; HYENA_ERR_UNSUPPORTED for an unknown
 * boundary or a shape outside its range. The cache must hold
 * hyena_nd_cache_bytes_ex(..., boundary) bytes. */
int hyena_nd_layer_init_ex(hyena_nd_layer *layer, int X, int Y, int Z, int C, int N, int boundary,
                           void *cache, size_t cache_bytes);

/* Evaluates K^n_c on the layer's (MX, MY, MZ) offset grid, (2X, 2Y, 2Z) zero padded
 * or (X, Y, Z) circular, and caches its 3D spectrum. If k_out is not NULL the
 * kernel is also written there as fp32 [N][C][MX][MY][MZ], entry [i][j][k] at
 * offset (i - MX/2, j - MY/2, k - MZ/2). ws must hold
 * hyena_nd_filter_workspace_bytes_ex(..., layer->boundary) bytes. */
int hyena_nd_filter_gen(hyena_nd_layer *layer, const hyena_nd_filter_params *p, float *k_out,
                        void *ws, size_t ws_bytes, hipStream_t stream);

/* Forward pass, fp32, with the layer's boundary:
 *   u, y [B][X][Y][Z][C]; w_in [C][(N+1)C]; dskip, gate_a, gate_b [N][C]; w_out [C][C].
 * ws must hold hyena_nd_workspace_bytes_ex(B, ..., layer->boundary) bytes. */
int hyena_nd_fwd(const hyena_nd_layer *layer, const float *u, const float *w_in,
                 const float *dskip, const float *gate_a, const float *gate_b,
                 const float *w_out, int B, float *y, void *ws, size_t ws_bytes,
                 hipStream_t stream);

/* Same launches as hyena_nd_fwd, plus hipEventRecord(events[i], stream) at the four
 * stage boundaries, for timing the stages on the launch stream:
 *   events[0] before the channel means and gates,
 *   events[1] after the in-projection (gates, weight transposes, GEMM),
 *   events[2] after the 3D FFT convolutions with gating (all orders),
 *   events[3] after the out-projection.
 * events: host array of 4 events the caller created (and destroys); nothing here
 * synchronises. A null `events` is HYENA_ERR_INVALID_ARG. */
int hyena_nd_fwd_profiled(const hyena_nd_layer *layer, const float *u, const float *w_in,
                          const float *dskip, const float *gate_a, const float *gate_b,
                          const float *w_out, int B, float *y, void *ws, size_t ws_bytes,
                          hipStream_t stream, const hipEvent_t *events);

/* ------------------------------------------------- 3D, register-conditioned ---- */
/*
 * HyenaND with the page's own input conditioning (HyenaND explainer,
 * gist.science, "Methodology: HyenaND": Input-Dependent Kernels via Registers
 * and FiLM; Kernel Synthesis; Kernel Parameterization). Per sample b, with the
 * R register activations reg[b] [R][C] (the layer input at the register tokens):
 *   w_r  = softmax over r of (reg[b][r] . q),  z = sum_r w_r reg[b][r]
 *   gamma_l = film_w[2l-2]^T z + film_b[2l-2],  beta_l = film_w[2l-1]^T z + film_b[2l-1]
 *   h_1 = sin(omega0 * gamma_1 * (W1^T c + b1) + beta_1)
 *   h_2 = sin(gamma_2 * (W2^T h_1 + b2) + beta_2)
 *   K^n_{b,c}(d) = exp(-a_c |c|^2) * (W3^T h_2 + b3)[(n-1)C + c]   (Gaussian window,
 *                  a = hyena_nd_filter_params.decay)
 * at the offsets and coordinates of the boundary (as hyena_nd_filter_gen), then
 * the projection / recurrence of hyena_nd_fwd, each sample convolved with its own
 * kernel and no channel-mean gate. The page gives the parts and their order,
 * not these formulas: they are the plainest reading of it. The kernels depend on
 * the input, so every call synthesises and transforms B of them.
 */
typedef struct {
  int registers;        /* R, 1 <= R <= 1024 */
  const float *q;       /* [C]     register score vector */
  const float *film_w;  /* [4][C][W]  gamma_1, beta_1, gamma_2, beta_2 maps of z */
  const float *film_b;  /* [4][W] */
  const float *omega0;  /* [W]     first-layer frequency factors */
} hyena_nd_film_params;

/* Scratch for hyena_nd_film_fwd: the hyena_nd_fwd workspace, B kernel spectra
 * (B N C MX MY (MZ/2+1) complex fp32), one kernel's synthesis buffers and the
 * FiLM vectors. 0 for unsupported shapes (those of hyena_nd_workspace_bytes_ex,
 * 1 <= width <= 128). */
size_t hyena_nd_film_workspace_bytes(int B, int X, int Y, int Z, int C, int N, int width, int boundary);

/* Forward pass of the register-conditioned layer. Shapes as hyena_nd_fwd, plus
 *   p       SIREN weights (width W) and, in `decay`, the Gaussian window rates [C]
 *   fp      register scoring and FiLM maps
 *   reg     [B][R][C] fp32 register activations
 *   k_out   NULL, or [B][N][C][MX][MY][MZ] fp32 receiving every sample's kernel on
 *           the offset grid (as hyena_nd_filter_gen's k_out)
 *   ws      scratch of hyena_nd_film_workspace_bytes(B, X, Y, Z, C, N, p->width, boundary)
 * Pointers 16-byte aligned; y may not alias the inputs. Errors as hyena_nd_fwd. */
int hyena_nd_film_fwd(int X, int Y, int Z, int C, int N, int boundary, const hyena_nd_filter_params *p,
                      const hyena_nd_film_params *fp, const float *u, const float *reg, const float *w_in,
                      const float *dskip, const float *w_out, int B, float *y, float *k_out, void *ws,
                      size_t ws_bytes, hipStream_t stream);

/* Same launches plus hipEventRecord(events[i], stream) at five points: [0] before
 * the kernel synthesis, [1] after it (FiLM vectors, B MLP evaluations and 3D
 * FFTs), [2] after the in-projection, [3] after the convolutions, [4] after the
 * out-projection. A null `events` is HYENA_ERR_INVALID_ARG. */
int hyena_nd_film_fwd_profiled(int X, int Y, int Z, int C, int N, int boundary, const hyena_nd_filter_params *p,
                               const hyena_nd_film_params *fp, const float *u, const float *reg,
                               const float *w_in, const float *dskip, const float *w_out, int B, float *y,
                               float *k_out, void *ws, size_t ws_bytes, hipStream_t stream,
                               const hipEvent_t *events);

#ifdef __cplusplus
}
#endif
#endif /* HYENA_H */
