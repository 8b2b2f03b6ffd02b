/*
 * Host-side checks of libhyena's C ABI, compiled as C (the header must be
 * usable from C) and linked against the library's host code built with
 * AddressSanitizer and UndefinedBehaviorSanitizer (any finding aborts).
 *
 * Size queries are swept over in-range, boundary and extreme arguments (INT_MIN,
 * INT_MAX, ...), and every entry point is called with arguments it must reject.
 * No call here reaches the GPU: apart from the size queries, each call carries
 * at least one argument that the library rejects before its first HIP call.
 * Pointers are host addresses that are never dereferenced as device memory.
 *
 * Exit status 0 when every expectation holds; the failures are printed.
 */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "hyena.h"

static int failures = 0;

#define EXPECT_EQ(expr, want)                                                                   \
  do {                                                                                          \
    long long got_ = (long long)(expr), want_ = (long long)(want);                              \
    if (got_ != want_) {                                                                        \
      fprintf(stderr, "%s:%d: %s = %lld, expected %lld\n", __FILE__, __LINE__, #expr, got_, want_); \
      ++failures;                                                                               \
    }                                                                                           \
  } while (0)

#define EXPECT_TRUE(cond, ...)                      \
  do {                                              \
    if (!(cond)) {                                  \
      fprintf(stderr, "%s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                 \
      fprintf(stderr, "\n");                        \
      ++failures;                                   \
    }                                               \
  } while (0)

static const int kSizes[] = {INT_MIN, -64, -1, 0, 1, 2, 3, 4, 8, 15, 16, 24, 32, 64, 96, 128,
                             256, 4096, 8192, 8256, 65536, 1 << 20, 1 << 21, INT_MAX};
#define NSIZES ((int)(sizeof(kSizes) / sizeof(kSizes[0])))
static const int kSmall[] = {INT_MIN, -1, 0, 1, 2, 4, 5, INT_MAX};
#define NSMALL ((int)(sizeof(kSmall) / sizeof(kSmall[0])))

static int pow2_in(long long x, long long lo, long long hi) {
  return x >= lo && x <= hi && (x & (x - 1)) == 0;
}

/* The supported 1D shapes as the header states them. */
static int shape_1d(int L, int D, int N) {
  return pow2_in(L, 16, 1 << 20) && D >= 64 && D <= 8192 && D % 64 == 0 && N >= 1 && N <= 4;
}

/* B*L*(N+1)*D < 2^31 without forming the product. */
static int fits_1d(int B, int L, int D, int N) {
  const long long per = (long long)L * (N + 1) * D;
  return B >= 1 && (long long)B <= ((1LL << 31) - 1) / per;
}

static void sweep_1d_sizes(void) {
  for (int i = 0; i < NSIZES; ++i)
    for (int j = 0; j < NSIZES; ++j)
      for (int k = 0; k < NSMALL; ++k) {
        const int L = kSizes[i], D = kSizes[j], N = kSmall[k];
        const int ok = shape_1d(L, D, N);
        const size_t cache = hyena_cache_bytes(L, D, N);
        EXPECT_TRUE((cache > 0) == ok, "hyena_cache_bytes(%d, %d, %d) = %zu", L, D, N, cache);
        for (int dir = -1; dir <= 2; ++dir) {
          const size_t f = hyena_filter_workspace_bytes_ex(L, D, N, dir);
          EXPECT_TRUE((f > 0) == (ok && (dir == 0 || dir == 1)), "filter ws (%d, %d, %d, dir %d) = %zu", L, D, N,
                      dir, f);
          for (int pe = 0; pe <= 33; pe += 11)
            for (int w = 0; w <= 144; w += 24) {
              const size_t fb = hyena_filter_bwd_workspace_bytes(L, D, N, pe, w, dir);
              const int fb_ok = ok && (dir == 0 || dir == 1) && pe >= 1 && pe <= 32 && w >= 16 && w <= 128 &&
                                w % 16 == 0;
              EXPECT_TRUE((fb > 0) == fb_ok, "filter bwd ws (%d, %d, %d, %d, %d, dir %d) = %zu", L, D, N, pe, w,
                          dir, fb);
            }
        }
        EXPECT_EQ(hyena_filter_workspace_bytes(L, D, N), hyena_filter_workspace_bytes_ex(L, D, N, HYENA_CAUSAL));
        for (int b = 0; b < NSIZES; ++b) {
          const int B = kSizes[b];
          for (int dt = -1; dt <= 2; ++dt) {
            const int fwd_ok = ok && (dt == 0 || dt == 1) && fits_1d(B, L, D, N);
            const size_t ws = hyena_workspace_bytes(B, L, D, N, dt);
            EXPECT_TRUE((ws > 0) == fwd_ok, "hyena_workspace_bytes(%d, %d, %d, %d, %d) = %zu", B, L, D, N, dt, ws);
            for (int dir = -1; dir <= 2; ++dir) {
              const int bwd_ok = fwd_ok && L >= 32 && (dir == 0 || dir == 1);
              const size_t bw = hyena_bwd_workspace_bytes(B, L, D, N, dt, dir);
              EXPECT_TRUE((bw > 0) == bwd_ok, "hyena_bwd_workspace_bytes(%d, %d, %d, %d, %d, %d) = %zu", B, L, D,
                          N, dt, dir, bw);
            }
          }
        }
      }
}

/* The supported 3D / 2D shapes as the header states them. */
static int shape_nd(int X, int Y, int Z, int C, int N, int bd) {
  if (bd != HYENA_ND_ZERO_PAD && bd != HYENA_ND_CIRCULAR) return 0;
  const int lo = bd == HYENA_ND_CIRCULAR ? 8 : 4, hi = bd == HYENA_ND_CIRCULAR ? 128 : 64;
  const int axes = (X == 1 || pow2_in(X, lo, hi)) && pow2_in(Y, lo, hi) && pow2_in(Z, lo, hi);
  return axes && C >= 64 && C <= 4096 && C % 64 == 0 && N >= 1 && N <= 4;
}

static int fits_nd(int B, int X, int Y, int Z, int C, int N) {
  const long long per = (long long)X * Y * Z * (N + 1) * C;
  return B >= 1 && (long long)B <= ((1LL << 31) - 1) / per;
}

static void sweep_nd_sizes(void) {
  static const int axes[] = {INT_MIN, -8, 0, 1, 2, 4, 8, 12, 16, 32, 64, 128, 256, INT_MAX};
  static const int chans[] = {INT_MIN, 0, 32, 64, 96, 128, 4096, 4160, INT_MAX};
  static const int batches[] = {INT_MIN, -1, 0, 1, 2, 3, 1 << 16, INT_MAX};
  const int na = (int)(sizeof(axes) / sizeof(axes[0]));
  const int nc = (int)(sizeof(chans) / sizeof(chans[0]));
  const int nb = (int)(sizeof(batches) / sizeof(batches[0]));
  for (int x = 0; x < na; ++x)
    for (int y = 0; y < na; ++y)
      for (int z = 0; z < na; ++z)
        for (int c = 0; c < nc; ++c)
          for (int n = 0; n < NSMALL; n += 2)
            for (int bd = -1; bd <= 2; ++bd) {
              const int X = axes[x], Y = axes[y], Z = axes[z], C = chans[c], N = kSmall[n];
              const int ok = shape_nd(X, Y, Z, C, N, bd);
              const size_t cache = hyena_nd_cache_bytes_ex(X, Y, Z, C, N, bd);
              EXPECT_TRUE((cache > 0) == ok, "nd cache (%d, %d, %d, %d, %d, bd %d) = %zu", X, Y, Z, C, N, bd, cache);
              const size_t f = hyena_nd_filter_workspace_bytes_ex(X, Y, Z, C, N, bd);
              EXPECT_TRUE((f > 0) == ok, "nd filter ws (%d, %d, %d, %d, %d, bd %d) = %zu", X, Y, Z, C, N, bd, f);
              if (bd == HYENA_ND_ZERO_PAD) {
                EXPECT_EQ(hyena_nd_cache_bytes(X, Y, Z, C, N), cache);
                EXPECT_EQ(hyena_nd_filter_workspace_bytes(X, Y, Z, C, N), f);
              }
              for (int b = 0; b < nb; ++b) {
                const int B = batches[b];
                const int fwd_ok = ok && fits_nd(B, X, Y, Z, C, N);
                const size_t ws = hyena_nd_workspace_bytes_ex(B, X, Y, Z, C, N, bd);
                EXPECT_TRUE((ws > 0) == fwd_ok, "nd ws (%d; %d, %d, %d, %d, %d, bd %d) = %zu", B, X, Y, Z, C, N,
                            bd, ws);
                if (bd == HYENA_ND_ZERO_PAD) EXPECT_EQ(hyena_nd_workspace_bytes(B, X, Y, Z, C, N), ws);
                for (int w = -1; w <= 129; w += 65) {
                  const size_t fw = hyena_nd_film_workspace_bytes(B, X, Y, Z, C, N, w, bd);
                  EXPECT_TRUE((fw > 0) == (fwd_ok && w >= 1 && w <= 128), "film ws (%d; %d, %d, %d, %d, %d, w %d) = %zu",
                              B, X, Y, Z, C, N, w, fw);
                }
              }
            }
}

/* 16-byte aligned host memory standing in for device buffers: never read. */
static _Alignas(256) unsigned char arena[4096];

static void checks_1d(void) {
  void *P = arena, *M = arena + 4;  /* aligned / misaligned */
  float *F = (float *)(void *)arena, *FM = (float *)(void *)(arena + 4);
  const int L = 1024, D = 64, N = 2;
  const size_t cache = hyena_cache_bytes(L, D, N);
  EXPECT_TRUE(cache > 0, "cache bytes");

  EXPECT_TRUE(strcmp(hyena_status_str(HYENA_OK), "ok") == 0, "status 0");
  for (int s = -2; s <= 8; ++s) EXPECT_TRUE(hyena_status_str(s) != NULL, "status string %d", s);
  EXPECT_TRUE(hyena_status_str(INT_MIN) != NULL && hyena_status_str(INT_MAX) != NULL, "extreme status strings");

  hyena_layer layer;
  memset(&layer, 0, sizeof(layer));
  EXPECT_EQ(hyena_layer_init(NULL, L, D, N, P, cache), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_layer_init(&layer, 1000, D, N, P, cache), HYENA_ERR_UNSUPPORTED);
  EXPECT_EQ(hyena_layer_init(&layer, INT_MIN, INT_MIN, INT_MIN, P, cache), HYENA_ERR_UNSUPPORTED);
  EXPECT_EQ(hyena_layer_init_ex(&layer, L, D, N, 2, P, cache), HYENA_ERR_UNSUPPORTED);
  EXPECT_EQ(hyena_layer_init_ex(&layer, L, D, N, -1, P, cache), HYENA_ERR_UNSUPPORTED);
  EXPECT_EQ(hyena_layer_init(&layer, L, D, N, NULL, cache), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_layer_init(&layer, L, D, N, M, cache), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_layer_init(&layer, L, D, N, P, cache - 1), HYENA_ERR_WORKSPACE);
  EXPECT_EQ(hyena_layer_init(&layer, L, D, N, P, cache), HYENA_OK);
  EXPECT_EQ(layer.built, 0);
  EXPECT_EQ(layer.direction, HYENA_CAUSAL);

  /* filter generation: bad parameter structs and workspace */
  hyena_filter_params fp;
  memset(&fp, 0, sizeof(fp));
  fp.pe_freqs = 8;
  fp.width = 64;
  fp.w1 = fp.b1 = fp.w2 = fp.b2 = fp.w3 = fp.b3 = fp.decay = F;
  const size_t fws = hyena_filter_workspace_bytes(L, D, N);
  EXPECT_EQ(hyena_filter_gen(NULL, &fp, NULL, P, fws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_filter_gen(&layer, NULL, NULL, P, fws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_filter_gen(&layer, &fp, NULL, P, fws - 1, NULL), HYENA_ERR_WORKSPACE);
  EXPECT_EQ(hyena_filter_gen(&layer, &fp, FM, P, fws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_filter_gen(&layer, &fp, NULL, M, fws, NULL), HYENA_ERR_INVALID_ARG);
  {
    hyena_filter_params bad = fp;
    bad.pe_freqs = 0;
    EXPECT_EQ(hyena_filter_gen(&layer, &bad, NULL, P, fws, NULL), HYENA_ERR_UNSUPPORTED);
    bad.pe_freqs = INT_MAX;
    EXPECT_EQ(hyena_filter_gen(&layer, &bad, NULL, P, fws, NULL), HYENA_ERR_UNSUPPORTED);
    bad = fp;
    bad.width = 129;
    EXPECT_EQ(hyena_filter_gen(&layer, &bad, NULL, P, fws, NULL), HYENA_ERR_UNSUPPORTED);
    bad = fp;
    bad.w3 = NULL;
    EXPECT_EQ(hyena_filter_gen(&layer, &bad, NULL, P, fws, NULL), HYENA_ERR_INVALID_ARG);
    bad = fp;
    bad.decay = FM;
    EXPECT_EQ(hyena_filter_gen(&layer, &bad, NULL, P, fws, NULL), HYENA_ERR_INVALID_ARG);
  }
  {
    hyena_layer small = layer;
    small.cache_bytes = cache - 1;
    EXPECT_EQ(hyena_filter_gen(&small, &fp, NULL, P, fws, NULL), HYENA_ERR_WORKSPACE);
    small = layer;
    small.L = 3;
    EXPECT_EQ(hyena_filter_gen(&small, &fp, NULL, P, fws, NULL), HYENA_ERR_UNSUPPORTED);
    small = layer;
    small.direction = 7;
    EXPECT_EQ(hyena_filter_gen(&small, &fp, NULL, P, fws, NULL), HYENA_ERR_UNSUPPORTED);
  }

  /* forward (plain, profiled, allocation-free): the layer is not built yet */
  const size_t ws = hyena_workspace_bytes(1, L, D, N, HYENA_F32);
  EXPECT_EQ(hyena_fwd(&layer, P, P, F, F, P, 1, HYENA_F32, P, P, ws, NULL), HYENA_ERR_LAYER_MISMATCH);
  EXPECT_EQ(hyena_fwd_noalloc(&layer, P, P, F, F, P, 1, HYENA_F32, P, NULL), HYENA_ERR_LAYER_MISMATCH);
  hyena_layer built = layer;
  built.built = 1;
  EXPECT_EQ(hyena_fwd(NULL, P, P, F, F, P, 1, HYENA_F32, P, P, ws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_fwd(&built, NULL, P, F, F, P, 1, HYENA_F32, P, P, ws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_fwd(&built, P, M, F, F, P, 1, HYENA_F32, P, P, ws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_fwd(&built, P, P, FM, F, P, 1, HYENA_F32, P, P, ws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_fwd(&built, P, P, F, NULL, P, 1, HYENA_F32, P, P, ws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_fwd(&built, P, P, F, F, NULL, 1, HYENA_F32, P, P, ws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_fwd(&built, P, P, F, F, P, 1, HYENA_F32, NULL, P, ws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_fwd(&built, P, P, F, F, P, 1, HYENA_F32, P, NULL, ws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_fwd(&built, P, P, F, F, P, 1, 2, P, P, ws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_fwd(&built, P, P, F, F, P, 1, -1, P, P, ws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_fwd(&built, P, P, F, F, P, 0, HYENA_F32, P, P, ws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_fwd(&built, P, P, F, F, P, INT_MIN, HYENA_F32, P, P, ws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_fwd(&built, P, P, F, F, P, INT_MAX, HYENA_F32, P, P, ws, NULL), HYENA_ERR_UNSUPPORTED);
  EXPECT_EQ(hyena_fwd(&built, P, P, F, F, P, 1, HYENA_F32, P, P, ws - 1, NULL), HYENA_ERR_WORKSPACE);
  EXPECT_EQ(hyena_fwd(&built, P, P, F, F, P, 1, HYENA_F32, P, P, 0, NULL), HYENA_ERR_WORKSPACE);
  EXPECT_EQ(hyena_fwd_profiled(&built, P, P, F, F, P, 1, HYENA_F32, P, P, ws, NULL, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_fwd_noalloc(&built, P, P, F, F, P, INT_MAX, HYENA_F32, P, NULL), HYENA_ERR_UNSUPPORTED);
  EXPECT_EQ(hyena_fwd_noalloc(&built, P, P, F, F, P, 0, HYENA_F32, P, NULL), HYENA_ERR_INVALID_ARG);
  {
    /* a batch whose workspace exceeds the fixed scratch array, within the shape limits */
    int B = 1;
    while (hyena_workspace_bytes(B, L, D, N, HYENA_F32) <= HYENA_NOALLOC_SCRATCH_BYTES &&
           hyena_workspace_bytes(B + 1, L, D, N, HYENA_F32) > 0)
      ++B;
    if (hyena_workspace_bytes(B, L, D, N, HYENA_F32) > HYENA_NOALLOC_SCRATCH_BYTES)
      EXPECT_EQ(hyena_fwd_noalloc(&built, P, P, F, F, P, B, HYENA_F32, P, NULL), HYENA_ERR_WORKSPACE);
  }
  {
    hyena_layer other = built;
    other.D = 128;  /* the cache was sized for D = 64 */
    EXPECT_EQ(hyena_fwd(&other, P, P, F, F, P, 1, HYENA_F32, P, P, hyena_workspace_bytes(1, L, 128, N, 0), NULL),
              HYENA_ERR_LAYER_MISMATCH);
    other = built;
    other.cache = M;
    EXPECT_EQ(hyena_fwd(&other, P, P, F, F, P, 1, HYENA_F32, P, P, ws, NULL), HYENA_ERR_LAYER_MISMATCH);
  }

  /* backward */
  const size_t bws = hyena_bwd_workspace_bytes(1, L, D, N, HYENA_F32, HYENA_CAUSAL);
  EXPECT_EQ(hyena_bwd(&layer, P, P, F, F, P, P, 1, HYENA_F32, P, F, F, F, F, F, P, bws, NULL),
            HYENA_ERR_LAYER_MISMATCH);
  EXPECT_EQ(hyena_bwd(NULL, P, P, F, F, P, P, 1, HYENA_F32, P, F, F, F, F, F, P, bws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_bwd(&built, P, P, F, F, P, NULL, 1, HYENA_F32, P, F, F, F, F, F, P, bws, NULL),
            HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_bwd(&built, P, P, F, F, P, P, 1, HYENA_F32, P, F, F, F, F, FM, P, bws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_bwd(&built, P, P, F, F, P, P, 1, 5, P, F, F, F, F, F, P, bws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_bwd(&built, P, P, F, F, P, P, -3, HYENA_F32, P, F, F, F, F, F, P, bws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_bwd(&built, P, P, F, F, P, P, INT_MAX, HYENA_F32, P, F, F, F, F, F, P, bws, NULL),
            HYENA_ERR_UNSUPPORTED);
  EXPECT_EQ(hyena_bwd(&built, P, P, F, F, P, P, 1, HYENA_F32, P, F, F, F, F, F, P, bws - 1, NULL), HYENA_ERR_WORKSPACE);
  {
    hyena_layer longl = built;
    longl.L = 8192;  /* four-step regime: a larger workspace */
    longl.cache_bytes = hyena_cache_bytes(8192, D, N);
    longl.direction = 5;
    EXPECT_EQ(hyena_bwd(&longl, P, P, F, F, P, P, 1, HYENA_F32, P, F, F, F, F, F, P, bws, NULL),
              HYENA_ERR_UNSUPPORTED);
    longl.direction = HYENA_NONCAUSAL;
    EXPECT_EQ(hyena_bwd(&longl, P, P, F, F, P, P, 1, HYENA_F32, P, F, F, F, F, F, P, bws, NULL),
              HYENA_ERR_WORKSPACE);
    longl.direction = HYENA_CAUSAL;
    EXPECT_EQ(hyena_bwd(&longl, P, P, F, F, P, P, 1, HYENA_F32, P, F, F, F, F, F, P, bws, NULL),
              HYENA_ERR_WORKSPACE);
  }
  {
    hyena_filter_params bp = fp;
    bp.width = 64;
    const size_t fbws = hyena_filter_bwd_workspace_bytes(L, D, N, bp.pe_freqs, bp.width, HYENA_CAUSAL);
    EXPECT_TRUE(fbws > 0, "filter bwd ws");
    EXPECT_EQ(hyena_filter_bwd(NULL, &bp, F, F, F, F, F, F, F, F, P, fbws, NULL), HYENA_ERR_INVALID_ARG);
    EXPECT_EQ(hyena_filter_bwd(&built, NULL, F, F, F, F, F, F, F, F, P, fbws, NULL), HYENA_ERR_INVALID_ARG);
    EXPECT_EQ(hyena_filter_bwd(&built, &bp, NULL, F, F, F, F, F, F, F, P, fbws, NULL), HYENA_ERR_INVALID_ARG);
    EXPECT_EQ(hyena_filter_bwd(&built, &bp, F, F, F, F, F, F, F, FM, P, fbws, NULL), HYENA_ERR_INVALID_ARG);
    EXPECT_EQ(hyena_filter_bwd(&built, &bp, F, F, F, F, F, F, F, F, P, fbws - 1, NULL), HYENA_ERR_WORKSPACE);
    bp.width = 24;  /* not a multiple of 16 */
    EXPECT_EQ(hyena_filter_bwd(&built, &bp, F, F, F, F, F, F, F, F, P, fbws, NULL), HYENA_ERR_UNSUPPORTED);
  }
}

static void checks_nd(void) {
  float *F = (float *)(void *)arena, *FM = (float *)(void *)(arena + 4);
  void *P = arena;
  const int X = 8, Y = 16, Z = 32, C = 64, N = 2;
  const size_t cache = hyena_nd_cache_bytes(X, Y, Z, C, N);
  EXPECT_TRUE(cache > 0, "nd cache");
  hyena_nd_layer nd;
  memset(&nd, 0, sizeof(nd));
  EXPECT_EQ(hyena_nd_layer_init(NULL, X, Y, Z, C, N, P, cache), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_nd_layer_init(&nd, X, Y, 24, C, N, P, cache), HYENA_ERR_UNSUPPORTED);
  EXPECT_EQ(hyena_nd_layer_init(&nd, 2, Y, Z, C, N, P, cache), HYENA_ERR_UNSUPPORTED);  /* X = 2 is no grid */
  EXPECT_EQ(hyena_nd_layer_init_ex(&nd, X, Y, Z, C, N, 9, P, cache), HYENA_ERR_UNSUPPORTED);
  EXPECT_EQ(hyena_nd_layer_init(&nd, X, Y, Z, C, N, NULL, cache), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_nd_layer_init(&nd, X, Y, Z, C, N, P, cache - 1), HYENA_ERR_WORKSPACE);
  EXPECT_EQ(hyena_nd_layer_init(&nd, X, Y, Z, C, N, P, cache), HYENA_OK);
  EXPECT_EQ(nd.boundary, HYENA_ND_ZERO_PAD);

  hyena_nd_filter_params p;
  memset(&p, 0, sizeof(p));
  p.width = 32;
  p.w1 = p.b1 = p.w2 = p.b2 = p.w3 = p.b3 = p.decay = F;
  const size_t fws = hyena_nd_filter_workspace_bytes(X, Y, Z, C, N);
  EXPECT_EQ(hyena_nd_filter_gen(NULL, &p, NULL, P, fws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_nd_filter_gen(&nd, NULL, NULL, P, fws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_nd_filter_gen(&nd, &p, FM, P, fws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_nd_filter_gen(&nd, &p, NULL, P, fws - 1, NULL), HYENA_ERR_WORKSPACE);
  {
    hyena_nd_filter_params bad = p;
    bad.width = 0;
    EXPECT_EQ(hyena_nd_filter_gen(&nd, &bad, NULL, P, fws, NULL), HYENA_ERR_UNSUPPORTED);
    bad = p;
    bad.b2 = NULL;
    EXPECT_EQ(hyena_nd_filter_gen(&nd, &bad, NULL, P, fws, NULL), HYENA_ERR_INVALID_ARG);
  }

  const size_t ws = hyena_nd_workspace_bytes(1, X, Y, Z, C, N);
  EXPECT_EQ(hyena_nd_fwd(&nd, F, F, F, F, F, F, 1, F, P, ws, NULL), HYENA_ERR_LAYER_MISMATCH);
  hyena_nd_layer built = nd;
  built.built = 1;
  EXPECT_EQ(hyena_nd_fwd(NULL, F, F, F, F, F, F, 1, F, P, ws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_nd_fwd(&built, F, F, F, NULL, F, F, 1, F, P, ws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_nd_fwd(&built, F, F, F, F, F, F, 1, FM, P, ws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_nd_fwd(&built, F, F, F, F, F, F, 0, F, P, ws, NULL), HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_nd_fwd(&built, F, F, F, F, F, F, INT_MAX, F, P, ws, NULL), HYENA_ERR_UNSUPPORTED);
  EXPECT_EQ(hyena_nd_fwd(&built, F, F, F, F, F, F, 1, F, P, ws - 1, NULL), HYENA_ERR_WORKSPACE);
  EXPECT_EQ(hyena_nd_fwd_profiled(&built, F, F, F, F, F, F, 1, F, P, ws, NULL, NULL), HYENA_ERR_INVALID_ARG);
  {
    hyena_nd_layer other = built;
    other.boundary = 5;
    EXPECT_EQ(hyena_nd_fwd(&other, F, F, F, F, F, F, 1, F, P, ws, NULL), HYENA_ERR_UNSUPPORTED);
    other = built;
    other.cache_bytes = cache - 1;
    EXPECT_EQ(hyena_nd_fwd(&other, F, F, F, F, F, F, 1, F, P, ws, NULL), HYENA_ERR_LAYER_MISMATCH);
  }

  hyena_nd_film_params fp;
  memset(&fp, 0, sizeof(fp));
  fp.registers = 4;
  fp.q = fp.film_w = fp.film_b = fp.omega0 = F;
  const size_t fw = hyena_nd_film_workspace_bytes(2, X, Y, Z, C, N, p.width, HYENA_ND_ZERO_PAD);
  EXPECT_TRUE(fw > ws, "film workspace holds the forward's");
  EXPECT_EQ(hyena_nd_film_fwd(X, Y, Z, C, N, 0, NULL, &fp, F, F, F, F, F, 2, F, NULL, P, fw, NULL),
            HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_nd_film_fwd(X, Y, Z, C, N, 0, &p, NULL, F, F, F, F, F, 2, F, NULL, P, fw, NULL),
            HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_nd_film_fwd(X, Y, Z, C, N, 0, &p, &fp, F, F, F, F, F, 2, F, FM, P, fw, NULL),
            HYENA_ERR_INVALID_ARG);
  EXPECT_EQ(hyena_nd_film_fwd(X, Y, Z, C, N, 0, &p, &fp, F, F, F, F, F, 2, F, NULL, P, fw - 1, NULL),
            HYENA_ERR_WORKSPACE);
  EXPECT_EQ(hyena_nd_film_fwd(X, Y, Z, C, N, 0, &p, &fp, F, F, F, F, F, INT_MAX, F, NULL, P, fw, NULL),
            HYENA_ERR_UNSUPPORTED);
  EXPECT_EQ(hyena_nd_film_fwd(X, Y, Z, C, N, 3, &p, &fp, F, F, F, F, F, 2, F, NULL, P, fw, NULL),
            HYENA_ERR_UNSUPPORTED);
  {
    hyena_nd_film_params bad = fp;
    bad.registers = 0;
    EXPECT_EQ(hyena_nd_film_fwd(X, Y, Z, C, N, 0, &p, &bad, F, F, F, F, F, 2, F, NULL, P, fw, NULL),
              HYENA_ERR_UNSUPPORTED);
    bad.registers = 1025;
    EXPECT_EQ(hyena_nd_film_fwd(X, Y, Z, C, N, 0, &p, &bad, F, F, F, F, F, 2, F, NULL, P, fw, NULL),
              HYENA_ERR_UNSUPPORTED);
    bad = fp;
    bad.omega0 = FM;
    EXPECT_EQ(hyena_nd_film_fwd(X, Y, Z, C, N, 0, &p, &bad, F, F, F, F, F, 2, F, NULL, P, fw, NULL),
              HYENA_ERR_INVALID_ARG);
  }
  EXPECT_EQ(hyena_nd_film_fwd_profiled(X, Y, Z, C, N, 0, &p, &fp, F, F, F, F, F, 2, F, NULL, P, fw, NULL, NULL),
            HYENA_ERR_INVALID_ARG);
}

int main(void) {
  sweep_1d_sizes();
  sweep_nd_sizes();
  checks_1d();
  checks_nd();
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("abi_check: all expectations hold\n");
  return 0;
}
