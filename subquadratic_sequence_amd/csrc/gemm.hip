// Dense projections of the Hyena operator on the MFMA units of gfx950.
//
// The in-projection (u [B*L][D] times W_in) and the out-projection
// (z [B][D][L] times W_out) are the only dense contractions of the operator.
// C = A * B with B supplied transposed (Bt [N][K], K contiguous) so that both
// MFMA operands are read from LDS as K-contiguous fragments.
//  * A_CM: A is channel-major [Bsz][K][Lseq] (the layout the long convolution
//    produces); tiles are loaded along M and transposed while stored to LDS.
//  * C_CM: C is written channel-major [Bsz][N][Lseq] (the layout the long
//    convolution consumes), staged through LDS for 16-byte stores.
//  * SC (with C_CM): the causal length-3 depthwise short convolution along the
//    sequence is applied in the epilogue, s_t = w0 p_t + w1 p_{t-1} + w2 p_{t-2}
//    (zero history at the start of every sequence). M-tiles then overlap by 8
//    rows: a tile computes rows [m0 - 8, m0 + 248) and writes [m0, m0 + 248), so
//    the two previous rows of every written row are on chip.
// Block tile 256 x 256, eight waves of 128 x 64 (8 accumulators of 32 x 32 per
// wave, two waves per SIMD), K step of 64 bytes per row; for N that 256 does
// not divide a 256 x 128 tile of eight waves of 64 x 64 wastes fewer MFMA
// columns, and fp32 products with a short K use 256 x 64 tiles (eight waves of
// 32 x 64, registers and LDS for two workgroups per CU). Three LDS tile
// buffers: while a step multiplies tile kt it already reads the first MMA
// fragments of tile kt + 1 (stored one step earlier) and stores tile kt + 2
// from registers, so that no step starts by waiting for all eight waves' LDS
// reads; global loads run three tiles ahead through two register sets. Tiles are numbered so that the
// workgroups dispatched to one XCD walk the N-tiles of one M-tile together
// (they share the A rows in that XCD's L2). bf16 storage uses v_mfma_f32_32x32x16_bf16, fp32 uses
// v_mfma_f32_32x32x2_f32; accumulation is fp32 in both cases.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hy {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int GBM = 256, GBN = 256;
constexpr int kScRows = GBM - 8;  // rows written per M-tile with the short-conv epilogue

template <typename T> struct GemmCfg {
  static constexpr int VEC = 16 / sizeof(T);    // elements per 16-byte chunk
  static constexpr int BK = 64 / sizeof(T);     // K elements per tile row (64 bytes)
  static constexpr int LDK = BK + VEC;          // padded LDS row (80 bytes)
  static constexpr int TILE = GBM * LDK;        // elements per operand tile
  static constexpr int CHUNKS = GBM * BK / VEC / 512;  // 16-byte chunks per thread per operand
};

// Wave layout of a GBM x TN block tile: TN / 64 wave columns of 64, the eight
// waves' rows split GBM (128 rows per wave for TN = 256, 64 for TN = 128).
template <int TN> struct WaveCfg {
  static constexpr int WCOLS = TN / 64;
  static constexpr int WR = GBM * WCOLS / 8;  // rows per wave
  static constexpr int MI = WR / 32;          // 32-row accumulator blocks per wave
};

constexpr int kCsLd = GBM + 4;  // staging row (floats), channel-major output: [RN n][256 m]
constexpr int kBufs = 3;                                 // LDS tile buffers
// staging of one epilogue round: RN = 128 columns (64 for 64-wide tiles) as
// [RN][kCsLd] (channel-major output) or [256][RN + 4] (row-major output)
constexpr size_t stage_bytes(int TN) {
  return TN >= 128 ? (128 * kCsLd * 4 > 256 * 132 * 4 ? 128 * kCsLd * 4 : 256 * 132 * 4)
                   : (64 * kCsLd * 4 > 256 * 68 * 4 ? 64 * kCsLd * 4 : 256 * 68 * 4);
}
// A (GBM rows) and B (TN rows) tiles per buffer, 80-byte rows; the epilogue
// staging reuses the space; then the short-conv taps of the tile's columns
constexpr size_t gemm_main_bytes(int TN) {
  return (size_t)kBufs * (GBM + TN) * 80 > stage_bytes(TN) ? (size_t)kBufs * (GBM + TN) * 80 : stage_bytes(TN);
}
constexpr size_t gemm_lds_bytes(int TN) { return gemm_main_bytes(TN) + (size_t)TN * 3 * 4; }

constexpr int kXcds = 8;

// tile number of workgroup `bid` when consecutive workgroups go round robin to
// the XCDs: XCD x receives the contiguous range of tile numbers it would get
// from a blocked split of [0, total)
__device__ __forceinline__ int xcd_tile(int bid, int total) {
  const int q = total / kXcds, r = total % kXcds;
  const int x = bid % kXcds, k = bid / kXcds;
  return x < r ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

template <typename T, bool A_CM, bool C_CM, bool SC, int TN = GBN>
__global__ __launch_bounds__(512, TN == 64 ? 4 : 1) void gemm_kernel(const T* __restrict__ A, const T* __restrict__ Bt,
                                                      T* __restrict__ C, int M, int N, int K, int Lseq,
                                                      const float* __restrict__ short_w, int ntn, int ntiles,
                                                      size_t sa, size_t sb, size_t sc, size_t ka, size_t kb,
                                                      int nsplit, int lda, int ldb) {
  using Cfg = GemmCfg<T>;
  using WC = WaveCfg<TN>;
  constexpr int BK = Cfg::BK, LDK = Cfg::LDK, VEC = Cfg::VEC, NCH = Cfg::CHUNKS;
  constexpr int BCH = TN * BK / VEC;             // 16-byte chunks of the B tile
  constexpr int NCHB = (BCH + 511) / 512;        // per thread (the last partly when BCH < 512)
  constexpr bool BPART = BCH % 512 != 0;
  constexpr int MI = WC::MI;
  extern __shared__ float4 smem4[];
  char* smem = reinterpret_cast<char*>(smem4);
  T* As0 = reinterpret_cast<T*>(smem);  // [kBufs][GBM][LDK] then Bs [kBufs][TN][LDK]
  T* Bs0 = As0 + kBufs * Cfg::TILE;

  {
    // product and K split of this grid row
    const int y = blockIdx.y, bz = y / nsplit, sz = y - bz * nsplit;
    A += bz * sa + sz * ka;
    Bt += bz * sb + sz * kb;
    C += (size_t)y * sc;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // waves of WR x 64; consecutive waves (which sit on different SIMDs) take
  // consecutive wave rows first, so that the waves staging one epilogue round
  // are spread over the four SIMDs
  constexpr int WROWS = 8 / WC::WCOLS;
  const int wm = wave % WROWS, wn = wave / WROWS;
  const int tile = xcd_tile(blockIdx.x, ntiles);
  const int tm = tile / ntn, tn = tile - tm * ntn;
  const int n0 = tn * TN;
  const int m0 = SC ? tm * kScRows - 8 : tm * GBM;  // first A row of the tile

  // short-conv taps of this tile's columns, staged once (read by the epilogue)
  float* sw = reinterpret_cast<float*>(smem + gemm_main_bytes(TN));
  if (SC) {
    for (int x = tid; x < TN * 3; x += 512) sw[x] = (n0 * 3 + x < N * 3) ? short_w[n0 * 3 + x] : 0.f;
  }

  f32x16 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  u32x4 ra2[2][NCH], rb2[2][NCH];  // two K tiles in flight
  // Per-thread global pointers, predicates and LDS offsets of the tile loads,
  // computed once; each K step only advances the pointers.
  const T* pa[NCH];
  const T* pb[NCH];
  int la[NCH], lb[NCH];
  size_t a_step;  // elements between consecutive K tiles
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + i * 512;
    const int row = c >> 2, kc = (c & 3) * VEC;
    if (!A_CM) {
      const int m = m0 + row;
      // rows outside [0, M) load row 0: they only feed output rows that are not
      // stored (with the short convolution, rows before a sequence start are
      // masked by position), and unconditional loads keep the compiler's count
      // of loads in flight exact
      pa[i] = A + (size_t)(m >= 0 && m < M ? m : 0) * lda + kc;
      la[i] = row * LDK + kc;
    } else {
      // chunks of VEC consecutive m for one k; ra[2j] and ra[2j + 1] hold
      // k = 2p and 2p + 1 of the same m chunk. Consecutive lanes take
      // consecutive k pairs (then chunks), so the interleaved LDS writes of
      // 16 lanes land on 16 consecutive words.
      constexpr int KP = BK / 2;  // k pairs per tile
      const int slot = tid + (i >> 1) * 512, hi = i & 1;
      const int k = 2 * (slot % KP) + hi, mc = (slot / KP) * VEC;
      const int m = m0 + mc;
      const int mm = m >= 0 && m < M ? m : 0;
      const int b = mm / Lseq, t = mm - b * Lseq;
      pa[i] = A + ((size_t)b * lda + k) * Lseq + t;
      la[i] = mc * LDK + (k & ~1);
    }
    if (i < NCHB) {
      const int n = n0 + (BPART && c >= BCH ? 0 : row);
      pb[i] = Bt + (size_t)(n < N ? n : 0) * ldb + kc;  // columns >= N are not stored
      lb[i] = row * LDK + kc;
    }
  }
  a_step = A_CM ? (size_t)BK * Lseq : (size_t)BK;

  // The register set is always a compile-time constant so that ra2/rb2 stay in VGPRs.
  // Loads and LDS stores are unconditional (past the last K tile the pointers
  // stay on it and the extra copies go unused): with no branch around them the
  // compiler waits for exactly the tile it stores, never for the one in flight.
  int tiles_left = K / BK;  // tiles from the current pointer position on
  auto load_tile = [&](auto set) {
    u32x4* ra = ra2[decltype(set)::value];
    u32x4* rb = rb2[decltype(set)::value];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      ra[i] = *reinterpret_cast<const u32x4*>(pa[i]);
      pa[i] += tiles_left > 1 ? a_step : 0;
      if (i < NCHB) {
        rb[i] = *reinterpret_cast<const u32x4*>(pb[i]);
        pb[i] += tiles_left > 1 ? BK : 0;
      }
    }
    --tiles_left;
  };
  // register set `set` -> LDS buffer `buf`
  auto store_tile = [&](auto set, auto bufc) {
    constexpr int sidx = decltype(set)::value, buf = decltype(bufc)::value;
    const u32x4* ra = ra2[sidx];
    const u32x4* rb = rb2[sidx];
    T* As = As0 + buf * Cfg::TILE;
    T* Bs = Bs0 + buf * (TN * LDK);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      if (!A_CM) {
        *reinterpret_cast<u32x4*>(As + la[i]) = ra[i];
      } else if (i % 2 == 0) {
        // ra[i] holds k = 2p, ra[i + 1] holds k = 2p + 1 for the same m chunk:
        // interleave them into 32-bit (bf16) or 64-bit (fp32) LDS writes
        // (register values only: no pointer into the register arrays, which
        // would send them to scratch)
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int q = 0; q < VEC; ++q) {
            const unsigned lo = (ra[i][q >> 1] >> (16 * (q & 1))) & 0xFFFFu;
            const unsigned hi = (ra[i + 1][q >> 1] >> (16 * (q & 1))) & 0xFFFFu;
            *reinterpret_cast<unsigned int*>(As + la[i] + q * LDK) = lo | (hi << 16);
          }
        } else {
#pragma unroll
          for (int q = 0; q < VEC; ++q)
            *reinterpret_cast<float2*>(As + la[i] + q * LDK) =
                make_float2(__uint_as_float(ra[i][q]), __uint_as_float(ra[i + 1][q]));
        }
      }
      if (i < NCHB && (!BPART || tid + i * 512 < BCH)) *reinterpret_cast<u32x4*>(Bs + lb[i]) = rb[i];
    }
  };

  // MMA fragments of one 16 (bf16) or 2 (fp32) wide K slice: MI of A, 2 of B
  using FragT = std::conditional_t<sizeof(T) == 2, bf16x8, float>;
  struct Frag {
    FragT a[MI], b[2];
  };
  const int ar = wm * WC::WR + (lane & 31), br = wn * 64 + (lane & 31);
  constexpr int KS = sizeof(T) == 2 ? 16 : 2;  // K per MMA
  auto read_frag = [&](Frag& f, int buf, int kk) {
    const T* As = As0 + buf * Cfg::TILE;
    const T* Bs = Bs0 + buf * (TN * LDK);
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
        f.a[i] = *reinterpret_cast<const bf16x8*>(As + (ar + i * 32) * LDK + kk + (lane >> 5) * 8);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        f.b[j] = *reinterpret_cast<const bf16x8*>(Bs + (br + j * 32) * LDK + kk + (lane >> 5) * 8);
    } else {
#pragma unroll
      for (int i = 0; i < MI; ++i) f.a[i] = As[(ar + i * 32) * LDK + kk + (lane >> 5)];
#pragma unroll
      for (int j = 0; j < 2; ++j) f.b[j] = Bs[(br + j * 32) * LDK + kk + (lane >> 5)];
    }
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (sizeof(T) == 2)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
      }
  };

  // Tile kt sits in LDS buffer kt % 3; it travels through register set kt & 1,
  // loaded three steps before it is multiplied and stored to LDS two steps
  // before. f0 holds the first K slice of the current tile on entry to a step.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  const int ktiles = K / BK;
  load_tile(S0{});
  store_tile(S0{}, std::integral_constant<int, 0>{});
  load_tile(S1{});
  store_tile(S1{}, std::integral_constant<int, 1>{});
  load_tile(S0{});
  __syncthreads();
  Frag f0;
  read_frag(f0, 0, 0);
  // step kt (compile-time phase P = kt % 6): multiply tile kt, read the first
  // slice of tile kt + 1, store tile kt + 2, fetch tile kt + 3
  auto step = [&](int kt, auto phase) {
    constexpr int P = decltype(phase)::value;
    constexpr int cur = P % 3, nxt = (P + 1) % 3, st = (P + 2) % 3;
    load_tile(std::integral_constant<int, (P + 1) & 1>{});  // tile kt + 3
    // keep the loads at the top of the step (the scheduler would otherwise sink
    // them toward their use and shorten the prefetch distance)
    __builtin_amdgcn_sched_barrier(0);
    if (kt < ktiles) {  // the steps past the last tile only move data
#pragma unroll
      for (int kk = 0; kk < BK; kk += KS) {
        Frag f;
        if (kk + KS < BK) read_frag(f, cur, kk + KS);
        else read_frag(f, nxt, 0);
        mma(f0);
        f0 = f;
      }
    }
    store_tile(std::integral_constant<int, P & 1>{}, std::integral_constant<int, st>{});  // tile kt + 2
    __syncthreads();
  };
  // groups of six steps cover both periods (register set 2, LDS buffer 3); the
  // loads and stores stay unconditional, which keeps the compiler's count of
  // loads in flight exact
  for (int kt = 0; kt < ktiles; kt += 6) {
    step(kt, std::integral_constant<int, 0>{});
    step(kt + 1, std::integral_constant<int, 1>{});
    step(kt + 2, std::integral_constant<int, 2>{});
    step(kt + 3, std::integral_constant<int, 3>{});
    step(kt + 4, std::integral_constant<int, 4>{});
    step(kt + 5, std::integral_constant<int, 5>{});
  }

  // Epilogue. Accumulator element e of lane l in block (i, j):
  //   row = i*32 + (e/4)*8 + (l/32)*4 + e%4, col = j*32 + l%32 (within the wave tile).
  // One round per RN-column slice (the waves whose 64 columns lie in it stage
  // them in LDS as fp32); the slice is written with 16-byte stores.
  constexpr int HC = WC::WCOLS < 2 ? WC::WCOLS : 2;  // wave columns per round
  constexpr int RN = HC * 64;                         // columns per round
  constexpr int RLD = RN + 4;                         // staging row (floats), row-major output
  float* Cs = reinterpret_cast<float*>(smem);
  // channel-major output: every thread keeps one chunk of 8 consecutive m for
  // the whole epilogue (only its n varies), so its sequence and position are
  // computed once; with the short convolution the first chunk of every row
  // (the 8 overlap rows) is not written
  const int mc = (tid & 31) * 8;
  const int mg = m0 + mc;
  const bool m_ok = mg >= 0 && mg < M && (!SC || mc >= 8);
  size_t cbase = 0;
  int tq = 0;
  if (C_CM) {
    const int mm = m_ok ? mg : 0;
    const int bq = mm / Lseq;
    tq = mm - bq * Lseq;
    cbase = (size_t)bq * N * Lseq + tq;
  }
#pragma unroll
  for (int h = 0; h < WC::WCOLS / HC; ++h) {
    if (wn / HC == h) {
      const int nb = (wn % HC) * 64;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const int ml = wm * WC::WR + i * 32 + e4 * 8 + (lane >> 5) * 4;
            const int nl = nb + j * 32 + (lane & 31);
            const float4 q = make_float4(acc[i][j][4 * e4], acc[i][j][4 * e4 + 1], acc[i][j][4 * e4 + 2],
                                         acc[i][j][4 * e4 + 3]);
            if (C_CM) {
              // [n][m]: the four rows of a lane are contiguous
              *reinterpret_cast<float4*>(Cs + nl * kCsLd + ml) = q;
            } else {
              // [m][n]
              Cs[(ml + 0) * RLD + nl] = q.x;
              Cs[(ml + 1) * RLD + nl] = q.y;
              Cs[(ml + 2) * RLD + nl] = q.z;
              Cs[(ml + 3) * RLD + nl] = q.w;
            }
          }
    }
    __syncthreads();
    if (C_CM) {
      // RN rows (n) x 256 (m): 16 rows per pass of the workgroup
#pragma unroll
      for (int it = 0; it < RN / 16; ++it) {
        const int nl = (tid >> 5) + it * 16;
        const int n = n0 + h * RN + nl;
        if (m_ok && n < N) {
          T* dst = C + cbase + (size_t)n * Lseq;
          const float* src = Cs + nl * kCsLd + mc;
          const float4 s0 = *reinterpret_cast<const float4*>(src);
          const float4 s1 = *reinterpret_cast<const float4*>(src + 4);
          float o[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
          if (SC) {
            // mc >= 8 here, so the two previous rows are in the staged row;
            // chunks start on multiples of 8, so only tq == 0 starts a sequence
            const float* wn3 = sw + 3 * (n - n0);
            const float w0 = wn3[0], w1 = wn3[1], w2 = wn3[2];
            const float r1 = src[-1], r2 = src[-2];
            float prev1 = tq ? r1 : 0.f, prev2 = tq ? r2 : 0.f;
#pragma unroll
            for (int v = 0; v < 8; ++v) {
              const float cur = o[v];
              o[v] = w0 * cur + w1 * prev1 + w2 * prev2;
              prev2 = prev1;
              prev1 = cur;
            }
          }
          if constexpr (sizeof(T) == 2) {
            bf16x8 ob;
#pragma unroll
            for (int v = 0; v < 8; ++v) ob[v] = (__bf16)o[v];
            *reinterpret_cast<bf16x8*>(dst) = ob;
          } else {
            *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
          }
        }
      }
    } else {
      // 256 rows (m) x RN (n) in chunks of 8 consecutive n
      constexpr int CPR = RN / 8;  // chunks per row
#pragma unroll
      for (int it = 0; it < 256 * CPR / 512; ++it) {
        const int c = tid + it * 512;
        const int ml = c / CPR, nc = (c % CPR) * 8;
        const int m = m0 + ml, n = n0 + h * RN + nc;
        if (m >= 0 && m < M && n < N) {
          const float* src = Cs + ml * RLD + nc;
          const float4 s0 = *reinterpret_cast<const float4*>(src);
          const float4 s1 = *reinterpret_cast<const float4*>(src + 4);
          T* dst = C + (size_t)m * N + n;
          if constexpr (sizeof(T) == 2) {
            bf16x8 ob;
            ob[0] = (__bf16)s0.x; ob[1] = (__bf16)s0.y; ob[2] = (__bf16)s0.z; ob[3] = (__bf16)s0.w;
            ob[4] = (__bf16)s1.x; ob[5] = (__bf16)s1.y; ob[6] = (__bf16)s1.z; ob[7] = (__bf16)s1.w;
            *reinterpret_cast<bf16x8*>(dst) = ob;
          } else {
            *reinterpret_cast<float4*>(dst) = s0;
            *reinterpret_cast<float4*>(dst + 4) = s1;
          }
        }
      }
    }
    __syncthreads();
  }
}

template <typename T, int TN>
static hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.K <= 0 || g.K % GemmCfg<T>::BK != 0) return hipErrorInvalidValue;  // whole K tiles
  const bool sc = g.short_w != nullptr;
  const int mtiles = sc ? (g.M + kScRows - 1) / kScRows : (g.M + GBM - 1) / GBM;
  const int ntn = (g.N + TN - 1) / TN;
  const int ntiles = ntn * mtiles;
  if (g.batch < 1 || g.nsplit < 1) return hipErrorInvalidValue;
  dim3 grid(ntiles, g.batch * g.nsplit), block(512);
  const int lda = g.lda ? g.lda : g.K, ldb = g.ldb ? g.ldb : g.K;
  const T* A = static_cast<const T*>(g.A);
  const T* B = static_cast<const T*>(g.Bt);
  T* C = static_cast<T*>(g.C);
#define GEMM_LAUNCH(acm, ccm, scv)                                                                    \
  do {                                                                                                \
    auto fn = gemm_kernel<T, acm, ccm, scv, TN>;                                                      \
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize,   \
                                       (int)gemm_lds_bytes(TN));                                      \
    if (e != hipSuccess) return e;                                                                    \
    hipLaunchKernelGGL(fn, grid, block, gemm_lds_bytes(TN), s, A, B, C, g.M, g.N, g.K, g.Lseq,        \
                       g.short_w, ntn, ntiles, g.sa, g.sb, g.sc, g.ka, g.kb, g.nsplit, lda, ldb);       \
  } while (0)
  if (sc) {
    if (!g.c_cm || g.a_cm) return hipErrorInvalidValue;
    GEMM_LAUNCH(false, true, true);
  } else if (g.a_cm && g.c_cm) {
    GEMM_LAUNCH(true, true, false);
  } else if (g.a_cm) {
    GEMM_LAUNCH(true, false, false);
  } else if (g.c_cm) {
    GEMM_LAUNCH(false, true, false);
  } else {
    GEMM_LAUNCH(false, false, false);
  }
#undef GEMM_LAUNCH
  return hipGetLastError();
}

// fp32 with a short K (the 3D and 2D projections, K = C): 256 x 64 tiles, two
// workgroups per CU, so that one's epilogue (a large share of the time when K
// is short) overlaps the other's K loop. Otherwise 256-wide tiles unless
// 128-wide ones leave fewer unused columns.
hipError_t gemm(const GemmArgs& g, bool bf16, hipStream_t s) {
  if (!bf16 && g.K <= 512) return launch_gemm<float, 64>(g, s);
  const int pad256 = (g.N + 255) / 256 * 256 - g.N, pad128 = (g.N + 127) / 128 * 128 - g.N;
  if (pad128 < pad256) return bf16 ? launch_gemm<__bf16, 128>(g, s) : launch_gemm<float, 128>(g, s);
  return bf16 ? launch_gemm<__bf16, 256>(g, s) : launch_gemm<float, 256>(g, s);
}

// ------------------------------------------------------------- transpose

template <typename U>
__global__ __launch_bounds__(256) void transpose_kernel(const U* __restrict__ src, U* __restrict__ dst, int rows,
                                                        int cols) {
  __shared__ U tile[32][33];
  // blockIdx.z: matrix of a batch, each rows x cols
  src += (size_t)blockIdx.z * rows * cols;
  dst += (size_t)blockIdx.z * rows * cols;
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int i = ty; i < 32; i += 8) {
    const int r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) tile[i][tx] = src[(size_t)r * cols + c];
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int c = c0 + i, r = r0 + tx;
    if (r < rows && c < cols) dst[(size_t)c * rows + r] = tile[tx][i];
  }
}

// Two matrices of different shapes in one launch (blockIdx.z picks the
// matrix; the grid covers the larger and the other's surplus blocks return).
// 64 x 64 tiles in 16-byte accesses: VEC consecutive columns of a source row
// per load, VEC consecutive rows of a source column per store (dimensions are
// multiples of 64; the padded LDS rows keep every row 16-byte aligned).
template <typename U>
__global__ __launch_bounds__(256) void transpose_pair_kernel(const U* __restrict__ s0, U* __restrict__ d0, int r0,
                                                             int c0, const U* __restrict__ s1, U* __restrict__ d1,
                                                             int r1, int c1) {
  constexpr int T = 64, VEC = 16 / (int)sizeof(U), CPR = T / VEC, LD = T + VEC;
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) U tile[T * LD];
  const bool second = blockIdx.z == 1;
  const U* src = second ? s1 : s0;
  U* dst = second ? d1 : d0;
  const int rows = second ? r1 : r0, cols = second ? c1 : c0;
  const int col0 = blockIdx.x * T, row0 = blockIdx.y * T;
  if (col0 >= cols || row0 >= rows) return;  // uniform per workgroup
#pragma unroll
  for (int q = threadIdx.x; q < T * CPR; q += 256) {
    const int r = q / CPR, c = (q % CPR) * VEC;
    *reinterpret_cast<u32x4v*>(tile + r * LD + c) =
        *reinterpret_cast<const u32x4v*>(src + (size_t)(row0 + r) * cols + col0 + c);
  }
  __syncthreads();
#pragma unroll
  for (int q = threadIdx.x; q < T * CPR; q += 256) {
    // CPR consecutive lanes write one destination row's 64 elements
    const int c = q / CPR, r = (q % CPR) * VEC;
    u32x4v o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (sizeof(U) == 2)
        o[k] = (unsigned)tile[(r + 2 * k) * LD + c] | ((unsigned)tile[(r + 2 * k + 1) * LD + c] << 16);
      else
        o[k] = __float_as_uint(tile[(r + k) * LD + c]);
    }
    *reinterpret_cast<u32x4v*>(dst + (size_t)(col0 + c) * rows + row0 + r) = o;
  }
}

hipError_t transpose2d_pair(const void* s0, void* d0, int r0, int c0, const void* s1, void* d1, int r1, int c1,
                            bool bf16, hipStream_t s) {
  if (r0 % 64 || c0 % 64 || r1 % 64 || c1 % 64) return hipErrorInvalidValue;
  const int cols = c0 > c1 ? c0 : c1, rows = r0 > r1 ? r0 : r1;
  dim3 grid(cols / 64, rows / 64, 2), block(256);
  if (bf16)
    hipLaunchKernelGGL(transpose_pair_kernel<unsigned short>, grid, block, 0, s, (const unsigned short*)s0,
                       (unsigned short*)d0, r0, c0, (const unsigned short*)s1, (unsigned short*)d1, r1, c1);
  else
    hipLaunchKernelGGL(transpose_pair_kernel<float>, grid, block, 0, s, (const float*)s0, (float*)d0, r0, c0,
                       (const float*)s1, (float*)d1, r1, c1);
  return hipGetLastError();
}

hipError_t transpose2d(const void* src, void* dst, int rows, int cols, bool bf16, hipStream_t s, int batch) {
  dim3 grid((cols + 31) / 32, (rows + 31) / 32, batch), block(256);
  if (bf16)
    hipLaunchKernelGGL(transpose_kernel<unsigned short>, grid, block, 0, s, (const unsigned short*)src,
                       (unsigned short*)dst, rows, cols);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, block, 0, s, (const float*)src, (float*)dst, rows, cols);
  return hipGetLastError();
}

}  // namespace hy
