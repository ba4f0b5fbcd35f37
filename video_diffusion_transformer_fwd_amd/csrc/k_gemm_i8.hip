// int8 product of the per-row / grouped int8 FC2 on the gfx950 matrix cores.
//
// C[M,N] = bf16(((sum_g float(acc_g) * SA[m,g]) * SW[n]) + bias[n]) with acc_g the exact int32
// sum of QA[m,k] QW[n,k] over K group g (groups ascending, each float operation rounded, no
// fused multiply-add).  Row mode has one group (the whole K).
//
// v_mfma_i32_32x32x32_i8: lane l supplies 16 consecutive k at 16(l/32) of row l%32 of each
// operand; accumulator register i of lane l is D[8(i/4) + 4(l/32) + i%4][l%32] with D = X Y^T.
// The weight tile is passed as the first operand (D = C^T), so lane l holds row m = l%32 of C
// at the four runs of 4 consecutive columns 8(i/4) + 4(l/32) + 0..3: one activation scale per
// lane and 16-byte vector stores.
//
// Same pipeline as the bf16 product: a K slice is 128 int8 = 128 bytes per row, so the LDS tile
// rows, their bank swizzle (chunk c of row r in slot c ^ ((r >> 1) & 7)) and the direct
// global -> LDS staging are identical; each 32-wide K step's fragment reads are issued while
// the previous step's MFMAs run.
//
// Row mode may split K over S workgroups per tile: each stores its int32 partial tile, and a
// second launch adds the S partials (integer addition: exact in any order) and dequantises, so
// the result equals the unsplit product bit for bit.  Grouped mode folds each group's int32
// sums into a float32 total in group order inside the kernel and is never split (the float
// fold order is fixed).  The dequantising epilogue, optionally followed by the bf16 product's
// GELU (erf form, erfc by A&S 7.1.26), runs from an LDS band in a rolled loop, as in the bf16
// product.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "h3_internal.h"

namespace h3 {

namespace {

typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(16))) int i32x16_t;

constexpr int kXcds = 8;
constexpr int kGroupM = 8;

typedef __attribute__((address_space(3))) unsigned char lds_u8;

template <int BM, int BN, int WM, int WN, int NS>
struct GemmI8Cfg {
  static constexpr int NT = 64 * WM * WN;
  static constexpr int BK = 128;  // int8 elements = bytes per row per slice
  static constexpr int TM = BM / WM / 32;
  static constexpr int TN = BN / WN / 32;
  static constexpr int STAGE = (BM + BN) * 128;
  static constexpr int EPI_LD = BN + 4;              // float32 row stride of the epilogue band
  static constexpr int EPI_BAND = WM * 32 * EPI_LD;  // one 32-row block of every wave row
  static constexpr size_t EPI_BYTES = (static_cast<size_t>(EPI_BAND) + 2 * BN) * 4;
  static constexpr size_t LDS_BYTES =
      NS * static_cast<size_t>(STAGE) > EPI_BYTES ? NS * static_cast<size_t>(STAGE) : EPI_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "tile does not fit the 160 KB LDS");
  static_assert(TM >= 1 && TN >= 1 && BM % (WM * 32) == 0 && BN % (WN * 32) == 0,
                "wave tile must be whole 32x32 blocks");
};

struct GemmI8Args {
  const int8_t *QA;
  const float *SA;  // [M, ngroups]
  const int8_t *QW;
  const float *SW;  // [N]
  const bf16_t *bias;
  bf16_t *C;
  int64_t ldc;
  int M, N, K, group;
  int32_t *part;  // split-K int32 partials [S][M][N] (row mode)
  QkEpi qk;       // QKV product with the Q/K RMSNorm + RoPE epilogue (QKD > 0)
};

// QKD > 0: the QKV product with heads of QKD channels, columns in QkMap<BN, QKD> order and the
// Q/K RMSNorm + RoPE applied to the q/k heads in the epilogue (row mode, unsplit, no GELU).
template <int BM, int BN, int WM, int WN, int NS, bool GROUPED, int SPLIT, int EPI, int QKD = 0>
__global__ __launch_bounds__(64 * WM * WN) void gemm_i8_kernel(GemmI8Args g) {
#pragma clang fp contract(off)
  static_assert(!(GROUPED && SPLIT > 1), "the grouped float fold is never split");
  static_assert(QKD == 0 || (!GROUPED && SPLIT == 1 && EPI == H3_EPI_NONE), "QKV epilogue form");
  using Cfg = GemmI8Cfg<BM, BN, WM, WN, NS>;
  constexpr int NT = Cfg::NT, BK = Cfg::BK, TM = Cfg::TM, TN = Cfg::TN;
  // static: constant parts of the fragment addresses fold into the LDS instructions' offsets
  __shared__ __align__(16) unsigned char smem8[Cfg::LDS_BYTES];

  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int tile_id = blockIdx.x / SPLIT;
  const int split = blockIdx.x % SPLIT;
  int tm, tn;
  {
    const int ntiles = tiles_m * tiles_n;
    int id = tile_id;
    if (ntiles % kXcds == 0) {
      const int per = ntiles / kXcds;
      id = (id % kXcds) * per + id / kXcds;
    }
    const int in_group = kGroupM * tiles_n;
    const int grp = id / in_group;
    const int first_m = grp * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM);
    const int r = id - grp * in_group;
    tm = first_m + r % gm;
    tn = r / gm;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int kc = g.K / SPLIT, kbeg = split * kc;
  // output column of local tile column j
  auto ncol = [&](int j) {
    if constexpr (QKD > 0)
      return QkMap<BN, QKD>::col(tn, j, g.qk.d);
    else
      return n0 + j;
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: copy targets are scalar
  const int wm = wave / WN, wn = wave % WN;

  // direct global -> LDS staging, as in the bf16 product (1 byte per element here); LDS holds
  // the NS A stages, then the NS B stages
  constexpr int NW = NT / 64;
  constexpr int ROW_BLOCKS = (BM + BN) / 8;
  constexpr int LOADS = ROW_BLOCKS / NW;
  static_assert(ROW_BLOCKS % NW == 0 && BM % 8 == 0, "row blocks must split evenly over waves");
  const unsigned char *abase = reinterpret_cast<const unsigned char *>(g.QA);
  const unsigned char *bbase = reinterpret_cast<const unsigned char *>(g.QW);
  uint32_t goff[LOADS];
  {
    const int lrow = lane >> 3;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int R = (i * NW + wave) * 8 + lrow;
      const int chunk = (lane & 7) ^ ((R >> 1) & 7);
      if (R < BM) {
        int r = m0 + R;
        r = r < g.M ? r : g.M - 1;
        goff[i] = static_cast<uint32_t>(static_cast<int64_t>(r) * g.K + kbeg + chunk * 16);
      } else {
        int r = ncol(R - BM);
        r = r < g.N ? r : g.N - 1;
        goff[i] = static_cast<uint32_t>(static_cast<int64_t>(r) * g.K + kbeg + chunk * 16);
      }
    }
  }
  constexpr int A_BYTES = NS * BM * 128;  // the B stages start here
  // stage: a compile-time constant (the unrolled loop: LDS offsets are immediates) or an int
  auto issue_slice = [&](int kt, auto stage) __attribute__((always_inline)) {
    const int S = stage;
    const uint32_t kb = static_cast<uint32_t>(kt * BK);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int R0 = (i * NW + wave) * 8;
      const unsigned char *base = (R0 < BM ? abase : bbase) + kb;  // uniform
      const unsigned char *src = base + goff[i];
      lds_u8 *dst = (lds_u8 *)smem8 +
                    (R0 < BM ? S * BM * 128 + R0 * 128 : A_BYTES + S * BN * 128 + (R0 - BM) * 128);
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(dst), 16, 0, 0);
    }
  };

  // fragment addresses, as in the bf16 product: chunk 2 ks + fh of A row (wm TM + i) 32 + fr
  // sits at a_lane ^ 32 ks + 4096 i (+ BM 128 S for stage S); B likewise from b_lane
  const int fr = lane & 31, fh = lane >> 5;
  const int a_lane = (wm * TM * 32 + fr) * 128 + ((fh ^ ((fr >> 1) & 7)) << 4);
  const int b_lane = A_BYTES + (wn * TN * 32 + fr) * 128 + ((fh ^ ((fr >> 1) & 7)) << 4);
  const lds_u8 *lds = (const lds_u8 *)smem8;

  // lane holds C[m_l][n_l + 8q + e], e = 0..3, in accumulator registers 4q + e of each block
  const int m_l = lane & 31, n_l = (lane >> 5) * 4;
  i32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = i32x16_t{};
  float tot[GROUPED ? TM : 1][GROUPED ? TN : 1][GROUPED ? 16 : 1];
  if constexpr (GROUPED) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) tot[i][j][r] = 0.f;
  }

  const int KT = kc / BK;
  const int slices_per_group = g.group / BK;
  const int ngroups = g.K / g.group;
  issue_slice(0, std::integral_constant<int, 0>{});
  if constexpr (NS == 3)
    if (KT > 1) issue_slice(1, std::integral_constant<int, 1>{});
  if (KT >= NS - 1)
    lds_dma_barrier<LOADS * (NS - 2)>();
  else
    lds_dma_barrier<0>();

  // one K slice out of stage S; the K loop is unrolled over the stages (rolled for the grouped
  // fold, whose float totals leave no registers for copies of the loop body)
  auto slice = [&](int kt, auto stage) __attribute__((always_inline)) {
    const int S = stage;
    const bool more = kt + NS - 1 < KT;
    // grouped: this slice ends a group -> fetch the group's activation scales now (before this
    // iteration's slice loads, so waiting for them never waits for those) and use them after
    // the MFMAs
    const bool fold = GROUPED && (kt + 1) % slices_per_group == 0;
    float sa_g[GROUPED ? TM : 1];
    if constexpr (GROUPED) {
      if (fold) {
        const int gi = (kt + 1) / slices_per_group - 1;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          int m = m0 + (wm * TM + i) * 32 + m_l;
          m = m < g.M ? m : g.M - 1;
          sa_g[i] = g.SA[static_cast<int64_t>(m) * ngroups + gi];
        }
      }
    }
    if (more) {
      if constexpr (std::is_same_v<decltype(stage), int>)
        issue_slice(kt + NS - 1, (S + NS - 1) % NS);
      else
        issue_slice(kt + NS - 1, std::integral_constant<int, (decltype(stage)::value + NS - 1) % NS>{});
    }
    auto afrag = [&](int i, int ks) {
      return *reinterpret_cast<const __attribute__((address_space(3))) i32x4_t *>(
          lds + ((a_lane ^ (32 * ks)) + S * BM * 128 + i * 4096));
    };
    auto bfrag = [&](int j, int ks) {
      return *reinterpret_cast<const __attribute__((address_space(3))) i32x4_t *>(
          lds + ((b_lane ^ (32 * ks)) + S * BN * 128 + j * 4096));
    };
    i32x4_t af[2][TM], bfr[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) af[0][i] = afrag(i, 0);
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[0][j] = bfrag(j, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < BK / 32) {
#pragma unroll
        for (int i = 0; i < TM; ++i) af[cur ^ 1][i] = afrag(i, ks + 1);
#pragma unroll
        for (int j = 0; j < TN; ++j) bfr[cur ^ 1][j] = bfrag(j, ks + 1);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bfr[cur][j], af[cur][i], acc[i][j], 0, 0, 0);
      if (ks + 1 < BK / 32) {
#pragma unroll
        for (int q = 0; q < TM + TN; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if (TM * TN > TM + TN) __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - (TM + TN), 0);
      }
    }
    if constexpr (GROUPED) {
      // group end: tot += float(acc) * SA[m, g], then clear acc (one scale per lane row)
      if (fold) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const float sa = sa_g[i];
#pragma unroll
          for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float t = static_cast<float>(acc[i][j][r]) * sa;
              tot[i][j][r] = tot[i][j][r] + t;
            }
            acc[i][j] = i32x16_t{};
          }
        }
      }
    }
    if (more)
      lds_dma_barrier<LOADS * (NS - 2)>();
    else
      lds_dma_barrier<0>();
  };
  if constexpr (GROUPED) {
    for (int kt = 0; kt < KT; ++kt) slice(kt, kt % NS);
  } else {
    for (int kt = 0; kt < KT; kt += NS) {
      slice(kt, std::integral_constant<int, 0>{});
      if (kt + 1 < KT) slice(kt + 1, std::integral_constant<int, 1>{});
      if constexpr (NS == 3)
        if (kt + 2 < KT) slice(kt + 2, std::integral_constant<int, 2>{});
    }
  }

  if constexpr (SPLIT > 1) {
    // row-mode split: store this K piece's int32 partial tile, row-major [piece][M][N] (N % 4 == 0)
    int32_t *part = g.part + static_cast<int64_t>(split) * g.M * g.N;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + (wm * TM + i) * 32 + m_l;
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + (wn * TN + j) * 32 + q * 8 + n_l;
          if (n < g.N)
            *reinterpret_cast<int4 *>(part + static_cast<int64_t>(m) * g.N + n) =
                make_int4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        }
    }
    return;
  }

  // Epilogue through LDS: per-column weight scale and bias staged once; per 32-row block index
  // i every wave writes its float32 activation-scaled sums (row mode: float(acc) * SA[m]) to a
  // band of WM * 32 rows x BN columns, then all threads dequantise 4-column chunks of the band
  // in a rolled loop: bf16((v * SW[n]) + bias[n]), 8-byte stores along the rows.
  constexpr int LD = Cfg::EPI_LD;
  float *band = reinterpret_cast<float *>(smem8);
  float *ssw = band + Cfg::EPI_BAND;
  float *sbias = ssw + BN;
  __syncthreads();
  for (int c = tid; c < BN; c += NT) {
    const int n = ncol(c);
    ssw[c] = n < g.N ? g.SW[n] : 0.f;
    sbias[c] = n < g.N ? bf2f(g.bias[n]) : 0.f;
  }
  const bool vec = (g.ldc % 4 == 0) && (reinterpret_cast<uintptr_t>(g.C) % 8 == 0);
  constexpr int CHUNKS_PER_ROW = BN / 4;
  constexpr int BAND_CHUNKS = WM * 32 * CHUNKS_PER_ROW;
  // QKV: rotation slices and gains of band 0's q/k-head tasks, fetched before the band fills
  QkHeadPass<BN, QKD ? QKD : 128, WM, TM, NT> hp(g.qk, tid, tn, m0, g.M);
  if constexpr (QKD > 0) hp.fetch(0);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    if (i > 0) __syncthreads();  // previous band fully read
    float sa = 0.f;
    if constexpr (!GROUPED) {
      int m = m0 + (wm * TM + i) * 32 + m_l;
      m = m < g.M ? m : g.M - 1;
      sa = g.SA[m];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (GROUPED)
            v[e] = tot[i][j][4 * q + e];
          else
            v[e] = static_cast<float>(acc[i][j][4 * q + e]) * sa;
        }
        *reinterpret_cast<float4 *>(band + (wm * 32 + m_l) * LD + (wn * TN + j) * 32 + q * 8 + n_l) =
            make_float4(v[0], v[1], v[2], v[3]);
      }
    __syncthreads();
    if constexpr (QKD > 0) {
      // QKV: q/k heads first (QkHeadPass: the bf16 value the plain product stores, then
      // RMSNorm + RoPE), then the other columns with the plain dequantising epilogue.  The host
      // guarantees 8 | ldc, a 16-byte aligned C and table.
      using Map = QkMap<BN, QKD>;
      const int hc = hp.hpr * QKD;
      const int pc4 = (BN - hc) / 4;
      hp.run(i, [&](int row, int col, float *a) {
        const float4 *bp = reinterpret_cast<const float4 *>(band + row * LD + col);
        const float4 *wp = reinterpret_cast<const float4 *>(ssw + col);
        const float4 *sp = reinterpret_cast<const float4 *>(sbias + col);
        const float4 v0 = bp[0], v1 = bp[1], w0 = wp[0], w1 = wp[1], b0 = sp[0], b1 = sp[1];
        const float t[8] = {v0.x * w0.x, v0.y * w0.y, v0.z * w0.z, v0.w * w0.w,
                            v1.x * w1.x, v1.y * w1.y, v1.z * w1.z, v1.w * w1.w};
        const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = bf2f(f2bf(t[e] + b[e]));
      }, g.C, g.ldc);
      if (i + 1 < TM) hp.fetch(i + 1);
      for (int c4 = tid; c4 < WM * 32 * pc4; c4 += NT) {
        const int row = c4 / pc4, col = hc + (c4 - row * pc4) * 4;
        const int m = m0 + ((row >> 5) * TM + i) * 32 + (row & 31);
        const int n = Map::col(tn, col, g.qk.d);
        if (m >= g.M || n >= g.N) continue;
        const float4 a4 = *reinterpret_cast<const float4 *>(band + row * LD + col);
        const float4 w4 = *reinterpret_cast<const float4 *>(ssw + col);
        const float4 b4 = *reinterpret_cast<const float4 *>(sbias + col);
        const float t0 = a4.x * w4.x, t1 = a4.y * w4.y, t2 = a4.z * w4.z, t3 = a4.w * w4.w;
        uint2 pk;
        pk.x = pack_bf2(t0 + b4.x, t1 + b4.y);
        pk.y = pack_bf2(t2 + b4.z, t3 + b4.w);
        *reinterpret_cast<uint2 *>(g.C + static_cast<int64_t>(m) * g.ldc + n) = pk;
      }
      continue;
    }
#pragma unroll 2
    for (int c4 = tid; c4 < BAND_CHUNKS; c4 += NT) {
      const int row = c4 / CHUNKS_PER_ROW, col = (c4 - row * CHUNKS_PER_ROW) * 4;
      const int m = m0 + ((row >> 5) * TM + i) * 32 + (row & 31);
      const int n = n0 + col;
      if (m >= g.M || n >= g.N) continue;
      const float4 a4 = *reinterpret_cast<const float4 *>(band + row * LD + col);
      const float4 w4 = *reinterpret_cast<const float4 *>(ssw + col);
      const float4 b4 = *reinterpret_cast<const float4 *>(sbias + col);
      const float t0 = a4.x * w4.x, t1 = a4.y * w4.y, t2 = a4.z * w4.z, t3 = a4.w * w4.w;
      float o[4] = {t0 + b4.x, t1 + b4.y, t2 + b4.z, t3 + b4.w};
      if constexpr (EPI == H3_EPI_GELU) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = gelu_erf(o[e]);
      }
      const int64_t off = static_cast<int64_t>(m) * g.ldc + n;
      if (vec && n + 3 < g.N) {
        uint2 pk;
        pk.x = pack_bf2(o[0], o[1]);
        pk.y = pack_bf2(o[2], o[3]);
        *reinterpret_cast<uint2 *>(g.C + off) = pk;
      } else {
        for (int e = 0; e < 4 && n + e < g.N; ++e) g.C[off + e] = static_cast<bf16_t>(f2bf(o[e]));
      }
    }
  }
}

// Adds the S int32 partials (exact) and dequantises: bf16(((float(sum) * SA[m]) * SW[n]) + b[n]),
// then GELU when EPI says so.
template <int S, int EPI>
__global__ __launch_bounds__(256) void splitk_i8_reduce_kernel(const int32_t *__restrict__ part,
                                                               int M, int N,
                                                               const float *__restrict__ SA,
                                                               const float *__restrict__ SW,
                                                               const bf16_t *__restrict__ bias,
                                                               bf16_t *__restrict__ C, int64_t ldc) {
#pragma clang fp contract(off)
  const int64_t total4 = static_cast<int64_t>(M) * N / 4;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total4) return;
  const int64_t e0 = idx * 4;
  const int m = static_cast<int>(e0 / N), n = static_cast<int>(e0 - static_cast<int64_t>(m) * N);
  int4 s = *reinterpret_cast<const int4 *>(part + e0);
#pragma unroll
  for (int p = 1; p < S; ++p) {
    const int4 t = *reinterpret_cast<const int4 *>(part + static_cast<int64_t>(p) * M * N + e0);
    s.x += t.x;
    s.y += t.y;
    s.z += t.z;
    s.w += t.w;
  }
  const float sa = SA[m];
  const int sv[4] = {s.x, s.y, s.z, s.w};
  float o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float v = static_cast<float>(sv[e]) * sa;
    const float t = v * SW[n + e];
    o[e] = t + bf2f(bias[n + e]);
    if constexpr (EPI == H3_EPI_GELU) o[e] = gelu_erf(o[e]);
  }
  bf16_t *dst = C + static_cast<int64_t>(m) * ldc + n;
  if (ldc % 4 == 0 && (reinterpret_cast<uintptr_t>(C) % 8) == 0) {
    uint2 pk;
    pk.x = pack_bf2(o[0], o[1]);
    pk.y = pack_bf2(o[2], o[3]);
    *reinterpret_cast<uint2 *>(dst) = pk;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = static_cast<bf16_t>(f2bf(o[e]));
  }
}

template <int BM, int BN, int WM, int WN, int NS, bool GROUPED, int SPLIT, int EPI, int QKD = 0,
          bool REDUCE = true>
void run_gemm_i8(const GemmI8Args &a, hipStream_t s) {
  using Cfg = GemmI8Cfg<BM, BN, WM, WN, NS>;
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  auto kern = gemm_i8_kernel<BM, BN, WM, WN, NS, GROUPED, SPLIT, EPI, QKD>;
  kern<<<tiles * SPLIT, Cfg::NT, 0, s>>>(a);
  if constexpr (SPLIT > 1 && REDUCE) {
    const int64_t total4 = static_cast<int64_t>(a.M) * a.N / 4;
    splitk_i8_reduce_kernel<SPLIT, EPI><<<static_cast<int>((total4 + 255) / 256), 256, 0, s>>>(
        a.part, a.M, a.N, a.SA, a.SW, a.bias, a.C, a.ldc);
  }
}

}  // namespace

// Tile choice (cfg * 8 + split), measured on the MI355X with random int8 operands:
//   grouped, M >= 4096                   192x192, 4 waves, three LDS stages (never split)
//   grouped, otherwise                   128x256, 4 waves, three LDS stages
//   row, M >= 4096                       256x256, 8 waves, two LDS stages
//   row, 1024 <= M < 4096                384x192, 8 waves; K split in 4 when N < 8192
//   row, 192 <= M < 1024                 192x192, 4 waves; K split in 4 when N < 8192
//   row, otherwise                       128x128, 4 waves
// A split needs K % (128 * split) == 0 and N % 4 == 0.
GemmPlan plan_gemm_i8(int M, int N, int K, int group) {
  GemmPlan p{};
  p.cfg = 0;
  p.split = 1;
  const int wide_split = N >= 8192 ? 1 : 4;
  if (group != K) {
    p.cfg = M >= 4096 ? 1 : 3;
  } else if (M >= 4096) {
    p.cfg = 2;
  } else if (M >= 1024) {
    p.cfg = 4;
    p.split = wide_split;
  } else if (M >= 192) {
    p.cfg = 1;
    p.split = wide_split;
  }
  if (p.split > 1 && (K % (128 * p.split) != 0 || N % 4 != 0)) p.split = 1;
  if (p.split > 1) p.part_bytes = static_cast<size_t>(p.split) * M * N * sizeof(int32_t);
  return p;
}

namespace {
template <int EPI>
void dispatch_i8(const GemmPlan &p, const GemmI8Args &a, bool grouped, hipStream_t s) {
  if (grouped) {
    if (p.cfg == 1)
      run_gemm_i8<192, 192, 2, 2, 3, true, 1, EPI>(a, s);
    else
      run_gemm_i8<128, 256, 2, 2, 3, true, 1, EPI>(a, s);
    return;
  }
  switch (p.cfg * 8 + p.split) {
    case 2 * 8 + 1: run_gemm_i8<256, 256, 2, 4, 2, false, 1, EPI>(a, s); break;
    case 4 * 8 + 1: run_gemm_i8<384, 192, 4, 2, 2, false, 1, EPI>(a, s); break;
    case 4 * 8 + 4: run_gemm_i8<384, 192, 4, 2, 2, false, 4, EPI>(a, s); break;
    case 1 * 8 + 1: run_gemm_i8<192, 192, 2, 2, 3, false, 1, EPI>(a, s); break;
    case 1 * 8 + 4: run_gemm_i8<192, 192, 2, 2, 3, false, 4, EPI>(a, s); break;
    default: run_gemm_i8<128, 128, 2, 2, 3, false, 1, EPI>(a, s); break;
  }
}

template <int QKD>
void qkv_dispatch_i8(const GemmPlan &p, const GemmI8Args &a, hipStream_t s) {
  switch (p.cfg) {
    case 2: run_gemm_i8<256, 256, 2, 4, 2, false, 1, H3_EPI_NONE, QKD>(a, s); break;
    case 4: run_gemm_i8<384, 192, 4, 2, 2, false, 1, H3_EPI_NONE, QKD>(a, s); break;
    case 1: run_gemm_i8<192, 192, 2, 2, 3, false, 1, H3_EPI_NONE, QKD>(a, s); break;
    default: run_gemm_i8<128, 128, 2, 2, 3, false, 1, H3_EPI_NONE, QKD>(a, s); break;
  }
}
}  // namespace

void launch_gemm_i8(const int8_t *QA, const float *SA, const int8_t *QW, const float *SW,
                    const bf16_t *bias, bf16_t *C, int64_t ldc, int M, int N, int K, int group,
                    hipStream_t s, const SplitScratch &sc, int epilogue) {
  GemmPlan p = plan_gemm_i8(M, N, K, group);
  if (p.split > 1 && (!sc.part || p.part_bytes > sc.part_bytes)) p.split = 1;
  GemmI8Args a{QA, SA, QW, SW, bias, C, ldc, M, N, K, group, reinterpret_cast<int32_t *>(sc.part)};
  if (epilogue == H3_EPI_GELU)
    dispatch_i8<H3_EPI_GELU>(p, a, group != K, s);
  else
    dispatch_i8<H3_EPI_NONE>(p, a, group != K, s);
}

int launch_gemm_i8_partials(const int8_t *QA, const float *SA, const int8_t *QW, const float *SW,
                            int M, int N, int K, hipStream_t s, const SplitScratch &sc) {
  const GemmPlan p = plan_gemm_i8(M, N, K, K);
  if (p.split <= 1 || !sc.part || p.part_bytes > sc.part_bytes) return 0;
  GemmI8Args a{QA, SA, QW, SW, nullptr, nullptr, 0, M, N, K, K, reinterpret_cast<int32_t *>(sc.part)};
  switch (p.cfg * 8 + p.split) {
    case 4 * 8 + 4: run_gemm_i8<384, 192, 4, 2, 2, false, 4, H3_EPI_NONE, 0, false>(a, s); return 4;
    case 1 * 8 + 4: run_gemm_i8<192, 192, 2, 2, 3, false, 4, H3_EPI_NONE, 0, false>(a, s); return 4;
    default: return 0;
  }
}

int launch_gemm_i8_qkv(const int8_t *QA, const float *SA, const int8_t *QW, const float *SW,
                       const bf16_t *bias, bf16_t *C, int64_t ldc, int M, int d, int K,
                       int head_dim, const QkEpi &qk, hipStream_t s) {
  const GemmPlan p = plan_gemm_i8(M, 4 * d, K, K);
  if (p.split > 1 || (head_dim != 64 && head_dim != 128) || d % 128 || ldc % 8 ||
      reinterpret_cast<uintptr_t>(C) % 16 ||
      reinterpret_cast<uintptr_t>(qk.table) % 16)
    return 0;
  GemmI8Args a{QA, SA, QW, SW, bias, C, ldc, M, 4 * d, K, K, nullptr, qk};
  if (head_dim == 128)
    qkv_dispatch_i8<128>(p, a, s);
  else
    qkv_dispatch_i8<64>(p, a, s);
  return 1;
}

}  // namespace h3
