// Dense products of the block on the gfx950 matrix cores.
//
// bf16: C[M,N] = A[M,K] B[N,K]^T (+ bias) (+ GELU), v_mfma_f32_32x32x16_bf16, float32
// accumulation.  int8: per-group int32 sums with v_mfma_i32_32x32x32_i8 and a float32
// dequantisation epilogue.
//
// Tiling: a 256-thread workgroup (4 wave64s, WM x WN) owns a BM x BN output tile and walks K in
// BK slices.  Both operands are K-contiguous, so A and B tiles are staged identically:
// 16-byte global loads (8 consecutive lanes cover one 128-byte row slice), registers, then a
// padded LDS tile (row stride BK + 16 bytes, which keeps the 16-byte MFMA-operand reads of 8
// consecutive rows on distinct banks).  LDS is double-buffered with one barrier per K slice:
// the next slice's global loads are in flight while the current slice feeds the MFMAs.
//
// Operand layouts (32x32x16 bf16): lane l supplies A[m = l%32][k = 8(l/32) .. +7] and
// B[n = l%32][k = 8(l/32) .. +7]; accumulator register i of lane l is
// C[8(i/4) + 4(l/32) + i%4][l%32].  (i8 32x32x32: 16 consecutive k per lane, k = 16(l/32).)
//
// Workgroup order is XCD-aware: consecutive workgroup ids land on different XCDs, so ids are
// regrouped so that each XCD walks a contiguous band of tiles, and tiles are visited in
// groups of GROUP_M tile-rows so neighbours share A rows and B columns in that XCD's L2.
#include <hip/hip_runtime.h>

#include "h3_internal.h"

namespace h3 {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(16))) int i32x16_t;

constexpr int kXcds = 8;
constexpr int kGroupM = 8;

// Maps the hardware workgroup id to a (tile_m, tile_n) pair.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int &tm, int &tn) {
  const int nwg = tiles_m * tiles_n;
  int id = blockIdx.x;
  // regroup: hardware id -> XCD-contiguous id (only when the grid divides evenly)
  if (nwg % kXcds == 0) {
    const int per = nwg / kXcds;
    id = (id % kXcds) * per + id / kXcds;
  }
  const int in_group = kGroupM * tiles_n;
  const int group = id / in_group;
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int r = id - group * in_group;
  tm = first_m + r % gm;
  tn = r / gm;
}

__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

// ------------------------------------------------------------------------ bf16 GEMM
template <int BM, int BN, int WM, int WN>
struct GemmCfg {
  static constexpr int BK = 64;
  static constexpr int LDS_STRIDE = BK + 8;  // elements
  static constexpr int TM = BM / WM / 32;
  static constexpr int TN = BN / WN / 32;
  static constexpr int A_CHUNKS = BM * BK / 8 / 256;  // 16-byte chunks per thread
  static constexpr int B_CHUNKS = BN * BK / 8 / 256;
  static constexpr int LDS_A = BM * LDS_STRIDE;
  static constexpr int LDS_B = BN * LDS_STRIDE;
  static constexpr size_t LDS_BYTES = 2 * (LDS_A + LDS_B) * sizeof(bf16_t);
};

template <int BM, int BN, int WM, int WN, int EPI, int OUT_F32>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(
    const bf16_t *__restrict__ A, int64_t lda, const bf16_t *__restrict__ B, int64_t ldb,
    void *__restrict__ C, int64_t ldc, int M, int N, int K, const bf16_t *__restrict__ bias,
    const bf16_t *__restrict__ bias2) {
  using Cfg = GemmCfg<BM, BN, WM, WN>;
  constexpr int BK = Cfg::BK, LS = Cfg::LDS_STRIDE, TM = Cfg::TM, TN = Cfg::TN;
  extern __shared__ __align__(16) bf16_t smem[];
  bf16_t *As = smem;                    // [2][BM][LS]
  bf16_t *Bs = smem + 2 * Cfg::LDS_A;   // [2][BN][LS]

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // global -> register staging coordinates: chunk c covers row (tid/8 + c*32), col (tid%8)*8
  const int ld_row = tid >> 3, ld_col = (tid & 7) * 8;
  const bf16_t *a_src[Cfg::A_CHUNKS];
  const bf16_t *b_src[Cfg::B_CHUNKS];
#pragma unroll
  for (int c = 0; c < Cfg::A_CHUNKS; ++c) {
    int r = m0 + ld_row + c * 32;
    r = r < M ? r : M - 1;
    a_src[c] = A + static_cast<int64_t>(r) * lda + ld_col;
  }
#pragma unroll
  for (int c = 0; c < Cfg::B_CHUNKS; ++c) {
    int r = n0 + ld_row + c * 32;
    r = r < N ? r : N - 1;
    b_src[c] = B + static_cast<int64_t>(r) * ldb + ld_col;
  }
  uint4 ra[Cfg::A_CHUNKS], rb[Cfg::B_CHUNKS];

  auto load_global = [&](int k0) {
#pragma unroll
    for (int c = 0; c < Cfg::A_CHUNKS; ++c) ra[c] = *reinterpret_cast<const uint4 *>(a_src[c] + k0);
#pragma unroll
    for (int c = 0; c < Cfg::B_CHUNKS; ++c) rb[c] = *reinterpret_cast<const uint4 *>(b_src[c] + k0);
  };
  auto store_lds = [&](int buf) {
    bf16_t *as = As + buf * Cfg::LDS_A;
    bf16_t *bs = Bs + buf * Cfg::LDS_B;
#pragma unroll
    for (int c = 0; c < Cfg::A_CHUNKS; ++c)
      *reinterpret_cast<uint4 *>(as + (ld_row + c * 32) * LS + ld_col) = ra[c];
#pragma unroll
    for (int c = 0; c < Cfg::B_CHUNKS; ++c)
      *reinterpret_cast<uint4 *>(bs + (ld_row + c * 32) * LS + ld_col) = rb[c];
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16_t{};

  const int KT = K / BK;
  load_global(0);
  store_lds(0);
  __syncthreads();

  const int frag_row = lane & 31, frag_k = (lane >> 5) * 8;
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load_global((kt + 1) * BK);
    const bf16_t *as = As + buf * Cfg::LDS_A + (wm * TM * 32 + frag_row) * LS + frag_k;
    const bf16_t *bs = Bs + buf * Cfg::LDS_B + (wn * TN * 32 + frag_row) * LS + frag_k;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t *>(as + i * 32 * LS + ks * 16);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t *>(bs + j * 32 * LS + ks * 16);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store_lds(buf ^ 1);
    __syncthreads();
  }

  // epilogue
  const int col_l = lane & 31, row_l = (lane >> 5) * 4;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = n0 + (wn * TN + j) * 32 + col_l;
    if (n >= N) continue;
    float bsum = 0.f;
    if (bias) bsum += bf2f(bias[n]);
    if (bias2) bsum += bf2f(bias2[n]);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + (wm * TM + i) * 32 + (r / 4) * 8 + row_l + (r % 4);
        if (m >= M) continue;
        float v = acc[i][j][r] + bsum;
        if constexpr (EPI == H3_EPI_GELU) v = gelu_erf(v);
        if constexpr (OUT_F32)
          reinterpret_cast<float *>(C)[static_cast<int64_t>(m) * ldc + n] = v;
        else
          reinterpret_cast<bf16_t *>(C)[static_cast<int64_t>(m) * ldc + n] =
              static_cast<bf16_t>(f2bf(v));
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int EPI, int OUT_F32>
void run_gemm(const bf16_t *A, int64_t lda, const bf16_t *B, int64_t ldb, void *C, int64_t ldc,
              int M, int N, int K, const bf16_t *bias, const bf16_t *bias2, hipStream_t s) {
  using Cfg = GemmCfg<BM, BN, WM, WN>;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  auto kern = gemm_bf16_kernel<BM, BN, WM, WN, EPI, OUT_F32>;
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                        hipFuncAttributeMaxDynamicSharedMemorySize,
                        static_cast<int>(Cfg::LDS_BYTES));
    attr_set = true;
  }
  kern<<<tiles, 256, Cfg::LDS_BYTES, s>>>(A, lda, B, ldb, C, ldc, M, N, K, bias, bias2);
}

template <int EPI, int OUT_F32>
void gemm_select(const bf16_t *A, int64_t lda, const bf16_t *B, int64_t ldb, void *C,
                 int64_t ldc, int M, int N, int K, const bf16_t *bias, const bf16_t *bias2,
                 hipStream_t s) {
  run_gemm<128, 128, 2, 2, EPI, OUT_F32>(A, lda, B, ldb, C, ldc, M, N, K, bias, bias2, s);
}

// ------------------------------------------------------------------------ int8 GEMM
// Same structure with int8 operands: BK = 128 bytes, 32x32x32 i8 MFMA.  acc holds the int32
// sum of the current K group; at each group end it is folded into the float32 total as
// tot = tot + float(acc) * SA[m, g] (two rounded operations, no fused multiply-add).
template <int BM, int BN, int WM, int WN>
struct GemmI8Cfg {
  static constexpr int BK = 128;
  static constexpr int LDS_STRIDE = BK + 16;  // bytes
  static constexpr int TM = BM / WM / 32;
  static constexpr int TN = BN / WN / 32;
  static constexpr int A_CHUNKS = BM * BK / 16 / 256;
  static constexpr int B_CHUNKS = BN * BK / 16 / 256;
  static constexpr int LDS_A = BM * LDS_STRIDE;
  static constexpr int LDS_B = BN * LDS_STRIDE;
  static constexpr size_t LDS_BYTES = 2 * (LDS_A + LDS_B);
};

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void gemm_i8_kernel(
    const int8_t *__restrict__ QA, const float *__restrict__ SA, const int8_t *__restrict__ QW,
    const float *__restrict__ SW, const bf16_t *__restrict__ bias, bf16_t *__restrict__ C,
    int64_t ldc, int M, int N, int K, int group) {
#pragma clang fp contract(off)
  using Cfg = GemmI8Cfg<BM, BN, WM, WN>;
  constexpr int BK = Cfg::BK, LS = Cfg::LDS_STRIDE, TM = Cfg::TM, TN = Cfg::TN;
  extern __shared__ __align__(16) int8_t smem8[];
  int8_t *As = smem8;
  int8_t *Bs = smem8 + 2 * Cfg::LDS_A;

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  const int ld_row = tid >> 3, ld_col = (tid & 7) * 16;
  const int8_t *a_src[Cfg::A_CHUNKS];
  const int8_t *b_src[Cfg::B_CHUNKS];
#pragma unroll
  for (int c = 0; c < Cfg::A_CHUNKS; ++c) {
    int r = m0 + ld_row + c * 32;
    r = r < M ? r : M - 1;
    a_src[c] = QA + static_cast<int64_t>(r) * K + ld_col;
  }
#pragma unroll
  for (int c = 0; c < Cfg::B_CHUNKS; ++c) {
    int r = n0 + ld_row + c * 32;
    r = r < N ? r : N - 1;
    b_src[c] = QW + static_cast<int64_t>(r) * K + ld_col;
  }
  uint4 ra[Cfg::A_CHUNKS], rb[Cfg::B_CHUNKS];
  auto load_global = [&](int k0) {
#pragma unroll
    for (int c = 0; c < Cfg::A_CHUNKS; ++c) ra[c] = *reinterpret_cast<const uint4 *>(a_src[c] + k0);
#pragma unroll
    for (int c = 0; c < Cfg::B_CHUNKS; ++c) rb[c] = *reinterpret_cast<const uint4 *>(b_src[c] + k0);
  };
  auto store_lds = [&](int buf) {
    int8_t *as = As + buf * Cfg::LDS_A;
    int8_t *bs = Bs + buf * Cfg::LDS_B;
#pragma unroll
    for (int c = 0; c < Cfg::A_CHUNKS; ++c)
      *reinterpret_cast<uint4 *>(as + (ld_row + c * 32) * LS + ld_col) = ra[c];
#pragma unroll
    for (int c = 0; c < Cfg::B_CHUNKS; ++c)
      *reinterpret_cast<uint4 *>(bs + (ld_row + c * 32) * LS + ld_col) = rb[c];
  };

  const int col_l = lane & 31, row_l = (lane >> 5) * 4;
  i32x16_t acc[TM][TN];
  float tot[TM][TN][16];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      acc[i][j] = i32x16_t{};
#pragma unroll
      for (int r = 0; r < 16; ++r) tot[i][j][r] = 0.f;
    }

  const int KT = K / BK;
  const int tiles_per_group = group / BK;
  const int ngroups = K / group;
  load_global(0);
  store_lds(0);
  __syncthreads();
  const int frag_row = lane & 31, frag_k = (lane >> 5) * 16;
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load_global((kt + 1) * BK);
    const int8_t *as = As + buf * Cfg::LDS_A + (wm * TM * 32 + frag_row) * LS + frag_k;
    const int8_t *bs = Bs + buf * Cfg::LDS_B + (wn * TN * 32 + frag_row) * LS + frag_k;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      i32x4_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const i32x4_t *>(as + i * 32 * LS + ks * 32);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = *reinterpret_cast<const i32x4_t *>(bs + j * 32 * LS + ks * 32);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if ((kt + 1) % tiles_per_group == 0) {
      const int g = (kt + 1) / tiles_per_group - 1;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          int m = m0 + (wm * TM + i) * 32 + (r / 4) * 8 + row_l + (r % 4);
          m = m < M ? m : M - 1;
          const float sa = SA[static_cast<int64_t>(m) * ngroups + g];
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const float t = static_cast<float>(acc[i][j][r]) * sa;
            tot[i][j][r] = tot[i][j][r] + t;
          }
        }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = i32x16_t{};
    }
    if (kt + 1 < KT) store_lds(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = n0 + (wn * TN + j) * 32 + col_l;
    if (n >= N) continue;
    const float sw = SW[n];
    const float b = bf2f(bias[n]);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + (wm * TM + i) * 32 + (r / 4) * 8 + row_l + (r % 4);
        if (m >= M) continue;
        const float v = tot[i][j][r] * sw;
        const float o = v + b;
        C[static_cast<int64_t>(m) * ldc + n] = static_cast<bf16_t>(f2bf(o));
      }
  }
}

}  // namespace

void launch_gemm_bf16(const bf16_t *A, int64_t lda, const bf16_t *B, int64_t ldb, void *C,
                      int64_t ldc, int M, int N, int K, const bf16_t *bias, const bf16_t *bias2,
                      int epilogue, int out_f32, hipStream_t s) {
  if (out_f32)
    gemm_select<H3_EPI_NONE, 1>(A, lda, B, ldb, C, ldc, M, N, K, bias, bias2, s);
  else if (epilogue == H3_EPI_GELU)
    gemm_select<H3_EPI_GELU, 0>(A, lda, B, ldb, C, ldc, M, N, K, bias, bias2, s);
  else
    gemm_select<H3_EPI_NONE, 0>(A, lda, B, ldb, C, ldc, M, N, K, bias, bias2, s);
}

void launch_gemm_i8(const int8_t *QA, const float *SA, const int8_t *QW, const float *SW,
                    const bf16_t *bias, bf16_t *C, int64_t ldc, int M, int N, int K, int group,
                    hipStream_t s) {
  constexpr int BM = 128, BN = 128;
  using Cfg = GemmI8Cfg<BM, BN, 2, 2>;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  auto kern = gemm_i8_kernel<BM, BN, 2, 2>;
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                        hipFuncAttributeMaxDynamicSharedMemorySize,
                        static_cast<int>(Cfg::LDS_BYTES));
    attr_set = true;
  }
  kern<<<tiles, 256, Cfg::LDS_BYTES, s>>>(QA, SA, QW, SW, bias, C, ldc, M, N, K, group);
}

}  // namespace h3
