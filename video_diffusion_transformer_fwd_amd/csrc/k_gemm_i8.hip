// int8 product of the per-row / grouped int8 FC2 on the gfx950 matrix cores.
//
// C[M,N] = bf16(((sum_g float(acc_g) * SA[m,g]) * SW[n]) + bias[n]) with acc_g the exact int32
// sum of QA[m,k] QW[n,k] over K group g (v_mfma_i32_32x32x32_i8: lane l supplies 16
// consecutive k at 16(l/32) of row l%32 for both operands).  Same tiling skeleton as the bf16
// product: 256-thread workgroup, 128x128 tile, BK = 128 bytes, padded LDS, double-buffered.
#include <hip/hip_runtime.h>

#include "h3_internal.h"

namespace h3 {

namespace {

typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(16))) int i32x16_t;

constexpr int kXcds = 8;
constexpr int kGroupM = 8;

__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int &tm, int &tn) {
  const int nwg = tiles_m * tiles_n;
  int id = blockIdx.x;
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
