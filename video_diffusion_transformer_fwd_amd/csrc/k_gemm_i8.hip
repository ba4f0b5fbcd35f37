// int8 product of the per-row / grouped int8 FC2 on the gfx950 matrix cores.
//
// C[M,N] = bf16(((sum_g float(acc_g) * SA[m,g]) * SW[n]) + bias[n]) with acc_g the exact int32
// sum of QA[m,k] QW[n,k] over K group g (groups ascending, each float operation rounded, no
// fused multiply-add), v_mfma_i32_32x32x32_i8: lane l supplies 16 consecutive k at 16(l/32) of
// row l%32 for both operands; accumulator register i of lane l is C[8(i/4) + 4(l/32) + i%4][l%32].
//
// Same pipeline as the bf16 product: a K slice is 128 int8 = 128 bytes per row, so the LDS tile
// rows, their bank swizzle (chunk c of row r in slot c ^ ((r >> 1) & 7)) and the direct
// global -> LDS staging are identical; three LDS stages; each 32-wide K step's fragment reads
// are issued while the previous step's MFMAs run.  At each group end the int32 sums are folded
// into a float32 total and cleared.
#include <hip/hip_runtime.h>

#include "h3_internal.h"

namespace h3 {

namespace {

typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(16))) int i32x16_t;

constexpr int kXcds = 8;
constexpr int kGroupM = 8;

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

constexpr int waitcnt_vm(int vm) { return (vm & 15) | (7 << 4) | (15 << 8) | ((vm >> 4) << 14); }

template <int VM>
__device__ __forceinline__ void lds_dma_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM));
  __builtin_amdgcn_s_barrier();
}

template <int BM, int BN, int WM, int WN, int NS>
struct GemmI8Cfg {
  static constexpr int NT = 64 * WM * WN;
  static constexpr int BK = 128;  // int8 elements = bytes per row per slice
  static constexpr int TM = BM / WM / 32;
  static constexpr int TN = BN / WN / 32;
  static constexpr int STAGE = (BM + BN) * 128;
  static constexpr size_t LDS_BYTES = NS * static_cast<size_t>(STAGE);
};

template <int BM, int BN, int WM, int WN, int NS>
__global__ __launch_bounds__(64 * WM * WN) void gemm_i8_kernel(
    const int8_t *__restrict__ QA, const float *__restrict__ SA, const int8_t *__restrict__ QW,
    const float *__restrict__ SW, const bf16_t *__restrict__ bias, bf16_t *__restrict__ C,
    int64_t ldc, int M, int N, int K, int group) {
#pragma clang fp contract(off)
  using Cfg = GemmI8Cfg<BM, BN, WM, WN, NS>;
  constexpr int NT = Cfg::NT, BK = Cfg::BK, TM = Cfg::TM, TN = Cfg::TN;
  extern __shared__ __align__(16) unsigned char smem8[];

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  {
    const int ntiles = tiles_m * tiles_n;
    int id = blockIdx.x;
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
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // direct global -> LDS staging, as in the bf16 product (1 byte per element here)
  constexpr int NW = NT / 64;
  constexpr int ROW_BLOCKS = (BM + BN) / 8;
  constexpr int LOADS = ROW_BLOCKS / NW;
  static_assert(ROW_BLOCKS % NW == 0 && BM % 8 == 0, "row blocks must split evenly over waves");
  const unsigned char *abase = reinterpret_cast<const unsigned char *>(QA);
  const unsigned char *bbase = reinterpret_cast<const unsigned char *>(QW);
  uint32_t goff[LOADS];
  {
    const int lrow = lane >> 3;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int R = (i * NW + wave) * 8 + lrow;
      const int chunk = (lane & 7) ^ ((R >> 1) & 7);
      if (R < BM) {
        int r = m0 + R;
        r = r < M ? r : M - 1;
        goff[i] = static_cast<uint32_t>(static_cast<int64_t>(r) * K + chunk * 16);
      } else {
        int r = n0 + R - BM;
        r = r < N ? r : N - 1;
        goff[i] = static_cast<uint32_t>(static_cast<int64_t>(r) * K + chunk * 16);
      }
    }
  }
  auto issue_slice = [&](int stage, int kt) {
    const uint32_t kb = static_cast<uint32_t>(kt * BK);
    unsigned char *st = smem8 + stage * Cfg::STAGE;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int R0 = (i * NW + wave) * 8;
      const unsigned char *src = (R0 < BM ? abase : bbase) + (goff[i] + kb);
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(st + R0 * 128), 16, 0, 0);
    }
  };

  const int fr = lane & 31, fh = lane >> 5;
  int a_row[TM], b_row[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) a_row[i] = (wm * TM + i) * 32 + fr;
#pragma unroll
  for (int j = 0; j < TN; ++j) b_row[j] = (wn * TN + j) * 32 + fr;

  const int row_l = fh * 4;
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
  const int slices_per_group = group / BK;
  const int ngroups = K / group;
#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
    if (p < KT) issue_slice(p, p);
  if (KT >= NS - 1)
    lds_dma_barrier<LOADS * (NS - 2)>();
  else
    lds_dma_barrier<0>();

  for (int kt = 0; kt < KT; ++kt) {
    const unsigned char *st = smem8 + (kt % NS) * Cfg::STAGE;
    const bool more = kt + NS - 1 < KT;
    if (more) issue_slice((kt + NS - 1) % NS, kt + NS - 1);
    i32x4_t af[2][TM], bfr[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) af[0][i] = *reinterpret_cast<const i32x4_t *>(st + swz(a_row[i], fh));
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[0][j] = *reinterpret_cast<const i32x4_t *>(st + BM * 128 + swz(b_row[j], fh));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < BK / 32) {
        const int ch = 2 * (ks + 1) + fh;
#pragma unroll
        for (int i = 0; i < TM; ++i) af[cur ^ 1][i] = *reinterpret_cast<const i32x4_t *>(st + swz(a_row[i], ch));
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bfr[cur ^ 1][j] = *reinterpret_cast<const i32x4_t *>(st + BM * 128 + swz(b_row[j], ch));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[cur][i], bfr[cur][j], acc[i][j], 0, 0, 0);
      if (ks + 1 < BK / 32) {
#pragma unroll
        for (int q = 0; q < TM + TN; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if (TM * TN > TM + TN) __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - (TM + TN), 0);
      }
    }
    // group end: tot += float(acc) * SA[m, g], then clear acc
    if ((kt + 1) % slices_per_group == 0) {
      const int g = (kt + 1) / slices_per_group - 1;
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
    if (more)
      lds_dma_barrier<LOADS * (NS - 2)>();
    else
      lds_dma_barrier<0>();
  }

  const int col_l = lane & 31;
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

template <int BM, int BN, int WM, int WN, int NS>
void run_gemm_i8(const int8_t *QA, const float *SA, const int8_t *QW, const float *SW,
                 const bf16_t *bias, bf16_t *C, int64_t ldc, int M, int N, int K, int group,
                 hipStream_t s) {
  using Cfg = GemmI8Cfg<BM, BN, WM, WN, NS>;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  auto kern = gemm_i8_kernel<BM, BN, WM, WN, NS>;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(Cfg::LDS_BYTES));
    attr_set = true;
  }
  kern<<<tiles, Cfg::NT, Cfg::LDS_BYTES, s>>>(QA, SA, QW, SW, bias, C, ldc, M, N, K, group);
}

}  // namespace

void launch_gemm_i8(const int8_t *QA, const float *SA, const int8_t *QW, const float *SW,
                    const bf16_t *bias, bf16_t *C, int64_t ldc, int M, int N, int K, int group,
                    hipStream_t s) {
  run_gemm_i8<128, 128, 2, 2, 3>(QA, SA, QW, SW, bias, C, ldc, M, N, K, group, s);
}

}  // namespace h3
