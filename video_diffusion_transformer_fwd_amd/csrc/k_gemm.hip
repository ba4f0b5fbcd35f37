// bf16 products of the block on the gfx950 matrix cores:
// C[M,N] = A[M,K] B[N,K]^T (+ bias) (+ bias2) (+ exact GELU), v_mfma_f32_32x32x16_bf16,
// float32 accumulation, bf16 or float32 output.
//
// Tiling: a workgroup of WM x WN wave64s owns a BM x BN output tile (each wave a
// (BM/WM) x (BN/WN) block of 32x32 MFMA tiles) and walks K in BK = 64 slices.  Both operands
// are K-contiguous, so A and B tiles are staged identically, straight from global memory into
// LDS (global_load_lds_dwordx4: 8 consecutive lanes cover one 128-byte row slice), NS slices
// in flight; a slice is consumed once its loads have landed (explicit vmcnt wait + barrier).
// The MFMAs of each slice's last K step are held across that barrier (XBO below).
//
// LDS rows are 64 bf16 = 128 bytes = 8 chunks of 16 bytes, stored without padding: chunk c of
// row r sits at slot c ^ ((r >> 1) & 7).  The MFMA-operand reads (16 bytes per lane, 32 rows at
// one chunk, served 16 lanes = 8 row pairs at a time) then hit distinct bank groups.
//
// Operand layouts (32x32x16 bf16): lane l supplies rows X[p = l%32][k = 8(l/32) .. +7] of the
// first operand and Y[q = l%32][k ...] of the second; accumulator register i of lane l is
// D[8(i/4) + 4(l/32) + i%4][l%32] with D = X Y^T.  The B tile is passed as the first operand
// (D = C^T), so lane l holds row m = l%32 of C at the four runs of 4 consecutive columns
// 8(i/4) + 4(l/32) + 0..3: the epilogue writes 8-byte (bf16) or 16-byte (float32) vectors.
//
// Tile shapes are chosen per problem by plan_gemm (measured on random bf16 operands): 384x192
// tiles (8 waves of 96x96, two per SIMD, two LDS stages), 256x256 or 192x192 tiles for the wide
// QKV / FC1 products by a wave-count model, 256x256 tiles with 8 waves of 128x64 for the narrow
// products at large M, and 192x192 tiles (three LDS stages) with K split in two for the narrow
// (N = d) products of the 1536-token workload and in four at 768 tokens.  192x192 tiles, split or
// not, are run by 8 waves in two K-step groups (KSG below).
//
// Split-K (S pieces of K per tile in separate workgroups): each piece stores its float32 partial
// tile with plain stores; a second launch sums the S partials in piece order 0..S-1 and applies
// the epilogue (for the block's out-projection and FC2 that launch is the gated-residual kernel
// that consumes the product, with the same sum), so the result is deterministic and no
// device-scope fence (which would write back and invalidate L2 under every workgroup) is
// needed.
//
// Workgroup order is XCD-aware: consecutive hardware ids land on different XCDs, so ids are
// regrouped so that each XCD walks a contiguous band of tiles, visited in groups of 8 tile
// rows so neighbours share A rows and B columns in that XCD's L2.
#include <hip/hip_runtime.h>

#include "h3_internal.h"

namespace h3 {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

constexpr int kXcds = 8;
constexpr int kGroupM = 8;

// LDS holds 64 banks of 4 bytes; a 16-byte-per-lane read is served 16 lanes per cycle.  Tile
// rows are 128 bytes, so two rows share one 256-byte bank line: 16-byte chunk c of row r is
// stored at byte r * 128 + ((c ^ ((r >> 1) & 7)) << 4), which puts the 16 rows an MFMA-operand
// read touches at one chunk on 16 distinct 16-byte bank groups.

template <int BM, int BN, int WM, int WN, int NS = 2>
struct GemmCfg {
  static constexpr int NT = 64 * WM * WN;
  static constexpr int BK = 64;
  static constexpr int TM = BM / WM / 32;
  static constexpr int TN = BN / WN / 32;
  static constexpr int A_CHUNKS = BM * 8 / NT;  // 16-byte chunks per thread
  static constexpr int B_CHUNKS = BN * 8 / NT;
  static constexpr int STAGE = (BM + BN) * 128;  // bytes
  static constexpr int EPI_LD = BN + 4;            // float32 row stride of the epilogue band
  static constexpr int EPI_BAND = WM * 32 * EPI_LD;  // floats: one 32-row block of every wave row
  static constexpr size_t EPI_BYTES = (static_cast<size_t>(EPI_BAND) + BN) * 4;
  static constexpr size_t LDS_BYTES =
      NS * static_cast<size_t>(STAGE) > EPI_BYTES ? NS * static_cast<size_t>(STAGE) : EPI_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "tile does not fit the 160 KB LDS");
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile rows must split evenly over threads");
  static_assert(TM >= 1 && TN >= 1 && BM % (WM * 32) == 0 && BN % (WN * 32) == 0,
                "wave tile must be whole 32x32 blocks");
};

struct GemmArgs {
  const bf16_t *A;
  int64_t lda;
  const bf16_t *B;
  int64_t ldb;
  void *C;
  int64_t ldc;
  int M, N, K;
  const bf16_t *bias, *bias2;
  float *part;  // split-K partials [S][M][N]
  QkEpi qk;     // QKV product with the Q/K RMSNorm + RoPE epilogue (QKD > 0)
  // ALN > 0: AdaLN shift and scale [K] applied to the A rows as they are staged
  const float *aln_shift = nullptr, *aln_scale = nullptr;
};

// ALN > 0 (the velocity head): A is the residual stream x [M, K = d] and the staged A tile is
// the final AdaLN of it, n = bf16(((x - mean) rstd) (1 + scale) + shift), formed while the tile
// is loaded (registers -> transform -> LDS) instead of read from a stored n.  The row statistics
// are computed first, for the tile's rows, in the exact order of the AdaLN row kernel with ALN
// waves per row (aln_row_stats), and the transform is that kernel's expression, so the staged
// values are the bits the AdaLN kernel stores and the product equals AdaLN + product bit for bit.
template <int ALN>
__device__ __forceinline__ void aln_row_stats(const bf16_t *__restrict__ x, int64_t ldx, int d,
                                              int row, int lane, float &mean, float &rstd) {
#pragma clang fp contract(off)
  // thread t of the AdaLN kernel's row holds the 8-channel chunks (i * 64 ALN + t) * 8; its
  // waves' butterfly totals are added wave 0 first.  This wave plays those ALN waves in turn.
  const bf16_t *xr = x + static_cast<int64_t>(row) * ldx;
  const int vpl = d / (512 * ALN);
  float tot[ALN];
#pragma unroll
  for (int h = 0; h < ALN; ++h) {
    float sum = 0.f;
    for (int i = 0; i < vpl; ++i) {
      float v[8];
      unpack8(*reinterpret_cast<const uint4 *>(xr + (i * 64 * ALN + h * 64 + lane) * 8), v);
#pragma unroll
      for (int k = 0; k < 8; ++k) sum += v[k];
    }
    tot[h] = wave_sum(sum);
  }
  float ssum = tot[0];
  if constexpr (ALN == 2) ssum = tot[0] + tot[1];
  mean = ssum / static_cast<float>(d);
#pragma unroll
  for (int h = 0; h < ALN; ++h) {
    float q = 0.f;
    for (int i = 0; i < vpl; ++i) {
      float v[8];
      unpack8(*reinterpret_cast<const uint4 *>(xr + (i * 64 * ALN + h * 64 + lane) * 8), v);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float c = v[k] - mean;
        q += c * c;
      }
    }
    tot[h] = wave_sum(q);
  }
  float qsum = tot[0];
  if constexpr (ALN == 2) qsum = tot[0] + tot[1];
  rstd = 1.0f / sqrtf(qsum / static_cast<float>(d) + kLnEps);
}
// One staged 8-channel chunk of the AdaLN output: the AdaLN row kernel's expression.
__device__ __forceinline__ uint4 aln_chunk(const uint4 &xv, float mean, float rstd,
                                           const float4 &sh0, const float4 &sh1, const float4 &sc0,
                                           const float4 &sc1) {
#pragma clang fp contract(off)
  float v[8], o[8];
  unpack8(xv, v);
  const float sh[8] = {sh0.x, sh0.y, sh0.z, sh0.w, sh1.x, sh1.y, sh1.z, sh1.w};
  const float sc[8] = {sc0.x, sc0.y, sc0.z, sc0.w, sc1.x, sc1.y, sc1.z, sc1.w};
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = ((v[k] - mean) * rstd) * (1.0f + sc[k]) + sh[k];
  return pack8(o);
}

// QKD > 0: the QKV product with heads of QKD channels; columns follow QkMap<BN, QKD> and the
// epilogue applies the Q/K RMSNorm + RoPE to the q/k heads (bias, no GELU, bf16, unsplit).
// KSG = 2: twice the waves, in two groups over the same WM x WN layout; each group takes half of
// the 16-wide K steps of every staged slice (two waves per SIMD where one group alone has one),
// and the second group hands its accumulators to the first through LDS: with split K the first
// adds them as it stores the partial tile, unsplit it adds them in registers and both groups run
// the epilogue (only the first writes the LDS band).
// XBO (the K loop without ALN): the MFMAs of every slice's last K step are issued after the
// slice's barrier, from fragments already in registers, so the matrix cores stay busy while
// the next slice's first fragments are read.  XBO = 1 issues them before the next slice's
// copies, XBO = 2 after them.  Measured in the 512x512x22f denoise step (weights streaming from
// HBM): the 192x192 split-K products gain most with 1 (-5.6%), the 384x192 products with 2
// (-2%; with 1 they lose 2%), and the 256x256 products of 61,488 rows with 2.  Every
// accumulator sees its K steps in the same order either way, so the results do not change.
template <int BM, int BN, int WM, int WN, int NS, int EPI, int OUT_F32, int SPLIT, int QKD = 0,
          int KSG = 1, int ALN = 0, int XBO = 1>
__global__ __launch_bounds__(64 * WM * WN * KSG) void gemm_bf16_kernel(GemmArgs g) {
  static_assert(QKD == 0 || (EPI == H3_EPI_NONE && !OUT_F32 && SPLIT == 1), "QKV epilogue form");
  static_assert(ALN == 0 || (QKD == 0 && KSG == 1 && SPLIT == 1 && NS == 3), "AdaLN A operand form");
  static_assert(KSG == 1 || KSG == 2, "one or two K-step groups");
  static_assert(XBO == 1 || XBO == 2, "cross-barrier order");
  using Cfg = GemmCfg<BM, BN, WM, WN, NS>;
  constexpr int NT = Cfg::NT * KSG, BK = Cfg::BK, TM = Cfg::TM, TN = Cfg::TN;
  constexpr int KS_PER = BK / 16 / KSG;  // K steps per slice and wave
  static_assert(KSG == 1 || WM * WN * TM * TN * 16 * 64 * 4 <= Cfg::LDS_BYTES,
                "the accumulator hand-over must fit the LDS");
  // static (its address is known when the kernel is compiled, so the constant parts of the
  // fragment addresses fold into the LDS instructions' offsets)
  __shared__ __align__(16) unsigned char smem[Cfg::LDS_BYTES + (ALN > 0 ? 2 * BM * 4 : 0)];

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
    const int group = id / in_group;
    const int first_m = group * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM);
    const int r = id - group * in_group;
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
  const int wv = wave % (WM * WN), kg = wave / (WM * WN);     // wave of the layout, K-step group
  const int wm = wv / WN, wn = wv % WN;

  // Staging: direct global -> LDS loads (global_load_lds_dwordx4).  One wave instruction fills
  // 8 consecutive tile rows = 1 KiB of LDS, lane L landing at byte 16 L: row R = R0 + L/8, slot
  // L%8, which holds chunk (L%8) ^ ((R >> 1) & 7) of that row.  Row blocks R0 = (i * NW + wave)
  // * 8 walk the A rows then the B rows.  LDS holds the NS A stages, then the NS B stages.
  constexpr int NW = NT / 64;
  constexpr int ROW_BLOCKS = (BM + BN) / 8;
  constexpr int LOADS = ROW_BLOCKS / NW;  // load instructions per wave per K slice
  static_assert(ROW_BLOCKS % NW == 0 && BM % 8 == 0, "row blocks must split evenly over waves");
  const unsigned char *abase = reinterpret_cast<const unsigned char *>(g.A);
  const unsigned char *bbase = reinterpret_cast<const unsigned char *>(g.B);
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
        goff[i] = static_cast<uint32_t>((static_cast<int64_t>(r) * g.lda + kbeg + chunk * 8) * 2);
      } else {
        int r = ncol(R - BM);
        r = r < g.N ? r : g.N - 1;
        goff[i] = static_cast<uint32_t>((static_cast<int64_t>(r) * g.ldb + kbeg + chunk * 8) * 2);
      }
    }
  }
  constexpr int A_BYTES = NS * BM * 128;  // the B stages start here
  // with ALN the A rows (the first LOADS_A row blocks of each wave) go through registers
  constexpr int LOADS_A = ALN > 0 ? BM / 8 / NW : 0;
  constexpr int LOADS_B = LOADS - LOADS_A;  // direct-to-LDS copies per wave per K slice
  static_assert(ALN == 0 || (BM / 8) % NW == 0, "A row blocks must split evenly over waves");
  // copies K slice kt into stage S (a compile-time constant: the LDS targets are scalar)
  auto issue_slice = [&](int kt, auto stage) __attribute__((always_inline)) {
    constexpr int S = decltype(stage)::value;
    const uint32_t kb = static_cast<uint32_t>(kt * BK * 2);
#pragma unroll
    for (int i = LOADS_A; i < LOADS; ++i) {
      const int R0 = (i * NW + wave) * 8;
      const unsigned char *base = (R0 < BM ? abase : bbase) + kb;  // uniform
      const unsigned char *src = base + goff[i];
      lds_u8 *dst = (lds_u8 *)smem +
                    (R0 < BM ? S * BM * 128 + R0 * 128 : A_BYTES + S * BN * 128 + (R0 - BM) * 128);
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(dst), 16, 0, 0);
    }
  };

  // ALN: row statistics of the tile's A rows (rows past M repeat row M - 1), then the A slices
  // are loaded into registers (aload) and written to LDS transformed (astore)
  float *s_stat = reinterpret_cast<float *>(smem + Cfg::LDS_BYTES);  // mean [BM], rstd [BM]
  uint4 areg[LOADS_A > 0 ? LOADS_A : 1];
  float4 ash[LOADS_A > 0 ? LOADS_A : 1][2], asc[LOADS_A > 0 ? LOADS_A : 1][2];
  if constexpr (ALN > 0) {
    for (int r = wave; r < BM; r += NW) {
      float mean, rstd;
      aln_row_stats<ALN>(g.A, g.lda, g.K, min(m0 + r, g.M - 1), lane, mean, rstd);
      if (lane == 0) {
        s_stat[r] = mean;
        s_stat[BM + r] = rstd;
      }
    }
    __syncthreads();
  }
  auto aload = [&](int kt) __attribute__((always_inline)) {
    const uint32_t kb = static_cast<uint32_t>(kt * BK * 2);
#pragma unroll
    for (int i = 0; i < LOADS_A; ++i) {
      const int R = (i * NW + wave) * 8 + (lane >> 3);
      const int col = kbeg + kt * BK + ((lane & 7) ^ ((R >> 1) & 7)) * 8;
      areg[i] = *reinterpret_cast<const uint4 *>(abase + kb + goff[i]);
      ash[i][0] = *reinterpret_cast<const float4 *>(g.aln_shift + col);
      ash[i][1] = *reinterpret_cast<const float4 *>(g.aln_shift + col + 4);
      asc[i][0] = *reinterpret_cast<const float4 *>(g.aln_scale + col);
      asc[i][1] = *reinterpret_cast<const float4 *>(g.aln_scale + col + 4);
    }
  };
  auto astore = [&](auto stage) __attribute__((always_inline)) {
    constexpr int S = decltype(stage)::value;
#pragma unroll
    for (int i = 0; i < LOADS_A; ++i) {
      const int R = (i * NW + wave) * 8 + (lane >> 3);
      const uint4 o = aln_chunk(areg[i], s_stat[R], s_stat[BM + R], ash[i][0], ash[i][1], asc[i][0], asc[i][1]);
      *reinterpret_cast<__attribute__((address_space(3))) u32x4_t *>(
          (lds_u8 *)smem + S * BM * 128 + R * 128 + (lane & 7) * 16) = u32x4_t{o.x, o.y, o.z, o.w};
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16_t{};

  // Fragment addresses.  Row (wm TM + i) 32 + fr of A has swizzle key (fr >> 1) & 7 for every i,
  // so the chunk 2 ks + fh of that row sits at a_lane ^ 32 ks + 4096 i (+ BM 128 S for stage S),
  // with a_lane the lane's row of block 0 and its swizzled chunk fh; B likewise from b_lane.
  const int fr = lane & 31, fh = lane >> 5;
  // (group kg starts at K step kg KS_PER: 32 kg KS_PER is folded into the lane bases)
  const int a_lane = ((wm * TM * 32 + fr) * 128 + ((fh ^ ((fr >> 1) & 7)) << 4)) ^ (32 * KS_PER * kg);
  const int b_lane = (A_BYTES + (wn * TN * 32 + fr) * 128 + ((fh ^ ((fr >> 1) & 7)) << 4)) ^ (32 * KS_PER * kg);
  const lds_u8 *lds = (const lds_u8 *)smem;

  // NS-stage pipeline: slices kt+1 .. kt+NS-1 stream into LDS while slice kt feeds the MFMAs.
  // The K loop is unrolled over the stages, so each stage's offsets are compile-time constants.
  const int KT = kc / BK;
  if constexpr (ALN > 0) {
    aload(0);
    issue_slice(0, std::integral_constant<int, 0>{});
    astore(std::integral_constant<int, 0>{});
    if (KT > 1) {
      aload(1);
      issue_slice(1, std::integral_constant<int, 1>{});
      astore(std::integral_constant<int, 1>{});
    }
    lds_dma_write_barrier<0>();
  } else {
    issue_slice(0, std::integral_constant<int, 0>{});
    if constexpr (NS == 3)
      if (KT > 1) issue_slice(1, std::integral_constant<int, 1>{});
    if (KT >= NS - 1)
      lds_dma_barrier<LOADS * (NS - 2)>();
    else
      lds_dma_barrier<0>();
  }

  // without ALN the last K step of each slice is held across the slice's barrier (XBO above);
  // fragment buffer 1 holds that step (KS_PER is even), buffer 0 the next slice's first step
  constexpr bool XB = ALN == 0;
  static_assert(KS_PER % 2 == 0, "the last K step's fragments must sit in buffer 1");
  bf16x8_t af[2][TM], bfr[2][TN];
  auto held_step = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[1][j], af[1][i], acc[i][j], 0, 0, 0);
  };
  auto slice = [&](int kt, auto stage) __attribute__((always_inline)) {
    constexpr int S = decltype(stage)::value;
    const bool more = kt + NS - 1 < KT;
    auto afrag = [&](int i, int ks) {
      return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t *>(
          lds + ((a_lane ^ (32 * ks)) + S * BM * 128 + i * 4096));
    };
    auto bfrag = [&](int j, int ks) {
      return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t *>(
          lds + ((b_lane ^ (32 * ks)) + S * BN * 128 + j * 4096));
    };
    if constexpr (!XB) {
      if (more) {
        aload(kt + NS - 1);
        issue_slice(kt + NS - 1, std::integral_constant<int, (S + NS - 1) % NS>{});
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) af[0][i] = afrag(i, 0);
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[0][j] = bfrag(j, 0);
    if constexpr (XB && XBO == 1) {
      if (kt > 0) held_step();
      if (more) issue_slice(kt + NS - 1, std::integral_constant<int, (S + NS - 1) % NS>{});
    } else if constexpr (XB) {
      if (more) issue_slice(kt + NS - 1, std::integral_constant<int, (S + NS - 1) % NS>{});
      __builtin_amdgcn_sched_barrier(0);
      if (kt > 0) held_step();
    }
    __builtin_amdgcn_sched_barrier(0);
    constexpr int KS_MMA = XB ? KS_PER - 1 : KS_PER;  // K steps whose MFMAs issue in this slice
#pragma unroll
    for (int ks = 0; ks < KS_MMA; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < KS_PER) {
#pragma unroll
        for (int i = 0; i < TM; ++i) af[cur ^ 1][i] = afrag(i, ks + 1);
#pragma unroll
        for (int j = 0; j < TN; ++j) bfr[cur ^ 1][j] = bfrag(j, ks + 1);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[cur][j], af[cur][i], acc[i][j], 0, 0, 0);
      // interleave: one MFMA, one fragment read of the next step, ... so the reads are in flight
      // while this step's MFMAs run
      if (ks + 1 < KS_PER) {
#pragma unroll
        for (int q = 0; q < TM + TN; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - (TM + TN), 0);
      }
    }
    // slice kt+1 must be complete (later slices may still be in flight); every wave must be
    // done reading stage S before the next slice refills it (with XB that includes the held
    // step's fragment reads, hence the LDS-count wait)
    if constexpr (ALN > 0) {
      // the A rows of slice kt + NS - 1, transformed into the stage this slice's loads target
      // (its registers have landed: the loads were issued before this slice's MFMAs)
      if (more) astore(std::integral_constant<int, (S + NS - 1) % NS>{});
      if (more)
        lds_dma_write_barrier<LOADS_B * (NS - 2)>();
      else
        lds_dma_write_barrier<0>();
    } else {
      if (more)
        lds_dma_write_barrier<LOADS * (NS - 2)>();
      else
        lds_dma_write_barrier<0>();
    }
  };
  for (int kt = 0; kt < KT; kt += NS) {
    slice(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < KT) slice(kt + 1, std::integral_constant<int, 1>{});
    if constexpr (NS == 3)
      if (kt + 2 < KT) slice(kt + 2, std::integral_constant<int, 2>{});
  }
  if constexpr (XB) {
    if (KT > 0) held_step();
  }

  // lane holds C[m_l][n_l + 8q + e], e = 0..3, in accumulator registers 4q + e of each 32x32 block
  const int m_l = lane & 31, n_l = (lane >> 5) * 4;
  // the second group's accumulators join the first's: float [wave][i][j][r][lane] in the
  // (now free) LDS, consecutive lanes on consecutive words
  const float *xch = reinterpret_cast<const float *>(smem) + wv * (TM * TN * 16 * 64);
  if constexpr (KSG == 2) {
    float *xw = reinterpret_cast<float *>(smem) + wv * (TM * TN * 16 * 64);
    __syncthreads();  // every wave is done with the staged slices (no copy is in flight)
    if (kg == 1) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) xw[((i * TN + j) * 16 + r) * 64 + lane] = acc[i][j][r];
    }
    __syncthreads();
    if constexpr (SPLIT > 1) {
      if (kg == 1) return;  // no barrier follows; the first group adds them as it stores
    } else {
      // the first group takes the sums; both groups then run the epilogue, whose opening
      // barrier also orders these LDS reads before the band overwrites them
      if (kg == 0) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = acc[i][j][r] + xch[((i * TN + j) * 16 + r) * 64 + lane];
      }
    }
  }
  if constexpr (SPLIT > 1) {
    // split-K: store this K piece's float32 partial tile, row-major [piece][M][N] (N % 4 == 0);
    // a separate reduction launch sums the pieces in order and applies the epilogue
    float *part = g.part + static_cast<int64_t>(split) * g.M * g.N;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + (wm * TM + i) * 32 + m_l;
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        // (with two K-step groups the second group's block is added here, one block at a
        // time: adding all of them first would hold a second copy of the accumulators)
        float v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          v[r] = acc[i][j][r];
          if constexpr (KSG == 2) v[r] += xch[((i * TN + j) * 16 + r) * 64 + lane];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + (wn * TN + j) * 32 + q * 8 + n_l;
          if (n < g.N)
            *reinterpret_cast<float4 *>(part + static_cast<int64_t>(m) * g.N + n) =
                make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        }
      }
    }
    return;
  }

  // Epilogue through LDS (free once the last slice is consumed): the column sums of the biases
  // are staged once; then, for each 32-row block index i, every wave writes its accumulators
  // of that block to a float32 band of WM * 32 rows x BN columns (row stride BN + 4: the 16
  // rows of a 16-lane write group land on distinct banks), and all threads walk the band in
  // 4-column chunks with a rolled loop: bias, GELU, conversion, one 8-byte (bf16) or 16-byte
  // (float32) store per chunk, consecutive threads on consecutive columns of a row.  The code
  // stays compact (a fully unrolled register epilogue is several thousand instructions that
  // every wave fetches once, cold, while the MFMAs sit idle).
  constexpr int LD = Cfg::EPI_LD;
  float *band = reinterpret_cast<float *>(smem);
  float *sbias = band + Cfg::EPI_BAND;
  __syncthreads();
  for (int c = tid; c < BN; c += NT) {
    const int n = ncol(c);
    float bs = 0.f;
    if (n < g.N) {
      if (g.bias) bs += bf2f(g.bias[n]);
      if (g.bias2) bs += bf2f(g.bias2[n]);
    }
    sbias[c] = bs;
  }
  // vector stores need 4 | ldc and an 8-byte (bf16) / 16-byte (float32) aligned C
  const bool vec = (g.ldc % 4 == 0) &&
                   (reinterpret_cast<uintptr_t>(g.C) % (OUT_F32 ? 16 : 8) == 0);
  constexpr int CHUNKS_PER_ROW = BN / 4;
  constexpr int BAND_CHUNKS = WM * 32 * CHUNKS_PER_ROW;
  if constexpr (QKD > 0) {
    // QKV: the leading hc columns of the tile are whole q/k heads, normalised and rotated by
    // QkHeadPass (the bf16 value the plain product stores, then RMSNorm + RoPE); the remaining
    // columns get the plain bias epilogue.  Each band's rotation slices and gains are fetched
    // while the previous band's plain columns are stored.  The host guarantees 8 | ldc, a
    // 16-byte aligned C and table.
    using Map = QkMap<BN, QKD>;
    QkHeadPass<BN, QKD, WM, TM, NT> hp(g.qk, tid, tn, m0, g.M);
    const int hc = hp.hpr * QKD;
    const int pc4 = (BN - hc) / 4;  // 4-column chunks per row after the heads
    bf16_t *C = reinterpret_cast<bf16_t *>(g.C);
    hp.fetch(0);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (i > 0) __syncthreads();
      if (KSG == 1 || kg == 0) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4 *>(band + (wm * 32 + m_l) * LD + (wn * TN + j) * 32 + q * 8 + n_l) =
                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
      }
      __syncthreads();
      hp.run(i, [&](int row, int col, float *a) {
        const float4 *bp = reinterpret_cast<const float4 *>(band + row * LD + col);
        const float4 *sp = reinterpret_cast<const float4 *>(sbias + col);
        const float4 v0 = bp[0], v1 = bp[1], b0 = sp[0], b1 = sp[1];
        const float v[8] = {v0.x + b0.x, v0.y + b0.y, v0.z + b0.z, v0.w + b0.w,
                            v1.x + b1.x, v1.y + b1.y, v1.z + b1.z, v1.w + b1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = bf2f(f2bf(v[e]));
      }, C, g.ldc);
      if (i + 1 < TM) hp.fetch(i + 1);
      for (int c4 = tid; c4 < WM * 32 * pc4; c4 += NT) {
        const int row = c4 / pc4, col = hc + (c4 - row * pc4) * 4;
        const int m = m0 + ((row >> 5) * TM + i) * 32 + (row & 31);
        const int n = Map::col(tn, col, g.qk.d);
        if (m >= g.M || n >= g.N) continue;
        const float4 a4 = *reinterpret_cast<const float4 *>(band + row * LD + col);
        const float4 b4 = *reinterpret_cast<const float4 *>(sbias + col);
        uint2 pk;
        pk.x = pack_bf2(a4.x + b4.x, a4.y + b4.y);
        pk.y = pack_bf2(a4.z + b4.z, a4.w + b4.w);
        *reinterpret_cast<uint2 *>(C + static_cast<int64_t>(m) * g.ldc + n) = pk;
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    if (i > 0) __syncthreads();  // previous band fully read
    if (KSG == 1 || kg == 0) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<float4 *>(band + (wm * 32 + m_l) * LD + (wn * TN + j) * 32 + q * 8 + n_l) =
              make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
    }
    __syncthreads();
#pragma unroll 2
    for (int c4 = tid; c4 < BAND_CHUNKS; c4 += NT) {
      const int row = c4 / CHUNKS_PER_ROW, col = (c4 - row * CHUNKS_PER_ROW) * 4;
      const int m = m0 + ((row >> 5) * TM + i) * 32 + (row & 31);
      const int n = n0 + col;
      if (m >= g.M || n >= g.N) continue;
      const float4 a4 = *reinterpret_cast<const float4 *>(band + row * LD + col);
      const float4 b4 = *reinterpret_cast<const float4 *>(sbias + col);
      float v[4] = {a4.x + b4.x, a4.y + b4.y, a4.z + b4.z, a4.w + b4.w};
      if constexpr (EPI == H3_EPI_GELU) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = gelu_erf(v[e]);
      }
      const int64_t off = static_cast<int64_t>(m) * g.ldc + n;
      if (vec && n + 3 < g.N) {
        if constexpr (OUT_F32) {
          *reinterpret_cast<float4 *>(reinterpret_cast<float *>(g.C) + off) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
          uint2 pk;
          pk.x = pack_bf2(v[0], v[1]);
          pk.y = pack_bf2(v[2], v[3]);
          *reinterpret_cast<uint2 *>(reinterpret_cast<bf16_t *>(g.C) + off) = pk;
        }
      } else {
        for (int e = 0; e < 4 && n + e < g.N; ++e) {
          if constexpr (OUT_F32)
            reinterpret_cast<float *>(g.C)[off + e] = v[e];
          else
            reinterpret_cast<bf16_t *>(g.C)[off + e] = static_cast<bf16_t>(f2bf(v[e]));
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int NS, int EPI, int OUT_F32, int SPLIT, int QKD = 0,
          int KSG = 1, int ALN = 0, int XBO = 1>
void run_gemm(const GemmArgs &a, hipStream_t s) {
  using Cfg = GemmCfg<BM, BN, WM, WN, NS>;
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  auto kern = gemm_bf16_kernel<BM, BN, WM, WN, NS, EPI, OUT_F32, SPLIT, QKD, KSG, ALN, XBO>;
  kern<<<tiles * SPLIT, Cfg::NT * KSG, 0, s>>>(a);
}

// Sums the split-K partials [S][M][N] in piece order and applies the bias / GELU epilogue.
template <int EPI, int OUT_F32, int S>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part, int M,
                                                            int N, const bf16_t *__restrict__ bias,
                                                            const bf16_t *__restrict__ bias2,
                                                            void *__restrict__ C, int64_t ldc) {
  const int64_t i4 = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  const int64_t total = static_cast<int64_t>(M) * N;
  if (i4 >= total) return;
  const int m = static_cast<int>(i4 / N), n = static_cast<int>(i4 - static_cast<int64_t>(m) * N);
  float4 t = *reinterpret_cast<const float4 *>(part + i4);
#pragma unroll
  for (int q = 1; q < S; ++q) {
    const float4 v = *reinterpret_cast<const float4 *>(part + q * total + i4);
    t.x += v.x; t.y += v.y; t.z += v.z; t.w += v.w;
  }
  float v[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float b = 0.f;
    if (bias) b += bf2f(bias[n + e]);
    if (bias2) b += bf2f(bias2[n + e]);
    v[e] = v[e] + b;
    if constexpr (EPI == H3_EPI_GELU) v[e] = gelu_erf(v[e]);
  }
  if constexpr (OUT_F32) {
    float *c = reinterpret_cast<float *>(C) + static_cast<int64_t>(m) * ldc + n;
    c[0] = v[0]; c[1] = v[1]; c[2] = v[2]; c[3] = v[3];
  } else {
    uint2 w;
    w.x = pack_bf2(v[0], v[1]);
    w.y = pack_bf2(v[2], v[3]);
    *reinterpret_cast<uint2 *>(reinterpret_cast<bf16_t *>(C) + static_cast<int64_t>(m) * ldc + n) = w;
  }
}

// One product: the tiled GEMM, then (split-K) the ordered reduction with the epilogue.
// split-K products and the unsplit 192x192 tiles run with two K-step groups (two waves per
// SIMD)
template <int BM, int BN, int WM, int WN, int NS, int EPI, int OUT_F32, int S, int XBO = 1,
          int KSG = (S > 1 ? 2 : 1)>
void run_product(const GemmArgs &a, hipStream_t s) {
  run_gemm<BM, BN, WM, WN, NS, EPI, OUT_F32, S, 0, KSG, 0, XBO>(a, s);
  if constexpr (S > 1) {
    const int64_t total = static_cast<int64_t>(a.M) * a.N;
    splitk_reduce_kernel<EPI, OUT_F32, S><<<static_cast<int>((total / 4 + 255) / 256), 256, 0, s>>>(
        a.part, a.M, a.N, a.bias, a.bias2, a.C, a.ldc);
  }
}

template <int EPI, int OUT_F32>
void gemm_dispatch(const GemmPlan &p, const GemmArgs &a, hipStream_t s) {
  switch (p.cfg * 8 + p.split) {
    case 4 * 8 + 1: run_product<384, 192, 4, 2, 2, EPI, OUT_F32, 1, 2>(a, s); break;
    case 2 * 8 + 1: run_product<256, 256, 2, 4, 2, EPI, OUT_F32, 1, 2>(a, s); break;
    case 1 * 8 + 1: run_product<192, 192, 2, 2, 3, EPI, OUT_F32, 1, 1, 2>(a, s); break;
    case 1 * 8 + 2: run_product<192, 192, 2, 2, 3, EPI, OUT_F32, 2>(a, s); break;
    case 1 * 8 + 4: run_product<192, 192, 2, 2, 3, EPI, OUT_F32, 4>(a, s); break;
    default: run_product<128, 128, 2, 2, 3, EPI, OUT_F32, 1>(a, s); break;
  }
}

}  // namespace

// The wide products (QKV, FC1: N >= 8192) take whichever of the 384x192, 256x256 and 192x192
// tiles needs the least time by a simple model: waves of tiles over the 256 CUs (a partly
// filled last wave costs a whole one) times the outputs per tile, 192x192 tiles weighted
// 1.15 for their lower per-output rate.  Measured (FC1-shaped, K = 3072): at 1536 rows the
// 384x192 tiles make exactly one wave (110 us; 256x256 165 us); at 2430 rows (864x480) the
// 384-row tiles leave a last row block a third full and 1.75 waves, 256x256 tiles 1.88 waves
// of smaller tiles (183-200 against 209-220 us); at 1260 rows (864x480 paired) 256x256 tiles
// make one wave (94 us against 110 for 384x192 and 126 for 192x192); at 768 rows 192x192
// (70 us); at 61,488 rows the model ties and 384x192 is 2% faster.
int wide_tile_cfg(int M, int N) {
  auto cost = [&](int bm, int bn, double w) {
    const int64_t tiles = static_cast<int64_t>((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    return static_cast<double>((tiles + 255) / 256) * bm * bn * w;
  };
  const double c4 = cost(384, 192, 1.0), c2 = cost(256, 256, 1.0), c1 = cost(192, 192, 1.15);
  // ties (within 2%) go to 384x192, then to 256x256
  if (c4 <= 1.02 * c2 && c4 <= 1.02 * c1) return 4;
  return c2 <= c1 ? 2 : 1;
}

// Tile choice measured on the MI355X with random bf16 operands:
//   N >= 8192, M >= 192             wide_tile_cfg above               (QKV, FC1)
//   M >= 4096, N >= 2048            256x256, 8 waves                 (narrow products, 768x1344)
//   1024 <= M < 4096, N < 8192      192x192, K split in 2            (out-proj, FC2 at 1536)
//   192 <= M < 1024, N < 8192       192x192, K split in 4            (out-proj, FC2 at 768)
//   otherwise                       128x128
// A split needs K % (64 * split) == 0 and N % 4 == 0, else the product runs unsplit.
GemmPlan plan_gemm(int M, int N, int K) {
  GemmPlan p{};
  p.cfg = 0;
  p.split = 1;
  if (N >= 8192 && M >= 192) {
    p.cfg = wide_tile_cfg(M, N);
  } else if (M >= 4096 && N >= 2048) {
    p.cfg = 2;
  } else if (M >= 1024 && N >= 256) {
    p.cfg = 1;
    p.split = 2;
  } else if (M >= 192 && N >= 192) {
    p.cfg = 1;
    p.split = 4;
  }
  if (p.split > 1 && (K % (64 * p.split) != 0 || N % 4 != 0 || K / p.split < 1024)) p.split = 1;
  if (p.split > 1) p.part_bytes = static_cast<size_t>(p.split) * M * N * sizeof(float);
  return p;
}

int launch_gemm_bf16_partials(const bf16_t *A, int64_t lda, const bf16_t *B, int64_t ldb, int M,
                              int N, int K, hipStream_t s, const SplitScratch &sc) {
  const GemmPlan p = plan_gemm(M, N, K);
  if (p.split <= 1 || !sc.part || p.part_bytes > sc.part_bytes) return 0;
  GemmArgs a{A, lda, B, ldb, nullptr, 0, M, N, K, nullptr, nullptr, sc.part};
  switch (p.cfg * 8 + p.split) {
    case 1 * 8 + 2: run_gemm<192, 192, 2, 2, 3, H3_EPI_NONE, 0, 2, 0, 2>(a, s); return 2;
    case 1 * 8 + 4: run_gemm<192, 192, 2, 2, 3, H3_EPI_NONE, 0, 4, 0, 2>(a, s); return 4;
    default: return 0;
  }
}

void launch_gemm_bf16(const bf16_t *A, int64_t lda, const bf16_t *B, int64_t ldb, void *C,
                      int64_t ldc, int M, int N, int K, const bf16_t *bias, const bf16_t *bias2,
                      int epilogue, int out_f32, hipStream_t s, const SplitScratch &sc) {
  GemmPlan p = plan_gemm(M, N, K);
  if (p.split > 1 && (!sc.part || p.part_bytes > sc.part_bytes))
    p.split = 1;  // no split-K scratch: run the whole K per tile
  GemmArgs a{A, lda, B, ldb, C, ldc, M, N, K, bias, bias2, sc.part};
  if (out_f32)
    gemm_dispatch<H3_EPI_NONE, 1>(p, a, s);
  else if (epilogue == H3_EPI_GELU)
    gemm_dispatch<H3_EPI_GELU, 0>(p, a, s);
  else
    gemm_dispatch<H3_EPI_NONE, 0>(p, a, s);
}

namespace {
template <int QKD>
void qkv_dispatch(const GemmPlan &p, const GemmArgs &a, hipStream_t s) {
  switch (p.cfg) {
    case 4: run_gemm<384, 192, 4, 2, 2, H3_EPI_NONE, 0, 1, QKD, 1, 0, 2>(a, s); break;
    case 2: run_gemm<256, 256, 2, 4, 2, H3_EPI_NONE, 0, 1, QKD, 1, 0, 2>(a, s); break;
    case 1: run_gemm<192, 192, 2, 2, 3, H3_EPI_NONE, 0, 1, QKD, 2>(a, s); break;
    default: run_gemm<128, 128, 2, 2, 3, H3_EPI_NONE, 0, 1, QKD>(a, s); break;
  }
}
}  // namespace

bool head_adaln_gemm_fits(const bf16_t *x, int64_t ldx, const float *shift, const float *scale,
                          int M, int N, int d) {
  // below 192 columns the plain product always takes the 128x128 unsplit tiles reproduced here
  const GemmPlan p = plan_gemm(M, N, d);
  return N < 192 && p.cfg == 0 && p.split == 1 && d % (512 * adaln_waves_per_row(M, d)) == 0 &&
         ldx % 8 == 0 &&
         reinterpret_cast<uintptr_t>(x) % 16 == 0 && reinterpret_cast<uintptr_t>(shift) % 16 == 0 &&
         reinterpret_cast<uintptr_t>(scale) % 16 == 0;
}

int launch_head_adaln_gemm(const bf16_t *x, int64_t ldx, const float *shift, const float *scale,
                           const bf16_t *W, int64_t ldw, const bf16_t *bias, float *out,
                           int64_t ldo, int M, int N, int d, hipStream_t s) {
  if (!head_adaln_gemm_fits(x, ldx, shift, scale, M, N, d)) return 0;
  const int wpr = adaln_waves_per_row(M, d);
  GemmArgs a{x, ldx, W, ldw, out, ldo, M, N, d, bias, nullptr, nullptr};
  a.aln_shift = shift;
  a.aln_scale = scale;
  if (wpr == 2)
    run_gemm<128, 128, 2, 2, 3, H3_EPI_NONE, 1, 1, 0, 1, 2>(a, s);
  else
    run_gemm<128, 128, 2, 2, 3, H3_EPI_NONE, 1, 1, 0, 1, 1>(a, s);
  return 1;
}

int launch_gemm_bf16_qkv(const bf16_t *A, int64_t lda, const bf16_t *W, int64_t ldw,
                         const bf16_t *bias, bf16_t *C, int64_t ldc, int M, int d, int K,
                         int head_dim, const QkEpi &qk, hipStream_t s) {
  const GemmPlan p = plan_gemm(M, 4 * d, K);
  if (p.split > 1 || (head_dim != 64 && head_dim != 128) || d % 128 || ldc % 8 ||
      reinterpret_cast<uintptr_t>(C) % 16 ||
      reinterpret_cast<uintptr_t>(qk.table) % 16)
    return 0;
  GemmArgs a{A, lda, W, ldw, C, ldc, M, 4 * d, K, bias, nullptr, nullptr, qk};
  if (head_dim == 128)
    qkv_dispatch<128>(p, a, s);
  else
    qkv_dispatch<64>(p, a, s);
  return 1;
}

}  // namespace h3
