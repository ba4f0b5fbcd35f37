// Internal declarations shared by the HIP sources of libh3dit.so.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/h3dit.h"

namespace h3 {

// ---------------------------------------------------------------- errors
void set_error(const std::string &msg);
void clear_error();
int32_t fail(int32_t code, const std::string &msg);
// Checks the launch status of the last kernel(s); returns H3_OK or H3_EHIP.
int32_t check_launch(const char *what);

// ---------------------------------------------------------------- bf16 helpers
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// Round-to-nearest-even float32 -> bf16 bits (v_cvt_pk_bf16_f32 on gfx950; NaN stays NaN).
typedef __attribute__((ext_vector_type(2))) __bf16 h3_bf16x2_t;
__device__ __forceinline__ uint32_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// s_waitcnt immediate that waits until at most `vm` vector-memory operations are outstanding
// (expcnt and lgkmcnt left unconstrained): vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14.
constexpr int waitcnt_vm(int vm) { return (vm & 15) | (7 << 4) | (15 << 8) | ((vm >> 4) << 14); }
// The same, and every LDS / scalar-memory operation done (lgkmcnt, bits 11:8, = 0).
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | (7 << 4) | ((vm >> 4) << 14); }

// Waits for this thread's direct-to-LDS loads down to `VM` outstanding, then meets the other
// waves at a barrier; afterwards every wave sees the LDS bytes those loads wrote.
template <int VM>
__device__ __forceinline__ void lds_dma_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM));
  __builtin_amdgcn_s_barrier();
}
// As lds_dma_barrier, for waves that also wrote LDS themselves (ds_write) since the last barrier.
template <int VM>
__device__ __forceinline__ void lds_dma_write_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(VM));
  __builtin_amdgcn_s_barrier();
}

// xor butterfly over the wave: lanes i and i^o add the same two values (commutative), so every
// lane ends with the identical total.  The AdaLN row statistics of every kernel use this sum.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Waves per row of the AdaLN row kernels for `rows` rows of width d: two below 16384 rows
// when d / 512 is even (twice the waves in flight), else one.  The row statistics' summation
// order depends on it, so every kernel that must reproduce an AdaLN bit for bit asks here.
inline int adaln_waves_per_row(int rows, int d) { return (rows >= 16384 || (d / 512) % 2) ? 1 : 2; }

constexpr float kLnEps = 1e-6f;

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  h3_bf16x2_t r;
  r.x = static_cast<__bf16>(lo);
  r.y = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ void unpack8(const uint4 &q, float *f) {
  f[0] = bf_lo(q.x); f[1] = bf_hi(q.x); f[2] = bf_lo(q.y); f[3] = bf_hi(q.y);
  f[4] = bf_lo(q.z); f[5] = bf_hi(q.z); f[6] = bf_lo(q.w); f[7] = bf_hi(q.w);
}
__device__ __forceinline__ uint4 pack8(const float *f) {
  uint4 q;
  q.x = pack_bf2(f[0], f[1]); q.y = pack_bf2(f[2], f[3]);
  q.z = pack_bf2(f[4], f[5]); q.w = pack_bf2(f[6], f[7]);
  return q;
}

// ---------------------------------------------------------------- Q/K RMSNorm + RoPE
// Per head of D channels: x <- x / sqrt(mean(x^2) + 1e-6) * gamma (when norm), then each
// interleaved pair (x_2j, x_2j+1) is rotated by the token's angle for that pair, given as
// (cos, sin) in a [tokens, D/2] table.  A lane owns 8 consecutive channels of a head (4 pairs);
// the D/8 lanes of a head are adjacent and start at a multiple of D/8, so a head is one DPP row
// of 16 lanes (D = 128) or half of one (D = 64).  The standalone kernel and the QKV products'
// fused epilogue both use these helpers, with the same lane grouping and no contraction, so
// their results agree bit for bit.
constexpr float kQkRmsEps = 1e-6f;
__device__ __forceinline__ float qk_sumsq8(const float *a) {
#pragma clang fp contract(off)
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) ss = ss + a[k] * a[k];
  return ss;
}
template <int CTRL>
__device__ __forceinline__ float dpp_take(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// The head's sum of the lanes' partial sums, on every lane of the head: pairs (l, l^1), then
// (l, l^2) (quad_perm), then the two quads of each 8 lanes (row_half_mirror: l <-> 7 - l), then
// the two halves of the 16-lane row (row_mirror: l <-> 15 - l).  Every lane adds the same two
// values, so all lanes of the head end with the same sum.
template <int D>
__device__ __forceinline__ float qk_head_sumsq(float ss) {
  static_assert(D == 64 || D == 128, "head of 8 or 16 lanes");
  ss = ss + dpp_take<0xB1>(ss);   // quad_perm [1, 0, 3, 2]
  ss = ss + dpp_take<0x4E>(ss);   // quad_perm [2, 3, 0, 1]
  ss = ss + dpp_take<0x141>(ss);  // row_half_mirror
  if constexpr (D == 128) ss = ss + dpp_take<0x140>(ss);  // row_mirror
  return ss;
}
// a: the lane's 8 channels; ss: the head's sum of squares; g: the 8 gains of those channels
// (read only when norm); cs: the (cos, sin) of the lane's 4 pairs.
template <int D>
__device__ __forceinline__ void qk_norm_rope8(float *a, float ss, const float *g, const float2 *cs,
                                              bool norm) {
#pragma clang fp contract(off)
  if (norm) {
    const float r = 1.0f / sqrtf(ss / static_cast<float>(D) + kQkRmsEps);
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = (a[k] * r) * g[k];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float x0 = a[2 * k], x1 = a[2 * k + 1];
    a[2 * k] = x0 * cs[k].x - x1 * cs[k].y;
    a[2 * k + 1] = x0 * cs[k].y + x1 * cs[k].x;
  }
}

// Output-column order of a QKV product tile whose epilogue applies the Q/K RMSNorm + RoPE.
// The product's columns are [q | k | v | qc], d each, heads of D channels.  When the tile
// width BN is a multiple of D, tiles keep the natural order and the q/k columns of a tile are
// whole heads.  For BN = 192 with D = 128 (a head does not divide the tile) the columns are
// regrouped: tile t < 2d/128 holds q/k head t (128 columns) followed by the 64 columns
// 2d + 64 t .. of v; the later tiles hold qc in natural order (3d + 192 (t - 2d/128) + j).  The
// B rows of a tile are gathered in that order and the epilogue scatters each column back, so
// the stored product is the plain one.
struct QkEpi {
  const bf16_t *q_gamma, *k_gamma;  // [D] each
  const float2 *table;              // [M, D/2] (cos, sin) of each token's rotation angles
  int d;                            // model width
  int norm;                         // 1: RMSNorm before the rotation
};
template <int BN, int D>
struct QkMap {
  static constexpr bool kMixed = BN % D != 0;
  static_assert(!kMixed || (BN == 192 && D == 128), "unsupported QKV tile / head combination");
  // canonical column of local column j of tile tn (may be >= 4d past the end)
  static __device__ __forceinline__ int col(int tn, int j, int d) {
    if constexpr (kMixed) {
      const int qk_tiles = 2 * d / 128;
      if (tn < qk_tiles) return j < 128 ? tn * 128 + j : 2 * d + tn * 64 + (j - 128);
      return 3 * d + (tn - qk_tiles) * 192 + j;
    } else {
      return tn * BN + j;
    }
  }
  // leading local columns of tile tn that are q/k channels (whole heads)
  static __device__ __forceinline__ int head_cols(int tn, int d) {
    if constexpr (kMixed) {
      return tn < 2 * d / 128 ? 128 : 0;
    } else {
      const int c = 2 * d - tn * BN;
      return c <= 0 ? 0 : (c < BN ? c : BN);
    }
  }
};

// The q/k-head part of a QKV product's fused epilogue, for one thread.  The tile's accumulators
// pass through an LDS band of WM * 32 rows (band row r = token m0 + ((r >> 5) TM + i) 32 + r % 32
// for band i) in TM bands; the leading hc columns of a band row are hc / QKD whole heads.  Task
// k of this thread (t = tid + k NT < items) is 8 channels of one (row, head), QKD / 8 adjacent
// lanes per head.  fetch(i) loads the rotation (cos, sin) slices and gains of band i's tasks
// into registers (issued ahead so their latency overlaps other work); run(i, ...) forms each
// task's bf16 values (value(row, col, a): what the plain product would store), applies the
// RMSNorm + rotation and stores 16 bytes.  items is a multiple of 64, so a wave is wholly in or
// out of a task and the DPP sums see only lanes of that head.
template <int BN, int QKD, int WM, int TM, int NT>
struct QkHeadPass {
  using Map = QkMap<BN, QKD>;
  static constexpr int LPH = QKD / 8;
  static constexpr int HI = (WM * 32 * (BN / QKD) * LPH + NT - 1) / NT;
  const QkEpi &qk;
  int tid, tn, m0, M, hpr, items;
  float4 tb[HI][2];
  uint4 gm[HI];

  __device__ QkHeadPass(const QkEpi &q, int tid_, int tn_, int m0_, int M_)
      : qk(q), tid(tid_), tn(tn_), m0(m0_), M(M_) {
    hpr = Map::head_cols(tn, qk.d) / QKD;
    items = WM * 32 * hpr * LPH;
  }
  __device__ __forceinline__ void task(int k, int i, int &row, int &col, int &m, int &n) const {
    const int t = tid + k * NT;
    const int item = t / LPH;
    row = item / hpr;
    col = (item - row * hpr) * QKD + (t % LPH) * 8;
    m = m0 + ((row >> 5) * TM + i) * 32 + (row & 31);
    n = Map::col(tn, col, qk.d);
  }
  __device__ __forceinline__ void fetch(int i) {
#pragma unroll
    for (int k = 0; k < HI; ++k) {
      if (tid + k * NT < items) {
        int row, col, m, n;
        task(k, i, row, col, m, n);
        const int mt = m < M ? m : M - 1;
        const int pos = col % QKD;
        const float4 *tp =
            reinterpret_cast<const float4 *>(qk.table + static_cast<int64_t>(mt) * (QKD / 2) + pos / 2);
        tb[k][0] = tp[0];
        tb[k][1] = tp[1];
        if (qk.norm) gm[k] = *reinterpret_cast<const uint4 *>((n < qk.d ? qk.q_gamma : qk.k_gamma) + pos);
      }
    }
  }
  template <class Value>
  __device__ __forceinline__ void run(int i, Value value, bf16_t *C, int64_t ldc) {
#pragma unroll
    for (int k = 0; k < HI; ++k) {
      if (tid + k * NT < items) {
        int row, col, m, n;
        task(k, i, row, col, m, n);
        float a[8], g[8];
        value(row, col, a);
        float ss = 0.f;
        if (qk.norm) {
          ss = qk_head_sumsq<QKD>(qk_sumsq8(a));
          unpack8(gm[k], g);
        }
        const float2 cs[4] = {make_float2(tb[k][0].x, tb[k][0].y), make_float2(tb[k][0].z, tb[k][0].w),
                              make_float2(tb[k][1].x, tb[k][1].y), make_float2(tb[k][1].z, tb[k][1].w)};
        qk_norm_rope8<QKD>(a, ss, g, cs, qk.norm != 0);
        if (m < M) *reinterpret_cast<uint4 *>(C + static_cast<int64_t>(m) * ldc + n) = pack8(a);
      }
    }
  }
};

// GELU(x) = x Phi(x) with Phi the standard normal CDF.  erfc by Abramowitz & Stegun, Handbook
// of Mathematical Functions, formula 7.1.26: erfc(z) = (a1 t + ... + a5 t^5) exp(-z^2) with
// t = 1 / (1 + p z), z >= 0, absolute error <= 1.5e-7.  With z = |x| / sqrt 2 and
// q = erfc(z) / 2 = Phi(-|x|), x Phi(x) = x / 2 + |x| (1/2 - q) holds for either sign of x, so
// the product needs no branch or select: one reciprocal, one exponential, eight FMA/multiplies.
// The factor 1/2 of q is folded into the coefficients, 1/sqrt 2 into p and the exponent.
__device__ __forceinline__ float gelu_erf(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.0f + (0.3275911f * 0.70710678118654752f) * ax);
  float h = 0.5f * 1.061405429f;
  h = h * t - 0.5f * 1.453152027f;
  h = h * t + 0.5f * 1.421413741f;
  h = h * t - 0.5f * 0.284496736f;
  h = h * t + 0.5f * 0.254829592f;
  h = h * t;
  const float e = __builtin_amdgcn_exp2f((x * -0.72134752044448170f) * x);  // exp(-x^2 / 2)
  const float q = h * e;
  return __builtin_fmaf(ax, 0.5f - q, 0.5f * x);
}

// ---------------------------------------------------------------- model
struct Model {
  h3_dims dims;
  int32_t head_dim;
  h3_global_weights g;
  h3_block_weights *blocks;  // n_blocks entries (host copy of the pointer table)
};

// Workspace plan for a token count and options (all offsets 256-byte aligned).
struct WsPlan {
  // block part
  size_t n1, qkvq, attn, y, n2, h, m, hq, hs, rope, gpart;
  size_t gpart_bytes;
  // forward / modulation part
  size_t mod, fin, tmp, x, xr, n1b, lat16, rope_r, x0;
  size_t total;
};
WsPlan plan_workspace(const Model &m, int32_t n_tokens, const h3_run_opts &o);

// ---------------------------------------------------------------- kernel launchers
// All launchers assume validated arguments and enqueue on `s`.
// Tile configuration and split-K choice of a bf16 or int8 product; part_bytes is the float32
// (int32 for int8) partial buffer [split][M][N] a split-K launch needs.
struct GemmPlan {
  int cfg;    // 0: 128x128, 1: 192x192, 2: 256x256, 3: 128x256 (int8 grouped only), 4: 384x192
  int split;  // pieces of K in separate workgroups (1, 2 or 4)
  size_t part_bytes;
};
GemmPlan plan_gemm(int M, int N, int K);
// Split-K scratch handed to a product (float32 or int32 partials) with its capacity.  A product whose
// plan needs more than the capacity (or gets none) runs without split-K.
struct SplitScratch {
  float *part = nullptr;
  size_t part_bytes = 0;
};
void launch_gemm_bf16(const bf16_t *A, int64_t lda, const bf16_t *B, int64_t ldb, void *C,
                      int64_t ldc, int M, int N, int K, const bf16_t *bias, const bf16_t *bias2,
                      int epilogue, int out_f32, hipStream_t s,
                      const SplitScratch &scratch = SplitScratch());
// Tile / split-K choice of an int8 product with `group` K channels per activation scale
// (group == K: row mode, which may split K; part_bytes is then the int32 partial buffer).
GemmPlan plan_gemm_i8(int M, int N, int K, int group);
// A split-K product without its reduction: the float32 partials [S][M][N] stay in the
// scratch for a consumer that sums them (launch_gate_adaln with a GateY source).  Returns S,
// or 0 when the plan does not split this product or the scratch is too small (nothing is
// launched then).
int launch_gemm_bf16_partials(const bf16_t *A, int64_t lda, const bf16_t *B, int64_t ldb, int M,
                              int N, int K, hipStream_t s, const SplitScratch &scratch);
// The same for a row-mode int8 product: its int32 partials [S][M][N] stay in the scratch for
// the gate kernel (GateY with ipart, sa, sw), which sums and dequantises them as the int8
// split-K reduction would.  Returns S, or 0 (nothing launched).
int launch_gemm_i8_partials(const int8_t *QA, const float *SA, const int8_t *QW, const float *SW,
                            int M, int N, int K, hipStream_t s, const SplitScratch &scratch);
void launch_gemm_i8(const int8_t *QA, const float *SA, const int8_t *QW, const float *SW,
                    const bf16_t *bias, bf16_t *C, int64_t ldc, int M, int N, int K, int group,
                    hipStream_t s, const SplitScratch &scratch = SplitScratch(),
                    int epilogue = H3_EPI_NONE);
// The velocity head with the final AdaLN applied while the A tiles are staged:
// out = float(AdaLN(x; shift, scale) W^T + bias), float32 [M, N] at row stride ldo, x bf16
// [M, d] at stride ldx, shift / scale float [d], W bf16 [N, d].  Bit-identical to
// launch_gate_adaln (AdaLN only) into a bf16 buffer followed by launch_gemm_bf16 with a float32
// output.  Returns 1 when launched, 0 when there is no such form (it needs N < 192, where the
// plain product takes 128x128 unsplit tiles; 16-byte aligned x, shift, scale; 8 | ldx): nothing
// is launched then.
int launch_head_adaln_gemm(const bf16_t *x, int64_t ldx, const float *shift, const float *scale,
                           const bf16_t *W, int64_t ldw, const bf16_t *bias, float *out,
                           int64_t ldo, int M, int N, int d, hipStream_t s);
// Matrix-core probe: `workgroups` workgroups of four waves, each wave issuing `iters` rounds of
// eight independent 32x32 bf16 (int8 = 0) or int8 (int8 = 1) MFMAs; out: float [workgroups * 256].
void launch_mfma_probe(int int8, int iters, int workgroups, float *out, hipStream_t s);
// Whether launch_head_adaln_gemm has a fused form for these arguments.
bool head_adaln_gemm_fits(const bf16_t *x, int64_t ldx, const float *shift, const float *scale,
                          int M, int N, int d);
// The QKV product [q | k | v | qc] = A W^T + bias (N = 4d) with the Q/K RMSNorm + RoPE of
// launch_qk_norm_rope applied in the product's epilogue (QkEpi; table rows are the M tokens),
// bit-identical to the product followed by that kernel.  Returns 1 when launched, 0 when the
// product's plan has no fused form (split K, head_dim not 64 or 128): nothing is launched then.
int launch_gemm_bf16_qkv(const bf16_t *A, int64_t lda, const bf16_t *W, int64_t ldw,
                         const bf16_t *bias, bf16_t *C, int64_t ldc, int M, int d, int K,
                         int head_dim, const QkEpi &qk, hipStream_t s);
int launch_gemm_i8_qkv(const int8_t *QA, const float *SA, const int8_t *QW, const float *SW,
                       const bf16_t *bias, bf16_t *C, int64_t ldc, int M, int d, int K,
                       int head_dim, const QkEpi &qk, hipStream_t s);
void launch_attention(const bf16_t *Q, int64_t ldq, const bf16_t *K, int64_t ldk,
                      const bf16_t *V, int64_t ldv, bf16_t *O, int64_t ldo, int nq, int nk,
                      int heads, int head_dim, hipStream_t s);
// Two independent attention problems of the same head layout in one launch.
void launch_attention_pair(const bf16_t *Q0, int64_t ldq0, const bf16_t *K0, int64_t ldk0,
                           const bf16_t *V0, int64_t ldv0, bf16_t *O0, int64_t ldo0, int nq0, int nk0,
                           const bf16_t *Q1, int64_t ldq1, const bf16_t *K1, int64_t ldk1,
                           const bf16_t *V1, int64_t ldv1, bf16_t *O1, int64_t ldo1, int nq1, int nk1,
                           int heads, int head_dim, hipStream_t s);
// x_out = bf16(x + gate*y) (if y != nullptr), then n_out = bf16(LN(x_out)(1+scale)+shift)
// (if n_out != nullptr).  With y == nullptr the row is read from x.  x_out may equal x.
// With q_out != nullptr the normalised row is not stored as bf16 but quantised: q_out int8
// [rows, d] and s_out float32 [rows] (one scale per row), bit-identical to storing n_out and
// quantising it with launch_quant_rows(group = d).
void launch_gate_adaln(const bf16_t *x, const bf16_t *y, const float *gate, bf16_t *x_out,
                       const float *shift, const float *scale, bf16_t *n_out, int rows, int d,
                       hipStream_t s, int8_t *q_out = nullptr, float *s_out = nullptr);
// The gated branch y given as S float32 split-K partials of a [rows, d] product (part +
// q * stride, q = 0..S-1, S = 2 or 4) with its biases (b1 required, b2 optional): y =
// bf16(((p_0 + p_1) + ...) + ((0 + b1) + b2)), the split-K reduction's own arithmetic,
// optionally stored to y_out; then as launch_gate_adaln.
struct GateY {
  const float *part;
  int S;
  int64_t stride;
  const bf16_t *b1, *b2;
  bf16_t *y_out;
  // int8 FC2 (row mode): the partials are int32 (ipart instead of part) and y is dequantised
  // with the activation scale sa [rows] and the weight scale sw [d], as the int8 split-K
  // reduction does
  const int32_t *ipart = nullptr;
  const float *sa = nullptr, *sw = nullptr;
};
void launch_gate_adaln_part(const bf16_t *x, const GateY &ysrc, const float *gate, bf16_t *x_out,
                            const float *shift, const float *scale, bf16_t *n_out, int rows, int d,
                            hipStream_t s, int8_t *q_out = nullptr, float *s_out = nullptr);
void launch_rope_table(float2 *table, const h3_geom &geom, int n_tokens, int head_dim,
                       hipStream_t s);
void launch_qk_norm_rope(bf16_t *qkvq, int64_t ld, int n_tokens, int d, int head_dim,
                         const bf16_t *q_gamma, const bf16_t *k_gamma, int qk_norm,
                         const float2 *table, hipStream_t s);
void launch_token_reduce(int direction, const h3_geom &geom, int d, const bf16_t *src,
                         const bf16_t *bypass, bf16_t *dst, hipStream_t s);
void launch_euler(float *x, const float *v, float dt, int64_t n, hipStream_t s);
// Core-residual reuse (n % 8 == 0): delta = float(x_core) - float(x_patch); x = bf16(float(x_patch)
// + delta) (x may equal x_patch).
void launch_core_delta(const bf16_t *x_core, const bf16_t *x_patch, float *delta, int64_t n,
                       hipStream_t s);
void launch_core_apply(const bf16_t *x_patch, const float *delta, bf16_t *x, int64_t n, hipStream_t s);
void launch_quant_rows(const bf16_t *X, int8_t *Q, float *S, int rows, int K, int group,
                       hipStream_t s);
void launch_f32_to_bf16(const float *src, bf16_t *dst, int64_t n, hipStream_t s);
void launch_timestep_sinusoid(float sigma, float *e, hipStream_t s);
// y[r] = act(sum_k W[r,k] x[k] + b[r]) + add[r]; act: 0 none, 1 SiLU.
void launch_gemv(const bf16_t *W, const float *x, const bf16_t *b, const bf16_t *add, float *y,
                 int rows, int K, int act, hipStream_t s);
// out[b, i] = M[i] + T[b, i] for b < nb, i < width (T bf16).
void launch_add_table(const float *Mv, const bf16_t *T, float *out, int nb, int width,
                      hipStream_t s);

inline size_t align_up(size_t v, size_t a = 256) { return (v + a - 1) / a * a; }

// Records a begin event now and an end event at scope exit on stream s when a profiling
// session selects this stage (h3_profile_begin); otherwise does nothing.
class ProfScope {
 public:
  ProfScope(int stage, hipStream_t s);
  ~ProfScope();
  ProfScope(const ProfScope &) = delete;
  ProfScope &operator=(const ProfScope &) = delete;

 private:
  int stage_;
  hipStream_t stream_;
  int pair_;
};

}  // namespace h3
