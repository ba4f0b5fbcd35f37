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
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  h3_bf16x2_t r;
  r.x = static_cast<__bf16>(lo);
  r.y = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, r);
}

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
// Tile configuration and split-K choice of a bf16 product; part_bytes is the float32 partial
// buffer [split][M][N] a split-K launch needs.
struct GemmPlan {
  int cfg;    // 0: 128x128, 1: 192x192, 2: 256x256, 3: 128x256, 4: 384x192 output tiles
  int split;  // pieces of K in separate workgroups (1, 2, 3 or 4)
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
void launch_gemm_i8(const int8_t *QA, const float *SA, const int8_t *QW, const float *SW,
                    const bf16_t *bias, bf16_t *C, int64_t ldc, int M, int N, int K, int group,
                    hipStream_t s, const SplitScratch &scratch = SplitScratch(),
                    int epilogue = H3_EPI_NONE);
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
// q * stride, q = 0..S-1) with its biases: y = bf16(((p_0 + p_1) + ...) + ((0 + b1) + b2)), the
// split-K reduction's own arithmetic, optionally stored to y_out; then as launch_gate_adaln.
struct GateY {
  const float *part;
  int S;
  int64_t stride;
  const bf16_t *b1, *b2;
  bf16_t *y_out;
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
