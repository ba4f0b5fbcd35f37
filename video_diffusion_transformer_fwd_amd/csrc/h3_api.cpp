// C ABI entry points: model handle, workspace plan, block / forward orchestration, and the
// single-operation entry points.  Every argument is validated before the first launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "h3_internal.h"

// Device scratch of h3_modulation_noalloc, for callers that cannot allocate device memory:
// every GPU the library runs on holds one copy of it until the process ends.  Host code never
// passes this name to a kernel (on the host it is only a stand-in for the symbol): it uses the
// device address looked up once per device (static_scratch below).
constexpr size_t kStaticScratchBytes = 264 * 1024;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

struct h3_model : h3::Model {};

namespace h3 {
namespace {

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// The products copy their operand tiles through 32-bit byte offsets from the operand's base:
// a [rows, K] operand at row stride ld (elements of esize bytes) must span less than 4 GiB.
bool fits_u32(int64_t rows, int64_t ld, int64_t K, int64_t esize) {
  return ((rows - 1) * ld + K) * esize < (int64_t{1} << 32);
}

bool supported_width(int d) {
  const int v = d / 512;
  return d % 512 == 0 && (v == 1 || v == 2 || v == 3 || v == 4 || v == 5 || v == 6 || v == 8 ||
                          v == 10 || v == 12 || v == 16);
}

int32_t check_opts(const h3_run_opts *o) {
  if (!o) return fail(H3_EINVAL, "run options are NULL");
  if (o->fc2_mode < H3_FC2_BF16 || o->fc2_mode > H3_FC2_INT8_GROUPED)
    return fail(H3_EINVAL, "fc2_mode must be 0, 1 or 2");
  if (o->int8_linear != 0 && o->int8_linear != 1) return fail(H3_EINVAL, "int8_linear must be 0 or 1");
  if (o->fused_qk_rope != 0 && o->fused_qk_rope != 1) return fail(H3_EINVAL, "fused_qk_rope must be 0 or 1");
  if (o->store_branches != 0 && o->store_branches != 1) return fail(H3_EINVAL, "store_branches must be 0 or 1");
  if (o->fused_head_adaln != 0 && o->fused_head_adaln != 1)
    return fail(H3_EINVAL, "fused_head_adaln must be 0 or 1");
  return H3_OK;
}

// The int8 weight copies a block needs under these options.
int32_t check_block_int8(const h3_block_weights &w, const h3_run_opts &o, const char *who) {
  if (o.fc2_mode != H3_FC2_BF16 && (!w.fc2_q || !w.fc2_s))
    return fail(H3_EINVAL, std::string(who) + ": int8 FC2 needs quantised weights");
  if (o.int8_linear && (!w.qkvq_q || !w.qkvq_s || !w.fc1_q || !w.fc1_s))
    return fail(H3_EINVAL, std::string(who) + ": int8_linear needs quantised QKV and FC1 weights");
  return H3_OK;
}

size_t bytes_bf16(int64_t n) { return static_cast<size_t>(n) * 2; }

}  // namespace

WsPlan plan_workspace(const Model &m, int32_t n, const h3_run_opts &o) {
  const int64_t d = m.dims.d_model, F = m.dims.ffn_dim, C = m.dims.latent_ch;
  const int64_t nb = m.dims.n_blocks, half = m.head_dim / 2;
  WsPlan p{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + align_up(bytes));
    return at;
  };
  p.n1 = take(bytes_bf16(n * d));
  p.qkvq = take(bytes_bf16(n * 4 * d));
  p.attn = take(bytes_bf16(n * 2 * d));
  p.y = take(bytes_bf16(n * d));
  p.n2 = take(bytes_bf16(n * d));
  p.h = take(bytes_bf16(n * F));
  p.m = take(bytes_bf16(n * d));
  const bool i8 = o.fc2_mode != H3_FC2_BF16;
  p.hq = take(i8 ? static_cast<size_t>(n * F) : 0);
  p.hs = take(i8 ? static_cast<size_t>(n * (F / 1024)) * sizeof(float) : 0);
  p.rope = take(static_cast<size_t>(n * half) * sizeof(float2));
  // split-K partials of the block's products
  size_t part = 0;
  // the block runs at n tokens, or at about n/2 between a token merge and its restore
  for (int64_t rows : {static_cast<int64_t>(n), static_cast<int64_t>((n + 1) / 2)}) {
    const int r = static_cast<int>(rows);
    const GemmPlan gp[] = {plan_gemm(r, 4 * d, d), plan_gemm(r, d, 2 * d), plan_gemm(r, F, d),
                           plan_gemm(r, d, F)};
    for (const GemmPlan &g : gp) part = std::max(part, g.part_bytes);
    if (i8) part = std::max(part, plan_gemm_i8(r, d, F, o.fc2_mode == H3_FC2_INT8_ROW ? F : 1024).part_bytes);
    if (o.int8_linear) {
      part = std::max(part, plan_gemm_i8(r, 4 * d, d, d).part_bytes);
      part = std::max(part, plan_gemm_i8(r, F, d, d).part_bytes);
    }
  }
  p.gpart = take(part);
  p.gpart_bytes = part;
  // forward / modulation
  p.mod = take(static_cast<size_t>(nb * 6 * d) * sizeof(float));
  p.fin = take(static_cast<size_t>(2 * d) * sizeof(float));
  p.tmp = take(static_cast<size_t>(256 + 2 * d + 6 * d) * sizeof(float));
  p.x = take(bytes_bf16(n * d));
  p.xr = take(bytes_bf16(n * d));
  p.n1b = take(bytes_bf16(n * d));
  p.lat16 = take(bytes_bf16(n * C));
  p.rope_r = take(static_cast<size_t>(n * half) * sizeof(float2));
  p.x0 = take(bytes_bf16(n * d));  // patch embedding kept for the core-residual delta
  p.total = off;
  return p;
}

}  // namespace h3

using namespace h3;

namespace {

int32_t validate_model(const h3_model *m) {
  if (!m) return fail(H3_EINVAL, "model is NULL");
  return H3_OK;
}

// Token counts of a block: its largest activation operands are the FC2 input [n, ffn_dim] and
// the out-projection input [n, 2 d_model] (bf16), each addressed within 4 GiB; the patch
// product's input, the bf16 latent [n, latent_ch], likewise.
int32_t check_tokens(const h3_model *m, int32_t n, const char *who) {
  if (n < 1) return fail(H3_ESHAPE, std::string(who) + ": n_tokens must be >= 1");
  const int64_t f = m->dims.ffn_dim, d2 = 2 * static_cast<int64_t>(m->dims.d_model);
  if (!fits_u32(n, f, f, 2) || !fits_u32(n, d2, d2, 2))
    return fail(H3_ESHAPE, std::string(who) + ": n_tokens x ffn_dim spans 4 GiB or more");
  const int64_t c = m->dims.latent_ch;
  if (!fits_u32(n, c, c, 2))
    return fail(H3_ESHAPE, std::string(who) + ": n_tokens x latent_ch spans 4 GiB or more");
  return H3_OK;
}

// A row-quantised AdaLN output: int8 [rows, d] followed by the float32 row scales [rows].
struct QRows {
  int8_t *q;
  float *s;
};
QRows qrows(const void *buf, int rows, int d) {
  char *b = reinterpret_cast<char *>(const_cast<void *>(buf));
  return {reinterpret_cast<int8_t *>(b), reinterpret_cast<float *>(b + static_cast<size_t>(rows) * d)};
}

// AdaLN (after the optional gate x <- x + g y) into dst: bf16 [rows, d], or row-quantised
// (QRows layout) when quant.  fused = gate and AdaLN in one kernel (bit-identical either way).
// yp (instead of y): the gate's y comes as split-K partials that the gate kernel reduces.
void gate_then_adaln(bf16_t *x, const bf16_t *y, const float *g, const float *sh, const float *sc,
                     void *dst, bool quant, bool fused, int rows, int d, hipStream_t s,
                     const GateY *yp = nullptr) {
  if (yp) {
    if (!fused) {
      launch_gate_adaln_part(x, *yp, g, x, nullptr, nullptr, nullptr, rows, d, s);
      y = nullptr;
    } else if (quant) {
      const QRows r = qrows(dst, rows, d);
      launch_gate_adaln_part(x, *yp, g, x, sh, sc, nullptr, rows, d, s, r.q, r.s);
      return;
    } else {
      launch_gate_adaln_part(x, *yp, g, x, sh, sc, reinterpret_cast<bf16_t *>(dst), rows, d, s);
      return;
    }
  }
  if (y && !fused) {
    launch_gate_adaln(x, y, g, x, nullptr, nullptr, nullptr, rows, d, s);
    y = nullptr;
  }
  if (quant) {
    const QRows r = qrows(dst, rows, d);
    launch_gate_adaln(x, y, g, y ? x : nullptr, sh, sc, nullptr, rows, d, s, r.q, r.s);
  } else {
    launch_gate_adaln(x, y, g, y ? x : nullptr, sh, sc, reinterpret_cast<bf16_t *>(dst), rows, d, s);
  }
}

// Launches the block on validated arguments.  rows = tokens of this geometry.  With
// o.int8_linear the block's n1 (given or computed) is row-quantised; n1_next is row-quantised
// when n1_next_q, else bf16.
int32_t run_block(const h3_model *m, int32_t b, const h3_geom &geom, int32_t rows,
                  const h3_run_opts &o, bf16_t *x, const void *n1_in, void *n1_next,
                  bool n1_next_q, const float *mod, const float *mod_next, const bf16_t *ctx_kv,
                  char *ws, const WsPlan &p, hipStream_t s, const float2 *rope_table) {
  const bool q8 = o.int8_linear != 0;
  const int d = m->dims.d_model, F = m->dims.ffn_dim, H = m->dims.n_heads, D = m->head_dim;
  const int L = m->dims.ctx_len;
  const h3_block_weights &w = m->blocks[b];
  void *n1 = ws + p.n1;
  bf16_t *qkvq = reinterpret_cast<bf16_t *>(ws + p.qkvq);
  bf16_t *attn = reinterpret_cast<bf16_t *>(ws + p.attn);
  bf16_t *y = reinterpret_cast<bf16_t *>(ws + p.y);
  void *n2 = ws + p.n2;
  bf16_t *h = reinterpret_cast<bf16_t *>(ws + p.h);
  bf16_t *mo = reinterpret_cast<bf16_t *>(ws + p.m);
  const float *sh1 = mod, *sc1 = mod + d, *g1 = mod + 2 * d;
  const float *sh2 = mod + 3 * d, *sc2 = mod + 4 * d, *g2 = mod + 5 * d;
  SplitScratch sk;
  sk.part = reinterpret_cast<float *>(ws + p.gpart);
  sk.part_bytes = p.gpart_bytes;

  // AdaLN-1 (unless the caller already has it, e.g. from the previous block's fused gate)
  if (!n1_in) {
    ProfScope ps(H3_ST_ADALN, s);
    gate_then_adaln(x, nullptr, nullptr, sh1, sc1, n1, q8, true, rows, d, s);
    n1_in = n1;
  }
  // [q | k | v | qc] = n1 W_qkvq^T + b, then Q/K RMSNorm + 3D RoPE (in the product's
  // epilogue when fused and the tiling allows, else in place by its own kernel)
  const QkEpi qe{reinterpret_cast<const bf16_t *>(w.q_gamma),
                 reinterpret_cast<const bf16_t *>(w.k_gamma), rope_table, d, o.qk_norm};
  bool qk_done = false;
  {
    ProfScope ps(H3_ST_QKV_GEMM, s);
    if (q8) {
      const QRows r = qrows(n1_in, rows, d);
      if (o.fused_qk_rope)
        qk_done = launch_gemm_i8_qkv(r.q, r.s, reinterpret_cast<const int8_t *>(w.qkvq_q),
                                     reinterpret_cast<const float *>(w.qkvq_s),
                                     reinterpret_cast<const bf16_t *>(w.qkvq_b), qkvq, 4 * d, rows,
                                     d, d, D, qe, s) != 0;
      if (!qk_done)
        launch_gemm_i8(r.q, r.s, reinterpret_cast<const int8_t *>(w.qkvq_q),
                       reinterpret_cast<const float *>(w.qkvq_s),
                       reinterpret_cast<const bf16_t *>(w.qkvq_b), qkvq, 4 * d, rows, 4 * d, d, d,
                       s, sk, H3_EPI_NONE);
    } else {
      if (o.fused_qk_rope)
        qk_done = launch_gemm_bf16_qkv(reinterpret_cast<const bf16_t *>(n1_in), d,
                                       reinterpret_cast<const bf16_t *>(w.qkvq_w), d,
                                       reinterpret_cast<const bf16_t *>(w.qkvq_b), qkvq, 4 * d, rows,
                                       d, d, D, qe, s) != 0;
      if (!qk_done)
        launch_gemm_bf16(reinterpret_cast<const bf16_t *>(n1_in), d,
                         reinterpret_cast<const bf16_t *>(w.qkvq_w), d, qkvq, 4 * d, rows, 4 * d, d,
                         reinterpret_cast<const bf16_t *>(w.qkvq_b), nullptr, H3_EPI_NONE, 0, s, sk);
    }
  }
  if (!qk_done) {
    ProfScope ps(H3_ST_QK_NORM_ROPE, s);
    launch_qk_norm_rope(qkvq, 4 * d, rows, d, D, qe.q_gamma, qe.k_gamma, o.qk_norm, rope_table, s);
  }
  // self-attention -> attn[:, 0:d] and cross-attention -> attn[:, d:2d], in one launch
  {
    ProfScope ps(H3_ST_SELF_ATTN, s);
    launch_attention_pair(qkvq, 4 * d, qkvq + d, 4 * d, qkvq + 2 * d, 4 * d, attn, 2 * d, rows, rows,
                          qkvq + 3 * d, 4 * d, ctx_kv, d, ctx_kv + static_cast<size_t>(L) * d, d,
                          attn + d, 2 * d, rows, L, H, D, s);
  }
  // y = [O | Oc] [W_o | W_oc]^T + b_o + b_oc.  When the product splits K, its partials go
  // straight to the gate kernel, which sums them exactly as the split-K reduction would (and
  // stores y only when asked to: nothing downstream reads it).
  GateY yp{sk.part, 0, static_cast<int64_t>(rows) * d, reinterpret_cast<const bf16_t *>(w.out_b),
           reinterpret_cast<const bf16_t *>(w.outc_b), o.store_branches ? y : nullptr};
  {
    ProfScope ps(H3_ST_OUT_GEMM, s);
    // (widths above 4096 keep the separate reduction: the gate kernel's registers would spill)
    if (d <= 4096)
      yp.S = launch_gemm_bf16_partials(attn, 2 * d, reinterpret_cast<const bf16_t *>(w.out_w),
                                       2 * d, rows, d, 2 * d, s, sk);
    if (!yp.S)
      launch_gemm_bf16(attn, 2 * d, reinterpret_cast<const bf16_t *>(w.out_w), 2 * d, y, d, rows,
                       d, 2 * d, yp.b1, yp.b2, H3_EPI_NONE, 0, s, sk);
  }
  // x <- x + g1 y ; n2 = AdaLN(x; sh2, sc2)
  {
    ProfScope ps(H3_ST_GATE_ADALN, s);
    gate_then_adaln(x, y, g1, sh2, sc2, n2, q8, o.fused_gate_adaln != 0, rows, d, s,
                    yp.S ? &yp : nullptr);
  }
  // h = GELU(n2 W1^T + b1)
  {
    ProfScope ps(H3_ST_FC1_GEMM, s);
    if (q8) {
      const QRows r = qrows(n2, rows, d);
      launch_gemm_i8(r.q, r.s, reinterpret_cast<const int8_t *>(w.fc1_q),
                     reinterpret_cast<const float *>(w.fc1_s),
                     reinterpret_cast<const bf16_t *>(w.fc1_b), h, F, rows, F, d, d, s, sk,
                     H3_EPI_GELU);
    } else {
      launch_gemm_bf16(reinterpret_cast<const bf16_t *>(n2), d,
                       reinterpret_cast<const bf16_t *>(w.fc1_w), d, h, F, rows, F, d,
                       reinterpret_cast<const bf16_t *>(w.fc1_b), nullptr, H3_EPI_GELU, 0, s, sk);
    }
  }
  // m = FC2(h) (bf16 FC2 with K split: partials reduced by the gate kernel, as above)
  GateY mp{sk.part, 0, static_cast<int64_t>(rows) * d, reinterpret_cast<const bf16_t *>(w.fc2_b),
           nullptr, o.store_branches ? mo : nullptr};
  if (o.fc2_mode == H3_FC2_BF16) {
    ProfScope ps(H3_ST_FC2_GEMM, s);
    if (d <= 4096)
      mp.S = launch_gemm_bf16_partials(h, F, reinterpret_cast<const bf16_t *>(w.fc2_w), F, rows, d,
                                       F, s, sk);
    if (!mp.S)
      launch_gemm_bf16(h, F, reinterpret_cast<const bf16_t *>(w.fc2_w), F, mo, d, rows, d, F,
                       mp.b1, nullptr, H3_EPI_NONE, 0, s, sk);
  } else {
    const int group = o.fc2_mode == H3_FC2_INT8_ROW ? F : 1024;
    int8_t *hq = reinterpret_cast<int8_t *>(ws + p.hq);
    float *hs = reinterpret_cast<float *>(ws + p.hs);
    {
      ProfScope ps(H3_ST_FC2_QUANT, s);
      launch_quant_rows(h, hq, hs, rows, F, group, s);
    }
    ProfScope ps(H3_ST_FC2_I8_GEMM, s);
    // row mode with K split: the int32 partials go to the gate kernel, which sums and
    // dequantises them exactly as the int8 split-K reduction would
    if (o.fc2_mode == H3_FC2_INT8_ROW && d <= 4096) {
      mp.S = launch_gemm_i8_partials(hq, hs, reinterpret_cast<const int8_t *>(w.fc2_q),
                                     reinterpret_cast<const float *>(w.fc2_s), rows, d, F, s, sk);
      if (mp.S) {
        mp.part = nullptr;
        mp.ipart = reinterpret_cast<const int32_t *>(sk.part);
        mp.sa = hs;
        mp.sw = reinterpret_cast<const float *>(w.fc2_s);
      }
    }
    if (!mp.S)
      launch_gemm_i8(hq, hs, reinterpret_cast<const int8_t *>(w.fc2_q),
                     reinterpret_cast<const float *>(w.fc2_s),
                     reinterpret_cast<const bf16_t *>(w.fc2_b), mo, d, rows, d, F, group, s, sk);
  }
  // x <- x + g2 m ; optionally n1_next = AdaLN(x; next shift, scale)
  {
    ProfScope ps(H3_ST_GATE_ADALN, s);
    if (n1_next)
      gate_then_adaln(x, mo, g2, mod_next, mod_next + d, n1_next, n1_next_q,
                      o.fused_cross_block != 0, rows, d, s, mp.S ? &mp : nullptr);
    else if (mp.S)
      launch_gate_adaln_part(x, mp, g2, x, nullptr, nullptr, nullptr, rows, d, s);
    else
      launch_gate_adaln(x, mo, g2, x, nullptr, nullptr, nullptr, rows, d, s);
  }
  (void)geom;
  return check_launch("h3_dit_block_fwd");
}

// Modulation intermediates (tmp, (256 + 8 d) floats): the sinusoid e [256], the two hidden
// activations [d] each and the shared projection [6 d]; each is written in full before it is read.
size_t modulation_tmp_bytes(int d) { return (256 + 8 * static_cast<size_t>(d)) * sizeof(float); }

int32_t run_modulation(const h3_model *m, float sigma, float *mod, float *mod_final, float *tmp,
                       hipStream_t s) {
  const int d = m->dims.d_model, nb = m->dims.n_blocks;
  const h3_global_weights &g = m->g;
  float *e = tmp, *h1 = tmp + 256, *u = h1 + d, *Mv = u + d;
  launch_timestep_sinusoid(sigma, e, s);
  launch_gemv(reinterpret_cast<const bf16_t *>(g.t1_w), e, reinterpret_cast<const bf16_t *>(g.t1_b),
              nullptr, h1, d, 256, 1, s);
  launch_gemv(reinterpret_cast<const bf16_t *>(g.t2_w), h1, reinterpret_cast<const bf16_t *>(g.t2_b),
              nullptr, u, d, d, 1, s);
  launch_gemv(reinterpret_cast<const bf16_t *>(g.mod_w), u, reinterpret_cast<const bf16_t *>(g.mod_b),
              nullptr, Mv, 6 * d, d, 0, s);
  launch_add_table(Mv, reinterpret_cast<const bf16_t *>(g.mod_table), mod, nb, 6 * d, s);
  launch_gemv(reinterpret_cast<const bf16_t *>(g.fin_w), u, reinterpret_cast<const bf16_t *>(g.fin_b),
              reinterpret_cast<const bf16_t *>(g.fin_t), mod_final, 2 * d, d, 0, s);
  return check_launch("h3_modulation");
}

}  // namespace

extern "C" {

int32_t h3_model_create(const h3_dims *dims, const h3_global_weights *g,
                        const h3_block_weights *blocks, int32_t n_blocks, h3_model **out) {
  if (!dims || !g || !blocks || !out) return fail(H3_EINVAL, "h3_model_create: NULL argument");
  *out = nullptr;
  const h3_dims &dm = *dims;
  if (dm.n_blocks != n_blocks || n_blocks < 1)
    return fail(H3_ESHAPE, "h3_model_create: n_blocks mismatch");
  if (!supported_width(dm.d_model))
    return fail(H3_ESHAPE, "h3_model_create: d_model must be 512 * {1,2,3,4,5,6,8,10,12,16}");
  if (dm.n_heads < 1 || dm.d_model % dm.n_heads)
    return fail(H3_ESHAPE, "h3_model_create: n_heads must divide d_model");
  const int D = dm.d_model / dm.n_heads;
  if (D != 64 && D != 128) return fail(H3_ESHAPE, "h3_model_create: head_dim must be 64 or 128");
  if (dm.ffn_dim < 1024 || dm.ffn_dim % 1024)
    return fail(H3_ESHAPE, "h3_model_create: ffn_dim must be a positive multiple of 1024");
  if (dm.ctx_len < 1) return fail(H3_ESHAPE, "h3_model_create: ctx_len must be >= 1");
  if (!fits_u32(dm.ffn_dim, dm.d_model, dm.d_model, 2) || !fits_u32(dm.ctx_len, dm.d_model, dm.d_model, 2))
    return fail(H3_ESHAPE, "h3_model_create: ffn_dim x d_model or ctx_len x d_model spans 4 GiB or more");
  if (dm.latent_ch < 64 || dm.latent_ch % 64)
    return fail(H3_ESHAPE, "h3_model_create: latent_ch must be a positive multiple of 64");
  // the patch weight [d, C] and the head weight [C, d] are product operands too
  if (!fits_u32(dm.d_model, dm.latent_ch, dm.latent_ch, 2) || !fits_u32(dm.latent_ch, dm.d_model, dm.d_model, 2))
    return fail(H3_ESHAPE, "h3_model_create: latent_ch x d_model spans 4 GiB or more");
  const void *gp[] = {g->t1_w, g->t1_b, g->t2_w, g->t2_b, g->mod_w, g->mod_b, g->fin_w,
                      g->fin_b, g->fin_t, g->mod_table, g->patch_w, g->patch_b, g->head_w,
                      g->head_b};
  for (const void *q : gp)
    if (!q) return fail(H3_EINVAL, "h3_model_create: NULL global weight");
  for (int b = 0; b < n_blocks; ++b) {
    const h3_block_weights &w = blocks[b];
    const void *bp[] = {w.qkvq_w, w.qkvq_b, w.kc_w, w.kc_b, w.vc_w, w.vc_b, w.out_w, w.out_b,
                        w.outc_b, w.q_gamma, w.k_gamma, w.fc1_w, w.fc1_b, w.fc2_w, w.fc2_b};
    for (const void *q : bp)
      if (!q) return fail(H3_EINVAL, "h3_model_create: NULL weight in block " + std::to_string(b));
  }
  h3_model *m = new (std::nothrow) h3_model();
  if (!m) return fail(H3_EINVAL, "h3_model_create: out of host memory");
  m->dims = dm;
  m->head_dim = D;
  m->g = *g;
  m->blocks = new (std::nothrow) h3_block_weights[n_blocks];
  if (!m->blocks) {
    delete m;
    return fail(H3_EINVAL, "h3_model_create: out of host memory");
  }
  std::memcpy(m->blocks, blocks, sizeof(h3_block_weights) * n_blocks);
  *out = m;
  clear_error();
  return H3_OK;
}

void h3_model_destroy(h3_model *m) {
  if (!m) return;
  delete[] m->blocks;
  delete m;
}

int32_t h3_workspace_size(const h3_model *m, int32_t n_tokens, const h3_run_opts *o,
                          size_t *bytes) {
  if (int32_t e = validate_model(m)) return e;
  if (int32_t e = check_opts(o)) return e;
  if (!bytes) return fail(H3_EINVAL, "h3_workspace_size: bytes is NULL");
  if (int32_t e = check_tokens(m, n_tokens, "h3_workspace_size")) return e;
  *bytes = plan_workspace(*m, n_tokens, *o).total;
  return H3_OK;
}

int32_t h3_workspace_layout(const h3_model *m, int32_t n_tokens, const h3_run_opts *o,
                            h3_ws_layout *layout) {
  if (int32_t e = validate_model(m)) return e;
  if (int32_t e = check_opts(o)) return e;
  if (!layout) return fail(H3_EINVAL, "h3_workspace_layout: layout is NULL");
  if (int32_t e = check_tokens(m, n_tokens, "h3_workspace_layout")) return e;
  const WsPlan p = plan_workspace(*m, n_tokens, *o);
  layout->n1 = p.n1; layout->qkvq = p.qkvq; layout->attn = p.attn; layout->y = p.y;
  layout->n2 = p.n2; layout->h = p.h; layout->m = p.m; layout->hq = p.hq; layout->hs = p.hs;
  layout->rope = p.rope; layout->total = p.total;
  return H3_OK;
}

int32_t h3_prepare_context(const h3_model *m, const void *ctx, void *ctx_kv, void *stream) {
  if (int32_t e = validate_model(m)) return e;
  if (!ctx || !ctx_kv) return fail(H3_EINVAL, "h3_prepare_context: NULL pointer");
  const int d = m->dims.d_model, L = m->dims.ctx_len;
  hipStream_t s = as_stream(stream);
  bf16_t *kv = reinterpret_cast<bf16_t *>(ctx_kv);
  for (int b = 0; b < m->dims.n_blocks; ++b) {
    const h3_block_weights &w = m->blocks[b];
    bf16_t *kb = kv + static_cast<size_t>(b) * 2 * L * d;
    launch_gemm_bf16(reinterpret_cast<const bf16_t *>(ctx), d, reinterpret_cast<const bf16_t *>(w.kc_w),
                     d, kb, d, L, d, d, reinterpret_cast<const bf16_t *>(w.kc_b), nullptr,
                     H3_EPI_NONE, 0, s);
    launch_gemm_bf16(reinterpret_cast<const bf16_t *>(ctx), d, reinterpret_cast<const bf16_t *>(w.vc_w),
                     d, kb + static_cast<size_t>(L) * d, d, L, d, d,
                     reinterpret_cast<const bf16_t *>(w.vc_b), nullptr, H3_EPI_NONE, 0, s);
  }
  return check_launch("h3_prepare_context");
}

int32_t h3_quantize_fc2_weights(const h3_model *m, void *stream) {
  if (int32_t e = validate_model(m)) return e;
  for (int b = 0; b < m->dims.n_blocks; ++b)
    if (!m->blocks[b].fc2_q || !m->blocks[b].fc2_s)
      return fail(H3_EINVAL, "h3_quantize_fc2_weights: fc2_q/fc2_s not set in block " + std::to_string(b));
  hipStream_t s = as_stream(stream);
  const int d = m->dims.d_model, F = m->dims.ffn_dim;
  for (int b = 0; b < m->dims.n_blocks; ++b) {
    const h3_block_weights &w = m->blocks[b];
    launch_quant_rows(reinterpret_cast<const bf16_t *>(w.fc2_w), reinterpret_cast<int8_t *>(w.fc2_q),
                      reinterpret_cast<float *>(w.fc2_s), d, F, F, s);
  }
  return check_launch("h3_quantize_fc2_weights");
}

int32_t h3_quantize_linear_weights(const h3_model *m, void *stream) {
  if (int32_t e = validate_model(m)) return e;
  for (int b = 0; b < m->dims.n_blocks; ++b) {
    const h3_block_weights &w = m->blocks[b];
    if (!w.qkvq_q || !w.qkvq_s || !w.fc1_q || !w.fc1_s)
      return fail(H3_EINVAL, "h3_quantize_linear_weights: qkvq_q/qkvq_s/fc1_q/fc1_s not set in block " +
                                 std::to_string(b));
  }
  hipStream_t s = as_stream(stream);
  const int d = m->dims.d_model, F = m->dims.ffn_dim;
  for (int b = 0; b < m->dims.n_blocks; ++b) {
    const h3_block_weights &w = m->blocks[b];
    launch_quant_rows(reinterpret_cast<const bf16_t *>(w.qkvq_w), reinterpret_cast<int8_t *>(w.qkvq_q),
                      reinterpret_cast<float *>(w.qkvq_s), 4 * d, d, d, s);
    launch_quant_rows(reinterpret_cast<const bf16_t *>(w.fc1_w), reinterpret_cast<int8_t *>(w.fc1_q),
                      reinterpret_cast<float *>(w.fc1_s), F, d, d, s);
  }
  return check_launch("h3_quantize_linear_weights");
}

int32_t h3_modulation(const h3_model *m, float sigma, float *mod, float *mod_final, void *ws,
                      size_t ws_bytes, void *stream) {
  if (int32_t e = validate_model(m)) return e;
  if (!mod || !mod_final) return fail(H3_EINVAL, "h3_modulation: NULL output");
  if (!std::isfinite(sigma)) return fail(H3_EINVAL, "h3_modulation: sigma must be finite");
  h3_run_opts o{};
  const WsPlan p = plan_workspace(*m, 1, o);
  if (!ws || ws_bytes < p.total) return fail(H3_EWORKSPACE, "h3_modulation: workspace too small");
  return run_modulation(m, sigma, mod, mod_final, reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + p.tmp),
                        as_stream(stream));
}

}  // extern "C"

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up on the first call on each
// device (with that device current) and kept.
int32_t static_scratch(void **out, const char *who) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(H3_EHIP, std::string(who) + ": no current device");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(H3_EHIP, std::string(who) + ": device address of the static scratch: " +
                               hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return H3_OK;
}
}  // namespace

extern "C" {

int32_t h3_modulation_noalloc(const h3_model *m, float sigma, float *mod, float *mod_final,
                              void *stream) {
  if (int32_t e = validate_model(m)) return e;
  if (!mod || !mod_final) return fail(H3_EINVAL, "h3_modulation_noalloc: NULL output");
  if (!std::isfinite(sigma)) return fail(H3_EINVAL, "h3_modulation_noalloc: sigma must be finite");
  const size_t need = modulation_tmp_bytes(m->dims.d_model);
  if (need > kStaticScratchBytes)
    return fail(H3_ESHAPE, "h3_modulation_noalloc: d_model " + std::to_string(m->dims.d_model) +
                               " needs " + std::to_string(need) + " bytes of scratch, above the " +
                               std::to_string(kStaticScratchBytes) + "-byte static buffer");
  void *sp = nullptr;
  if (int32_t e = static_scratch(&sp, "h3_modulation_noalloc")) return e;
  return run_modulation(m, sigma, mod, mod_final, reinterpret_cast<float *>(sp), as_stream(stream));
}

int32_t h3_dit_block_fwd(const h3_model *m, int32_t block, const h3_geom *geom,
                         const h3_run_opts *o, void *x, const void *n1_in, void *n1_next,
                         const float *mod, const float *mod_next, const void *ctx_kv, void *ws,
                         size_t ws_bytes, void *stream) {
  if (int32_t e = validate_model(m)) return e;
  if (int32_t e = check_opts(o)) return e;
  if (block < 0 || block >= m->dims.n_blocks) return fail(H3_EINVAL, "h3_dit_block_fwd: bad block index");
  int32_t n = 0;
  if (int32_t e = h3_geom_tokens(geom, &n)) return e;
  if (int32_t e = check_tokens(m, n, "h3_dit_block_fwd")) return e;
  if (!x || !mod || !ctx_kv) return fail(H3_EINVAL, "h3_dit_block_fwd: NULL x, mod or ctx_kv");
  if (n1_next && !mod_next) return fail(H3_EINVAL, "h3_dit_block_fwd: n1_next needs mod_next");
  if (int32_t e = check_block_int8(m->blocks[block], *o, "h3_dit_block_fwd")) return e;
  const WsPlan p = plan_workspace(*m, n, *o);
  if (!ws || ws_bytes < p.total) return fail(H3_EWORKSPACE, "h3_dit_block_fwd: workspace too small");
  hipStream_t s = as_stream(stream);
  char *w = reinterpret_cast<char *>(ws);
  float2 *rope = reinterpret_cast<float2 *>(w + p.rope);
  launch_rope_table(rope, *geom, n, m->head_dim, s);
  return run_block(m, block, *geom, n, *o, reinterpret_cast<bf16_t *>(x), n1_in, n1_next,
                   o->int8_linear != 0, mod, mod_next, reinterpret_cast<const bf16_t *>(ctx_kv), w,
                   p, s, rope);
}

namespace {
enum CoreMode { kCorePlain = 0, kCoreFresh = 1, kCoreReuse = 2 };

// The velocity head v = AdaLN_final(x) W_h^T + b_h, float32 [n, C].  n_final: the final AdaLN,
// already stored (the last block's MLP gate computed it, which costs nothing extra), or NULL
// (after a bypass restore before the head, or for a cached core): then it is formed here,
// inside the head product's tile loads when o.fused_head_adaln is set and the product has that
// form, else by the AdaLN kernel into `scratch` (bf16 [n, d]) before the product.
void run_head(const h3_model *m, const h3_run_opts &o, const bf16_t *x, const bf16_t *n_final,
              const float *fin, float *velocity, int n, void *scratch, hipStream_t s) {
  const int d = m->dims.d_model, C = m->dims.latent_ch;
  const bf16_t *hw = reinterpret_cast<const bf16_t *>(m->g.head_w);
  const bf16_t *hb = reinterpret_cast<const bf16_t *>(m->g.head_b);
  if (!n_final && o.fused_head_adaln && head_adaln_gemm_fits(x, d, fin, fin + d, n, C, d)) {
    ProfScope ps(H3_ST_HEAD, s);
    launch_head_adaln_gemm(x, d, fin, fin + d, hw, d, hb, velocity, C, n, C, d, s);
    return;
  }
  if (!n_final) {
    ProfScope ps(H3_ST_ADALN, s);
    launch_gate_adaln(x, nullptr, nullptr, nullptr, fin, fin + d, reinterpret_cast<bf16_t *>(scratch),
                      n, d, s);
    n_final = reinterpret_cast<const bf16_t *>(scratch);
  }
  ProfScope ps(H3_ST_HEAD, s);
  launch_gemm_bf16(n_final, d, hw, d, velocity, C, n, C, d, hb, nullptr, H3_EPI_NONE, 1, s);
}
}  // namespace

// One evaluation.  kCorePlain: the forward.  kCoreFresh: the forward, and core_delta =
// x_L - x_0 (stream after the last active block minus the patch embedding).  kCoreReuse:
// x = bf16(x_0 + core_delta), then the final AdaLN of sigma and the head; the blocks are
// skipped.
static int32_t forward_impl(const h3_model *m, const h3_geom *geom, const h3_run_opts *o,
                            const float *latent, float sigma, const int32_t *active,
                            int32_t n_active, int32_t eval_index, const void *ctx_kv,
                            float *velocity, void *ws, size_t ws_bytes, void *stream,
                            int core_mode, float *core_delta) {
  if (int32_t e = validate_model(m)) return e;
  if (int32_t e = check_opts(o)) return e;
  if (!geom || geom->paired) return fail(H3_EINVAL, "h3_dit_forward: geom must be the full grid");
  int32_t n = 0;
  if (int32_t e = h3_geom_tokens(geom, &n)) return e;
  if (int32_t e = check_tokens(m, n, "h3_dit_forward")) return e;
  if (!latent || !velocity || !active || !ctx_kv) return fail(H3_EINVAL, "h3_dit_forward: NULL pointer");
  if (!std::isfinite(sigma)) return fail(H3_EINVAL, "h3_dit_forward: sigma must be finite");
  const int nb = m->dims.n_blocks;
  if (n_active < 1 || n_active > nb) return fail(H3_EINVAL, "h3_dit_forward: bad n_active");
  for (int i = 0; i < n_active; ++i) {
    if (active[i] < 0 || active[i] >= nb) return fail(H3_EINVAL, "h3_dit_forward: active index out of range");
    if (i && active[i] <= active[i - 1]) return fail(H3_EINVAL, "h3_dit_forward: active must ascend");
    if (int32_t e = check_block_int8(m->blocks[active[i]], *o, "h3_dit_forward")) return e;
  }
  if (eval_index < 0) return fail(H3_EINVAL, "h3_dit_forward: eval_index must be >= 0");
  int32_t merge_after = 0, restore_before = 0, n_red = 0;
  if (o->token_reduction) {
    if (int32_t e = h3_token_plan(geom->f_lat, geom->grid_h, geom->grid_w, eval_index, n_active,
                                  &merge_after, &restore_before, nullptr, &n_red))
      return e;
  }
  const WsPlan p = plan_workspace(*m, n, *o);
  if (!ws || ws_bytes < p.total) return fail(H3_EWORKSPACE, "h3_dit_forward: workspace too small");

  hipStream_t s = as_stream(stream);
  char *w = reinterpret_cast<char *>(ws);
  const int d = m->dims.d_model, C = m->dims.latent_ch, L = m->dims.ctx_len;
  float *mod = reinterpret_cast<float *>(w + p.mod);
  float *fin = reinterpret_cast<float *>(w + p.fin);
  bf16_t *x = reinterpret_cast<bf16_t *>(w + p.x);
  bf16_t *xr = reinterpret_cast<bf16_t *>(w + p.xr);
  void *na = w + p.n1b;
  void *nb_ = w + p.n1;
  const bool q8 = o->int8_linear != 0;
  bf16_t *lat16 = reinterpret_cast<bf16_t *>(w + p.lat16);
  float2 *rope_full = reinterpret_cast<float2 *>(w + p.rope);
  float2 *rope_red = reinterpret_cast<float2 *>(w + p.rope_r);
  const bf16_t *kv = reinterpret_cast<const bf16_t *>(ctx_kv);

  {
    ProfScope ps(H3_ST_MODULATION, s);
    if (int32_t e = run_modulation(m, sigma, mod, fin, reinterpret_cast<float *>(w + p.tmp), s)) return e;
  }
  {
    // patch embedding: x = bf16(latent) W_p^T + b_p
    ProfScope ps(H3_ST_PATCH, s);
    launch_f32_to_bf16(latent, lat16, static_cast<int64_t>(n) * C, s);
    launch_gemm_bf16(lat16, C, reinterpret_cast<const bf16_t *>(m->g.patch_w), C, x, d, n, d, C,
                     reinterpret_cast<const bf16_t *>(m->g.patch_b), nullptr, H3_EPI_NONE, 0, s);
  }
  const int64_t nd = static_cast<int64_t>(n) * d;
  bf16_t *x0 = reinterpret_cast<bf16_t *>(w + p.x0);
  if (core_mode == kCoreReuse) {
    // cached core: x = bf16(x_0 + delta); final AdaLN of this sigma; head
    launch_core_apply(x, core_delta, x, nd, s);
    run_head(m, *o, x, nullptr, fin, velocity, n, w + p.n1b, s);
    return check_launch("h3_dit_forward_cached");
  }
  if (core_mode == kCoreFresh) {
    if (hipMemcpyAsync(x0, x, static_cast<size_t>(nd) * sizeof(bf16_t), hipMemcpyDeviceToDevice, s) !=
        hipSuccess)
      return fail(H3_EHIP, "h3_dit_forward_cached: copy of the patch embedding failed");
  }
  launch_rope_table(rope_full, *geom, n, m->head_dim, s);
  h3_geom red = *geom;
  red.paired = 1;
  if (o->token_reduction) launch_rope_table(rope_red, red, n_red, m->head_dim, s);

  // n1 of the first block; the n1 buffers alternate between na and the block plan's n1 slot
  bf16_t *cur = x;
  int rows = n;
  const float2 *rope = rope_full;
  const h3_geom *g_cur = geom;
  void *n1 = na, *n1_other = nb_;
  bool n1_valid = false;
  for (int pos = 0; pos < n_active; ++pos) {
    const int b = active[pos];
    const float *mb = mod + static_cast<size_t>(b) * 6 * d;
    if (o->token_reduction && pos == merge_after) {
      ProfScope ps(H3_ST_TOKEN_REDUCE, s);
      launch_token_reduce(0, *geom, d, x, nullptr, xr, s);
      cur = xr; rows = n_red; rope = rope_red; g_cur = &red; n1_valid = false;
    }
    if (o->token_reduction && pos == restore_before - 1) {
      ProfScope ps(H3_ST_TOKEN_REDUCE, s);
      launch_token_reduce(1, *geom, d, xr, x, x, s);
      cur = x; rows = n; rope = rope_full; g_cur = geom; n1_valid = false;
    }
    if (!n1_valid) {
      ProfScope ps(H3_ST_ADALN, s);
      gate_then_adaln(cur, nullptr, nullptr, mb, mb + d, n1, q8, true, rows, d, s);
    }
    // the next AdaLN can be fused into this block's MLP gate when no token op sits between
    const bool last = pos + 1 == n_active;
    const bool token_op_next = o->token_reduction && !last &&
                               (pos + 1 == merge_after || pos + 1 == restore_before - 1);
    const bool restore_before_head = o->token_reduction && last && restore_before == n_active + 1 &&
                                     merge_after < n_active;
    const float *mnext = nullptr;
    void *n1n = nullptr;
    if (!last && !token_op_next) {
      mnext = mod + static_cast<size_t>(active[pos + 1]) * 6 * d;
      n1n = n1_other;
    } else if (last && !restore_before_head) {
      mnext = fin;
      n1n = n1_other;
    }
    // n1 is always supplied, so the block never writes its own n1 slot (p.n1), which serves
    // here as the second of the two alternating n1 buffers
    // the final AdaLN (mnext == fin) feeds the bf16 head, so it is never quantised
    int32_t e = run_block(m, b, *g_cur, rows, *o, cur, n1, n1n, q8 && mnext != fin, mb, mnext,
                          kv + static_cast<size_t>(b) * 2 * L * d, w, p, s, rope);
    if (e) return e;
    if (n1n) {
      std::swap(n1, n1_other);
      n1_valid = true;
    } else {
      n1_valid = false;
    }
    if (last && restore_before_head) {
      {
        ProfScope ps(H3_ST_TOKEN_REDUCE, s);
        launch_token_reduce(1, *geom, d, xr, x, x, s);
      }
      cur = x; rows = n;
      n1_valid = false;
    }
  }
  if (core_mode == kCoreFresh) launch_core_delta(x, x0, core_delta, nd, s);
  // head: velocity = AdaLN_final(x) W_h^T + b_h, float32 (n1 holds the final AdaLN when the
  // last block's MLP gate computed it)
  run_head(m, *o, x, n1_valid ? reinterpret_cast<const bf16_t *>(n1) : nullptr, fin, velocity, n,
           n1_other, s);
  return check_launch("h3_dit_forward");
}

int32_t h3_dit_forward(const h3_model *m, const h3_geom *geom, const h3_run_opts *o,
                       const float *latent, float sigma, const int32_t *active, int32_t n_active,
                       int32_t eval_index, const void *ctx_kv, float *velocity, void *ws,
                       size_t ws_bytes, void *stream) {
  return forward_impl(m, geom, o, latent, sigma, active, n_active, eval_index, ctx_kv, velocity,
                      ws, ws_bytes, stream, kCorePlain, nullptr);
}

int32_t h3_dit_forward_cached(const h3_model *m, const h3_geom *geom, const h3_run_opts *o,
                              const float *latent, float sigma, const int32_t *active,
                              int32_t n_active, int32_t eval_index, const void *ctx_kv,
                              int32_t refresh_core, float *core_delta, float *velocity, void *ws,
                              size_t ws_bytes, void *stream) {
  if (!core_delta) return fail(H3_EINVAL, "h3_dit_forward_cached: core_delta is NULL");
  if (refresh_core != 0 && refresh_core != 1)
    return fail(H3_EINVAL, "h3_dit_forward_cached: refresh_core must be 0 or 1");
  return forward_impl(m, geom, o, latent, sigma, active, n_active, eval_index, ctx_kv, velocity,
                      ws, ws_bytes, stream, refresh_core ? kCoreFresh : kCoreReuse, core_delta);
}

int32_t h3_euler_step(float *latent, const float *velocity, float sigma_cur, float sigma_next,
                      int64_t n_elems, void *stream) {
  if (!latent || !velocity) return fail(H3_EINVAL, "h3_euler_step: NULL pointer");
  if (n_elems < 0) return fail(H3_EINVAL, "h3_euler_step: n_elems must be >= 0");
  if (!std::isfinite(sigma_cur) || !std::isfinite(sigma_next))
    return fail(H3_EINVAL, "h3_euler_step: sigmas must be finite");
  if (reinterpret_cast<uintptr_t>(latent) % 16 || reinterpret_cast<uintptr_t>(velocity) % 16)
    return fail(H3_EINVAL, "h3_euler_step: pointers must be 16-byte aligned");
  if (n_elems == 0) return H3_OK;
  const float dt = sigma_next - sigma_cur;
  ProfScope ps(H3_ST_EULER, as_stream(stream));
  launch_euler(latent, velocity, dt, n_elems, as_stream(stream));
  return check_launch("h3_euler_step");
}

int32_t h3_token_reduce(int32_t direction, const h3_geom *geom, int32_t d_model, const void *src,
                        const void *bypass, void *dst, void *stream) {
  if (direction != 0 && direction != 1) return fail(H3_EINVAL, "h3_token_reduce: direction must be 0 or 1");
  int32_t n = 0;
  if (int32_t e = h3_geom_tokens(geom, &n)) return e;
  if (geom->paired) return fail(H3_EINVAL, "h3_token_reduce: geom must be the full grid");
  if (d_model < 8 || d_model % 8) return fail(H3_ESHAPE, "h3_token_reduce: d_model must be a multiple of 8");
  if (!src || !dst || (direction == 1 && !bypass)) return fail(H3_EINVAL, "h3_token_reduce: NULL pointer");
  if (dst == src) return fail(H3_EINVAL, "h3_token_reduce: dst must not alias src");
  if (direction == 0 && bypass) return fail(H3_EINVAL, "h3_token_reduce: merge takes no bypass");
  launch_token_reduce(direction, *geom, d_model, reinterpret_cast<const bf16_t *>(src),
                      reinterpret_cast<const bf16_t *>(bypass), reinterpret_cast<bf16_t *>(dst),
                      as_stream(stream));
  return check_launch("h3_token_reduce");
}

int32_t h3_gemm_bf16(const void *A, int64_t lda, const void *B, int64_t ldb, void *C, int64_t ldc,
                     int32_t M, int32_t N, int32_t K, const void *bias, const void *bias2,
                     int32_t epilogue, int32_t out_f32, void *stream) {
  if (!A || !B || !C) return fail(H3_EINVAL, "h3_gemm_bf16: NULL pointer");
  if (M < 1 || N < 1 || K < 64 || K % 64) return fail(H3_ESHAPE, "h3_gemm_bf16: need M,N >= 1 and K % 64 == 0");
  if (lda < K || ldb < K || ldc < N || lda % 8 || ldb % 8)
    return fail(H3_ESHAPE, "h3_gemm_bf16: strides too small or not multiples of 8");
  if (!fits_u32(M, lda, K, 2) || !fits_u32(N, ldb, K, 2))
    return fail(H3_ESHAPE, "h3_gemm_bf16: an operand spans 4 GiB or more");
  if (epilogue != H3_EPI_NONE && epilogue != H3_EPI_GELU) return fail(H3_EINVAL, "h3_gemm_bf16: bad epilogue");
  if (out_f32 && epilogue != H3_EPI_NONE) return fail(H3_EUNSUPPORTED, "h3_gemm_bf16: GELU with float output");
  launch_gemm_bf16(reinterpret_cast<const bf16_t *>(A), lda, reinterpret_cast<const bf16_t *>(B), ldb,
                   C, ldc, M, N, K, reinterpret_cast<const bf16_t *>(bias),
                   reinterpret_cast<const bf16_t *>(bias2), epilogue, out_f32, as_stream(stream));
  return check_launch("h3_gemm_bf16");
}

int32_t h3_attention(const void *Q, int64_t ldq, const void *K, int64_t ldk, const void *V,
                     int64_t ldv, void *O, int64_t ldo, int32_t n_q, int32_t n_k, int32_t n_heads,
                     int32_t head_dim, void *stream) {
  if (!Q || !K || !V || !O) return fail(H3_EINVAL, "h3_attention: NULL pointer");
  if (head_dim != 64 && head_dim != 128) return fail(H3_EUNSUPPORTED, "h3_attention: head_dim must be 64 or 128");
  if (n_q < 1 || n_k < 1 || n_heads < 1 || n_heads > 65535) return fail(H3_ESHAPE, "h3_attention: need n_q, n_k >= 1 and 1 <= n_heads <= 65535");
  const int64_t w = static_cast<int64_t>(n_heads) * head_dim;
  if (ldq < w || ldk < w || ldv < w || ldo < w || ldq % 8 || ldk % 8 || ldv % 8 || ldo % 8)
    return fail(H3_ESHAPE, "h3_attention: strides too small or not multiples of 8");
  if (ldk > (int64_t{1} << 24) || ldv > (int64_t{1} << 24))
    return fail(H3_ESHAPE, "h3_attention: key / value strides above 2^24 elements");
  launch_attention(reinterpret_cast<const bf16_t *>(Q), ldq, reinterpret_cast<const bf16_t *>(K), ldk,
                   reinterpret_cast<const bf16_t *>(V), ldv, reinterpret_cast<bf16_t *>(O), ldo, n_q,
                   n_k, n_heads, head_dim, as_stream(stream));
  return check_launch("h3_attention");
}

int32_t h3_quant_rows(const void *X, void *Q, float *S, int32_t rows, int32_t K, int32_t group,
                      void *stream) {
  if (!X || !Q || !S) return fail(H3_EINVAL, "h3_quant_rows: NULL pointer");
  if (group != K && group != 1024) return fail(H3_EINVAL, "h3_quant_rows: group must be K or 1024");
  if (rows < 1 || K < 512 || K % 512 || (group == 1024 && K % 1024))
    return fail(H3_ESHAPE, "h3_quant_rows: need rows >= 1 and K a multiple of 512 (of 1024 with groups)");
  launch_quant_rows(reinterpret_cast<const bf16_t *>(X), reinterpret_cast<int8_t *>(Q), S, rows, K,
                    group, as_stream(stream));
  return check_launch("h3_quant_rows");
}

int32_t h3_gemm_i8(const void *QA, const float *SA, const void *QW, const float *SW,
                   const void *bias, void *C, int64_t ldc, int32_t M, int32_t N, int32_t K,
                   int32_t group, int32_t epilogue, void *stream) {
  if (!QA || !SA || !QW || !SW || !bias || !C) return fail(H3_EINVAL, "h3_gemm_i8: NULL pointer");
  if (group != K && group != 1024) return fail(H3_EINVAL, "h3_gemm_i8: group must be K or 1024");
  if (M < 1 || N < 1 || K < 128 || K % 128 || (group == 1024 && K % 1024))
    return fail(H3_ESHAPE, "h3_gemm_i8: need M, N >= 1 and K a multiple of 128 (of 1024 with groups)");
  if (ldc < N) return fail(H3_ESHAPE, "h3_gemm_i8: ldc < N");
  if (!fits_u32(M, K, K, 1) || !fits_u32(N, K, K, 1))
    return fail(H3_ESHAPE, "h3_gemm_i8: an operand spans 4 GiB or more");
  if (epilogue != H3_EPI_NONE && epilogue != H3_EPI_GELU) return fail(H3_EINVAL, "h3_gemm_i8: bad epilogue");
  launch_gemm_i8(reinterpret_cast<const int8_t *>(QA), SA, reinterpret_cast<const int8_t *>(QW), SW,
                 reinterpret_cast<const bf16_t *>(bias), reinterpret_cast<bf16_t *>(C), ldc, M, N, K,
                 group, as_stream(stream), SplitScratch(), epilogue);
  return check_launch("h3_gemm_i8");
}

int32_t h3_gate_adaln(const void *x, const void *y, const float *gate, void *x_out,
                      const float *shift, const float *scale, void *n_out, int32_t rows,
                      int32_t d_model, void *stream) {
  if (!x) return fail(H3_EINVAL, "h3_gate_adaln: x is NULL");
  if (!y && !n_out) return fail(H3_EINVAL, "h3_gate_adaln: nothing to compute");
  if (y && (!gate || !x_out)) return fail(H3_EINVAL, "h3_gate_adaln: gate needs gate and x_out");
  if (n_out && (!shift || !scale)) return fail(H3_EINVAL, "h3_gate_adaln: AdaLN needs shift and scale");
  if (rows < 1) return fail(H3_ESHAPE, "h3_gate_adaln: rows must be >= 1");
  if (!supported_width(d_model)) return fail(H3_ESHAPE, "h3_gate_adaln: unsupported d_model");
  launch_gate_adaln(reinterpret_cast<const bf16_t *>(x), reinterpret_cast<const bf16_t *>(y), gate,
                    reinterpret_cast<bf16_t *>(x_out), shift, scale, reinterpret_cast<bf16_t *>(n_out),
                    rows, d_model, as_stream(stream));
  return check_launch("h3_gate_adaln");
}

int32_t h3_gate_adaln_quant(const void *x, const void *y, const float *gate, void *x_out,
                            const float *shift, const float *scale, void *q_out, float *s_out,
                            int32_t rows, int32_t d_model, void *stream) {
  if (!x || !shift || !scale || !q_out || !s_out) return fail(H3_EINVAL, "h3_gate_adaln_quant: NULL pointer");
  if (y && (!gate || !x_out)) return fail(H3_EINVAL, "h3_gate_adaln_quant: gate needs gate and x_out");
  if (rows < 1) return fail(H3_ESHAPE, "h3_gate_adaln_quant: rows must be >= 1");
  if (!supported_width(d_model)) return fail(H3_ESHAPE, "h3_gate_adaln_quant: unsupported d_model");
  launch_gate_adaln(reinterpret_cast<const bf16_t *>(x), reinterpret_cast<const bf16_t *>(y), gate,
                    reinterpret_cast<bf16_t *>(x_out), shift, scale, nullptr, rows, d_model,
                    as_stream(stream), reinterpret_cast<int8_t *>(q_out), s_out);
  return check_launch("h3_gate_adaln_quant");
}

int32_t h3_head_adaln_gemm(const void *x, const float *shift, const float *scale, const void *W,
                           const void *bias, float *out, int32_t rows, int32_t d_model,
                           int32_t n_out, void *stream) {
  if (!x || !shift || !scale || !W || !out) return fail(H3_EINVAL, "h3_head_adaln_gemm: NULL pointer");
  if (rows < 1) return fail(H3_ESHAPE, "h3_head_adaln_gemm: rows must be >= 1");
  if (!supported_width(d_model)) return fail(H3_ESHAPE, "h3_head_adaln_gemm: unsupported d_model");
  if (n_out < 1 || n_out % 8) return fail(H3_ESHAPE, "h3_head_adaln_gemm: n_out must be a positive multiple of 8");
  if (!fits_u32(rows, d_model, d_model, 2) || !fits_u32(n_out, d_model, d_model, 2))
    return fail(H3_ESHAPE, "h3_head_adaln_gemm: an operand spans 4 GiB or more");
  const bf16_t *xb = reinterpret_cast<const bf16_t *>(x);
  if (!head_adaln_gemm_fits(xb, d_model, shift, scale, rows, n_out, d_model))
    return fail(H3_EUNSUPPORTED,
                "h3_head_adaln_gemm: no fused form (n_out >= 192, or x / shift / scale not 16-byte aligned)");
  launch_head_adaln_gemm(xb, d_model, shift, scale, reinterpret_cast<const bf16_t *>(W), d_model,
                         reinterpret_cast<const bf16_t *>(bias), out, n_out, rows, n_out, d_model,
                         as_stream(stream));
  return check_launch("h3_head_adaln_gemm");
}

int32_t h3_mfma_probe(int32_t int8, int32_t iters, int32_t workgroups, float *out, void *stream) {
  if (int8 != 0 && int8 != 1) return fail(H3_EINVAL, "h3_mfma_probe: int8 must be 0 or 1");
  if (!out) return fail(H3_EINVAL, "h3_mfma_probe: out is NULL");
  if (iters < 1 || workgroups < 1 || workgroups > (1 << 20))
    return fail(H3_ESHAPE, "h3_mfma_probe: iters must be >= 1 and workgroups in [1, 2^20]");
  launch_mfma_probe(int8, iters, workgroups, out, as_stream(stream));
  return check_launch("h3_mfma_probe");
}

int32_t h3_rope_table(const h3_geom *geom, int32_t head_dim, void *table, void *stream) {
  int32_t n = 0;
  if (int32_t e = h3_geom_tokens(geom, &n)) return e;
  if (!table) return fail(H3_EINVAL, "h3_rope_table: table is NULL");
  if (head_dim != 64 && head_dim != 128) return fail(H3_EUNSUPPORTED, "h3_rope_table: head_dim must be 64 or 128");
  launch_rope_table(reinterpret_cast<float2 *>(table), *geom, n, head_dim, as_stream(stream));
  return check_launch("h3_rope_table");
}

int32_t h3_qk_norm_rope(void *qkvq, int64_t ld, int32_t n_tokens, int32_t d_model,
                        int32_t head_dim, const void *q_gamma, const void *k_gamma,
                        int32_t qk_norm, const void *table, void *stream) {
  if (!qkvq || !table || (qk_norm && (!q_gamma || !k_gamma)))
    return fail(H3_EINVAL, "h3_qk_norm_rope: NULL pointer");
  if (head_dim != 64 && head_dim != 128) return fail(H3_EUNSUPPORTED, "h3_qk_norm_rope: head_dim must be 64 or 128");
  if (n_tokens < 1 || d_model < 512 || d_model % 512 || d_model % head_dim)
    return fail(H3_ESHAPE, "h3_qk_norm_rope: need n_tokens >= 1 and d_model a multiple of 512 and of head_dim");
  if (ld < 2 * d_model || ld % 8) return fail(H3_ESHAPE, "h3_qk_norm_rope: ld too small or not a multiple of 8");
  launch_qk_norm_rope(reinterpret_cast<bf16_t *>(qkvq), ld, n_tokens, d_model, head_dim,
                      reinterpret_cast<const bf16_t *>(q_gamma), reinterpret_cast<const bf16_t *>(k_gamma),
                      qk_norm, reinterpret_cast<const float2 *>(table), as_stream(stream));
  return check_launch("h3_qk_norm_rope");
}

int32_t h3_qkv_gemm(const void *A, int64_t lda, const float *SA, const void *W, int64_t ldw,
                    const float *SW, const void *bias, void *C, int64_t ldc, int32_t M,
                    int32_t d_model, int32_t K, int32_t head_dim, const void *q_gamma,
                    const void *k_gamma, int32_t qk_norm, const void *table, int32_t a_q8,
                    int32_t fused, int32_t *fused_used, void *stream) {
  if (fused_used) *fused_used = 0;
  if (!A || !W || !bias || !C || !table || (a_q8 && (!SA || !SW)) || (qk_norm && (!q_gamma || !k_gamma)))
    return fail(H3_EINVAL, "h3_qkv_gemm: NULL pointer");
  if ((a_q8 != 0 && a_q8 != 1) || (fused != 0 && fused != 1) || (qk_norm != 0 && qk_norm != 1))
    return fail(H3_EINVAL, "h3_qkv_gemm: a_q8, fused and qk_norm must be 0 or 1");
  if (head_dim != 64 && head_dim != 128) return fail(H3_EUNSUPPORTED, "h3_qkv_gemm: head_dim must be 64 or 128");
  if (M < 1 || d_model < 512 || d_model % 512 || d_model % head_dim)
    return fail(H3_ESHAPE, "h3_qkv_gemm: need M >= 1 and d_model a multiple of 512 and of head_dim");
  if (ldc < 4 * static_cast<int64_t>(d_model) || ldc % 8) return fail(H3_ESHAPE, "h3_qkv_gemm: ldc too small or not a multiple of 8");
  if (a_q8) {
    if (K < 128 || K % 128 || lda != K || ldw != K) return fail(H3_ESHAPE, "h3_qkv_gemm: int8 needs K % 128 == 0 and lda = ldw = K");
  } else {
    if (K < 64 || K % 64 || lda < K || ldw < K || lda % 8 || ldw % 8)
      return fail(H3_ESHAPE, "h3_qkv_gemm: need K % 64 == 0, lda, ldw >= K and multiples of 8");
  }
  if (!fits_u32(M, lda, K, a_q8 ? 1 : 2) || !fits_u32(4 * static_cast<int64_t>(d_model), ldw, K, a_q8 ? 1 : 2))
    return fail(H3_ESHAPE, "h3_qkv_gemm: an operand spans 4 GiB or more");
  const hipStream_t s = as_stream(stream);
  const QkEpi qe{reinterpret_cast<const bf16_t *>(q_gamma), reinterpret_cast<const bf16_t *>(k_gamma),
                 reinterpret_cast<const float2 *>(table), d_model, qk_norm};
  bf16_t *c = reinterpret_cast<bf16_t *>(C);
  const bf16_t *b = reinterpret_cast<const bf16_t *>(bias);
  int done = 0;
  if (a_q8) {
    const int8_t *qa = reinterpret_cast<const int8_t *>(A), *qw = reinterpret_cast<const int8_t *>(W);
    if (fused) done = launch_gemm_i8_qkv(qa, SA, qw, SW, b, c, ldc, M, d_model, K, head_dim, qe, s);
    if (!done) launch_gemm_i8(qa, SA, qw, SW, b, c, ldc, M, 4 * d_model, K, K, s);
  } else {
    const bf16_t *a = reinterpret_cast<const bf16_t *>(A), *w = reinterpret_cast<const bf16_t *>(W);
    if (fused) done = launch_gemm_bf16_qkv(a, lda, w, ldw, b, c, ldc, M, d_model, K, head_dim, qe, s);
    if (!done) launch_gemm_bf16(a, lda, w, ldw, c, ldc, M, 4 * d_model, K, b, nullptr, H3_EPI_NONE, 0, s);
  }
  if (!done)
    launch_qk_norm_rope(c, ldc, M, d_model, head_dim, qe.q_gamma, qe.k_gamma, qk_norm, qe.table, s);
  if (fused_used) *fused_used = done;
  return check_launch("h3_qkv_gemm");
}

}  // extern "C"
