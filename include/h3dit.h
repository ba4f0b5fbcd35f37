/*
 * h3dit.h -- C ABI of the MiniMax-H3 DiT denoiser hot path for AMD MI355X (gfx950).
 *
 * The library (libh3dit.so) computes one fresh DiT denoiser evaluation over video latent
 * tokens, the blocks it is made of, the Euler transition that consumes its velocity, the
 * horizontal token pairing and the integer host logic of the sampler (frame alignment,
 * token grid, sigma schedule, layer thinning, pairing plan).
 *
 * Citation keys (the public pages describing the h3.c / h3-metal engine):
 *   P1 news.ditty.ir  "h3: native MiniMax-H3 on Apple Silicon"
 *   P2 aihot.vn       "H3-metal: running MiniMax-H3 directly on Apple Silicon", tutorial §1-§5
 *   P3 dothoosh.com   "How h3.c cuts MiniMax-H3 video inference to 3.5 seconds on M5"
 *                     sections "DiT fusions and memory", "aggressive levers", "the int8 path",
 *                     "memory and resolution limits", "temporal shapes and prompting"
 *   P4 wqu.guru       "h3-metal: native MiniMax-H3 inference for Apple Silicon", §1-§4, preset table
 *   P5 iitog.ru       "H3-metal: native inference of the MiniMax-H3 video model", key facts
 *
 * Conventions (all entry points):
 *   - Return value: H3_OK (0) or a negative H3_E* code.  h3_last_error() returns a
 *     thread-local message for the last failure on the calling thread.
 *   - Arguments are validated before anything is launched: a call that fails validation
 *     leaves device memory untouched.  No C++ exception crosses this boundary.
 *   - Device memory is owned by the caller.  The library never allocates or frees device
 *     memory; intermediate buffers live in a caller-provided workspace sized by
 *     h3_workspace_size().  The only library-owned object is the host-side h3_model.
 *   - "device" pointers must be HIP device allocations on the current device; "host"
 *     pointers are ordinary CPU memory.
 *   - stream: a hipStream_t passed as void* (NULL = the default stream).  All device work
 *     is enqueued asynchronously on it; no call synchronises the device except where noted.
 *   - Layouts are row-major.  Activations are [tokens, width] bf16 stored as uint16_t with
 *     token order n = (f * grid_h + h) * grid_w + w.  Weights are [out, in] bf16 (the "in"
 *     dimension contiguous).  Latent and velocity are [tokens, latent_ch] float32.
 *   - bf16 values are rounded to nearest-even on every store.
 *   - A handle is not safe for concurrent use from two host threads.
 */
#ifndef H3DIT_H
#define H3DIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  H3_OK = 0,
  H3_EINVAL = -1,        /* bad argument value or NULL pointer */
  H3_ESHAPE = -2,        /* shapes inconsistent with the model or with each other */
  H3_EUNSUPPORTED = -3,  /* valid request outside what this path implements */
  H3_EWORKSPACE = -4,    /* workspace missing or too small */
  H3_EHIP = -5           /* a HIP runtime call or kernel launch failed */
};

/* Message for the last error on this thread ("" if none). Never NULL. */
const char *h3_last_error(void);
/* ABI version of this header (major * 100 + minor). */
int32_t h3_abi_version(void);

/* ------------------------------------------------------------------------------------
 * Host integer logic (no device work; results are exact and match the oracle bit for bit)
 * ---------------------------------------------------------------------------------- */

/* P2 §5, P3 "temporal shapes": frame requests round up to the next 5 + 17 n, n >= 0
 * (23 -> 39).  requested >= 1, else H3_EINVAL.  *frames receives the aligned count. */
int32_t h3_align_frames(int32_t requested, int32_t *frames);

/* P5 key facts: `--seconds s` asks for ceil(24 s) frames at 24 fps, then aligns
 * (10 s -> 243).  seconds > 0 and ceil(24 s) <= INT32_MAX, else H3_EINVAL. */
int32_t h3_frames_for_seconds(double seconds, int32_t *frames);

/* Latent frames of an aligned clip: 1 + floor((frames - 1) / 4) (5 -> 2, 22 -> 6,
 * 243 -> 61; the pages do not give this mapping).  frames >= 1. */
int32_t h3_latent_frames(int32_t frames, int32_t *f_lat);

/* P2 §5, P3 "memory and resolution limits": width and height are multiples of 32, at
 * least 32, with width * height <= 768 * 1344, else H3_EINVAL.  One token per 32x32
 * pixels: grid_h = height / 32, grid_w = width / 32.  P2 §5: the spatial RoPE coordinates
 * are halved at the 8x8 grid (256x256 output) unless reference_rope != 0:
 * *rope_spatial_scale = 0.5 there, else 1.0. */
int32_t h3_token_grid(int32_t width, int32_t height, int32_t reference_rope,
                      int32_t *grid_h, int32_t *grid_w, float *rope_spatial_scale);

/* Sigma grid and fresh-evaluation mask of the Euler loop.  P2 §2: `--steps N` runs
 * exactly N denoising passes on a linear grid with one endpoint; P3 "aggressive levers"
 * and P4 table: `--reuse r` evaluates the denoiser at 20/11/8 of 20 steps for r = 1/2/3
 * and extrapolates the skipped transitions; P2 §4: --reuse and --core-reuse exclude each
 * other, and --core-reuse k (k <= 6) runs the core less often while the patch and the
 * timestep-dependent head stay fresh (h3_dit_forward_cached).
 *   sigmas (host, float[steps + 1]): sigma_i = (float)(steps - i) / (float)steps.
 *   fresh  (host, uint8[steps]): 1 iff i % r == 0 or i == steps - 1, r = reuse, or
 *          core_reuse when that is > 1 (then: the steps whose core runs fresh).
 *   n_fresh: number of fresh evaluations (of the core, with core_reuse > 1).
 * 1 <= steps <= 2^20, reuse >= 1, 1 <= core_reuse <= 6 (H3_EINVAL); reuse > 1 with
 * core_reuse > 1 is H3_EINVAL. */
int32_t h3_schedule(int32_t steps, int32_t reuse, int32_t core_reuse, float *sigmas,
                    uint8_t *fresh, int32_t *n_fresh);

/* `--layers L` (P3 "aggressive levers": rank blocks by their AdaLN gates, protect the
 * first and last).  mod_table (host, bf16 [n_blocks, 6, d_model], rows sh1 sc1 g1 sh2 sc2
 * g2 of the learned per-block modulation table).  Key of block b = sum over channels of
 * |g1| + |g2| in double, channels ascending; blocks 0 and n_blocks-1 are always kept; the
 * n_blocks - n_active smallest keys are dropped (ties: higher index first).
 * active (host, int32[n_active]) receives the kept block indices ascending.
 * 2 <= n_active <= n_blocks, else H3_EINVAL. */
int32_t h3_select_layers(const uint16_t *mod_table, int32_t n_blocks, int32_t d_model,
                         int32_t n_active, int32_t *active);

/* Horizontal token pairing plan for one fresh evaluation (P1; P3 "aggressive levers":
 * pairs after block 3; the bypass restores full resolution before block 40 in the first 10
 * evaluations, before block 30 later).  Positions are 1-based in the active list:
 * *merge_after = 3; *restore_before = 40 (eval_index < 10) or 30, capped at n_active + 1
 * (= before the head).  Reduced token j of row (f, h) pairs full tokens at columns 2j and
 * 2j+1 (an odd last column pairs with itself).  pairs (host, int32[2 * n_reduced], may be
 * NULL) receives (src0, src1) per reduced token; *n_reduced = f_lat*grid_h*ceil(grid_w/2).
 * n_active > 3, all sizes >= 1, else H3_EINVAL; more than 2^24 full-grid tokens: H3_ESHAPE
 * (the cap of h3_geom_tokens). */
int32_t h3_token_plan(int32_t f_lat, int32_t grid_h, int32_t grid_w, int32_t eval_index,
                      int32_t n_active, int32_t *merge_after, int32_t *restore_before,
                      int32_t *pairs, int32_t *n_reduced);

/* ------------------------------------------------------------------------------------
 * Model
 * ---------------------------------------------------------------------------------- */

typedef struct h3_dims {
  int32_t d_model;    /* d: residual width (multiple of 512) */
  int32_t n_heads;    /* H; head_dim = d_model / n_heads must be 64 or 128 */
  int32_t ffn_dim;    /* F: MLP width (multiple of 1024) */
  int32_t ctx_len;    /* L_ctx: text-context tokens (>= 1) */
  int32_t latent_ch;  /* C: latent channels per token (multiple of 64) */
  int32_t n_blocks;   /* number of DiT blocks (>= 1) */
} h3_dims;

/* Global weights (device, bf16 unless noted).  Modulation (reading of P3 "DiT fusions":
 * AdaLN shift/scale/gate come from the timestep): temb = t2(SiLU(t1(sinusoid(1000 sigma))));
 * block b uses mod(SiLU(temb)) + mod_table[b]; the final AdaLN uses fin(SiLU(temb)) + fin_t. */
typedef struct h3_global_weights {
  const void *t1_w, *t1_b;       /* [d, 256], [d] */
  const void *t2_w, *t2_b;       /* [d, d], [d] */
  const void *mod_w, *mod_b;     /* [6d, d], [6d] */
  const void *fin_w, *fin_b;     /* [2d, d], [2d] */
  const void *fin_t;             /* [2, d] */
  const void *mod_table;         /* [n_blocks, 6, d] */
  const void *patch_w, *patch_b; /* [d, C], [d] */
  const void *head_w, *head_b;   /* [C, d], [C] */
} h3_global_weights;

/* Per-block weights (device, bf16 unless noted). */
typedef struct h3_block_weights {
  const void *qkvq_w;  /* [4d, d]: rows W_q; W_k; W_v (self-attention) then W_qc (cross Q) */
  const void *qkvq_b;  /* [4d] */
  const void *kc_w, *kc_b;   /* cross-attention K of the text context: [d, d], [d] */
  const void *vc_w, *vc_b;   /* cross-attention V: [d, d], [d] */
  const void *out_w;   /* [d, 2d]: columns [W_o | W_oc] (self and cross output projections) */
  const void *out_b, *outc_b;  /* [d] each, both added */
  const void *q_gamma, *k_gamma;  /* [head_dim] RMSNorm gains */
  const void *fc1_w, *fc1_b;  /* [F, d], [F] */
  const void *fc2_w, *fc2_b;  /* [d, F], [d] */
  void *fc2_q;   /* int8 [d, F] or NULL: written by h3_quantize_fc2_weights */
  void *fc2_s;   /* float [d] or NULL: per-output-channel scales, same */
  /* int8 copies for the int8 QKV / FC1 path (h3_run_opts.int8_linear), or NULL; written by
   * h3_quantize_linear_weights with the same per-output-channel rule */
  void *qkvq_q;  /* int8 [4d, d] */
  void *qkvq_s;  /* float [4d] */
  void *fc1_q;   /* int8 [F, d] */
  void *fc1_s;   /* float [F] */
} h3_block_weights;

typedef struct h3_model h3_model;

/* Copies the dims and pointer tables (not the tensors, which stay caller-owned and must
 * outlive the model).  H3_EINVAL on NULL weights, H3_ESHAPE on unsupported dims (also when
 * the FFN weight [F, d] or the context [L_ctx, d], bf16, spans 4 GiB or more: the products
 * address each operand through 32-bit byte offsets). */
int32_t h3_model_create(const h3_dims *dims, const h3_global_weights *g,
                        const h3_block_weights *blocks, int32_t n_blocks, h3_model **out);
void h3_model_destroy(h3_model *m);

/* Token geometry of one latent.  paired = 0: the full grid, n = f_lat*grid_h*grid_w;
 * paired = 1: horizontally paired tokens, n = f_lat*grid_h*ceil(grid_w/2), RoPE w
 * coordinate = mean of the pair's columns (reading of P3 "aggressive levers"). */
typedef struct h3_geom {
  int32_t f_lat, grid_h, grid_w;
  float rope_spatial_scale;  /* from h3_token_grid: 1.0 or 0.5 */
  int32_t paired;
} h3_geom;

enum { H3_FC2_BF16 = 0, H3_FC2_INT8_ROW = 1, H3_FC2_INT8_GROUPED = 2 };

typedef struct h3_run_opts {
  int32_t fc2_mode;           /* H3_FC2_*: P2 §4 `--use-int8-row-fc2` (row), P3 "the int8 path" (grouped, 1024 channels per scale) */
  int32_t fused_gate_adaln;   /* 1: attention gate + MLP AdaLN in one kernel (P3 "DiT fusions"); 0: two kernels, bit-identical */
  int32_t fused_cross_block;  /* 1: MLP gate + next block's AdaLN in one kernel; 0: two kernels, bit-identical */
  int32_t qk_norm;            /* 1: per-head RMSNorm of Q and K before RoPE (P3 "the int8 path") */
  int32_t token_reduction;    /* 1: horizontal token pairing per h3_token_plan (forward only) */
  int32_t int8_linear;        /* 1: int8 QKV and FC1 products (P3 "the int8 path": quantised QKV
                               * projections and the int8 MLP, with the activation quantisation
                               * fused into the gated-AdaLN kernel).  The AdaLN rows n1, n2 are
                               * rounded to bf16 and quantised with one scale per token row
                               * (absmax / 127, the rule of h3_quant_rows); the weights need the
                               * copies of h3_quantize_linear_weights. */
  int32_t fused_qk_rope;      /* 1: the Q/K RMSNorm + RoPE run inside the QKV product's epilogue
                               * (P3 "the int8 path", fused epilogues; bf16 and int8 QKV) where
                               * its tiling allows (h3_qkv_gemm); 0: separate kernel, as the
                               * pages' `--use-slower-unfused-qkv-rope`.  Bit-identical. */
  int32_t store_branches;     /* 1: the attention and MLP branch outputs y and m are written to
                               * the workspace (h3_workspace_layout) also where the gate kernel
                               * sums the products' split-K partials itself; 0: there they are
                               * not written (nothing downstream reads them).  Results are
                               * identical either way. */
  int32_t fused_head_adaln;   /* Where the final AdaLN is not already computed by the last block's
                               * MLP gate (after a bypass restore before the head, or for a cached
                               * core): 1: it runs inside the velocity head's product, applied to
                               * the residual rows as its tiles are staged (P3 "DiT fusions and
                               * memory": the final heads apply AdaLN while loading their
                               * projection tiles; h3_head_adaln_gemm), where the head's tiling
                               * allows it (latent_ch < 192); 0: the AdaLN kernel, then the head.
                               * Bit-identical.  The fused form is the slower of the two at these
                               * sizes (few tiles; measured), so callers leave it 0. */
} h3_run_opts;

/* Tokens of a geometry (validates it). */
int32_t h3_geom_tokens(const h3_geom *geom, int32_t *n_tokens);

/* Bytes of workspace h3_dit_block_fwd / h3_dit_forward / h3_modulation /
 * h3_prepare_context need for n_tokens full-resolution tokens and these options.  Token
 * counts whose FC2 input [n_tokens, F] (bf16) spans 4 GiB or more are refused (H3_ESHAPE),
 * here and by the block and forward calls. */
int32_t h3_workspace_size(const h3_model *m, int32_t n_tokens, const h3_run_opts *o,
                          size_t *bytes);

/* Offsets (bytes from the workspace base) of the block intermediates after
 * h3_dit_block_fwd, for inspection.  Each is [n_tokens, width] bf16 unless noted:
 * n1 [N,d], qkvq [N,4d] (q,k after RMSNorm+RoPE), attn [N,2d] (self | cross outputs),
 * y [N,d] (summed output projection), n2 [N,d], h [N,F] (GELU output), m [N,d] (FC2
 * output), hq int8 [N,F], hs float [N, F/1024 or 1].  With int8_linear, n1 and n2 hold the
 * row-quantised AdaLN outputs: int8 [N,d] followed by float [N].  y and m hold the branches
 * only with store_branches = 1, or where the product is not split (the unfused gate, widths
 * above 4096, the int8 FC2). */
typedef struct h3_ws_layout {
  size_t n1, qkvq, attn, y, n2, h, m, hq, hs, rope, total;
} h3_ws_layout;
int32_t h3_workspace_layout(const h3_model *m, int32_t n_tokens, const h3_run_opts *o,
                            h3_ws_layout *layout);

/* Cross-attention K and V of the text context for every block, computed once per run
 * (the context does not depend on the timestep).  ctx (device, bf16 [ctx_len, d]);
 * ctx_kv (device, bf16 [n_blocks, 2, ctx_len, d]): K then V per block. */
int32_t h3_prepare_context(const h3_model *m, const void *ctx, void *ctx_kv, void *stream);

/* Per-output-channel int8 copy of every block's FC2 weight (P3 "the int8 path": per-output
 * channel weight scales): s = absmax_row / 127, q = clamp(rint(w / s), -127, 127), float32
 * division, ties to even, s = 0 -> q = 0.  Writes blocks[b].fc2_q / fc2_s (must be set). */
int32_t h3_quantize_fc2_weights(const h3_model *m, void *stream);

/* Same rule for the QKV(+cross Q) and FC1 weights of every block: writes
 * blocks[b].qkvq_q / qkvq_s ([4d, d] int8, [4d] float) and fc1_q / fc1_s ([F, d], [F]) (all
 * must be set); needed by h3_run_opts.int8_linear. */
int32_t h3_quantize_linear_weights(const h3_model *m, void *stream);

/* AdaLN parameters of every block for one timestep sigma (reading of P3 "DiT fusions").
 * mod (device, float [n_blocks, 6, d]) rows sh1 sc1 g1 sh2 sc2 g2; mod_final (device,
 * float [2, d]) rows shift, scale.  ws: at least h3_workspace_size bytes. */
int32_t h3_modulation(const h3_model *m, float sigma, float *mod, float *mod_final, void *ws,
                      size_t ws_bytes, void *stream);

/* h3_modulation without a workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, hosts that forbid allocation): the modulation MLP's
 * intermediates (256 + 8 d_model floats) live in a static device buffer of 264 KiB inside the
 * library, one per GPU, held until the process ends; nothing is allocated.  Same kernels and
 * results as h3_modulation (bit for bit).  d_model <= 8192 (H3_ESHAPE above that).  Every
 * intermediate is written before it is read, so the buffer needs no clearing; calls that
 * overlap on one GPU (several streams or host threads at once) race on the buffer and must be
 * serialised by the caller.  mod, mod_final as in h3_modulation. */
int32_t h3_modulation_noalloc(const h3_model *m, float sigma, float *mod, float *mod_final,
                              void *stream);

/* One DiT block on the residual stream (P3 "DiT fusions and memory"):
 *   n1 = AdaLN(x; sh1, sc1) (or the caller's n1_in);  [q|k|v|qc] = n1 W_qkvq^T + b;
 *   q,k <- RoPE(RMSNorm(q)), RoPE(RMSNorm(k));  O = softmax(q k^T / sqrt(D)) v per head;
 *   Oc = softmax(qc Kc^T / sqrt(D)) Vc with the context K/V;  y = [O|Oc] W_out^T + b_o + b_oc;
 *   x <- x + g1 y;  n2 = AdaLN(x; sh2, sc2);  h = GELU(n2 W1^T + b1);  m = FC2(h);
 *   x <- x + g2 m;  if n1_next != NULL: n1_next = AdaLN(x; mod_next sh1, sc1).
 * x (device, bf16 [N, d], in/out) with N = h3_geom_tokens(geom); n1_in (device, bf16 [N,d]
 * or NULL); n1_next (device, bf16 [N,d] or NULL, then mod_next != NULL: float [6,d] or
 * [2,d] rows shift, scale -- the next AdaLN's parameters); mod (device, float [6, d]);
 * ctx_kv (device, bf16 [2, ctx_len, d]: this block's K then V).  block in [0, n_blocks).
 * With o->int8_linear, n1_in and n1_next hold the quantised AdaLN row instead: int8 [N, d]
 * followed (at byte N*d) by the float32 row scales [N] -- N*d + 4N bytes; QKV and FC1 run as
 * int8 products with the block's qkvq_q / fc1_q copies. */
int32_t h3_dit_block_fwd(const h3_model *m, int32_t block, const h3_geom *geom,
                         const h3_run_opts *o, void *x, const void *n1_in, void *n1_next,
                         const float *mod, const float *mod_next, const void *ctx_kv,
                         void *ws, size_t ws_bytes, void *stream);

/* One fresh denoiser evaluation (P2 §2: `--steps N` runs N complete passes of the denoiser,
 * one per fresh step; P3 "DiT fusions and memory": modulation, patch, the active blocks with
 * the gate + AdaLN fusions, final AdaLN and the velocity head; P3 "aggressive levers": the
 * token pairing after the third active block and the bypass restore): timestep modulation,
 * patch embedding, the active blocks (h3_dit_block_fwd, with each MLP gate fused with the
 * next block's AdaLN), the token-pairing merge / restore when o->token_reduction is set, the
 * final AdaLN and the head.  latent (device, float [N, C]) at sigma -> velocity
 * (device, float [N, C]).  geom: the full grid (paired = 0).  active (host, int32
 * [n_active]): ascending block indices (h3_select_layers).  eval_index: 0-based count of
 * fresh evaluations before this one (selects the token-pairing restore point).
 * ctx_kv (device, bf16 [n_blocks, 2, ctx_len, d]) from h3_prepare_context. */
int32_t h3_dit_forward(const h3_model *m, const h3_geom *geom, const h3_run_opts *o,
                       const float *latent, float sigma, const int32_t *active,
                       int32_t n_active, int32_t eval_index, const void *ctx_kv,
                       float *velocity, void *ws, size_t ws_bytes, void *stream);

/* One evaluation under core-residual reuse (P2 §4, P3 "aggressive levers": --core-reuse k
 * runs the expensive core less often while the patch and the timestep-dependent head stay
 * fresh on every step; h3_schedule(.., core_reuse = k, ..) marks the core steps).
 *   refresh_core = 1: exactly h3_dit_forward, and core_delta (device, float [N, d]) receives
 *     x_L - x_0: the bf16 stream after the last active block (full resolution, after any
 *     bypass restore) minus the bf16 patch embedding, subtracted in float32.
 *   refresh_core = 0: the blocks are skipped: x = bf16(patch(latent) + core_delta) goes through
 *     the final AdaLN of sigma and the head (active, eval_index and the token reduction
 *     option are then unused).
 * Other arguments as h3_dit_forward. */
int32_t h3_dit_forward_cached(const h3_model *m, const h3_geom *geom, const h3_run_opts *o,
                              const float *latent, float sigma, const int32_t *active,
                              int32_t n_active, int32_t eval_index, const void *ctx_kv,
                              int32_t refresh_core, float *core_delta, float *velocity, void *ws,
                              size_t ws_bytes, void *stream);

/* Euler transition (P4 §2): latent[i] += (sigma_next - sigma_cur) * velocity[i], float32,
 * the step computed on the host in float32.  latent, velocity: device float [n_elems]. */
int32_t h3_euler_step(float *latent, const float *velocity, float sigma_cur,
                      float sigma_next, int64_t n_elems, void *stream);

/* Horizontal token pairing (P3 "aggressive levers").  geom: the full grid (paired = 0).
 * direction 0 (merge): dst[j] = (src[p0] + src[p1]) / 2, src bf16 [N, d] -> dst bf16
 * [N_r, d]; bypass unused.
 * direction 1 (restore): src = reduced stream bf16 [N_r, d], bypass = the full stream S
 * saved at the merge (bf16 [N, d]); dst[p] = S[p] + (src[j] - merge(S)[j]) for both members
 * p of pair j (bf16 [N, d]); merge(S) is recomputed exactly as direction 0 stores it, so a
 * merge followed by a restore with nothing between returns S bit for bit.  dst must not
 * alias src; for a restore dst may equal bypass (in-place restore of the saved stream). */
int32_t h3_token_reduce(int32_t direction, const h3_geom *geom, int32_t d_model,
                        const void *src, const void *bypass, void *dst, void *stream);

/* ------------------------------------------------------------------------------------
 * Single operations of the path (the same kernels the block uses), for callers that
 * compose their own block and for per-operation testing.  A row, token, head or column
 * count of zero is an error (H3_ESHAPE, nothing launched), not an empty no-op; only
 * h3_euler_step takes n_elems = 0 (returns H3_OK without a launch).
 * ---------------------------------------------------------------------------------- */

enum { H3_EPI_NONE = 0, H3_EPI_GELU = 1 };

/* C = A B^T + bias (+ bias2), bf16 MFMA with float32 accumulation.  A (device, bf16
 * [M, K], row stride lda elements), B (device, bf16 [N, K], row stride ldb), bias / bias2
 * (device, bf16 [N] or NULL).  out_f32 = 0: C bf16 [M, N] (stride ldc), epilogue
 * H3_EPI_GELU applies GELU after the bias; out_f32 = 1: C float [M, N].  GELU is the erf
 * form x * Phi(x), with erfc evaluated by Abramowitz & Stegun formula 7.1.26 (absolute error
 * of x * Phi(x) at most 3.7e-7 over [-12, 12], far below the bf16 rounding of the output).
 * K % 64 == 0, M, N >= 1, strides >= row widths and multiples of 8, and each operand
 * ((rows - 1) * ld + K elements) under 4 GiB (H3_ESHAPE otherwise). */
int32_t h3_gemm_bf16(const void *A, int64_t lda, const void *B, int64_t ldb, void *C,
                     int64_t ldc, int32_t M, int32_t N, int32_t K, const void *bias,
                     const void *bias2, int32_t epilogue, int32_t out_f32, void *stream);

/* Multi-head attention O = softmax(Q K^T / sqrt(D)) V, unmasked, float32 softmax, bf16
 * MFMA.  Q (device, bf16 [Nq, H*D] at row stride ldq), K/V ([Nk, H*D] at ldk/ldv), O
 * ([Nq, H*D] at ldo).  head_dim 64 or 128; Nq, Nk >= 1; strides multiples of 8, ldk and
 * ldv at most 2^24 elements (H3_ESHAPE otherwise). */
int32_t h3_attention(const void *Q, int64_t ldq, const void *K, int64_t ldk, const void *V,
                     int64_t ldv, void *O, int64_t ldo, int32_t n_q, int32_t n_k,
                     int32_t n_heads, int32_t head_dim, void *stream);

/* Dynamic int8 quantisation of rows (P2 §4 per-row scale; P3 "the int8 path" one scale per
 * 1024 channels): X (device, bf16 [rows, K]) -> Q (device, int8 [rows, K]) and S (device,
 * float [rows, K / group]); s = absmax / 127 in float32, q = clamp(rint(x / s), +-127),
 * ties to even, s = 0 -> q = 0.  group = K (per row; K % 512 == 0) or 1024 (K % 1024 == 0). */
int32_t h3_quant_rows(const void *X, void *Q, float *S, int32_t rows, int32_t K,
                      int32_t group, void *stream);

/* int8 product with float32 dequantisation: for each output (r, n),
 * acc_g = sum_{k in group g} QA[r,k] QW[n,k] (exact int32), out = bf16(((sum_g
 * float(acc_g) * SA[r,g]) * SW[n]) + bias[n]), groups ascending, each float operation
 * rounded (no fused multiply-add).  QA int8 [M, K], QW int8 [N, K], SA float [M, K/group],
 * SW float [N], bias bf16 [N], C bf16 [M, ldc].  group = K (K % 128 == 0) or 1024
 * (K % 1024 == 0); QA and QW each under 4 GiB.  epilogue: H3_EPI_NONE, or H3_EPI_GELU
 * (the GELU of h3_gemm_bf16 -- erf form, A&S 7.1.26, absolute error <= 3.7e-7 -- applied to
 * the dequantised value before the bf16 rounding: the int8 FC1 of P3 "the int8 path"). */
int32_t h3_gemm_i8(const void *QA, const float *SA, const void *QW, const float *SW,
                   const void *bias, void *C, int64_t ldc, int32_t M, int32_t N, int32_t K,
                   int32_t group, int32_t epilogue, void *stream);

/* Gated residual and/or AdaLN on rows of width d_model (P3 "DiT fusions and memory"):
 *   if y != NULL:     x_out = bf16(x + gate * y)                      (gate: device float [d])
 *   if n_out != NULL: n_out = bf16(LN(v) * (1 + scale) + shift), v = x_out if y != NULL else x,
 *                     LN without affine, biased variance, eps 1e-6   (shift, scale: float [d])
 * With both, the rounded x_out row is normalised from registers (one kernel); the two-call
 * sequence (gate, then AdaLN of x_out) gives bit-identical results.  x, y, x_out, n_out:
 * device bf16 [rows, d_model]; x_out may equal x.  d_model as in h3_dims. */
int32_t h3_gate_adaln(const void *x, const void *y, const float *gate, void *x_out,
                      const float *shift, const float *scale, void *n_out, int32_t rows,
                      int32_t d_model, void *stream);

/* The same with the AdaLN output quantised instead of stored (P3 "the int8 path": the
 * activation quantisation fused into the gated-AdaLN kernel): the bf16-rounded AdaLN row is
 * written as q_out (device int8 [rows, d_model]) and s_out (device float [rows]) by the rule
 * of h3_quant_rows with group = d_model -- bit-identical to h3_gate_adaln into n_out followed
 * by h3_quant_rows(n_out).  shift, scale, q_out, s_out must be set; y / gate / x_out as in
 * h3_gate_adaln. */
int32_t h3_gate_adaln_quant(const void *x, const void *y, const float *gate, void *x_out,
                            const float *shift, const float *scale, void *q_out, float *s_out,
                            int32_t rows, int32_t d_model, void *stream);

/* The velocity head with the final AdaLN applied while its tiles are staged (P3 "DiT fusions and
 * memory": the final BF16 heads apply AdaLN while loading their projection tiles):
 *   out = AdaLN(x; shift, scale) W^T + bias, float32,
 * with AdaLN as h3_gate_adaln computes it (n = bf16(LN(x) (1 + scale) + shift)).  The staged
 * tile holds exactly the bf16 values h3_gate_adaln would store, and the product runs as
 * h3_gemm_bf16 runs it, so the result equals h3_gate_adaln (into a bf16 buffer) followed by
 * h3_gemm_bf16 (out_f32 = 1) bit for bit.  x (device, bf16 [rows, d_model], 16-byte aligned);
 * shift, scale (device, float [d_model], 16-byte aligned); W (device, bf16 [n_out, d_model]);
 * bias (device, bf16 [n_out] or NULL); out (device, float [rows, n_out]).  d_model as in
 * h3_dims; n_out a positive multiple of 8 (H3_ESHAPE) and below 192, the widths at which the
 * plain product takes the 128x128 tiles reproduced here (H3_EUNSUPPORTED above); x and W under
 * 4 GiB (H3_ESHAPE). */
int32_t h3_head_adaln_gemm(const void *x, const float *shift, const float *scale, const void *W,
                           const void *bias, float *out, int32_t rows, int32_t d_model,
                           int32_t n_out, void *stream);

/* RoPE table of a geometry: table (device, float2 [n_tokens, head_dim/2]) = (cos, sin) of
 * coord * 10000^(-2j/D_axis) for the [t | h | w] channel slices of D - 4 floor(D/6),
 * 2 floor(D/6), 2 floor(D/6) channels (interleaved pairs j), coordinates (f, h*s, w*s) with s
 * = rope_spatial_scale; paired tokens use the mean of their two columns.  head_dim 64/128. */
int32_t h3_rope_table(const h3_geom *geom, int32_t head_dim, void *table, void *stream);

/* In place on the first 2 d_model channels of each row of qkvq (device bf16 [n_tokens, ld]):
 * per head of head_dim channels, q <- q / sqrt(mean(q^2) + 1e-6) * q_gamma (k likewise with
 * k_gamma; skipped when qk_norm == 0), then the RoPE rotation (a, b) -> (a cos - b sin,
 * a sin + b cos) of every interleaved pair with table from h3_rope_table. */
int32_t h3_qk_norm_rope(void *qkvq, int64_t ld, int32_t n_tokens, int32_t d_model,
                        int32_t head_dim, const void *q_gamma, const void *k_gamma,
                        int32_t qk_norm, const void *table, void *stream);

/* The block's QKV product C = [q | k | v | qc] = A W^T + bias (N = 4 d_model columns, device
 * bf16 [M, ldc]) followed by the Q/K RMSNorm + RoPE of h3_qk_norm_rope on the q and k heads
 * (P3 "the int8 path": the fused epilogues apply the RMS norm and RoPE of Q/K inside the QKV
 * projection tile).  a_q8 = 0: A bf16 [M, K] (row stride lda), W bf16 [4 d_model, K] (ldw),
 * SA and SW unused; K % 64 == 0, lda, ldw >= K and multiples of 8.  a_q8 = 1: the int8 QKV of
 * h3_run_opts.int8_linear: A int8 [M, K] with row scales SA float [M], W int8 [4 d_model, K]
 * with SW float [4 d_model] (h3_quantize_linear_weights), lda = ldw = K, K % 128 == 0.
 * bias bf16 [4 d_model]; table float2 [M, head_dim / 2] from h3_rope_table for the M tokens;
 * q_gamma, k_gamma bf16 [head_dim] (unused when qk_norm == 0); d_model % 512 == 0;
 * ldc >= 4 d_model, ldc % 8 == 0.  fused = 1: the norm and rotation run in the product's
 * epilogue when its tiling allows it (not for tiles that split K, nor for a C or table that is
 * not 16-byte aligned; *fused_used, if not NULL, says which ran); fused = 0, or no fused form: the product, then h3_qk_norm_rope.  The two are
 * bit-identical.  Errors: H3_EINVAL (NULL pointers, flags), H3_EUNSUPPORTED (head_dim not 64
 * or 128), H3_ESHAPE (sizes, strides, an A or W operand of 4 GiB or more). */
int32_t h3_qkv_gemm(const void *A, int64_t lda, const float *SA, const void *W, int64_t ldw,
                    const float *SW, const void *bias, void *C, int64_t ldc, int32_t M,
                    int32_t d_model, int32_t K, int32_t head_dim, const void *q_gamma,
                    const void *k_gamma, int32_t qk_norm, const void *table, int32_t a_q8,
                    int32_t fused, int32_t *fused_used, void *stream);

/* Matrix-core throughput probe (measurement only, not part of the path): `workgroups`
 * workgroups of four waves, each wave issuing `iters` rounds of eight independent 32x32 MFMAs
 * on register operands -- bf16 (v_mfma_f32_32x32x16_bf16, 32768 FLOP each) or, with int8 = 1,
 * int8 (v_mfma_i32_32x32x32_i8, 65536 OP each) -- with no memory traffic in the loop.  Timing
 * it gives the dense matrix-core rate the GPU sustains at its running clock.  out (device,
 * float [workgroups * 256]) receives per-thread sums.  iters >= 1, 1 <= workgroups <= 2^20. */
int32_t h3_mfma_probe(int32_t int8, int32_t iters, int32_t workgroups, float *out, void *stream);

/* ------------------------------------------------------------------------------------
 * Per-stage timing (HIP events recorded on the launch stream around every launch of the
 * selected stages).  One session per process; not thread-safe.  Inside a block the self- and
 * cross-attention run as one launch, timed under H3_ST_SELF_ATTN (H3_ST_CROSS_ATTN then
 * counts no launch).
 * ---------------------------------------------------------------------------------- */
enum {
  H3_ST_MODULATION = 0, H3_ST_PATCH, H3_ST_ADALN, H3_ST_QKV_GEMM, H3_ST_QK_NORM_ROPE,
  H3_ST_SELF_ATTN, H3_ST_CROSS_ATTN, H3_ST_OUT_GEMM, H3_ST_GATE_ADALN, H3_ST_FC1_GEMM,
  H3_ST_FC2_GEMM, H3_ST_FC2_QUANT, H3_ST_FC2_I8_GEMM, H3_ST_TOKEN_REDUCE, H3_ST_HEAD,
  H3_ST_EULER, H3_ST_COUNT
};
/* Opens a session: stage_mask bit i selects stage i; at most max_launches launches are
 * timed (host-side event pool).  H3_EINVAL if a session is open or max_launches is out of
 * [1, 2^20]. */
int32_t h3_profile_begin(uint32_t stage_mask, int32_t max_launches);
/* Closes the session: waits for the recorded events and writes, per stage, the summed
 * milliseconds (ms_per_stage, host double[H3_ST_COUNT]) and the launch count
 * (launches_per_stage, host int32[H3_ST_COUNT]).  Both NULL: closes without reading.
 * H3_EINVAL if more launches than max_launches were selected (the excess were not timed). */
int32_t h3_profile_end(double *ms_per_stage, int32_t *launches_per_stage);

#ifdef __cplusplus
}
#endif
#endif /* H3DIT_H */
