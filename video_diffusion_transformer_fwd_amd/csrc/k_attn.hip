// Flash-style multi-head attention on the gfx950 matrix cores (self-attention over the video
// tokens and cross-attention to the text context use the same kernel).
//
// A workgroup holds WAVES wave64s and 32 WAVES query rows of one head; every wave owns 32
// queries.  Keys and values stream through LDS in tiles of 64 rows, loaded straight from
// global memory into LDS (global_load_lds_dwordx4) one tile ahead of the one in use, in two
// stages; the tile loop is unrolled over the two stages, so every LDS read address is a
// loop-invariant per-lane base plus an immediate offset.
//
// Per tile a wave computes the transposed scores S^T = K Q^T (32 keys x 32 queries per
// v_mfma_f32_32x32x16_bf16 block), so every lane holds scores of a single query (lane % 32)
// and the row max / row sum need only the partner lane (lane ^ 32): one cross-lane swap
// instead of a 32-lane reduction.  The exponentiated scores stay in registers and are fed
// straight back as the B operand of O^T += V^T P^T: the 16 keys of each PV step are taken in
// the order the score accumulator already holds them.  The matching A operand (one channel,
// 4 + 4 keys per lane) comes from row-major V through two transposing LDS reads
// (ds_read_b64_tr_b16): within each 16-lane group, output lane j receives element j % 4 of the
// 8-byte pieces that lanes j / 4 + {0, 4, 8, 12} point at, so pointing lane i at key
// 4 (i / 4) + ... and channels 4 (i % 4) + ... hands every lane its channel across 4 keys.
// Softmax is online (running max m, running sum l, float32, base-2 exponentials).
// Keys beyond n_k are masked to -inf; query rows beyond n_q are computed and not stored.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "h3_internal.h"

namespace h3 {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
// LDS pointers in the LDS address space: 32-bit arithmetic whose constant parts fold into the
// offset fields of the DS instructions
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) const bf16x8_t lds_bf16x8;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

constexpr int kBlockN = 64;   // keys per tile
constexpr float kLazy = 8.0f; // log2 headroom of the lazily moved softmax reference
constexpr float kLazyBound = 256.0f;  // 2^kLazy

// LDS layout of a staged K or V tile: 64 key rows of D bf16, unpadded (2D bytes a row, so one
// 256-byte bank line holds 256 / 2D rows).  The 16-byte unit u of bank line `line` sits in
// slot u ^ lds_key(line): the sixteen rows one K-fragment read touches at one unit land on
// sixteen distinct slots, and the four rows x four units of a transposing V read on sixteen,
// so neither read has bank conflicts.  The layout satisfies (x < 16, c' < 4)
//   lds_off(r, 2k + g)  = lds_off(r, g) ^ 32k       lds_off(r + 32, c)  = lds_off(r, c) + 64 D
//   lds_off(r, 4b + c') = lds_off(r, c') ^ 64b      lds_off(16s + x, c) = lds_off(x, c) + 32 s D
// so every read address is a per-lane base combined with a compile-time constant.
template <int D>
__device__ __forceinline__ int lds_key(int line) {
  if constexpr (D == 128)
    return ((line & 3) << 2) | ((line >> 2) & 3);
  else
    return ((line & 1) << 2) | ((line >> 1) & 3);
}
// byte offset of 16-byte unit c (channels 8c .. 8c+7) of key row r within a tile
template <int D>
__device__ __forceinline__ int lds_off(int r, int c) {
  constexpr int RPL = 256 / (2 * D), UPR = D / 8;
  const int line = r / RPL, u = (r % RPL) * UPR + c;
  return line * 256 + ((u ^ lds_key<D>(line)) << 4);
}

// KG key groups: with KG = 2 the waves form WAVES / 2 query groups twice over, each stage holds
// two 64-key tiles, and the second group of waves takes the second tile of every stage; the
// groups' partial softmax sums are merged through LDS at the end.
template <int D, int WAVES, int KG>
struct AttnCfg {
  static constexpr int NT = 64 * WAVES;
  static constexpr int QG = WAVES / KG;                // query groups (32 queries each)
  static constexpr int BM = 32 * QG;                   // queries per workgroup
  static constexpr int KT = kBlockN * KG;              // keys per stage
  static constexpr int ROW = 2 * D;                    // bytes per staged key row
  static constexpr int TILE = KT * ROW;                // bytes per K (or V) stage
  static constexpr int STAGE = 2 * TILE;               // K rows, then V rows
  static constexpr int LDS = 2 * STAGE;                // two stages (64 KiB at D = 128, KG = 1)
  static constexpr int LOADS = TILE / (1024 * WAVES);  // DMA instructions per wave per K or V stage
  static constexpr int OW = D / 2 + 2;                 // floats per lane handed over by the merge
  static_assert(KG == 1 || KG == 2, "one or two key groups");
  static_assert(LOADS >= 1 && TILE % (1024 * WAVES) == 0, "a stage must split over the waves");
  static_assert(KG == 1 || QG * 64 * OW * 4 <= LDS, "the merge buffer must fit the stages");
};

// One attention problem; a launch may carry two (blockIdx.z selects), e.g. the self- and the
// cross-attention of a block, so the short one fills the CUs the other leaves idle.
struct AttnProblem {
  const bf16_t *Q;
  int64_t ldq;
  const bf16_t *K;
  int64_t ldk;
  const bf16_t *V;
  int64_t ldv;
  bf16_t *O;
  int64_t ldo;
  int nq, nk;
};
struct AttnProblems {
  AttnProblem p[2];
};

template <int D, int WAVES, int KG>
__global__ __launch_bounds__(64 * WAVES, WAVES == 4 ? 2 : 1) void attention_kernel(
    AttnProblems probs, float scale_log2) {
  using Cfg = AttnCfg<D, WAVES, KG>;
  // static (its address known when the kernel is compiled, so constant parts of LDS addresses
  // fold into the instructions' offsets; a dynamic array's base is a link-time symbol)
  __shared__ __align__(16) unsigned char smem[Cfg::LDS];
  lds_u8 *const lds = (lds_u8 *)smem;
  // select the problem with scalar conditionals (indexing the argument array by blockIdx.z
  // would copy it to private memory)
  const bool second = blockIdx.z != 0;
  const AttnProblem &p0 = probs.p[0], &p1 = probs.p[1];
  const bf16_t *__restrict__ Q = second ? p1.Q : p0.Q;
  const bf16_t *__restrict__ K = second ? p1.K : p0.K;
  const bf16_t *__restrict__ V = second ? p1.V : p0.V;
  bf16_t *__restrict__ O = second ? p1.O : p0.O;
  const int64_t ldq = second ? p1.ldq : p0.ldq, ldk = second ? p1.ldk : p0.ldk;
  const int64_t ldv = second ? p1.ldv : p0.ldv, ldo = second ? p1.ldo : p0.ldo;
  const int nq = second ? p1.nq : p0.nq, nk = second ? p1.nk : p0.nk;
  // (query tile, head) of this workgroup.  Hardware ids go round-robin over the 8 XCDs; each XCD
  // takes a contiguous run of (tile, head) pairs instead, so the query tiles of one head share
  // its keys and values in that XCD's L2 (1536 tokens, 24 heads: three heads' K / V, 2.4 MB, per
  // XCD instead of pieces of eighteen: -0.1% to -1.1% per 512x512x22f step on two machines with
  // 8-wave workgroups, bit-identical output; no change at 61,488 tokens)
  int tile = blockIdx.x, head = blockIdx.y;
  {
    const int per_plane = gridDim.x * gridDim.y;
    if (per_plane % 8 == 0) {
      int pid = blockIdx.x + gridDim.x * blockIdx.y;
      pid = (pid % 8) * (per_plane / 8) + pid / 8;
      tile = pid % gridDim.x;
      head = pid / gridDim.x;
    }
  }
  if (tile * Cfg::BM >= nq) return;  // this problem has fewer query tiles

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // query group, key group (compile-time 0 with one key group)
  const int qg = KG == 1 ? wave : wave % Cfg::QG, kh = KG == 1 ? 0 : wave / Cfg::QG;
  const int q_base = tile * Cfg::BM + qg * 32;
  const int hoff = head * D;
  const int l32 = lane & 31, g = lane >> 5;

  // Q fragments: B operand of S^T = K Q^T; lane holds Q[q_base + l32][ks*16 + 8g .. +7]
  bf16x8_t qf[D / 16];
  {
    const int q = q_base + l32;
    if (q < nq) {
      const bf16_t *qp = Q + static_cast<int64_t>(q) * ldq + hoff + 8 * g;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t *>(qp + ks * 16);
    } else {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) qf[ks] = bf16x8_t{};
    }
  }

  f32x16_t o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16_t{};
  // m_ref: running reference maximum (raw score units) of this lane's query; -inf until the
  // first tile, whose maximum always raises it (alpha = 2^-inf = 0 clears nothing yet stored)
  float m_ref = -INFINITY, l_run = 0.f;

  // Staging: DMA instruction j of this wave fills tile bytes 1024 (j WAVES + wave) + 16 lane,
  // i.e. bank line 4 (j WAVES + wave) + lane / 16, slot lane % 16, which holds unit
  // (lane % 16) ^ lds_key(line) of the line; src_row_unit names that key row and unit
  auto src_row_unit = [&](int j, int &r, int &c) {
    constexpr int RPL = 256 / Cfg::ROW, UPR = D / 8;
    const int line = 4 * (j * WAVES + wave) + (lane >> 4);
    const int u = (lane & 15) ^ lds_key<D>(line);
    r = line * RPL + u / UPR;
    c = u % UPR;
  };
  // byte offsets of this lane's sources relative to the tile's first key row (strides are
  // at most 2^24 elements, so they fit 32 bits)
  uint32_t koff[Cfg::LOADS], voff[Cfg::LOADS];
#pragma unroll
  for (int j = 0; j < Cfg::LOADS; ++j) {
    int r, c;
    src_row_unit(j, r, c);
    koff[j] = static_cast<uint32_t>((r * ldk + hoff + 8 * c) * 2);
    voff[j] = static_cast<uint32_t>((r * ldv + hoff + 8 * c) * 2);
  }
  const int n_tiles = (nk + Cfg::KT - 1) / Cfg::KT;  // stages
  // loads tile t into stage S (S a compile-time constant: the LDS destinations are immediates)
  auto issue = [&](int t, auto stage) {
    constexpr int S = decltype(stage)::value;
    const int kv0 = t * Cfg::KT;
    const unsigned char *kb = reinterpret_cast<const unsigned char *>(K + static_cast<int64_t>(kv0) * ldk);
    const unsigned char *vb = reinterpret_cast<const unsigned char *>(V + static_cast<int64_t>(kv0) * ldv);
    uint32_t ko[Cfg::LOADS], vo[Cfg::LOADS];
    if (kv0 + Cfg::KT <= nk) {  // workgroup-uniform
#pragma unroll
      for (int j = 0; j < Cfg::LOADS; ++j) ko[j] = koff[j], vo[j] = voff[j];
    } else {
      // last tile: rows past n_k repeat row n_k - 1 (their scores are masked, so P is 0)
#pragma unroll
      for (int j = 0; j < Cfg::LOADS; ++j) {
        int r, c;
        src_row_unit(j, r, c);
        r = r < nk - 1 - kv0 ? r : nk - 1 - kv0;
        ko[j] = static_cast<uint32_t>((r * ldk + hoff + 8 * c) * 2);
        vo[j] = static_cast<uint32_t>((r * ldv + hoff + 8 * c) * 2);
      }
    }
    // (source and destination as named pointers: written inline into the builtin's arguments,
    // the host pass drops the kernel's launch stub)
#pragma unroll
    for (int j = 0; j < Cfg::LOADS; ++j) {
      const unsigned char *src = kb + ko[j];
      lds_u8 *dst = lds + S * Cfg::STAGE + (j * WAVES + wave) * 1024;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(dst), 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < Cfg::LOADS; ++j) {
      const unsigned char *src = vb + vo[j];
      lds_u8 *dst = lds + S * Cfg::STAGE + Cfg::TILE + (j * WAVES + wave) * 1024;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(dst), 16, 0, 0);
    }
  };

  // Loop-invariant read addresses (bytes from the stage start).  K fragment of step ks and
  // 32-key block kb: lds_off(32 kb + l32, 2 ks + g) = ka[ks] + 64 D kb.  V^T fragment of PV
  // step st, channel block db, first / second read: va[h][db] + 32 D st, where lane
  // l = 16 q + i points at key 4 (q / 2) + i / 4 (+ 8) of the step and channels
  // db*32 + 16 (q % 2) + 4 (i % 4) .. +3; it receives channel db*32 + l % 32 at keys
  // 4 (l / 32) + 0..3 (and + 8..11) of the step
  int ka[D / 16], va[2][D / 32];
  {
    const int k_base = lds_off<D>(l32, g);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) ka[ks] = k_base ^ (32 * ks);
    const int vq = lane >> 4, vi = lane & 15;
    const int x = 4 * (vq >> 1) + (vi >> 2);
    const int cp = 2 * (vq & 1) + ((vi & 3) >> 1);
    const int vb0 = Cfg::TILE + lds_off<D>(x, cp) + 8 * (vi & 1);
    const int vb1 = Cfg::TILE + lds_off<D>(x + 8, cp) + 8 * (vi & 1);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      va[0][db] = vb0 ^ (64 * db);
      va[1][db] = vb1 ^ (64 * db);
    }
  }

  // one 64-key tile: keys kv0 .. kv0+63, K rows at st, V rows at st + TILE
  auto key_tile = [&](const lds_u8 *st, int kv0) __attribute__((always_inline)) {

    // S^T = K Q^T for keys kv0 .. kv0+63 (two 32-key blocks).  The K fragments of step
    // ks + 2 are read while step ks's two MFMAs run (a ring of three), so the LDS latency is
    // covered instead of waited out before every MFMA.
    f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
    {
      constexpr int KSTEPS = D / 16;
      auto kfrag = [&](int ks, int kb) {
        return *reinterpret_cast<lds_bf16x8 *>(st + ka[ks] + kb * 64 * D);
      };
      bf16x8_t kf[3][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        kf[ks][0] = kfrag(ks, 0);
        kf[ks][1] = kfrag(ks, 1);
      }
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        if (ks + 2 < KSTEPS) {
          kf[(ks + 2) % 3][0] = kfrag(ks + 2, 0);
          kf[(ks + 2) % 3][1] = kfrag(ks + 2, 1);
        }
        // keep those reads here: the scheduler would otherwise sink them next to their use
        __builtin_amdgcn_sched_barrier(0);
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks % 3][0], qf[ks], s[0], 0, 0, 0);
        s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks % 3][1], qf[ks], s[1], 0, 0, 0);
      }
    }
    // Online softmax with the scale folded into the exponent: p = 2^(s c - m c) with the raw
    // score s, c = log2(e) / sqrt(D) and m a running reference maximum in raw units.  The
    // reference only moves up when some lane's tile maximum exceeds it by more than
    // kLazy / c (p stays <= 2^kLazy); O and l are rescaled then, which leaves O / l exact.
    // A tile is first exponentiated against the current reference: if every lane's sum of p
    // stays within 2^kLazy, no p exceeds it, so the reference would not move and the tile
    // needs no maximum.  Otherwise (the first tile of a wave, a score far above the
    // reference, or many near it) the maximum is taken and the reference moved as above, and
    // the exponentials are redone if it moved.
    if (kv0 + kBlockN > nk) {  // keys beyond n_k (last tile only)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kv0 + kb * 32 + 8 * (i / 4) + 4 * g + (i % 4);
          if (key >= nk) s[kb][i] = -INFINITY;
        }
    }
    f32x16_t p[2];
    float psum;
    auto exponentiate = [&](float mc) __attribute__((always_inline)) {
      psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          p[kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], scale_log2, -mc));
          psum += p[kb][i];
        }
    };
    // (m_ref = -inf makes every p +inf or NaN here, so a wave's first tile takes the slow path)
    exponentiate(m_ref * scale_log2);
    if (__builtin_amdgcn_ballot_w64(!(psum <= kLazyBound)) != 0) {  // wave-uniform, rare
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[kb][i]);
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const bool raise = mt * scale_log2 > m_ref * scale_log2 + kLazy;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float m_new = raise ? mt : m_ref;
        const float alpha = __builtin_amdgcn_exp2f((m_ref - m_new) * scale_log2);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        m_ref = m_new;
      }
      // (with two key groups a wave may have seen no key yet (n_k <= 64): then every score and
      // the reference are -inf, and P must come out 0 rather than 2^(-inf + inf))
      exponentiate(KG == 1 || m_ref != -INFINITY ? m_ref * scale_log2 : 0.f);
    }
    l_run += psum;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s[kb] = p[kb];

    // O^T += V^T P^T over 4 steps of 16 keys; the V^T fragments of step st + 1 are read while
    // step st's MFMAs run
    {
      auto vfrag = [&](int step, int db) {
        const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(st + va[0][db] + 32 * D * step));
        const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(st + va[1][db] + 32 * D * step));
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8_t vf[2][D / 32];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) vf[0][db] = vfrag(0, db);
#pragma unroll
      for (int step = 0; step < 4; ++step) {
        const int kb = step >> 1, half = step & 1, cur = step & 1;
        if (step + 1 < 4) {
#pragma unroll
          for (int db = 0; db < D / 32; ++db) vf[cur ^ 1][db] = vfrag(step + 1, db);
        }
        __builtin_amdgcn_sched_barrier(0);
        bf16x8_t pb;
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[j] = static_cast<__bf16>(s[kb][8 * half + j]);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[cur][db], pb, o[db], 0, 0, 0);
      }
    }
  };

  // one stage out of LDS stage S: this wave's key group takes its 64-key tile
  auto stage_step = [&](int t, auto stage) __attribute__((always_inline)) {
    constexpr int S = decltype(stage)::value;
    const int kv0 = t * Cfg::KT + kh * kBlockN;
    // stage t has landed (this thread's loads, then every thread's at the barrier), and every
    // wave is done with the other stage, which the next issue refills
    lds_dma_barrier<0>();
    if (t + 1 < n_tiles) issue(t + 1, std::integral_constant<int, S ^ 1>{});
    if (KG == 1 || kv0 < nk) key_tile(lds + S * Cfg::STAGE + kh * kBlockN * Cfg::ROW, kv0);
  };

  if (n_tiles > 0) issue(0, std::integral_constant<int, 0>{});
  for (int t = 0; t < n_tiles; t += 2) {
    stage_step(t, std::integral_constant<int, 0>{});
    if (t + 1 < n_tiles) stage_step(t + 1, std::integral_constant<int, 1>{});
  }

  if constexpr (KG == 2) {
    // merge the key groups: the second group's waves hand (m, l, O) over LDS to the first
    // group's wave of the same queries, which rescales both to the larger reference
    float *xch = reinterpret_cast<float *>(smem) + qg * 64 * Cfg::OW;
    __syncthreads();  // every wave is done with the staged tiles (no copy is in flight)
    if (kh == 1) {
      xch[lane] = m_ref;
      xch[64 + lane] = l_run;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) xch[(2 + db * 16 + i) * 64 + lane] = o[db][i];
    }
    __syncthreads();
    if (kh == 1) return;
    const float m1 = xch[lane], l1 = xch[64 + lane];
    const float m = fmaxf(m_ref, m1);  // finite: key 0 belongs to the first group
    const float a0 = __builtin_amdgcn_exp2f((m_ref - m) * scale_log2);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m1 - m) * scale_log2);
    l_run = l_run * a0 + l1 * a1;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[db][i] = o[db][i] * a0 + xch[(2 + db * 16 + i) * 64 + lane] * a1;
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  const int q = q_base + l32;
  if (q < nq) {
    bf16_t *op = O + static_cast<int64_t>(q) * ldo + hoff;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dch = db * 32 + 8 * r4 + 4 * g;
        uint2 w;
        w.x = pack_bf2(o[db][4 * r4 + 0] * inv, o[db][4 * r4 + 1] * inv);
        w.y = pack_bf2(o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv);
        *reinterpret_cast<uint2 *>(op + dch) = w;
      }
  }
}

template <int D, int WAVES, int KG>
void launch_cfg(const AttnProblems &pr, int n_problems, int heads, float scale_log2, hipStream_t s) {
  using Cfg = AttnCfg<D, WAVES, KG>;
  int tiles = 0;
  for (int i = 0; i < n_problems; ++i) tiles = std::max(tiles, (pr.p[i].nq + Cfg::BM - 1) / Cfg::BM);
  dim3 grid(tiles, heads, n_problems), block(Cfg::NT);
  attention_kernel<D, WAVES, KG><<<grid, block, 0, s>>>(pr, scale_log2);
}

// 8192+ queries: 8-wave workgroups of 256 queries.  Fewer: 128 queries per workgroup, with 8
// waves in two key groups when the (128-query tile, head) grid of the longest problem leaves
// CUs idle (at most 256 workgroups: two waves per SIMD on each occupied CU, every wave half the
// key tiles); otherwise 8-wave workgroups of 256 queries again when their grid takes at most
// three quarters of the CUs, leaving the rest to the short cross-attention of the same launch
// (1536 tokens, 24 heads: 144 workgroups; -0.8% per 512x512x22f step against the next form),
// else 4 waves (two workgroups per CU; 2430 tokens: 240 workgroups of 256 queries would take
// a second round with the cross-attention's, +0.6% per step).
void launch_problems(const AttnProblems &pr, int n_problems, int heads, int head_dim, hipStream_t s) {
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(head_dim));
  int nq = 0;
  for (int i = 0; i < n_problems; ++i) nq = std::max(nq, pr.p[i].nq);
  const bool sparse = static_cast<int64_t>((nq + 127) / 128) * heads <= 256;
  const bool wide8 = static_cast<int64_t>((nq + 255) / 256) * heads <= 192;
  if (head_dim == 128 && (nq >= 8192 || (!sparse && wide8)))
    launch_cfg<128, 8, 1>(pr, n_problems, heads, scale_log2, s);
  else if (head_dim == 128)
    sparse ? launch_cfg<128, 8, 2>(pr, n_problems, heads, scale_log2, s)
           : launch_cfg<128, 4, 1>(pr, n_problems, heads, scale_log2, s);
  else
    sparse ? launch_cfg<64, 8, 2>(pr, n_problems, heads, scale_log2, s)
           : launch_cfg<64, 4, 1>(pr, n_problems, heads, scale_log2, s);
}

}  // namespace

void launch_attention(const bf16_t *Q, int64_t ldq, const bf16_t *K, int64_t ldk,
                      const bf16_t *V, int64_t ldv, bf16_t *O, int64_t ldo, int nq, int nk,
                      int heads, int head_dim, hipStream_t s) {
  AttnProblems pr{};
  pr.p[0] = AttnProblem{Q, ldq, K, ldk, V, ldv, O, ldo, nq, nk};
  launch_problems(pr, 1, heads, head_dim, s);
}

void launch_attention_pair(const bf16_t *Q0, int64_t ldq0, const bf16_t *K0, int64_t ldk0,
                           const bf16_t *V0, int64_t ldv0, bf16_t *O0, int64_t ldo0, int nq0, int nk0,
                           const bf16_t *Q1, int64_t ldq1, const bf16_t *K1, int64_t ldk1,
                           const bf16_t *V1, int64_t ldv1, bf16_t *O1, int64_t ldo1, int nq1, int nk1,
                           int heads, int head_dim, hipStream_t s) {
  AttnProblems pr{};
  pr.p[0] = AttnProblem{Q0, ldq0, K0, ldk0, V0, ldv0, O0, ldo0, nq0, nk0};
  pr.p[1] = AttnProblem{Q1, ldq1, K1, ldk1, V1, ldv1, O1, ldo1, nq1, nk1};
  launch_problems(pr, 2, heads, head_dim, s);
}

}  // namespace h3
