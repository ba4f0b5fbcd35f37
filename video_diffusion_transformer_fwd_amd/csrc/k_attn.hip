// Flash-style multi-head attention on the gfx950 matrix cores (self-attention over the video
// tokens and cross-attention to the text context use the same kernel).
//
// Workgroup = 4 wave64s = 128 query rows of one head; each wave owns 32 queries.  Keys and
// values stream through LDS in tiles of 64.  Per tile a wave computes the transposed scores
// S^T = K Q^T (32 keys x 32 queries per v_mfma_f32_32x32x16_bf16 block), so every lane holds
// scores of a single query (lane % 32) and the row max / row sum need only the partner lane
// (lane ^ 32): one cross-lane swap instead of a 32-lane reduction.  The exponentiated scores
// stay in registers and are fed straight back as the B operand of O^T += V^T P^T: the 16 keys of
// each PV step are taken in the order the score accumulator already holds them.  V is staged
// row-major in LDS ([key][channel], 16-byte stores straight from the loaded rows) and the
// matching A operand (one channel, 4 + 4 keys per lane) comes from two transposing LDS reads
// (ds_read_b64_tr_b16): within each 16-lane group, output lane j receives element j % 4 of
// the 8-byte pieces that lanes j / 4 + {0, 4, 8, 12} point at, so pointing lane i at key
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
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int kBlockN = 64;   // keys per tile
constexpr float kLazy = 8.0f; // log2 headroom of the lazily moved softmax reference

// WAVES wave64s per workgroup, 32 queries each: 4 (two workgroups per CU) for short
// sequences, 8 (one per CU, still two waves per SIMD) for long ones, where the same K/V tile
// then serves twice the queries and each thread stages half of it.
template <int D, int WAVES>
struct AttnCfg {
  static constexpr int NT = 64 * WAVES;
  static constexpr int BM = 32 * WAVES;    // queries per workgroup
  static constexpr int KS = D + 8;         // K tile row stride (elements)
  static constexpr int VS = D + 16;        // V row stride (elements): rows 288 bytes apart, so the
                                           // four 32-byte row pieces of a transposing read use
                                           // distinct banks
  static constexpr int CH = D / 8;         // 16-byte chunks per row
  static constexpr int K_PASSES = kBlockN * CH / NT;
  static_assert(K_PASSES >= 1 && kBlockN * CH % NT == 0, "K / V tile must split over the threads");
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

template <int D, int WAVES>
__global__ __launch_bounds__(64 * WAVES, WAVES == 4 ? 2 : 1) void attention_kernel(
    AttnProblems probs, float scale_log2) {
  using Cfg = AttnCfg<D, WAVES>;
  constexpr int kBlockM = Cfg::BM;
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
  if (static_cast<int>(blockIdx.x) * kBlockM >= nq) return;  // this problem has fewer query tiles
  __shared__ __align__(16) bf16_t Ks[kBlockN * Cfg::KS];
  __shared__ __align__(16) bf16_t Vs[kBlockN * Cfg::VS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int head = blockIdx.y;
  const int q_base = blockIdx.x * kBlockM + wave * 32;
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

  // staging registers for the next K/V tile
  uint4 kreg[Cfg::K_PASSES];
  uint4 vreg[Cfg::K_PASSES];
  // K and V rows alike: thread t stages 16-byte chunk t % CH of row t / CH (+ NT/CH per pass)
  const int k_row = tid / Cfg::CH, k_chunk = tid % Cfg::CH;

  // with 8 waves (long sequences) interior tiles load unconditionally; otherwise, and for the
  // last (ragged) tile, keys beyond n_k are zero-filled (measured: the 4-wave shape is faster
  // with the single guarded form)
  auto load_tile = [&](int kv0) {
    if (WAVES >= 8 && kv0 + kBlockN <= nk) {  // wave-uniform
#pragma unroll
      for (int p = 0; p < Cfg::K_PASSES; ++p) {
        const int r = kv0 + k_row + p * (Cfg::NT / Cfg::CH);
        kreg[p] = *reinterpret_cast<const uint4 *>(K + static_cast<int64_t>(r) * ldk + hoff + k_chunk * 8);
      }
#pragma unroll
      for (int p = 0; p < Cfg::K_PASSES; ++p) {
        const int r = kv0 + k_row + p * (Cfg::NT / Cfg::CH);
        vreg[p] = *reinterpret_cast<const uint4 *>(V + static_cast<int64_t>(r) * ldv + hoff + k_chunk * 8);
      }
      return;
    }
#pragma unroll
    for (int p = 0; p < Cfg::K_PASSES; ++p) {
      const int r = kv0 + k_row + p * (Cfg::NT / Cfg::CH);
      kreg[p] = r < nk ? *reinterpret_cast<const uint4 *>(K + static_cast<int64_t>(r) * ldk + hoff + k_chunk * 8)
                       : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < Cfg::K_PASSES; ++p) {
      const int r = kv0 + k_row + p * (Cfg::NT / Cfg::CH);
      vreg[p] = r < nk ? *reinterpret_cast<const uint4 *>(V + static_cast<int64_t>(r) * ldv + hoff + k_chunk * 8)
                       : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int p = 0; p < Cfg::K_PASSES; ++p)
      *reinterpret_cast<uint4 *>(Ks + (k_row + p * (Cfg::NT / Cfg::CH)) * Cfg::KS + k_chunk * 8) = kreg[p];
#pragma unroll
    for (int p = 0; p < Cfg::K_PASSES; ++p)
      *reinterpret_cast<uint4 *>(Vs + (k_row + p * (Cfg::NT / Cfg::CH)) * Cfg::VS + k_chunk * 8) = vreg[p];
  };

  const int n_tiles = (nk + kBlockN - 1) / kBlockN;
  load_tile(0);
  for (int t = 0; t < n_tiles; ++t) {
    const int kv0 = t * kBlockN;
    __syncthreads();  // previous tile fully consumed
    store_tile();
    __syncthreads();
    if (t + 1 < n_tiles) load_tile(kv0 + kBlockN);

    // S^T = K Q^T for keys kv0 .. kv0+63 (two 32-key blocks).  The K fragments of step
    // ks + 2 are read while step ks's two MFMAs run (a ring of three), so the LDS latency is
    // covered instead of waited out before every MFMA.
    f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
    {
      constexpr int KSTEPS = D / 16;
      const bf16_t *kp0 = Ks + l32 * Cfg::KS + 8 * g;
      const bf16_t *kp1 = kp0 + 32 * Cfg::KS;
      bf16x8_t kf[3][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        kf[ks][0] = *reinterpret_cast<const bf16x8_t *>(kp0 + ks * 16);
        kf[ks][1] = *reinterpret_cast<const bf16x8_t *>(kp1 + ks * 16);
      }
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        if (ks + 2 < KSTEPS) {
          kf[(ks + 2) % 3][0] = *reinterpret_cast<const bf16x8_t *>(kp0 + (ks + 2) * 16);
          kf[(ks + 2) % 3][1] = *reinterpret_cast<const bf16x8_t *>(kp1 + (ks + 2) * 16);
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
    if (kv0 + kBlockN > nk) {  // keys beyond n_k (last tile only)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kv0 + kb * 32 + 8 * (i / 4) + 4 * g + (i % 4);
          if (key >= nk) s[kb][i] = -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[kb][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const bool raise = mt * scale_log2 > m_ref * scale_log2 + kLazy;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // wave-uniform: rare after the first tiles
      const float m_new = raise ? mt : m_ref;
      const float alpha = __builtin_amdgcn_exp2f((m_ref - m_new) * scale_log2);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
      m_ref = m_new;
    }
    const float mc = m_ref * scale_log2;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], scale_log2, -mc));
        s[kb][i] = p;
        psum += p;
      }
    l_run += psum;

    // O^T += V^T P^T over 4 steps of 16 keys; the V^T fragments of step st + 1 are read
    // while step st's MFMAs run
    {
      // lane l = 16 q + i points at key 4 (q / 2) + i / 4 (+ 8 for the second read) of the
      // step and channels db*32 + 16 (q % 2) + 4 (i % 4) .. +3; it receives channel
      // db*32 + l % 32 at keys 4 (l / 32) + 0..3 (and + 8..11) of the step
      const int vq = lane >> 4, vi = lane & 15;
      const int v_lane = (4 * (vq >> 1) + (vi >> 2)) * Cfg::VS + 16 * (vq & 1) + 4 * (vi & 3);
      auto vfrag = [&](int st, int db) {
        const bf16_t *vp = Vs + ((st >> 1) * 32 + 16 * (st & 1)) * Cfg::VS + db * 32 + v_lane;
        typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
        const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vp));
        const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vp + 8 * Cfg::VS));
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8_t vf[2][D / 32];
#pragma unroll
      for (int db = 0; db < D / 32; ++db) vf[0][db] = vfrag(0, db);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int kb = st >> 1, half = st & 1, cur = st & 1;
        if (st + 1 < 4) {
#pragma unroll
          for (int db = 0; db < D / 32; ++db) vf[cur ^ 1][db] = vfrag(st + 1, db);
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

}  // namespace

namespace {
template <int D, int WAVES>
void launch_cfg(const AttnProblems &pr, int n_problems, int heads, float scale_log2, hipStream_t s) {
  constexpr int BM = AttnCfg<D, WAVES>::BM;
  int tiles = 0;
  for (int i = 0; i < n_problems; ++i) tiles = std::max(tiles, (pr.p[i].nq + BM - 1) / BM);
  dim3 grid(tiles, heads, n_problems), block(64 * WAVES);
  attention_kernel<D, WAVES><<<grid, block, 0, s>>>(pr, scale_log2);
}

void launch_problems(const AttnProblems &pr, int n_problems, int heads, int head_dim, hipStream_t s) {
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(head_dim));
  int nq = 0;
  for (int i = 0; i < n_problems; ++i) nq = std::max(nq, pr.p[i].nq);
  if (head_dim == 128 && nq >= 8192)
    launch_cfg<128, 8>(pr, n_problems, heads, scale_log2, s);
  else if (head_dim == 128)
    launch_cfg<128, 4>(pr, n_problems, heads, scale_log2, s);
  else
    launch_cfg<64, 4>(pr, n_problems, heads, scale_log2, s);
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
