// Memory-bound kernels of the block: gated residual + AdaLN (fused and unfused), Q/K
// RMSNorm + 3D RoPE, the RoPE table, horizontal token pairing, Euler update, dynamic int8
// row quantisation, and the small timestep/modulation kernels.
//
// Row kernels map one row to one 64-lane wavefront (4 rows per 256-thread workgroup): a row
// of d bf16 values is d/512 16-byte vectors per lane, loaded with consecutive lanes on
// consecutive 16-byte chunks (1 KiB per wave instruction), kept in registers, reduced with
// cross-lane butterflies.  No LDS and no barriers are needed.
#include <hip/hip_runtime.h>

#include <cmath>

#include <type_traits>

#include "h3_internal.h"

namespace h3 {

namespace {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ void load8f(const float *p, float *f) {
  float4 a = reinterpret_cast<const float4 *>(p)[0];
  float4 b = reinterpret_cast<const float4 *>(p)[1];
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// ------------------------------------------------------------------ int8 row quantisation
// Per group of channels: s = absmax / 127 (IEEE float32 division), q = clamp(rint(x / s),
// -127, 127) with x / s the correctly rounded float32 quotient and ties to even; s == 0 gives
// q = 0.  The quotient is formed as x * r with r = rcp(s) (within 1 ulp): for |x / s| <= 127
// that differs from the correctly rounded quotient by at most 3.1e-5, so both round to the
// same integer unless the value lies within that distance of a half-integer; those rare
// elements (|frac - 1/2| < 4e-5) take the exact division.  The result is the exact rule's.
__device__ __forceinline__ uint32_t quant4(const float *x, float s, float r) {
  float t[4];
  int near = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    t[k] = x[k] * r;
    const float f = t[k] - floorf(t[k]);
    if (fabsf(f - 0.5f) < 4e-5f) near |= 1 << k;
  }
  // a reciprocal that is not a finite positive number (s tiny) sends every element to the
  // exact division; s == 0 is handled below
  if (s > 0.f && !(r > 0.f && r < 3.0e38f)) near = 0xF;
  // wave-uniform branch: the divisions run only when some lane of the wave needs one
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(near != 0) != 0, 0)) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (near & (1 << k)) t[k] = x[k] / s;
  }
  uint32_t w = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float u = fminf(fmaxf(rintf(t[k]), -127.f), 127.f);
    const int q = s > 0.f ? static_cast<int>(u) : 0;
    w |= (static_cast<uint32_t>(q) & 0xFFu) << (8 * k);
  }
  return w;
}
__device__ __forceinline__ float quant_rcp(float s) { return s > 0.f ? __builtin_amdgcn_rcpf(s) : 0.f; }

// ------------------------------------------------------------------ gate + AdaLN
// GATE: x' = bf16(x + g*y) stored to x_out.  NORM: n = bf16((v - mean) * rstd * (1 + sc) + sh)
// over the row v (= x' when GATE, else the row of x).  The fused variant (GATE && NORM)
// normalises the bf16-rounded x' held in registers; the unfused pair writes x' and reads it
// back.  Both run the identical NORM code below (same lane mapping, order and operations),
// so their outputs are bit-identical.
// QUANT (with NORM): instead of n, the row of bf16-rounded n is quantised to int8 with one
// scale per row by the quant4 rule above and written as q_out (int8) and s_out (float32), the
// same bits as storing n and quantising it with the row quantiser.
// YS > 0 (with GATE): y is not read as bf16 but formed from YS split-K partials (GateY): the
// partials summed in piece order plus the bias sum, rounded to bf16 -- the reduction kernel's
// arithmetic -- and optionally stored to ysrc.y_out.  An absent second bias adds +0, which
// leaves every sum's bits unchanged, so the bias loads need no branch.
// YI8 (with YS): the partials are the int32 sums of the row-mode int8 FC2 (ysrc.ipart), added
// in piece order and dequantised as the int8 split-K reduction does:
// y = bf16((float(sum) * sa[row]) * sw[col] + b1[col]), without contraction.
// All loads of a chunk are issued before its values are used (no branches, no runtime loops),
// and the AdaLN shift / scale are loaded before the row reductions.
// WPR waves per row: 1 (four rows per 256-thread block) or 2 (one row per 128-thread block,
// the two waves' butterfly sums added wave 0 first through LDS); thread t of the row holds
// the VPL 8-channel chunks at (i * 64 WPR + t) * 8.
template <int WPR>
__device__ __forceinline__ float row_sum(float v, float *red, int t) {
  v = wave_sum(v);
  if constexpr (WPR == 2) {
    if ((t & 63) == 0) red[t >> 6] = v;
    __syncthreads();
    v = red[0] + red[1];
  }
  return v;
}
template <int WPR>
__device__ __forceinline__ float row_max(float v, float *red, int t) {
  v = wave_max(v);
  if constexpr (WPR == 2) {
    if ((t & 63) == 0) red[t >> 6] = v;
    __syncthreads();
    v = fmaxf(red[0], red[1]);
  }
  return v;
}

template <int VPL, int WPR, bool GATE, bool NORM, bool QUANT, int YS, bool YI8 = false>
__global__ __launch_bounds__(256) void gate_adaln_kernel(
    const bf16_t *__restrict__ x, const bf16_t *__restrict__ y, GateY ysrc,
    const float *__restrict__ gate, bf16_t *x_out, const float *__restrict__ shift,
    const float *__restrict__ scale, bf16_t *__restrict__ n_out, int8_t *__restrict__ q_out,
    float *__restrict__ s_out, int rows, int d) {
#pragma clang fp contract(off)
  static_assert(WPR == 1 || WPR == 2, "one or two waves per row");
  constexpr int TPR = 64 * WPR;
  __shared__ float red[3][2];  // (sum, sum of squares, absmax) x wave of the row
  const int lane = threadIdx.x % TPR;  // thread of the row
  const int row = WPR == 2 ? static_cast<int>(blockIdx.x) : blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // WPR == 2: the grid has exactly `rows` blocks
  const size_t base = static_cast<size_t>(row) * d;
  float v[VPL][8];
  // the branch values y (stored afterwards when y_out is given)
  float yk[YS > 0 ? VPL : 1][8];
  // all loads of the row first, stores after: x_out may alias x, so a store between them would
  // hold the later chunks' loads back
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = (i * TPR + lane) * 8;
    uint4 xv = *reinterpret_cast<const uint4 *>(x + base + e);
    unpack8(xv, v[i]);
    if constexpr (GATE) {
      float yv[8], gv[8];
      if constexpr (YS > 0 && YI8) {
        int32_t t[8];
        float sw[8], b1[8];
        {
          const int4 *pp = reinterpret_cast<const int4 *>(ysrc.ipart + base + e);
          const int4 p0 = pp[0], p1 = pp[1];
          t[0] = p0.x; t[1] = p0.y; t[2] = p0.z; t[3] = p0.w;
          t[4] = p1.x; t[5] = p1.y; t[6] = p1.z; t[7] = p1.w;
        }
#pragma unroll
        for (int q = 1; q < YS; ++q) {
          const int4 *pp = reinterpret_cast<const int4 *>(ysrc.ipart + q * ysrc.stride + base + e);
          const int4 p0 = pp[0], p1 = pp[1];
          t[0] += p0.x; t[1] += p0.y; t[2] += p0.z; t[3] += p0.w;
          t[4] += p1.x; t[5] += p1.y; t[6] += p1.z; t[7] += p1.w;
        }
        load8f(ysrc.sw + e, sw);
        unpack8(*reinterpret_cast<const uint4 *>(ysrc.b1 + e), b1);
        const float sa = ysrc.sa[row];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float v = static_cast<float>(t[k]) * sa;
          const float w = v * sw[k];
          yv[k] = bf2f(f2bf(w + b1[k]));
          yk[i][k] = yv[k];
        }
      } else if constexpr (YS > 0) {
        float t[8], u[8], b1[8], b2[8];
        load8f(ysrc.part + base + e, t);
        unpack8(*reinterpret_cast<const uint4 *>(ysrc.b1 + e), b1);
        unpack8(*reinterpret_cast<const uint4 *>((ysrc.b2 ? ysrc.b2 : ysrc.b1) + e), b2);
#pragma unroll
        for (int q = 1; q < YS; ++q) {
          load8f(ysrc.part + q * ysrc.stride + base + e, u);
#pragma unroll
          for (int k = 0; k < 8; ++k) t[k] = t[k] + u[k];
        }
        const bool has_b2 = ysrc.b2 != nullptr;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          float b = 0.f;
          b += b1[k];
          b += has_b2 ? b2[k] : 0.f;
          yv[k] = bf2f(f2bf(t[k] + b));
          yk[i][k] = yv[k];
        }
      } else {
        unpack8(*reinterpret_cast<const uint4 *>(y + base + e), yv);
      }
      load8f(gate + e, gv);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[i][k] = bf2f(f2bf(v[i][k] + gv[k] * yv[k]));
    }
  }
  float shv[NORM ? VPL : 1][8], scv[NORM ? VPL : 1][8];
  // AdaLN shift / scale: with one wave per row loaded before the reductions; with two (fewer
  // rows) after the mean, in flight during the variance reduction, which keeps the registers
  // low enough for three waves per SIMD
  auto load_mod = [&]() {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = (i * TPR + lane) * 8;
      load8f(shift + e, shv[i]);
      load8f(scale + e, scv[i]);
    }
  };
  if constexpr (NORM && WPR == 1) load_mod();
  if constexpr (GATE) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = (i * TPR + lane) * 8;
      if constexpr (YS > 0) {
        if (ysrc.y_out) *reinterpret_cast<uint4 *>(ysrc.y_out + base + e) = pack8(yk[i]);
      }
      *reinterpret_cast<uint4 *>(x_out + base + e) = pack8(v[i]);
    }
  }
  if constexpr (NORM) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
#pragma unroll
      for (int k = 0; k < 8; ++k) s += v[i][k];
    s = row_sum<WPR>(s, red[0], lane);
    if constexpr (WPR == 2) load_mod();
    const float mean = s / static_cast<float>(d);
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float c = v[i][k] - mean;
        q += c * c;
      }
    q = row_sum<WPR>(q, red[1], lane);
    const float rstd = 1.0f / sqrtf(q / static_cast<float>(d) + kLnEps);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = (i * TPR + lane) * 8;
      float o[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = ((v[i][k] - mean) * rstd) * (1.0f + scv[i][k]) + shv[i][k];
      if constexpr (QUANT) {
        // keep the bf16-rounded output in place of the (no longer needed) input vector
#pragma unroll
        for (int k = 0; k < 8; ++k) v[i][k] = bf2f(f2bf(o[k]));
      } else {
        *reinterpret_cast<uint4 *>(n_out + base + e) = pack8(o);
      }
    }
    if constexpr (QUANT) {
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
#pragma unroll
        for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[i][k]));
      m = row_max<WPR>(m, red[2], lane);
      const float sq = m / 127.0f, rq = quant_rcp(sq);
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = (i * TPR + lane) * 8;
        uint2 w;
        w.x = quant4(v[i], sq, rq);
        w.y = quant4(v[i] + 4, sq, rq);
        *reinterpret_cast<uint2 *>(q_out + base + e) = w;
      }
      if (lane == 0) s_out[row] = sq;
    }
  }
}

template <bool GATE, bool NORM, bool QUANT, int YS = 0, bool YI8 = false>
void dispatch_gate_adaln(const bf16_t *x, const bf16_t *y, const float *gate, bf16_t *x_out,
                         const float *shift, const float *scale, bf16_t *n_out, int8_t *q_out,
                         float *s_out, int rows, int d, hipStream_t s, const GateY &ysrc = GateY{}) {
  // few rows (under 16384) and an even number of 512-channel chunks: two waves per row, twice
  // the waves in flight for the same rows; otherwise one (with many rows the GPU is full
  // anyway and the second wave's LDS exchange only costs: measured at 61,488 rows)
  const dim3 grid1((rows + 3) / 4), block1(256), grid2(rows), block2(128);
  const int v512 = d / 512;
  if (adaln_waves_per_row(rows, d) == 1) {
    switch (v512) {
#define H3_CASE1(V)                                                                         \
  case V:                                                                                   \
    gate_adaln_kernel<V, 1, GATE, NORM, QUANT, YS, YI8><<<grid1, block1, 0, s>>>(           \
        x, y, ysrc, gate, x_out, shift, scale, n_out, q_out, s_out, rows, d);               \
    break;
      H3_CASE1(1) H3_CASE1(2) H3_CASE1(3) H3_CASE1(4) H3_CASE1(5) H3_CASE1(6) H3_CASE1(8)
      H3_CASE1(10) H3_CASE1(12) H3_CASE1(16)
#undef H3_CASE1
      default: break;
    }
    return;
  }
  switch (v512) {
#define H3_CASE2(V)                                                                         \
  case 2 * V:                                                                               \
    gate_adaln_kernel<V, 2, GATE, NORM, QUANT, YS, YI8><<<grid2, block2, 0, s>>>(           \
        x, y, ysrc, gate, x_out, shift, scale, n_out, q_out, s_out, rows, d);               \
    break;
    H3_CASE2(1) H3_CASE2(2) H3_CASE2(3) H3_CASE2(4) H3_CASE2(5) H3_CASE2(6) H3_CASE2(8)
#undef H3_CASE2
    default: break;
  }
}

// ------------------------------------------------------------------ RoPE table
// table[n * (D/2) + p] = (cos, sin) of coord_axis(n) * 10000^(-2 j / D_axis) for pair p, where
// the head splits into [t | h | w] slices of D - 4 floor(D/6), 2 floor(D/6), 2 floor(D/6)
// channels and j is the pair index inside its slice.  Computed in double.
__global__ void rope_table_kernel(float2 *table, int n_tokens, int half, int pairs_t,
                                  int pairs_h, int gh, int gw, int paired, float sscale) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_tokens * half) return;
  const int n = idx / half, p = idx - n * half;
  double f, h, w;
  if (!paired) {
    w = n % gw;
    h = (n / gw) % gh;
    f = n / (gw * gh);
  } else {
    const int wr = (gw + 1) / 2;
    const int c = n % wr;
    h = (n / wr) % gh;
    f = n / (wr * gh);
    const int w0 = 2 * c, w1 = (2 * c + 1 < gw) ? 2 * c + 1 : 2 * c;
    w = 0.5 * (w0 + w1);
  }
  h *= sscale;
  w *= sscale;
  double coord;
  int j, da;
  if (p < pairs_t) {
    coord = f; j = p; da = 2 * pairs_t;
  } else if (p < pairs_t + pairs_h) {
    coord = h; j = p - pairs_t; da = 2 * pairs_h;
  } else {
    coord = w; j = p - pairs_t - pairs_h; da = 2 * pairs_h;
  }
  const double ang = coord * pow(10000.0, -2.0 * j / da);
  table[idx] = make_float2(static_cast<float>(cos(ang)), static_cast<float>(sin(ang)));
}

// ------------------------------------------------------------------ Q/K RMSNorm + RoPE
// One wave per token.  The [q | k] span (2d channels at the start of the qkvq row) is walked
// in 512-channel chunks; each lane owns 8 consecutive channels = 4 rotation pairs, so a head
// of D channels lives on D/8 adjacent lanes and its RMS is a butterfly over those lanes.
template <int D>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(
    bf16_t *qkvq, int64_t ld, int n_tokens, int d, const bf16_t *__restrict__ q_gamma,
    const bf16_t *__restrict__ k_gamma, int qk_norm, const float2 *__restrict__ table) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n_tokens) return;
  bf16_t *rp = qkvq + static_cast<size_t>(row) * ld;
  const float2 *tr = table + static_cast<size_t>(row) * (D / 2);
  const int chunks = (2 * d) / 512;
  const int pos = (lane * 8) % D;  // channel offset inside the head
  for (int c = 0; c < chunks; ++c) {
    const int e = c * 512 + lane * 8;
    float a[8], g[8];
    float2 cs[4];
    unpack8(*reinterpret_cast<const uint4 *>(rp + e), a);
    float ss = 0.f;
    if (qk_norm) {
      ss = qk_head_sumsq<D>(qk_sumsq8(a));
      unpack8(*reinterpret_cast<const uint4 *>((e < d ? q_gamma : k_gamma) + pos), g);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) cs[k] = tr[pos / 2 + k];
    qk_norm_rope8<D>(a, ss, g, cs, qk_norm != 0);
    *reinterpret_cast<uint4 *>(rp + e) = pack8(a);
  }
}

// ------------------------------------------------------------------ token pairing
// One thread per (reduced token, 8-channel vector).  The pair of reduced token j in row
// (f, h) is (row*gw + 2c, row*gw + min(2c+1, gw-1)) with c = j % ceil(gw/2).
__device__ __forceinline__ void pair_of(int j, int gw, int &p0, int &p1) {
  const int wr = (gw + 1) / 2;
  const int row = j / wr, c = j - row * wr;
  p0 = row * gw + 2 * c;
  p1 = (2 * c + 1 < gw) ? p0 + 1 : p0;
}

__global__ void token_merge_kernel(const bf16_t *__restrict__ src, bf16_t *__restrict__ dst,
                                   int n_red, int gw, int d) {
  const int vecs = d / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(n_red) * vecs) return;
  const int j = static_cast<int>(idx / vecs), v = static_cast<int>(idx - static_cast<int64_t>(j) * vecs);
  int p0, p1;
  pair_of(j, gw, p0, p1);
  float a[8], b[8], o[8];
  unpack8(*reinterpret_cast<const uint4 *>(src + static_cast<size_t>(p0) * d + v * 8), a);
  unpack8(*reinterpret_cast<const uint4 *>(src + static_cast<size_t>(p1) * d + v * 8), b);
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = (a[k] + b[k]) * 0.5f;
  *reinterpret_cast<uint4 *>(dst + static_cast<size_t>(j) * d + v * 8) = pack8(o);
}

// dst may equal bypass: each thread reads both pair members before writing them and pairs
// are disjoint.
__global__ void token_restore_kernel(const bf16_t *__restrict__ xr, const bf16_t *bypass,
                                     bf16_t *dst, int n_red, int gw, int d) {
#pragma clang fp contract(off)
  const int vecs = d / 8;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(n_red) * vecs) return;
  const int j = static_cast<int>(idx / vecs), v = static_cast<int>(idx - static_cast<int64_t>(j) * vecs);
  int p0, p1;
  pair_of(j, gw, p0, p1);
  float a[8], b[8], r[8], o0[8], o1[8];
  unpack8(*reinterpret_cast<const uint4 *>(bypass + static_cast<size_t>(p0) * d + v * 8), a);
  unpack8(*reinterpret_cast<const uint4 *>(bypass + static_cast<size_t>(p1) * d + v * 8), b);
  unpack8(*reinterpret_cast<const uint4 *>(xr + static_cast<size_t>(j) * d + v * 8), r);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float m0 = bf2f(f2bf((a[k] + b[k]) * 0.5f));  // the merge value exactly as stored
    const float delta = r[k] - m0;
    o0[k] = a[k] + delta;
    o1[k] = b[k] + delta;
  }
  *reinterpret_cast<uint4 *>(dst + static_cast<size_t>(p0) * d + v * 8) = pack8(o0);
  if (p1 != p0) *reinterpret_cast<uint4 *>(dst + static_cast<size_t>(p1) * d + v * 8) = pack8(o1);
}

// ------------------------------------------------------------------ Euler
__global__ void euler_kernel(float *__restrict__ x, const float *__restrict__ v, float dt,
                             int64_t n) {
#pragma clang fp contract(off)
  const int64_t i4 = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i4 + 3 < n) {
    float4 a = *reinterpret_cast<float4 *>(x + i4);
    const float4 b = *reinterpret_cast<const float4 *>(v + i4);
    a.x = a.x + dt * b.x; a.y = a.y + dt * b.y; a.z = a.z + dt * b.z; a.w = a.w + dt * b.w;
    *reinterpret_cast<float4 *>(x + i4) = a;
  } else {
    for (int64_t i = i4; i < n; ++i) x[i] = x[i] + dt * v[i];
  }
}

// ------------------------------------------------------------------ core-residual reuse
// delta = float(x_core) - float(x_patch) over n elements (8 per thread).
__global__ void core_delta_kernel(const bf16_t *__restrict__ x_core, const bf16_t *__restrict__ x_patch,
                                  float *__restrict__ delta, int64_t n) {
#pragma clang fp contract(off)
  const int64_t i8 = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 8;
  if (i8 >= n) return;
  float a[8], b[8];
  unpack8(*reinterpret_cast<const uint4 *>(x_core + i8), a);
  unpack8(*reinterpret_cast<const uint4 *>(x_patch + i8), b);
  float4 lo, hi;
  lo.x = a[0] - b[0]; lo.y = a[1] - b[1]; lo.z = a[2] - b[2]; lo.w = a[3] - b[3];
  hi.x = a[4] - b[4]; hi.y = a[5] - b[5]; hi.z = a[6] - b[6]; hi.w = a[7] - b[7];
  reinterpret_cast<float4 *>(delta + i8)[0] = lo;
  reinterpret_cast<float4 *>(delta + i8)[1] = hi;
}

// x = bf16(float(x_patch) + delta), in place on x_patch allowed (8 per thread).
__global__ void core_apply_kernel(const bf16_t *x_patch, const float *__restrict__ delta,
                                  bf16_t *x, int64_t n) {
#pragma clang fp contract(off)
  const int64_t i8 = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 8;
  if (i8 >= n) return;
  float a[8];
  unpack8(*reinterpret_cast<const uint4 *>(x_patch + i8), a);
  const float4 lo = reinterpret_cast<const float4 *>(delta + i8)[0];
  const float4 hi = reinterpret_cast<const float4 *>(delta + i8)[1];
  a[0] = a[0] + lo.x; a[1] = a[1] + lo.y; a[2] = a[2] + lo.z; a[3] = a[3] + lo.w;
  a[4] = a[4] + hi.x; a[5] = a[5] + hi.y; a[6] = a[6] + hi.z; a[7] = a[7] + hi.w;
  *reinterpret_cast<uint4 *>(x + i8) = pack8(a);
}

// group == 1024: one wave per (row, group), 16 channels per lane.
__global__ __launch_bounds__(256) void quant_groups_kernel(const bf16_t *__restrict__ X,
                                                           int8_t *__restrict__ Q,
                                                           float *__restrict__ S, int rows, int K) {
  const int lane = threadIdx.x & 63;
  const int ng = K / 1024;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);  // row * ng + g
  if (item >= static_cast<int64_t>(rows) * ng) return;
  const int64_t row = item / ng;
  const int g = static_cast<int>(item - row * ng);
  const bf16_t *xr = X + row * K;
  int8_t *qr = Q + row * K;
  float a[16];
  const int e0 = g * 1024 + lane * 8, e1 = e0 + 512;
  unpack8(*reinterpret_cast<const uint4 *>(xr + e0), a);
  unpack8(*reinterpret_cast<const uint4 *>(xr + e1), a + 8);
  float m = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) m = fmaxf(m, fabsf(a[k]));
  m = wave_max(m);
  const float s = m / 127.0f, r = quant_rcp(s);
  uint2 w0, w1;
  w0.x = quant4(a, s, r); w0.y = quant4(a + 4, s, r);
  w1.x = quant4(a + 8, s, r); w1.y = quant4(a + 12, s, r);
  *reinterpret_cast<uint2 *>(qr + e0) = w0;
  *reinterpret_cast<uint2 *>(qr + e1) = w1;
  if (lane == 0) S[item] = s;
}

// Row mode with K = 8 V T: T threads (T / 64 waves) per row, the row held in registers (V
// 16-byte vectors per thread, consecutive threads on consecutive vectors), one pass over HBM.
// The row maximum is exact in any order, so the thread count does not change the result.
template <int V, int T>
__global__ __launch_bounds__(T) void quant_row_kernel(const bf16_t *__restrict__ X,
                                                      int8_t *__restrict__ Q,
                                                      float *__restrict__ S) {
  constexpr int K = V * 8 * T, W = T / 64;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const bf16_t *xr = X + row * K;
  int8_t *qr = Q + row * K;
  uint4 raw[V];
#pragma unroll
  for (int v = 0; v < V; ++v) raw[v] = *reinterpret_cast<const uint4 *>(xr + (v * T + tid) * 8);
  float m = 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    float a[8];
    unpack8(raw[v], a);
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(a[k]));
  }
  m = wave_max(m);
  __shared__ float red[W];
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < W; ++w) m = fmaxf(m, red[w]);
  const float s = m / 127.0f, r = quant_rcp(s);
#pragma unroll
  for (int v = 0; v < V; ++v) {
    float a[8];
    unpack8(raw[v], a);
    uint2 w;
    w.x = quant4(a, s, r);
    w.y = quant4(a + 4, s, r);
    *reinterpret_cast<uint2 *>(qr + (v * T + tid) * 8) = w;
  }
  if (tid == 0) S[row] = s;
}

// Row mode, any K (multiple of 512): one wave per row, two passes over the row.
__global__ __launch_bounds__(256) void quant_row_any_kernel(const bf16_t *__restrict__ X,
                                                            int8_t *__restrict__ Q,
                                                            float *__restrict__ S, int rows, int K) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const bf16_t *xr = X + static_cast<size_t>(row) * K;
  int8_t *qr = Q + static_cast<size_t>(row) * K;
  float m = 0.f;
  for (int e = lane * 8; e < K; e += 512) {
    float a[8];
    unpack8(*reinterpret_cast<const uint4 *>(xr + e), a);
#pragma unroll
    for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(a[k]));
  }
  m = wave_max(m);
  const float s = m / 127.0f, r = quant_rcp(s);
  for (int e = lane * 8; e < K; e += 512) {
    float a[8];
    unpack8(*reinterpret_cast<const uint4 *>(xr + e), a);
    uint2 w;
    w.x = quant4(a, s, r);
    w.y = quant4(a + 4, s, r);
    *reinterpret_cast<uint2 *>(qr + e) = w;
  }
  if (lane == 0) S[row] = s;
}

// ------------------------------------------------------------------ small kernels
__global__ void f32_to_bf16_kernel(const float *__restrict__ src, bf16_t *__restrict__ dst,
                                   int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = static_cast<bf16_t>(f2bf(src[i]));
}

// e = [cos(t w_j) | sin(t w_j)], j < 128, t = 1000 sigma, w_j = 10000^(-j/128), in double.
__global__ void sinusoid_kernel(float sigma, float *e) {
  const int j = threadIdx.x;
  if (j >= 128) return;
  const double t = 1000.0 * static_cast<double>(sigma);
  const double w = pow(10000.0, -static_cast<double>(j) / 128.0);
  e[j] = static_cast<float>(cos(t * w));
  e[128 + j] = static_cast<float>(sin(t * w));
}

// One wave per output row; float32 accumulation.
__global__ __launch_bounds__(256) void gemv_kernel(const bf16_t *__restrict__ W,
                                                   const float *__restrict__ x,
                                                   const bf16_t *__restrict__ b,
                                                   const bf16_t *__restrict__ add,
                                                   float *__restrict__ y, int rows, int K,
                                                   int act) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const bf16_t *wr = W + static_cast<size_t>(r) * K;
  float acc = 0.f;
  for (int e = lane * 8; e < K; e += 512) {
    float w[8], xv[8];
    unpack8(*reinterpret_cast<const uint4 *>(wr + e), w);
    load8f(x + e, xv);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += w[k] * xv[k];
  }
  acc = wave_sum(acc);
  if (lane == 0) {
    float v = acc + (b ? bf2f(b[r]) : 0.f);
    if (act == 1) v = v / (1.0f + expf(-v));
    if (add) v += bf2f(add[r]);
    y[r] = v;
  }
}

__global__ void add_table_kernel(const float *__restrict__ Mv, const bf16_t *__restrict__ T,
                                 float *__restrict__ out, int nb, int width) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(nb) * width) return;
  out[i] = Mv[i % width] + bf2f(T[i]);
}

}  // namespace

void launch_gate_adaln(const bf16_t *x, const bf16_t *y, const float *gate, bf16_t *x_out,
                       const float *shift, const float *scale, bf16_t *n_out, int rows, int d,
                       hipStream_t s, int8_t *q_out, float *s_out) {
  if (rows <= 0) return;
  if (q_out) {
    if (y)
      dispatch_gate_adaln<true, true, true>(x, y, gate, x_out, shift, scale, nullptr, q_out, s_out, rows, d, s);
    else
      dispatch_gate_adaln<false, true, true>(x, y, gate, x_out, shift, scale, nullptr, q_out, s_out, rows, d, s);
  } else if (y && n_out) {
    dispatch_gate_adaln<true, true, false>(x, y, gate, x_out, shift, scale, n_out, nullptr, nullptr, rows, d, s);
  } else if (y) {
    dispatch_gate_adaln<true, false, false>(x, y, gate, x_out, shift, scale, n_out, nullptr, nullptr, rows, d, s);
  } else {
    dispatch_gate_adaln<false, true, false>(x, y, gate, x_out, shift, scale, n_out, nullptr, nullptr, rows, d, s);
  }
}

void launch_gate_adaln_part(const bf16_t *x, const GateY &ysrc, const float *gate, bf16_t *x_out,
                            const float *shift, const float *scale, bf16_t *n_out, int rows, int d,
                            hipStream_t s, int8_t *q_out, float *s_out) {
  if (rows <= 0) return;
  const auto go = [&](auto ys, auto yi8) {
    constexpr int YS = decltype(ys)::value;
    constexpr bool YI8 = decltype(yi8)::value;
    if (q_out)
      dispatch_gate_adaln<true, true, true, YS, YI8>(x, nullptr, gate, x_out, shift, scale, nullptr,
                                                     q_out, s_out, rows, d, s, ysrc);
    else if (n_out)
      dispatch_gate_adaln<true, true, false, YS, YI8>(x, nullptr, gate, x_out, shift, scale, n_out,
                                                      nullptr, nullptr, rows, d, s, ysrc);
    else
      dispatch_gate_adaln<true, false, false, YS, YI8>(x, nullptr, gate, x_out, shift, scale,
                                                       nullptr, nullptr, nullptr, rows, d, s, ysrc);
  };
  // the int8 FC2's partials are always four pieces (its row-mode plan splits K in 4)
  if (ysrc.ipart)
    go(std::integral_constant<int, 4>(), std::true_type());
  else if (ysrc.S == 4)
    go(std::integral_constant<int, 4>(), std::false_type());
  else
    go(std::integral_constant<int, 2>(), std::false_type());
}

void launch_rope_table(float2 *table, const h3_geom &geom, int n_tokens, int head_dim,
                       hipStream_t s) {
  const int half = head_dim / 2;
  const int hw = 2 * (head_dim / 6);
  const int pairs_h = hw / 2, pairs_t = (head_dim - 2 * hw) / 2;
  const int total = n_tokens * half;
  rope_table_kernel<<<(total + 255) / 256, 256, 0, s>>>(table, n_tokens, half, pairs_t, pairs_h,
                                                        geom.grid_h, geom.grid_w, geom.paired,
                                                        geom.rope_spatial_scale);
}

void launch_qk_norm_rope(bf16_t *qkvq, int64_t ld, int n_tokens, int d, int head_dim,
                         const bf16_t *q_gamma, const bf16_t *k_gamma, int qk_norm,
                         const float2 *table, hipStream_t s) {
  dim3 grid((n_tokens + 3) / 4), block(256);
  if (head_dim == 128)
    qk_norm_rope_kernel<128><<<grid, block, 0, s>>>(qkvq, ld, n_tokens, d, q_gamma, k_gamma,
                                                     qk_norm, table);
  else
    qk_norm_rope_kernel<64><<<grid, block, 0, s>>>(qkvq, ld, n_tokens, d, q_gamma, k_gamma,
                                                    qk_norm, table);
}

void launch_token_reduce(int direction, const h3_geom &geom, int d, const bf16_t *src,
                         const bf16_t *bypass, bf16_t *dst, hipStream_t s) {
  const int n_red = geom.f_lat * geom.grid_h * ((geom.grid_w + 1) / 2);
  const int64_t total = static_cast<int64_t>(n_red) * (d / 8);
  const int blocks = static_cast<int>((total + 255) / 256);
  if (direction == 0)
    token_merge_kernel<<<blocks, 256, 0, s>>>(src, dst, n_red, geom.grid_w, d);
  else
    token_restore_kernel<<<blocks, 256, 0, s>>>(src, bypass, dst, n_red, geom.grid_w, d);
}

void launch_core_delta(const bf16_t *x_core, const bf16_t *x_patch, float *delta, int64_t n,
                       hipStream_t s) {
  const int64_t threads = n / 8;
  core_delta_kernel<<<static_cast<int>((threads + 255) / 256), 256, 0, s>>>(x_core, x_patch, delta, n);
}

void launch_core_apply(const bf16_t *x_patch, const float *delta, bf16_t *x, int64_t n, hipStream_t s) {
  const int64_t threads = n / 8;
  core_apply_kernel<<<static_cast<int>((threads + 255) / 256), 256, 0, s>>>(x_patch, delta, x, n);
}

void launch_euler(float *x, const float *v, float dt, int64_t n, hipStream_t s) {
  const int64_t threads = (n + 3) / 4;
  euler_kernel<<<static_cast<int>((threads + 255) / 256), 256, 0, s>>>(x, v, dt, n);
}

void launch_quant_rows(const bf16_t *X, int8_t *Q, float *S, int rows, int K, int group,
                       hipStream_t s) {
  if (group == 1024) {
    const int64_t items = static_cast<int64_t>(rows) * (K / 1024);
    quant_groups_kernel<<<static_cast<int>((items + 3) / 4), 256, 0, s>>>(X, Q, S, rows, K);
    return;
  }
  // long rows (K = 2048 n >= 8192): four waves per row, for more waves in flight
  switch (K % 2048 == 0 && K >= 8192 ? K / 2048 : 0) {
#define H3_QROW4(V) \
  case V: quant_row_kernel<V, 256><<<rows, 256, 0, s>>>(X, Q, S); return;
    H3_QROW4(4) H3_QROW4(5) H3_QROW4(6) H3_QROW4(8) H3_QROW4(10)
#undef H3_QROW4
    default: break;
  }
  switch (K % 1024 == 0 ? K / 1024 : 0) {
#define H3_QROW(V) \
  case V: quant_row_kernel<V, 128><<<rows, 128, 0, s>>>(X, Q, S); return;
    H3_QROW(1) H3_QROW(2) H3_QROW(3) H3_QROW(4) H3_QROW(5) H3_QROW(6) H3_QROW(8) H3_QROW(10)
    H3_QROW(12) H3_QROW(16) H3_QROW(20)
#undef H3_QROW
    default: quant_row_any_kernel<<<(rows + 3) / 4, 256, 0, s>>>(X, Q, S, rows, K);
  }
}

void launch_f32_to_bf16(const float *src, bf16_t *dst, int64_t n, hipStream_t s) {
  f32_to_bf16_kernel<<<static_cast<int>((n + 255) / 256), 256, 0, s>>>(src, dst, n);
}

void launch_timestep_sinusoid(float sigma, float *e, hipStream_t s) {
  sinusoid_kernel<<<1, 128, 0, s>>>(sigma, e);
}

void launch_gemv(const bf16_t *W, const float *x, const bf16_t *b, const bf16_t *add, float *y,
                 int rows, int K, int act, hipStream_t s) {
  gemv_kernel<<<(rows + 3) / 4, 256, 0, s>>>(W, x, b, add, y, rows, K, act);
}

void launch_add_table(const float *Mv, const bf16_t *T, float *out, int nb, int width,
                      hipStream_t s) {
  const int64_t total = static_cast<int64_t>(nb) * width;
  add_table_kernel<<<static_cast<int>((total + 255) / 256), 256, 0, s>>>(Mv, T, out, nb, width);
}

}  // namespace h3
