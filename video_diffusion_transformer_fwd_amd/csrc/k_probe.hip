// Matrix-core throughput probe: the dense bf16 (or int8) MFMA rate this GPU sustains at the
// clock it runs, the reference against which the products' and attention's rates are judged.
//
// Every wave issues `iters` rounds of eight independent 32x32 MFMAs (v_mfma_f32_32x32x16_bf16,
// or v_mfma_i32_32x32x32_i8) on register operands: no memory traffic and no dependent chain
// shorter than eight instructions, so the matrix core of every SIMD stays busy.  The
// accumulators are summed and written once per thread so the loop is kept.  The launch puts
// two workgroups of four waves on every CU (two waves per SIMD).
#include <hip/hip_runtime.h>

#include "h3_internal.h"

namespace h3 {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;
typedef __attribute__((ext_vector_type(16))) int i32x16_t;

template <int I8>
__global__ __launch_bounds__(256) void mfma_probe_kernel(float *__restrict__ out, int iters) {
  const int t = threadIdx.x;
  float r = 0.f;
  if constexpr (I8) {
    i32x4_t a, b;
    for (int i = 0; i < 4; ++i) {
      a[i] = 0x01020304 * (t + i);
      b[i] = 0x05060708 ^ (t * 7 + i);
    }
    i32x16_t c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = i32x16_t{};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) r += static_cast<float>(c[j][i]);
  } else {
    bf16x8_t a, b;
    for (int i = 0; i < 8; ++i) {
      a[i] = static_cast<__bf16>(0.001f * (t + i));
      b[i] = static_cast<__bf16>(0.5f - 0.01f * i);
    }
    f32x16_t c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = f32x16_t{};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) r += c[j][i];
  }
  out[static_cast<int64_t>(blockIdx.x) * 256 + t] = r;
}

}  // namespace

void launch_mfma_probe(int int8, int iters, int workgroups, float *out, hipStream_t s) {
  if (int8)
    mfma_probe_kernel<1><<<workgroups, 256, 0, s>>>(out, iters);
  else
    mfma_probe_kernel<0><<<workgroups, 256, 0, s>>>(out, iters);
}

}  // namespace h3
