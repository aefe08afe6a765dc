// Shared device helpers for libdflash's gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

#define DF_DEV __device__ __forceinline__

DF_DEV float to_f(float x) { return x; }
DF_DEV float to_f(bf16 x) { return (float)x; }
template <typename T> DF_DEV T from_f(float x);
template <> DF_DEV float from_f<float>(float x) { return x; }
template <> DF_DEV bf16 from_f<bf16>(float x) { return (bf16)x; }

// Wave64 reductions (xor butterflies over all 64 lanes).
DF_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
DF_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum over a workgroup of up to 1024 threads; `red` must hold >= 16 floats.  All threads
// receive the total.  Deterministic: a fixed butterfly then a fixed-order sum.
DF_DEV float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// RoPE angle for position p and pair index i of a head of width d, evaluated in float64
// and rounded to float32 (cos, sin).
DF_DEV void rope_cs(int64_t p, int i, int d, double base, float* c, float* s) {
  const double theta = pow(base, -2.0 * (double)i / (double)d);
  const double a = (double)p * theta;
  *c = (float)cos(a);
  *s = (float)sin(a);
}

// Device error bits (mirror of DFLASH_DEVERR_*).
#define DEVERR_PAGE 1
#define DEVERR_TOKEN 2
#define DEVERR_TAU 4
DF_DEV void flag_error(int32_t* flags, int bit) {
  if (flags) atomicOr(flags, bit);
}
