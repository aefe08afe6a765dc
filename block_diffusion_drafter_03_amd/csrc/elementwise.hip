// Row-wise and elementwise kernels of the drafter / verifier step (all deterministic:
// fixed reduction trees, no floating-point atomics).
#include "common.h"
#include "kernels.h"

namespace dflash {

// ---------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* ids, const int32_t* anchor,
                                                    int mode, int B, int mask_id,
                                                    const T* __restrict__ E, int V, int D,
                                                    float* __restrict__ h, float* hdbg,
                                                    int32_t* err) {
  const int row = blockIdx.x, b = row / B, j = row % B;
  int tok = mode == 0 ? (j == 0 ? anchor[b] : mask_id) : ids[row];
  if (tok < 0 || tok >= V) {
    if (threadIdx.x == 0) flag_error(err, DEVERR_TOKEN);
    tok = 0;
  }
  const T* e = E + (size_t)tok * D;
  for (int c = threadIdx.x; c < D; c += 256) {
    const float x = to_f(e[c]);
    h[(size_t)row * D + c] = x;
    if (hdbg) hdbg[(size_t)row * D + c] = x;
  }
}

hipError_t launch_embed(int dt, const int32_t* ids, const int32_t* anchor, int mode, int batch,
                        int B, int mask_id, const void* E, int V, int D, float* h, float* hdbg,
                        int32_t* err, hipStream_t st) {
  const int rows = batch * B;
  if (dt == BF16)
    hipLaunchKernelGGL(embed_kernel<bf16>, dim3(rows), dim3(256), 0, st, ids, anchor, mode, B,
                       mask_id, (const bf16*)E, V, D, h, hdbg, err);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(rows), dim3(256), 0, st, ids, anchor, mode, B,
                       mask_id, (const float*)E, V, D, h, hdbg, err);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// x = [h +] sum_s C_s ; optional h = x, hdbg = x, tap = x ; optional u = RMSNorm(x) * g.
template <typename T>
__global__ __launch_bounds__(256) void row_finalize_kernel(RowFin f) {
  extern __shared__ float xs[];
  __shared__ float red[16];
  const int row = blockIdx.x, N = f.N;
  float ss = 0.f;
  for (int c = threadIdx.x; c < N; c += 256) {
    float x = (f.h && f.add_resid) ? f.h[(size_t)row * N + c] : 0.f;
    if (f.C)
      for (int s = 0; s < f.S; ++s) x += f.C[(size_t)s * f.split_stride + (size_t)row * N + c];
    xs[c] = x;
    ss += x * x;
    if (f.h && f.write_h) f.h[(size_t)row * N + c] = x;
    if (f.hdbg) f.hdbg[(size_t)row * N + c] = x;
    if (f.tap) ((T*)f.tap)[(size_t)row * f.tap_ld + f.tap_col + c] = from_f<T>(x);
  }
  if (!f.g) return;
  ss = block_sum(ss, red);
  int orow = row;
  if (f.compact_B) {
    const int j = row % f.compact_B;
    if (j == 0) return;
    orow = row - row / f.compact_B - 1;
  }
  const float rs = 1.0f / sqrtf(ss / (float)N + f.eps);
  const T* g = (const T*)f.g;
  T* u = (T*)f.u + (size_t)orow * N;
  for (int c = threadIdx.x; c < N; c += 256) u[c] = from_f<T>(xs[c] * rs * to_f(g[c]));
}

hipError_t launch_row_finalize(int dt, const RowFin& f, int rows, hipStream_t st) {
  const size_t sm = (size_t)f.N * sizeof(float);
  if (dt == BF16)
    hipLaunchKernelGGL(row_finalize_kernel<bf16>, dim3(rows), dim3(256), sm, st, f);
  else
    hipLaunchKernelGGL(row_finalize_kernel<float>, dim3(rows), dim3(256), sm, st, f);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void qkv_post_kernel(const float* __restrict__ C, int S,
                                                       size_t split_stride, int B, int Bp, int Hq,
                                                       int Hkv, int d, double base,
                                                       const int32_t* seq_len, T* q, T* kblk,
                                                       T* vblkT, KvLayer cache, int has_cache) {
  extern __shared__ float cs[];   // [d/2] cos then [d/2] sin
  const int row = blockIdx.x, b = row / B, j = row % B;
  const int half = d / 2;
  const int N = (Hq + 2 * Hkv) * d;
  const int pos = seq_len[b] + j;
  for (int i = threadIdx.x; i < half; i += 256) rope_cs(pos, i, d, base, &cs[i], &cs[half + i]);
  __syncthreads();
  const float* Cr = C + (size_t)row * N;
  auto val = [&](int col) {
    float x = 0.f;
    for (int s = 0; s < S; ++s) x += Cr[(size_t)s * split_stride + col];
    return x;
  };
  // cache slot of this row (target verification writes the block's K/V)
  bool cache_ok = false;
  size_t kbase = 0, vbase = 0;
  if (has_cache) {
    const int pg = pos >> 6;
    const int page = (pos >= 0 && pg < cache.max_pages) ? cache.block_table[(size_t)b * cache.max_pages + pg] : -1;
    cache_ok = page >= 0 && page < cache.num_pages;
    if (!cache_ok && threadIdx.x == 0) flag_error(cache.err, DEVERR_PAGE);
    kbase = (size_t)page * Hkv * 64 * d + (size_t)(pos & 63) * d;   // + h*64*d + c
    vbase = (size_t)page * Hkv * d * 64 + (size_t)(pos & 63);       // + (h*d + c)*64
  }
  // rotated q and k heads
  for (int idx = threadIdx.x; idx < (Hq + Hkv) * half; idx += 256) {
    const int hh = idx / half, i = idx % half;
    const int col = hh * d + i;
    const float x1 = val(col), x2 = val(col + half);
    const float c = cs[i], s = cs[half + i];
    const float y1 = x1 * c - x2 * s, y2 = x2 * c + x1 * s;
    if (hh < Hq) {
      T* dst = q + (size_t)row * Hq * d + (size_t)hh * d;
      dst[i] = from_f<T>(y1);
      dst[i + half] = from_f<T>(y2);
    } else {
      const int kh = hh - Hq;
      T* dst = kblk + (size_t)row * Hkv * d + (size_t)kh * d;
      dst[i] = from_f<T>(y1);
      dst[i + half] = from_f<T>(y2);
      if (cache_ok) {
        T* kc = (T*)cache.k + kbase + (size_t)kh * 64 * d;
        kc[i] = from_f<T>(y1);
        kc[i + half] = from_f<T>(y2);
      }
    }
  }
  // v heads, stored transposed per (sequence, head): vblkT[b][h][c][j]
  for (int idx = threadIdx.x; idx < Hkv * d; idx += 256) {
    const int vh = idx / d, c = idx % d;
    const float x = val((Hq + Hkv) * d + idx);
    vblkT[((size_t)(b * Hkv + vh) * d + c) * Bp + j] = from_f<T>(x);
    if (j == B - 1)
      for (int jj = B; jj < Bp; ++jj) vblkT[((size_t)(b * Hkv + vh) * d + c) * Bp + jj] = from_f<T>(0.f);
    if (cache_ok) ((T*)cache.v)[vbase + ((size_t)vh * d + c) * 64] = from_f<T>(x);
  }
}

hipError_t launch_qkv_post(int dt, const float* C, int S, size_t split_stride, int batch, int B,
                           int Bp, int Hq, int Hkv, int d, double rope_base,
                           const int32_t* seq_len, void* q, void* kblk, void* vblkT,
                           const KvLayer* cache, hipStream_t st) {
  KvLayer c{};
  if (cache) c = *cache;
  const size_t sm = (size_t)d * sizeof(float);
  if (dt == BF16)
    hipLaunchKernelGGL(qkv_post_kernel<bf16>, dim3(batch * B), dim3(256), sm, st, C, S,
                       split_stride, B, Bp, Hq, Hkv, d, rope_base, seq_len, (bf16*)q, (bf16*)kblk,
                       (bf16*)vblkT, c, cache ? 1 : 0);
  else
    hipLaunchKernelGGL(qkv_post_kernel<float>, dim3(batch * B), dim3(256), sm, st, C, S,
                       split_stride, B, Bp, Hq, Hkv, d, rope_base, seq_len, (float*)q,
                       (float*)kblk, (float*)vblkT, c, cache ? 1 : 0);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void swiglu_kernel(const float* __restrict__ C, int S,
                                                     size_t split_stride, int M, int F,
                                                     T* __restrict__ act) {
  const size_t n = (size_t)M * F;
  for (size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x; idx < n; idx += (size_t)gridDim.x * 256) {
    const size_t m = idx / F, jj = idx % F;
    float gt = 0.f, up = 0.f;
    for (int s = 0; s < S; ++s) {
      gt += C[(size_t)s * split_stride + m * 2 * F + jj];
      up += C[(size_t)s * split_stride + m * 2 * F + F + jj];
    }
    act[idx] = from_f<T>(gt / (1.f + expf(-gt)) * up);
  }
}

hipError_t launch_swiglu(int dt, const float* C, int S, size_t split_stride, int M, int F,
                         void* act, hipStream_t st) {
  const size_t n = (size_t)M * F;
  int grid = (int)((n + 255) / 256);
  if (grid > 8192) grid = 8192;
  if (dt == BF16)
    hipLaunchKernelGGL(swiglu_kernel<bf16>, dim3(grid), dim3(256), 0, st, C, S, split_stride, M, F,
                       (bf16*)act);
  else
    hipLaunchKernelGGL(swiglu_kernel<float>, dim3(grid), dim3(256), 0, st, C, S, split_stride, M,
                       F, (float*)act);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
struct InjArgs {
  const float* C2;
  int S;
  size_t split_stride;
  int L, Hkv, d;
  double base;
  const int32_t* row_seq;
  const int32_t* row_pos;
  int pos_relative;
  void* kp[8];
  void* vp[8];
  const int32_t* block_table;
  const int32_t* seq_len;
  int max_pages, num_pages, batch;
  int32_t* err;
};

template <typename T>
__global__ __launch_bounds__(256) void inject_scatter_kernel(InjArgs a) {
  extern __shared__ float cs[];
  const int row = blockIdx.x;
  const int d = a.d, half = d / 2;
  const int b = a.row_seq[row];
  bool ok = b >= 0 && b < a.batch;
  int pos = 0, page = -1;
  if (ok) {
    pos = a.row_pos[row] + (a.pos_relative ? a.seq_len[b] : 0);
    const int pg = pos >> 6;
    ok = pos >= 0 && pg < a.max_pages;
    if (ok) page = a.block_table[(size_t)b * a.max_pages + pg];
    ok = ok && page >= 0 && page < a.num_pages;
  }
  if (!ok) {
    if (threadIdx.x == 0) flag_error(a.err, DEVERR_PAGE);
    return;
  }
  for (int i = threadIdx.x; i < half; i += 256) rope_cs(pos, i, d, a.base, &cs[i], &cs[half + i]);
  __syncthreads();
  const int per_layer = 2 * a.Hkv * d;
  const float* Cr = a.C2 + (size_t)row * a.L * per_layer;
  auto val = [&](int col) {
    float x = 0.f;
    for (int s = 0; s < a.S; ++s) x += Cr[(size_t)s * a.split_stride + col];
    return x;
  };
  const int slot = pos & 63;
  for (int l = 0; l < a.L; ++l) {
    T* kpool = (T*)a.kp[l];
    T* vpool = (T*)a.vp[l];
    for (int idx = threadIdx.x; idx < a.Hkv * half; idx += 256) {
      const int h = idx / half, i = idx % half;
      const int col = l * per_layer + h * d + i;
      const float x1 = val(col), x2 = val(col + half);
      const float c = cs[i], s = cs[half + i];
      T* dst = kpool + (((size_t)page * a.Hkv + h) * 64 + slot) * d;
      dst[i] = from_f<T>(x1 * c - x2 * s);
      dst[i + half] = from_f<T>(x2 * c + x1 * s);
    }
    for (int idx = threadIdx.x; idx < a.Hkv * d; idx += 256) {
      const int h = idx / d, c = idx % d;
      const float x = val(l * per_layer + a.Hkv * d + idx);
      vpool[(((size_t)page * a.Hkv + h) * d + c) * 64 + slot] = from_f<T>(x);
    }
  }
}

hipError_t launch_inject_scatter(int dt, const float* C2, int S, size_t split_stride, int rows,
                                 int L, int Hkv, int d, double rope_base,
                                 const int32_t* row_seq, const int32_t* row_pos, int pos_relative,
                                 void* const* kpools, void* const* vpools,
                                 const int32_t* block_table, const int32_t* seq_len,
                                 int max_pages, int num_pages, int batch, int32_t* err,
                                 hipStream_t st) {
  InjArgs a;
  a.C2 = C2;
  a.S = S;
  a.split_stride = split_stride;
  a.L = L;
  a.Hkv = Hkv;
  a.d = d;
  a.base = rope_base;
  a.row_seq = row_seq;
  a.row_pos = row_pos;
  a.pos_relative = pos_relative;
  for (int i = 0; i < 8; ++i) {
    a.kp[i] = i < L ? kpools[i] : nullptr;
    a.vp[i] = i < L ? vpools[i] : nullptr;
  }
  a.block_table = block_table;
  a.seq_len = seq_len;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.batch = batch;
  a.err = err;
  const size_t sm = (size_t)d * sizeof(float);
  if (dt == BF16)
    hipLaunchKernelGGL(inject_scatter_kernel<bf16>, dim3(rows), dim3(256), sm, st, a);
  else
    hipLaunchKernelGGL(inject_scatter_kernel<float>, dim3(rows), dim3(256), sm, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
DF_DEV bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__global__ __launch_bounds__(256) void argmax_kernel(const float* __restrict__ logits, int V,
                                                     int32_t* ids) {
  const int row = blockIdx.x;
  const float* z = logits + (size_t)row * V;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int v = threadIdx.x; v < V; v += 256) {
    const float x = z[v];
    if (better(x, v, bv, bi)) {
      bv = x;
      bi = v;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  __shared__ float sv[4];
  __shared__ int si[4];
  if ((threadIdx.x & 63) == 0) {
    sv[threadIdx.x >> 6] = bv;
    si[threadIdx.x >> 6] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    bv = sv[0];
    bi = si[0];
    for (int w = 1; w < 4; ++w)
      if (better(sv[w], si[w], bv, bi)) {
        bv = sv[w];
        bi = si[w];
      }
    ids[row] = bi == 0x7fffffff ? 0 : bi;
  }
}

hipError_t launch_argmax(const float* logits, int rows, int V, int32_t* ids, hipStream_t st) {
  hipLaunchKernelGGL(argmax_kernel, dim3(rows), dim3(256), 0, st, logits, V, ids);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
__global__ void accept_kernel(const int32_t* block_ids, const int32_t* g, int batch, int B,
                              int32_t* tau, int32_t* bonus) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  int a = 0;
  while (a < B - 1 && block_ids[(size_t)b * B + a + 1] == g[(size_t)b * B + a]) ++a;
  tau[b] = a + 1;
  bonus[b] = g[(size_t)b * B + a];
}

hipError_t launch_accept(const int32_t* block_ids, const int32_t* g, int batch, int B,
                         int32_t* tau, int32_t* bonus, hipStream_t st) {
  hipLaunchKernelGGL(accept_kernel, dim3((batch + 63) / 64), dim3(64), 0, st, block_ids, g, batch,
                     B, tau, bonus);
  return hipGetLastError();
}

__global__ void commit_kernel(int32_t* seq_t, int32_t* seq_d, int32_t* err_t, int32_t* err_d,
                              const int32_t* tau, int batch, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  int t = tau[b];
  if (t < 1 || t > B) {
    flag_error(err_t, DEVERR_TAU);
    flag_error(err_d, DEVERR_TAU);
    t = t < 1 ? 1 : B;
  }
  if (seq_t) seq_t[b] += t;
  if (seq_d) seq_d[b] += t;
}

hipError_t launch_commit(int32_t* seq_t, int32_t* seq_d, int32_t* err_t, int32_t* err_d,
                         const int32_t* tau, int batch, int B, hipStream_t st) {
  hipLaunchKernelGGL(commit_kernel, dim3((batch + 63) / 64), dim3(64), 0, st, seq_t, seq_d, err_t,
                     err_d, tau, batch, B);
  return hipGetLastError();
}

}  // namespace dflash
