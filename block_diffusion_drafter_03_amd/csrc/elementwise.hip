// Row kernels of the drafter / verifier step that are not GEMM epilogues: the block
// embedding, argmax decoding, greedy acceptance and the commit of sequence lengths.
#include "epilogue.h"

namespace dflash {

// ---------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs a) {
  const int B = a.B, D = a.D;
  const int row = blockIdx.x, b = row / B, j = row % B;
  // mode 0: [anchor, mask ...]; mode 1: [anchor, drafts ...] with ids = drafts [batch, B-1]
  int tok = j == 0 ? a.anchor[b] : (a.mode == 0 ? a.mask_id : a.ids[(size_t)b * (B - 1) + j - 1]);
  if (tok < 0 || tok >= a.V) {
    if (threadIdx.x == 0) flag_error(a.err, DEVERR_TOKEN);
    tok = 0;
  }
  const T* e = (const T*)a.E + (size_t)tok * D;
  bool done = false;
  if constexpr (sizeof(T) == 2) {
    if (a.afrag && D % 8 == 0) {
      // bf16 rows into the A-fragment order: 8 channels per thread, one 16-byte load and
      // two float4 stores (channels 8q .. 8q+3 and 8q+4 .. 8q+7 are contiguous in the two
      // halves of their fragment)
      for (int c = threadIdx.x * 8; c < D; c += 256 * 8) {
        const bf16x8 v = *(const bf16x8*)(e + c);
        const float4 lo = make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
        const float4 hi = make_float4((float)v[4], (float)v[5], (float)v[6], (float)v[7]);
        *(float4*)(a.h + afrag_off(row, c, D >> 5)) = lo;
        *(float4*)(a.h + afrag_off(row, c + 4, D >> 5)) = hi;
        if (a.hdbg) {
          *(float4*)(a.hdbg + (size_t)row * D + c) = lo;
          *(float4*)(a.hdbg + (size_t)row * D + c + 4) = hi;
        }
      }
      done = true;
    }
  }
  if (!done) {
    for (int c = threadIdx.x; c < D; c += 256) {
      const float x = to_f(e[c]);
      a.h[a.afrag ? afrag_off(row, c, D >> 5) : (size_t)row * D + c] = x;
      if (a.hdbg) a.hdbg[(size_t)row * D + c] = x;
    }
  }
  // RoPE angles of this row's position (float64, rounded to float32)
  const int pos = a.seq_len[b] + j;
  for (int i = threadIdx.x; i < a.hd / 2; i += 256) {
    float c, s;
    rope_cs(pos, i, a.hd, a.rope_base, &c, &s);
    a.rope[(size_t)row * (a.hd / 2) + i] = make_float2(c, s);
  }
  // arm this call's argmax keys and arrival counters
  if (row == 0) {
    for (int i = threadIdx.x; i < a.n_keys; i += 256) a.keys[i] = 0ull;
    for (int i = threadIdx.x; i < a.n_zero; i += 256) a.zero[i] = 0u;
  }
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
template <bool NT>
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* src, size_t n16, u32x4* sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    acc ^= NT ? __builtin_nontemporal_load(src + i) : src[i];
  __shared__ u32x4 red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    u32x4 x = red[0];
    for (int t = 1; t < 256; ++t) x ^= red[t];
    sink[blockIdx.x] = x;
  }
}

hipError_t launch_probe_read(const void* src, size_t n16, int nontemporal, void* sink, hipStream_t st) {
  if (nontemporal)
    hipLaunchKernelGGL(probe_read_kernel<true>, dim3(1024), dim3(256), 0, st, (const u32x4*)src, n16, (u32x4*)sink);
  else
    hipLaunchKernelGGL(probe_read_kernel<false>, dim3(1024), dim3(256), 0, st, (const u32x4*)src, n16, (u32x4*)sink);
  return hipGetLastError();
}

hipError_t launch_embed(int dt, const EmbedArgs& a, hipStream_t st) {
  const int rows = a.batch * a.B;
  if (dt == BF16)
    hipLaunchKernelGGL(embed_kernel<bf16>, dim3(rows), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(64) void rope_rows_kernel(const int32_t* row_seq, const int32_t* row_pos,
                                                       int pos_relative, const int32_t* seq_len,
                                                       int batch, int hd, double base, float2* rope) {
  const int row = blockIdx.x;
  const int b = row_seq[row];
  const int pos = row_pos[row] + ((pos_relative && b >= 0 && b < batch) ? seq_len[b] : 0);
  for (int i = threadIdx.x; i < hd / 2; i += 64) {
    float c, s;
    rope_cs(pos, i, hd, base, &c, &s);
    rope[(size_t)row * (hd / 2) + i] = make_float2(c, s);
  }
}

hipError_t launch_rope_rows(const int32_t* row_seq, const int32_t* row_pos, int pos_relative,
                            const int32_t* seq_len, int batch, int rows, int hd, double base,
                            float2* rope, hipStream_t st) {
  hipLaunchKernelGGL(rope_rows_kernel, dim3(rows), dim3(64), 0, st, row_seq, row_pos, pos_relative,
                     seq_len, batch, hd, base, rope);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------

// draft ids of the masked rows j = 1 .. B-1 of every block (the anchor rows' argmax is unused)
__global__ void unpack_ids_kernel(const unsigned long long* keys, int n, int B, int32_t* ids) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) ids[i] = unpack_argmax_idx(keys[(i / (B - 1)) * B + i % (B - 1) + 1]);
}

hipError_t launch_unpack_ids(const unsigned long long* keys, int batch, int B, int32_t* ids,
                             hipStream_t st) {
  const int n = batch * (B - 1);
  hipLaunchKernelGGL(unpack_ids_kernel, dim3((n + 255) / 256), dim3(256), 0, st, keys, n, B, ids);
  return hipGetLastError();
}

// Greedy acceptance, one wavefront per sequence (B <= 64): lane j decodes g_j, the target's
// argmax after row j, from its packed key; lane j >= 1 compares draft d_j with g_{j-1} (its
// neighbour's id); a ballot of the mismatches gives the leading run of matches a by a bit
// scan; tau = a + 1 and bonus = g_a.
__global__ __launch_bounds__(64) void accept_kernel(const unsigned long long* keys, const int32_t* drafts,
                                                    int B, int32_t* g, int32_t* tau, int32_t* bonus) {
  accept_wave<false>(keys, drafts, B, blockIdx.x, g, tau, bonus);
}

hipError_t launch_accept(const unsigned long long* keys, const int32_t* drafts, int batch, int B,
                         int32_t* g, int32_t* tau, int32_t* bonus, hipStream_t st) {
  if (B < 1 || B > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(accept_kernel, dim3(batch), dim3(64), 0, st, keys, drafts, B, g, tau, bonus);
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

// ---------------------------------------------------------------------------------------
// Sampling verification ([DF] section 6.2 and the DFlash 2 notes, section 7.2: lossless
// rejection sampling at temperature T; the standard speculative-sampling rule).

namespace dflash {

// Four launches, each spread over the vocabulary so that a row's V logits are scanned by
// many workgroups at once:
//  1. lse_partial: (max, sum exp(z/T - max)) of every chunk of every target and drafter row;
//  2. accept_decide: one workgroup per sequence folds the chunk partials into each row's
//     log-sum-exp, then decides the accepted prefix a and writes tau = a + 1;
//  3. sample_chunk: the Gumbel-max key of each chunk of the row the emitted token comes from;
//  4. sample_finish: the largest chunk key of each sequence gives the emitted token.
// The reduction order is fixed by the chunking, so results do not depend on timing.
#define SAMPLE_THREADS 256

int sample_chunks(int V) { return std::min(SAMPLE_MAX_CHUNKS, std::max(1, (V + 4095) / 4096)); }

// grid (rows, chunks): rows 0 .. nt-1 are the target's, the rest the drafter's
__global__ __launch_bounds__(SAMPLE_THREADS) void lse_partial_kernel(const float* zt, const float* zd,
                                                                     int nt, int V, int clen,
                                                                     float inv_t, float2* part) {
  __shared__ float red[SAMPLE_THREADS / 64];
  const int row = blockIdx.x, c = blockIdx.y;
  const float* z = row < nt ? zt + (size_t)row * V : zd + (size_t)(row - nt) * V;
  const int v0 = c * clen, v1 = min(V, v0 + clen);
  float m = -INFINITY;
  for (int v = v0 + threadIdx.x; v < v1; v += 4 * SAMPLE_THREADS) {
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = z[min(v + u * SAMPLE_THREADS, v1 - 1)];   // v1 > v here
#pragma unroll
    for (int u = 0; u < 4; ++u) m = fmaxf(m, x[u] * inv_t);
  }
  m = wave_max(m);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float s = 0.f;
  if (m > -INFINITY) {   // an empty chunk keeps (-inf, 0)
    for (int v = v0 + threadIdx.x; v < v1; v += 4 * SAMPLE_THREADS) {
      float x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = z[min(v + u * SAMPLE_THREADS, v1 - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (v + u * SAMPLE_THREADS < v1) s += expf(x[u] * inv_t - m);
    }
  }
  s = block_sum(s, red);
  if (threadIdx.x == 0) part[(size_t)row * gridDim.y + c] = make_float2(m, s);
}

// one wave: lse of a row from its nch (<= 64) chunk partials
DF_DEV float fold_lse(const float2* p, int nch) {
  const int l = threadIdx.x & 63;
  const float2 q = l < nch ? p[l] : make_float2(-INFINITY, 0.f);
  const float m = wave_max(q.x);
  const float s = wave_sum(q.x > -INFINITY ? q.y * expf(q.x - m) : 0.f);
  return m + logf(s);
}

// grid (batch), 1024 threads.  Draft d_i (i = 1 .. B-1) is judged by target row i-1: accepted
// while u_i < p_{i-1}(d_i) / q_i(d_i), u_i the uniform of draw (counter, 1, b, i, 0);
// a = the accepted prefix, tau = a + 1.  lse: target rows [batch * B] then drafter rows
// [batch * (B-1)].
__global__ __launch_bounds__(1024) void accept_decide_kernel(
    const float* zt, const float* zd, const float2* part, int nch, const int32_t* drafts, int B,
    int V, float inv_t, unsigned long long seed, unsigned counter, float* lse, int32_t* acc,
    int32_t* tau, int32_t* err) {
  __shared__ float lt_s[64], ld_s[64];
  const int b = blockIdx.x, batch = gridDim.x, w = threadIdx.x >> 6, l = threadIdx.x & 63;
  for (int r = w; r < 2 * B - 1; r += 16) {
    const int row = r < B ? b * B + r : batch * B + b * (B - 1) + (r - B);
    const float v = fold_lse(part + (size_t)row * nch, nch);
    if (l == 0) {
      lse[row] = v;
      if (r < B) lt_s[r] = v; else ld_s[r - B] = v;
    }
  }
  __syncthreads();
  if (w == 0) {
    bool reject = false;
    if (l >= 1 && l < B) {
      const int d = drafts[(size_t)b * (B - 1) + l - 1];
      if (d < 0 || d >= V) {   // not a token: rejected, and reported
        flag_error(err, DEVERR_TOKEN);
        reject = true;
      } else {
        const float lp = zt[((size_t)b * B + l - 1) * V + d] * inv_t - lt_s[l - 1];
        const float lq = zd[((size_t)b * (B - 1) + l - 1) * V + d] * inv_t - ld_s[l - 1];
        reject = !(rng_uniform(seed, counter, 1, b, l, 0) < expf(lp - lq));
      }
    }
    const unsigned long long rej = __ballot(reject);
    if (l == 0) {
      const int a = rej ? __builtin_ctzll(rej) - 1 : B - 1;
      acc[b] = a;
      tau[b] = a + 1;
    }
  }
}

// grid (batch, chunks): the emitted token is the argmax over v of key(v) + Gumbel noise of
// draw (counter, 2, b, a, v), key = log max(0, p_a - q_{a+1}) after a rejection (the
// residual distribution; its normaliser does not move the argmax), else log p_{B-1}.
__global__ __launch_bounds__(SAMPLE_THREADS) void sample_chunk_kernel(
    const float* zt, const float* zd, const float* lse, const int32_t* acc, int B, int V, int clen,
    float inv_t, unsigned long long seed, unsigned counter, unsigned long long* keys) {
  __shared__ unsigned long long best_s[SAMPLE_THREADS / 64];
  const int b = blockIdx.x, c = blockIdx.y, batch = gridDim.x;
  const int a = acc[b];
  const bool resid = a < B - 1;
  const float* pt = zt + ((size_t)b * B + a) * V;
  const float lt = lse[b * B + a];
  const float* pd = zd + ((size_t)b * (B - 1) + (resid ? a : 0)) * V;
  const float ld = resid ? lse[batch * B + b * (B - 1) + a] : 0.f;
  const int v0 = c * clen, v1 = min(V, v0 + clen);
  unsigned long long best = 0ull;
  for (int v = v0 + threadIdx.x; v < v1; v += 4 * SAMPLE_THREADS) {
    float xt[4], xd[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int vv = min(v + u * SAMPLE_THREADS, v1 - 1);
      xt[u] = pt[vv];
      xd[u] = resid ? pd[vv] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int vv = v + u * SAMPLE_THREADS;
      if (vv >= v1) continue;
      float key;
      if (resid) {
        const float r = expf(xt[u] * inv_t - lt) - expf(xd[u] * inv_t - ld);
        key = r > 0.f ? logf(r) : -INFINITY;
      } else {
        key = xt[u] * inv_t - lt;
      }
      if (key > -INFINITY) {
        const unsigned long long k = pack_argmax_key(key + gumbel_noise(seed, counter, 2, b, a, vv), vv);
        best = k > best ? k : best;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned lo = __shfl_xor((unsigned)(best & 0xFFFFFFFFull), o, 64);
    const unsigned hi = __shfl_xor((unsigned)(best >> 32), o, 64);
    const unsigned long long k = ((unsigned long long)hi << 32) | lo;
    best = k > best ? k : best;
  }
  if ((threadIdx.x & 63) == 0) best_s[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long k = best_s[0];
    for (int w = 1; w < SAMPLE_THREADS / 64; ++w) k = best_s[w] > k ? best_s[w] : k;
    keys[(size_t)b * gridDim.y + c] = k;
  }
}

// grid (batch), one wave: largest chunk key (ties in value go to the lowest id, as packed)
__global__ __launch_bounds__(64) void sample_finish_kernel(const unsigned long long* keys, int nch,
                                                           int32_t* next_token) {
  const int b = blockIdx.x, l = threadIdx.x;
  unsigned long long best = l < nch ? keys[(size_t)b * nch + l] : 0ull;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned lo = __shfl_xor((unsigned)(best & 0xFFFFFFFFull), o, 64);
    const unsigned hi = __shfl_xor((unsigned)(best >> 32), o, 64);
    const unsigned long long k = ((unsigned long long)hi << 32) | lo;
    best = k > best ? k : best;
  }
  if (l == 0) next_token[b] = best ? unpack_argmax_idx(best) : 0;
}

hipError_t launch_verify_sampled(const float* zt, const float* zd, const int32_t* drafts, int batch,
                                 int B, int V, float temperature, unsigned long long seed,
                                 unsigned counter, const SampleWs& ws, int32_t* tau,
                                 int32_t* next_token, int32_t* err, hipStream_t st) {
  if (batch <= 0) return hipSuccess;
  if (B < 2 || B > 64 || V < 1) return hipErrorInvalidValue;
  const int nch = sample_chunks(V), clen = (V + nch - 1) / nch;
  const float inv_t = 1.f / temperature;
  const int rows = batch * B + batch * (B - 1);
  hipLaunchKernelGGL(lse_partial_kernel, dim3(rows, nch), dim3(SAMPLE_THREADS), 0, st, zt, zd,
                     batch * B, V, clen, inv_t, ws.part);
  hipLaunchKernelGGL(accept_decide_kernel, dim3(batch), dim3(1024), 0, st, zt, zd,
                     (const float2*)ws.part, nch, drafts, B, V, inv_t, seed, counter, ws.lse,
                     ws.acc, tau, err);
  hipLaunchKernelGGL(sample_chunk_kernel, dim3(batch, nch), dim3(SAMPLE_THREADS), 0, st, zt, zd,
                     (const float*)ws.lse, (const int32_t*)ws.acc, B, V, clen, inv_t, seed, counter,
                     ws.keys);
  hipLaunchKernelGGL(sample_finish_kernel, dim3(batch), dim3(64), 0, st,
                     (const unsigned long long*)ws.keys, nch, next_token);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// DFlash 2 two-tap dynamic convolution ([DF] section 7.1, Problem 2): grid (rows, D / 256),
// one channel per thread; with the norm each workgroup first sums the squares of its row
// and of the row it reads (16 loads per thread in flight at once).
#define DCONV_CH 256
__global__ __launch_bounds__(DCONV_CH) void dconv_kernel(DconvArgs a) {
  __shared__ float red[8];
  const int r = blockIdx.x, D = a.D, j = r % a.B;
  const int p = j == 0 ? r : r - 1;
  auto at = [&](int row, int c) -> size_t {
    return a.afrag ? afrag_off(row, c, D >> 5) : (size_t)row * D + c;
  };
  float sr = 1.f, sp = 1.f;
  if (a.norm_g) {
    float s0 = 0.f, s1 = 0.f;
    for (int c0 = threadIdx.x; c0 < D; c0 += DCONV_CH * 8) {
      float x0[8], x1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = min(c0 + u * DCONV_CH, D - 1);
        x0[u] = a.x[at(r, c)];
        x1[u] = a.x[at(p, c)];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (c0 + u * DCONV_CH < D) {
          s0 += x0[u] * x0[u];
          s1 += x1[u] * x1[u];
        }
    }
    s0 = block_sum(s0, red);
    s1 = block_sum(s1, red + 4);
    sr = 1.0f / sqrtf(s0 / (float)D + a.eps);
    sp = 1.0f / sqrtf(s1 / (float)D + a.eps);
  }
  const int c = blockIdx.y * DCONV_CH + threadIdx.x;
  if (c >= D) return;
  float xr = a.x[at(r, c)] * sr, xp = a.x[at(p, c)] * sp;
  float b0, b1;
  if (a.bf16) {
    b0 = (float)((const bf16*)a.base)[c];
    b1 = (float)((const bf16*)a.base)[D + c];
    if (a.norm_g) {
      const float g = (float)((const bf16*)a.norm_g)[c];
      xr *= g;
      xp *= g;
    }
  } else {
    b0 = ((const float*)a.base)[c];
    b1 = ((const float*)a.base)[D + c];
    if (a.norm_g) {
      const float g = ((const float*)a.norm_g)[c];
      xr *= g;
      xp *= g;
    }
  }
  const float* cr = a.corr + (size_t)r * (D >> 3) + 2 * (c >> 4);
  const float y = (b0 + cr[0]) * xr + (b1 + cr[1]) * xp;
  const size_t o = at(r, c);
  const float v = a.accumulate ? a.out[o] + y : y;
  a.out[o] = v;
  if (a.hdbg) a.hdbg[(size_t)r * D + c] = v;
}

hipError_t launch_dconv(const DconvArgs& a, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  if (a.D % 16 || a.B < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dconv_kernel, dim3(a.M, (a.D + DCONV_CH - 1) / DCONV_CH), dim3(DCONV_CH), 0, st, a);
  return hipGetLastError();
}

}  // namespace dflash
