// Block attention over [injected / cached context ; block] for the drafter (bidirectional
// inside the block) and for the target's verification pass (causal inside the block).
//
// bf16 path (head_dim 128): one workgroup per (sequence, KV head, 64-row query group,
// key split).  The G*B query rows that share a KV head are kept in registers as MFMA
// operands, so every context K/V byte is read from HBM once.  Each of the 4 waves walks
// 32-key chunks of its split with its own online softmax; S^T = K Q^T and O^T = V^T P^T
// run on v_mfma_f32_16x16x32_bf16:
//   * the K rows of the two 16-key S^T tiles of a chunk are interleaved so that lane
//     group g ends up holding keys 8g .. 8g+7 of the chunk for its query column - exactly
//     the P^T operand layout of the PV product, with no data movement;
//   * V pages are stored transposed ([d][64 keys]) so the V^T operand is a plain 16-byte
//     load per lane.
// The 4 waves' states are merged in LDS (fixed order) and the workgroup writes one
// partial (m, l, O); a second kernel merges the splits with log-sum-exp weights.
// Scores are kept in the log2 domain (scaled by log2(e)/sqrt(d)) and exponentiated with
// exp2.
#include "common.h"
#include "kernels.h"

namespace dflash {

#define AD 128      // head dim of the MFMA path
#define ACHUNK 32   // keys per wave step

struct AttnArgs {
  const bf16* q;       // [batch*B, Hq*AD]
  const bf16* kblk;    // [batch*B, Hkv*AD]
  const bf16* vblkT;   // [batch, Hkv, AD, Bp]
  const bf16* kpool;   // [num_pages, Hkv, 64, AD]
  const bf16* vpool;   // [num_pages, Hkv, AD, 64]
  const int32_t* block_table;
  const int32_t* seq_len;
  int32_t* err;
  int max_pages, num_pages;
  int B, Bp, Hq, Hkv, G;
  int n_ctx_splits, split_len, n_rg, causal;
  float scale_log2;
  float* part;         // [(b, kvh, rg, s)][64][AD + 2]  (O then m, l per row)
};

__global__ __launch_bounds__(256) void attn_splitk_bf16(AttnArgs a) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int s = blockIdx.x;
  const int kvh = blockIdx.y % a.Hkv, rg = blockIdx.y / a.Hkv;
  const int b = blockIdx.z;
  const int R = a.G * a.B;
  const int S_total = a.n_ctx_splits + 1;
  const bool is_block = (s == a.n_ctx_splits);

  int n_ctx = a.seq_len[b];
  n_ctx = max(0, min(n_ctx, a.max_pages * 64));
  int kbeg, kend;
  if (is_block) {
    kbeg = 0;
    kend = a.B;
  } else {
    kbeg = s * a.split_len;
    kend = min(kbeg + a.split_len, n_ctx);
  }

  // Q^T operand fragments for the 4 query tiles of this row group.
  bf16x8 qf[4][4];
  int jrow[4];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    const int rho = rg * 64 + qt * 16 + r;
    jrow[qt] = rho < R ? rho % a.B : 0x7fffffff;
    if (rho < R) {
      const int gq = rho / a.B, j = rho % a.B;
      const bf16* src = a.q + (size_t)(b * a.B + j) * a.Hq * AD + (size_t)(kvh * a.G + gq) * AD + g * 8;
#pragma unroll
      for (int cs = 0; cs < 4; ++cs) qf[qt][cs] = *(const bf16x8*)(src + cs * 32);
    } else {
#pragma unroll
      for (int cs = 0; cs < 4; ++cs)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[qt][cs][e] = (bf16)0.f;
    }
  }

  float m[4], lsum[4];
  f32x4 o[8][4];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    m[qt] = -INFINITY;
    lsum[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // key row that this lane feeds into S^T tile t (interleaved so P^T needs no shuffle)
  const int krow0 = 8 * (r >> 2) + (r & 3);

  for (int c0 = kbeg + w * ACHUNK; c0 < kend; c0 += 4 * ACHUNK) {
    const bf16* kp0;
    const bf16* kp1;
    const bf16* vp;
    if (is_block) {
      const int j0 = min(c0 + krow0, a.B - 1), j1 = min(c0 + krow0 + 4, a.B - 1);
      kp0 = a.kblk + (size_t)(b * a.B + j0) * a.Hkv * AD + (size_t)kvh * AD + g * 8;
      kp1 = a.kblk + (size_t)(b * a.B + j1) * a.Hkv * AD + (size_t)kvh * AD + g * 8;
      vp = a.vblkT + ((size_t)(b * a.Hkv + kvh) * AD + r) * a.Bp + c0 + g * 8;
    } else {
      const int page = a.block_table[(size_t)b * a.max_pages + (c0 >> 6)];
      if (page < 0 || page >= a.num_pages) {
        if (lane == 0) flag_error(a.err, DEVERR_PAGE);
        continue;
      }
      const int off = c0 & 63;
      const size_t pb = (size_t)page * a.Hkv + kvh;
      kp0 = a.kpool + (pb * 64 + off + krow0) * AD + g * 8;
      kp1 = kp0 + 4 * AD;
      vp = a.vpool + (pb * AD + r) * 64 + off + g * 8;
    }
    bf16x8 kf0[4], kf1[4], vf[8];
#pragma unroll
    for (int cs = 0; cs < 4; ++cs) {
      kf0[cs] = *(const bf16x8*)(kp0 + cs * 32);
      kf1[cs] = *(const bf16x8*)(kp1 + cs * 32);
    }
    const int vstride = is_block ? 16 * a.Bp : 16 * 64;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) vf[dt] = *(const bf16x8*)(vp + (size_t)dt * vstride);
    // keys past the end of the range: zero V so stale or uninitialised page bytes
    // cannot leak NaN through a zero probability
    const int vkey = c0 + g * 8;
    if (vkey + 8 > kend) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (vkey + e >= kend) vf[dt][e] = (bf16)0.f;
    }

#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cs = 0; cs < 4; ++cs) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf0[cs], qf[qt][cs], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf1[cs], qf[qt][cs], s1, 0, 0, 0);
      }
      // this lane: keys c0 + 8g + i (s0) and c0 + 8g + 4 + i (s1), query column r
      float sc[8];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k0 = c0 + g * 8 + i, k1 = k0 + 4;
        bool v0 = k0 < kend, v1 = k1 < kend;
        if (is_block && a.causal) {
          v0 = v0 && (k0 <= jrow[qt]);
          v1 = v1 && (k1 <= jrow[qt]);
        }
        sc[i] = v0 ? s0[i] * a.scale_log2 : -INFINITY;
        sc[4 + i] = v1 ? s1[i] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, fmaxf(sc[i], sc[4 + i]));
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(m[qt], mx);
      float alpha, ps = 0.f;
      bf16x8 pf;
      if (mnew == -INFINITY) {
        alpha = 1.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = (bf16)0.f;
      } else {
        alpha = exp2f(m[qt] - mnew);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = exp2f(sc[e] - mnew);
          ps += p;
          pf[e] = (bf16)p;
        }
      }
      m[qt] = mnew;
      lsum[qt] = lsum[qt] * alpha + ps;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        o[dt][qt] *= alpha;
        o[dt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pf, o[dt][qt], 0, 0, 0);
      }
    }
  }

  // ---- merge the 4 waves (fixed order) ----
  __shared__ float sm_m[4][64], sm_l[4][64];
  __shared__ float sm_o[64][AD + 4];
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    const float lt = lsum[qt] + __shfl_xor(lsum[qt], 16, 64);
    lsum[qt] = lt + __shfl_xor(lt, 32, 64);
    if (g == 0) {
      sm_m[w][qt * 16 + r] = m[qt];
      sm_l[w][qt * 16 + r] = lsum[qt];
    }
  }
  __syncthreads();
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    const int q = qt * 16 + r;
    const float ms = fmaxf(fmaxf(sm_m[0][q], sm_m[1][q]), fmaxf(sm_m[2][q], sm_m[3][q]));
    const float sc = (m[qt] == -INFINITY) ? 0.f : exp2f(m[qt] - ms);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt][qt] *= sc;
  }
  for (int ww = 0; ww < 4; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          float* dst = &sm_o[qt * 16 + r][dt * 16 + g * 4];
          if (ww == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[e] = o[dt][qt][e];
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[e] += o[dt][qt][e];
          }
        }
    }
    __syncthreads();
  }
  float* dst = a.part + ((((size_t)b * a.Hkv + kvh) * a.n_rg + rg) * S_total + s) * 64 * (AD + 2);
  for (int idx = threadIdx.x; idx < 64 * AD; idx += 256) {
    const int q = idx / AD, d = idx % AD;
    dst[q * (AD + 2) + d] = sm_o[q][d];
  }
  if (threadIdx.x < 64) {
    const int q = threadIdx.x;
    const float ms = fmaxf(fmaxf(sm_m[0][q], sm_m[1][q]), fmaxf(sm_m[2][q], sm_m[3][q]));
    float lt = 0.f;
    for (int ww = 0; ww < 4; ++ww)
      if (sm_m[ww][q] != -INFINITY) lt += sm_l[ww][q] * exp2f(sm_m[ww][q] - ms);
    dst[q * (AD + 2) + AD] = ms;
    dst[q * (AD + 2) + AD + 1] = lt;
  }
}

// Merge the key splits of every query row: O = sum_s O_s 2^(m_s - m*) / sum_s l_s 2^(m_s - m*).
template <typename T>
__global__ __launch_bounds__(AD) void attn_merge(const float* __restrict__ part, int S_total,
                                                 int n_rg, int B, int Hq, int Hkv, int G,
                                                 T* __restrict__ out) {
  const int rho = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int R = G * B;
  if (rho >= R) return;
  const int rg = rho / 64, q = rho % 64;
  const float* base = part + (((size_t)b * Hkv + kvh) * n_rg + rg) * S_total * 64 * (AD + 2) +
                      (size_t)q * (AD + 2);
  const size_t sstride = 64 * (AD + 2);
  float ms = -INFINITY;
  for (int s = 0; s < S_total; ++s) ms = fmaxf(ms, base[s * sstride + AD]);
  float lt = 0.f, acc = 0.f;
  const int d = threadIdx.x;
  for (int s = 0; s < S_total; ++s) {
    const float mv = base[s * sstride + AD];
    if (mv == -INFINITY) continue;
    const float wgt = exp2f(mv - ms);
    lt += base[s * sstride + AD + 1] * wgt;
    acc += base[s * sstride + d] * wgt;
  }
  const int gq = rho / B, j = rho % B;
  out[(size_t)(b * B + j) * Hq * AD + (size_t)(kvh * G + gq) * AD + d] = from_f<T>(acc / lt);
}

// ---------------------------------------------------------------------------------------
// float32 path: one workgroup per (sequence, block row, query head), keys in chunks of
// 256 with an online softmax; plain VALU.
struct AttnF32Args {
  const float* q;
  const float* kblk;
  const float* vblkT;
  const float* kpool;
  const float* vpool;
  const int32_t* block_table;
  const int32_t* seq_len;
  int32_t* err;
  int max_pages, num_pages;
  int B, Bp, Hq, Hkv, G, d, causal;
  float scale;
  float* out;
};

__global__ __launch_bounds__(256) void attn_f32(AttnF32Args a) {
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / a.G, d = a.d;
  extern __shared__ float smem[];
  float* qs = smem;            // [d]
  float* ps = smem + d;        // [256]
  __shared__ float red[16];
  __shared__ int pages[4];
  const int tid = threadIdx.x;
  for (int c = tid; c < d; c += 256) qs[c] = a.q[(size_t)(b * a.B + j) * a.Hq * d + (size_t)h * d + c];
  int n_ctx = max(0, min(a.seq_len[b], a.max_pages * 64));
  const int nblk = a.causal ? j + 1 : a.B;
  const int total = n_ctx + nblk;
  float m = -INFINITY, l = 0.f;
  float acc0 = 0.f, acc1 = 0.f;   // output columns tid and tid + 256 (d <= 512)
  __syncthreads();
  for (int k0 = 0; k0 < total; k0 += 256) {
    const int kk = k0 + tid;
    float sc = -INFINITY;
    if (kk < total) {
      const float* kr;
      bool ok = true;
      if (kk < n_ctx) {
        const int page = a.block_table[(size_t)b * a.max_pages + (kk >> 6)];
        ok = page >= 0 && page < a.num_pages;
        if (!ok) flag_error(a.err, DEVERR_PAGE);
        kr = a.kpool + (((size_t)page * a.Hkv + kvh) * 64 + (kk & 63)) * d;
      } else {
        kr = a.kblk + (size_t)(b * a.B + (kk - n_ctx)) * a.Hkv * d + (size_t)kvh * d;
      }
      if (ok) {
        float t = 0.f;
        for (int c = 0; c < d; ++c) t = fmaf(qs[c], kr[c], t);
        sc = t * a.scale;
      }
    }
    // chunk max
    float mx = wave_max(sc);
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float mnew = fmaxf(m, mx);
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - mnew);
    const float p = (sc == -INFINITY) ? 0.f : expf(sc - mnew);
    ps[tid] = p;
    const float psum = block_sum(p, red + 4);
    l = l * alpha + psum;
    m = mnew;
    __syncthreads();
    const int nk = min(256, total - k0);
    for (int cc = 0; cc < 2; ++cc) {
      const int c = tid + cc * 256;
      if (c >= d) break;
      float t = 0.f;
      for (int e = 0; e < nk; ++e) {
        const int kk2 = k0 + e;
        const float pe = ps[e];
        if (pe == 0.f) continue;
        float v;
        if (kk2 < n_ctx) {
          const int page = a.block_table[(size_t)b * a.max_pages + (kk2 >> 6)];
          v = a.vpool[(((size_t)page * a.Hkv + kvh) * d + c) * 64 + (kk2 & 63)];
        } else {
          v = a.vblkT[((size_t)(b * a.Hkv + kvh) * d + c) * a.Bp + (kk2 - n_ctx)];
        }
        t = fmaf(pe, v, t);
      }
      if (cc == 0) acc0 = acc0 * alpha + t;
      else acc1 = acc1 * alpha + t;
    }
    __syncthreads();
  }
  float* o = a.out + (size_t)(b * a.B + j) * a.Hq * d + (size_t)h * d;
  if (tid < d) o[tid] = acc0 / l;
  if (tid + 256 < d) o[tid + 256] = acc1 / l;
}

// ---------------------------------------------------------------------------------------
AttnPlan attn_plan(int dt, int batch, int Hkv, int G, int B, int ctx_cap) {
  AttnPlan p;
  p.n_rg = (G * B + 63) / 64;
  if (dt != BF16) {
    p.n_ctx_splits = 0;
    p.split_len = 0;
    return p;
  }
  const int cap = ctx_cap > 0 ? ctx_cap : 1;
  const int units = batch * Hkv * p.n_rg;
  int want = (512 + units - 1) / units;                       // ~2 workgroups per CU
  const int max_splits = (cap + 127) / 128;
  if (want > max_splits) want = max_splits;
  if (want < 1) want = 1;
  int len = (cap + want - 1) / want;
  len = (len + 127) / 128 * 128;
  p.split_len = len;
  p.n_ctx_splits = (cap + len - 1) / len;
  return p;
}

size_t attn_partial_floats(const AttnPlan& p, int batch, int Hkv, int d) {
  return (size_t)batch * Hkv * p.n_rg * (p.n_ctx_splits + 1) * 64 * (d + 2);
}

hipError_t launch_attention(int dt, const AttnPlan& p, const void* q, const void* kblk,
                            const void* vblkT, const KvLayer& kv, int batch, int B, int Bp,
                            int Hq, int Hkv, int d, int causal, float* part, void* o,
                            hipStream_t st) {
  const int G = Hq / Hkv;
  if (dt == BF16) {
    AttnArgs a;
    a.q = (const bf16*)q;
    a.kblk = (const bf16*)kblk;
    a.vblkT = (const bf16*)vblkT;
    a.kpool = (const bf16*)kv.k;
    a.vpool = (const bf16*)kv.v;
    a.block_table = kv.block_table;
    a.seq_len = kv.seq_len;
    a.err = kv.err;
    a.max_pages = kv.max_pages;
    a.num_pages = kv.num_pages;
    a.B = B;
    a.Bp = Bp;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = G;
    a.n_ctx_splits = p.n_ctx_splits;
    a.split_len = p.split_len;
    a.n_rg = p.n_rg;
    a.causal = causal;
    a.scale_log2 = 1.4426950408889634f / sqrtf((float)d);
    a.part = part;
    dim3 grid(p.n_ctx_splits + 1, Hkv * p.n_rg, batch);
    hipLaunchKernelGGL(attn_splitk_bf16, grid, dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 g2(p.n_rg * 64, Hkv, batch);
    hipLaunchKernelGGL(attn_merge<bf16>, g2, dim3(AD), 0, st, (const float*)part,
                       p.n_ctx_splits + 1, p.n_rg, B, Hq, Hkv, G, (bf16*)o);
    return hipGetLastError();
  }
  AttnF32Args a;
  a.q = (const float*)q;
  a.kblk = (const float*)kblk;
  a.vblkT = (const float*)vblkT;
  a.kpool = (const float*)kv.k;
  a.vpool = (const float*)kv.v;
  a.block_table = kv.block_table;
  a.seq_len = kv.seq_len;
  a.err = kv.err;
  a.max_pages = kv.max_pages;
  a.num_pages = kv.num_pages;
  a.B = B;
  a.Bp = Bp;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = G;
  a.d = d;
  a.causal = causal;
  a.scale = 1.0f / sqrtf((float)d);
  a.out = (float*)o;
  dim3 grid(B, Hq, batch);
  hipLaunchKernelGGL(attn_f32, grid, dim3(256), (size_t)(d + 256) * sizeof(float), st, a);
  return hipGetLastError();
}

}  // namespace dflash
