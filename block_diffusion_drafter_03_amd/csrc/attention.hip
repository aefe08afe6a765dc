// Block attention over [injected / cached context ; block] for the drafter (bidirectional
// inside the block) and for the target's verification pass (causal inside the block).
//
// bf16 path (head_dim 128): one workgroup of 8 waves per CU and per (sequence, KV head,
// 64-row query group, key split); the last split also takes the block's own B keys.  The
// G*B query rows that share a KV head are split into 4 tiles of 16 rows (held in registers
// as MFMA operands) and each tile is taken by two waves, one per 32-key half of every step,
// so every context K/V byte is read from HBM once per workgroup.  A step is one 64-token
// page slice of the head (16 KB of K, 16 KB of V^T, both contiguous), loaded with 16-byte
// coalesced loads into a 3-deep ring of registers and copied into double-buffered LDS, so
// up to three steps are in flight while one is computed.  S^T = K Q^T and O^T = V^T P^T use
// v_mfma_f32_16x16x32_bf16 with the float32 operand (q, scaled into the log2 domain, and
// the probabilities P) taken as a compensated (hi, lo) bf16 pair against the stored bf16
// K / V:
//   * the K rows are placed in LDS so that the two 16-key S^T tiles of a 32-key half come
//     out with lane group g holding keys 8g .. 8g+7 of the half for its query column -
//     exactly the P^T operand layout of the PV product, with no data movement - while the
//     16 lanes of every K read still hit 16 different banks;
//   * V pages are stored transposed ([d][64 keys]) so a V^T operand is one 16-byte read.
// Each wave runs an online softmax over its half with a lazily moved reference maximum; the
// halves are merged through LDS and the workgroup writes one partial (m, l, unnormalised O)
// per row; a second launch merges the splits with log-sum-exp weights.  Scores are kept in
// the log2 domain (scaled by log2(e)/sqrt(d)) and exponentiated with exp2.
#include "common.h"
#include "kernels.h"

namespace dflash {

#define AD 128      // head dim of the MFMA path
#define PSTRIDE (AD + 4)    // floats per partial row: O[AD], m, l, 2 pad (16-byte rows)

struct AttnArgs {
  const float* q;      // [batch*B, Hq*AD]
  const bf16* kblk;    // [batch*B, Hkv*AD]
  const bf16* vblkT;   // [batch, Hkv, AD, Bp]
  const bf16* kblk_lo;    // low parts of the block's own K / V^T (same layouts): the block
  const bf16* vblkT_lo;   // keys enter as compensated (hi, lo) pairs; zero when stored
  const bf16* kpool;   // [num_pages, Hkv, 64, AD]
  const bf16* vpool;   // [num_pages, Hkv, AD, 64]
  const int32_t* block_table;
  const int32_t* seq_len;
  int32_t* err;
  int max_pages, num_pages;
  int B, Bp, Hq, Hkv, G;
  int n_splits, split_len, n_rg, causal;
  float scale_log2;
  float* part;         // [(b, kvh, rg, s)][64][PSTRIDE]  (O, then m, l per row)
  float* out;          // [batch*B, Hq*AD], A-fragment order when out_afrag == 1, operand
  int out_afrag;       // planes (bf16 pairs, pfrag_off) when 2
};

// LDS layouts of one 64-key step (one page slice of one KV head), padded by 16 bytes per row
#define KROW (AD + 8)     // bf16 per K row   [64 keys][AD]
#define VROW (64 + 8)     // bf16 per V^T row [AD][64 keys]
#define KTILE (64 * KROW)
#define VTILE (AD * VROW)
#define ATTN_MAX_SPLIT_PAGES 1024   // keys per split <= 65536: the split's page list fits LDS

// LDS row of key kk (0..63) of a K tile.  The S^T tile t of lane (r, g) in key half h needs
// key 32h + 8(r >> 2) + (r & 3) + 4t (so that the accumulator comes out in the P^T operand
// layout); storing key kk at row (kk & 35) | ((kk >> 1) & 12) | ((kk << 2) & 16) (bit 2
// moved to bit 4, bits 3-4 to bits 2-3) puts that key at row 32h + 16t + r, so the 16
// lanes of a read hit 16 consecutive rows: distinct banks at the 68-dword row stride.
DF_DEV int krow_phys(int kk) { return (kk & 35) | ((kk >> 1) & 12) | ((kk << 2) & 16); }

// One workgroup of 8 waves per CU (two per SIMD).  Waves w and w + 4 hold the same 16
// query rows; w < 4 takes keys 0..31 of every 64-key step and w + 4 keys 32..63, each with
// its own online softmax, and the two halves are merged through LDS at the end.  The K/V
// loads of a step are spread over all 512 threads (4 x 16 B each), which leaves room for a
// 3-deep ring of register-staged steps: up to 96 KB of K/V in flight per CU while a fourth
// step is computed from LDS.
#define ATTN_THREADS 512
// KV_NT: the context K/V loads carry the non-temporal hint (a context far larger than the
// caches: the 64K and 262K layers 64.2 -> 60.6 and 193.6 -> 185.8 us; at 4K, where the K/V
// of every layer stays in the 256 MB last-level cache from one block to the next, plain
// loads are faster)
template <bool KV_NT>
__global__ __launch_bounds__(ATTN_THREADS, 1) void attn_splitk_bf16(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 kt[2][KTILE];
  __shared__ __attribute__((aligned(16))) bf16 vt[2][VTILE];
  __shared__ float xo[4][64][33];      // key-half merge: O of waves 4..7
  __shared__ float xm[4][64], xl[4][64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wq = w & 3, kh = w >> 2;
  const int r = lane & 15, g = lane >> 4;
  const int s = blockIdx.x;
  const int kvh = blockIdx.y % a.Hkv, rg = blockIdx.y / a.Hkv;
  const int b = blockIdx.z;
  const int R = a.G * a.B;

  // the page-table entries of the planned layout (split s from s * split_len on) are read
  // together with seq_len: when this sequence's context fills planned splits (a context
  // within about a step per split of the capacity, as for a cache sized to its sequence)
  // they are the split's own and the start-up waits for one round trip less; otherwise
  // they are read again below, once seq_len is known
  constexpr int PPT = ATTN_MAX_SPLIT_PAGES / ATTN_THREADS;
  int pg[PPT];
#pragma unroll
  for (int j = 0; j < PPT; ++j)
    pg[j] = a.block_table[(size_t)b * a.max_pages +
                          min(((s * a.split_len) >> 6) + tid + j * ATTN_THREADS, a.max_pages - 1)];
  int n_ctx = a.seq_len[b];
  n_ctx = max(0, min(n_ctx, a.max_pages * 64));
  // keys per split: this sequence's context spread evenly over the splits in whole pages
  // (never more than the planned split length, which sizes the page list), so a grid sized
  // for the cache capacity stays balanced at any context length
  const int slen = min(a.split_len, ((n_ctx + a.n_splits - 1) / a.n_splits + 63) / 64 * 64);
  const int kbeg = s * slen;                         // multiple of 64
  const int kend = min(kbeg + slen, n_ctx);
  const int n_ctx_steps = kend > kbeg ? (kend - kbeg + 63) / 64 : 0;
  // one split also takes the block's own keys: the last one when it holds fewer context
  // steps than the first (the splits before it are full), so that the longest workgroup is
  // one of the context's and not one with a step more; the first one when all are equal
  // (it starts first)
  const int last_steps = max(0, (n_ctx - (a.n_splits - 1) * slen + 63) / 64);
  const bool own = s == (last_steps < min(slen, n_ctx + 63) / 64 ? a.n_splits - 1 : 0);

  // Start-up takes two memory round trips: the query rows, the block's own keys (own)
  // and the split's page-table entries are fetched together, then the first context steps
  // (their addresses need the page table), while the queries are converted.

  // this wave's query tile: rows rho = rg*64 + wq*16 + r as the Q^T MFMA operand, scaled
  // into the log2 domain and split into a compensated (hi, lo) pair (after the page table)
  const int rho = rg * 64 + wq * 16 + r;
  const int jq = rho < R ? rho % a.B : 0x7fffffff;
  float qv[4][8];
  bf16x8 qh[4], ql[4];
  {
    const int gq = rho < R ? rho / a.B : 0;
    const float* src = a.q + (size_t)(b * a.B + (rho < R ? jq : 0)) * a.Hq * AD +
                       (size_t)(kvh * a.G + gq) * AD + g * 8;
#pragma unroll
    for (int cs = 0; cs < 4; ++cs) load8(src + cs * 32, qv[cs]);
  }

  // the split's physical pages, read and checked once (a page index used straight from
  // global memory would make every step wait for all loads in flight)
  __shared__ int pages_s[ATTN_MAX_SPLIT_PAGES];

  // ---- global -> register staging of one step: 4 x 16 B per thread (K then V^T) ----
  // Every ring slot issues exactly these 4 loads, unconditionally and to valid addresses,
  // so the compiler can count them and keep several steps in flight; masking happens when
  // a step is copied to LDS.  A slot past the split's last step (the ring's tail, or a
  // split of fewer steps than the ring is deep) is never computed: its loads all point at
  // the first 16 bytes of the last page, one cache line per load instead of 1 KB of K / V
  // fetched again.  An unmapped page is flagged and read as page 0 (the outputs of that
  // sequence are then invalid, which the error flag reports).
  bf16x8 st0[4], st1[4], st2[4];
  auto load_ctx = [&](int i, bf16x8 (&st)[4]) {
    const bool tail = i >= n_ctx_steps;
    const size_t pb = (size_t)pages_s[tail ? n_ctx_steps - 1 : i] * a.Hkv + kvh;
    const size_t per = tail ? 0 : 8;   // elements per thread index
    const bf16* ks = a.kpool + pb * 64 * AD;
    const bf16* vs = a.vpool + pb * AD * 64;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int idx = tid + ATTN_THREADS * j;
      if constexpr (KV_NT) {
        st[j] = __builtin_nontemporal_load((const bf16x8*)(ks + (size_t)idx * per));
        st[2 + j] = __builtin_nontemporal_load((const bf16x8*)(vs + (size_t)idx * per));
      } else {
        st[j] = *(const bf16x8*)(ks + (size_t)idx * per);
        st[2 + j] = *(const bf16x8*)(vs + (size_t)idx * per);
      }
    }
  };
  // the block's own keys (last split only): K rows from k_blk, V^T columns from v_blk^T
  // (B <= 64), high or low parts; rows and columns past B are read from valid places and
  // masked at the copy
  auto load_blk = [&](bf16x8 (&st)[4], const bf16* kb, const bf16* vb) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int idx = tid + ATTN_THREADS * j;
      const int key = min(idx >> 4, a.B - 1);
      const int k8 = min((idx & 7) * 8, a.Bp - 8);
      st[j] = *(const bf16x8*)(kb + (size_t)(b * a.B + key) * a.Hkv * AD + (size_t)kvh * AD + (idx & 15) * 8);
      st[2 + j] = *(const bf16x8*)(vb + ((size_t)(b * a.Hkv + kvh) * AD + (idx >> 3)) * a.Bp + k8);
    }
  };
  // keys at or past `lim` (a partial last page, the block's padding): their V^T columns are
  // zeroed so stale bytes cannot leak NaN through a zero probability (their scores are
  // masked to -inf, so K needs no masking)
  auto store_step = [&](int buf, int lim, bf16x8 (&st)[4]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int idx = tid + ATTN_THREADS * j;
      *(bf16x8*)&kt[buf][krow_phys(idx >> 4) * KROW + (idx & 15) * 8] = st[j];
      bf16x8 v = st[2 + j];
      const int k0 = (idx & 7) * 8;
      if (lim < 64 && k0 + 8 > lim) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (k0 + e >= lim) v[e] = (bf16)0.f;
      }
      *(bf16x8*)&vt[buf][(idx >> 3) * VROW + k0] = v;
    }
  };
  auto step_lim = [&](int i) { return min(64, kend - (kbeg + i * 64)); };

  float m = -INFINITY, lsum = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this wave's half (keys kh*32 .. kh*32+31) of the step in LDS buffer `buf` (keys >= lim
  // masked; the block's own step is causal for the verifier).  The block's own step (blk)
  // holds the low parts of its K / V^T in the other buffer: scores K_hi q_hi + K_hi q_lo +
  // K_lo q_hi, outputs V_hi p_hi + V_hi p_lo + V_lo p_hi (the lo x lo terms are below
  // float32 resolution).
  auto compute = [&](int buf, bool blk, int lim) {
    const bf16* K = kt[buf];
    const bf16* VT = vt[buf];
    // every K and V^T fragment of the step is read from LDS up front, so the V^T reads are
    // in flight across the score MFMAs and the softmax instead of waited for pair by pair
    bf16x8 kf[2][4], vf[8];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int cs = 0; cs < 4; ++cs)   // key kh*32 + 8(r>>2) + (r&3) + 4t
        kf[t][cs] = *(const bf16x8*)(K + (kh * 32 + 16 * t + r) * KROW + g * 8 + cs * 32);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) vf[dt] = *(const bf16x8*)(VT + (dt * 16 + r) * VROW + kh * 32 + g * 8);
    f32x4 sc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cs = 0; cs < 4; ++cs)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[t][cs], qh[cs], sc[t], 0, 0, 0);
        sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[t][cs], ql[cs], sc[t], 0, 0, 0);
      }
    if (blk) {
      const bf16* KL = kt[buf ^ 1];
#pragma unroll
      for (int cs = 0; cs < 4; ++cs)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 kl = *(const bf16x8*)(KL + (kh * 32 + 16 * t + r) * KROW + g * 8 + cs * 32);
          sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kl, qh[cs], sc[t], 0, 0, 0);
        }
    }
    // lane holds keys kh*32 + 8g + 4t + e (e < 4) of the step for query column r
    float p[8];
    float mx = -INFINITY;
    if (!blk && lim == 64) {   // a full context page: nothing to mask
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[4 * t + e] = sc[t][e];
          mx = fmaxf(mx, sc[t][e]);
        }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = kh * 32 + g * 8 + 4 * t + e;
          bool ok = key < lim;
          if (blk && a.causal) ok = ok && key <= jq;
          const float x = ok ? sc[t][e] : -INFINITY;
          p[4 * t + e] = x;
          mx = fmaxf(mx, x);
        }
    }
    // the reference max moves only when a step's column max exceeds it by more than 8
    // (log2 domain): probabilities relative to it stay <= 256, the softmax is the same for
    // any reference, and deep into a context the O rescale is mostly skipped.  No column
    // max can exceed it unless some lane's own max does, so the cross-lane max is formed
    // only then (the same reference values, with no lane exchange in the common case).
    float mnew = m;
    if (__any(mx > m + 8.f)) {
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      mnew = mx > m + 8.f ? mx : m;
    }
    const float alpha = mnew == m ? 1.f : (m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mnew));
    const float msub = mnew == -INFINITY ? 0.f : mnew;   // all scores -inf: p = 0
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pe = __builtin_amdgcn_exp2f(p[e] - msub);
      ps += pe;
      p[e] = pe;
    }
    bf16x8 ph, pl;
    split8(p, ph, pl);
    m = mnew;
    lsum = lsum * alpha + ps;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], ph, o[dt], 0, 0, 0);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pl, o[dt], 0, 0, 0);
    }
    if (blk) {
      const bf16* VL = vt[buf ^ 1];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x8 vl = *(const bf16x8*)(VL + (dt * 16 + r) * VROW + kh * 32 + g * 8);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vl, ph, o[dt], 0, 0, 0);
      }
    }
  };
  // the block's own keys first (last split), high and low parts
  bf16x8 stb[4], stl[4];
  const int last = n_ctx_steps - 1;
  if (own) {
    load_blk(stb, a.kblk, a.vblkT);
    load_blk(stl, a.kblk_lo, a.vblkT_lo);
  }
  // (every thread reads and writes its slots unconditionally - past the split's last page
  // the index is clamped to a valid entry - so every thread waits here for its loads and
  // the query conversion below needs no wait on the context loads issued after it)
  if (slen != a.split_len) {
#pragma unroll
    for (int j = 0; j < PPT; ++j)
      pg[j] = a.block_table[(size_t)b * a.max_pages + (kbeg >> 6) + min(tid + j * ATTN_THREADS, max(n_ctx_steps - 1, 0))];
  }
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int i = tid + j * ATTN_THREADS;
    int page = pg[j];
    if (page < 0 || page >= a.num_pages) {
      if (i < n_ctx_steps) flag_error(a.err, DEVERR_PAGE);
      page = 0;
    }
    pages_s[i] = page;
  }
  __syncthreads();
  if (n_ctx_steps > 0) {
    load_ctx(0, st0);
    load_ctx(1, st1);
    load_ctx(2, st2);
  }
#pragma unroll
  for (int cs = 0; cs < 4; ++cs) {
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[cs][e] = rho < R ? qv[cs][e] * a.scale_log2 : 0.f;
    split8(qv[cs], qh[cs], ql[cs]);
  }
  if (own) {
    store_step(0, a.B, stb);
    store_step(1, a.B, stl);
    __syncthreads();
    compute(0, true, a.B);
    __syncthreads();
  }
  // ring over the context steps: while step i is computed from LDS buffer i % 2, steps
  // i+1 .. i+3 are in flight in the staging registers; step i+1 then moves to the other
  // LDS buffer.  Loads and copies run for every slot (past the last step, loads of one
  // cache line) so each ring slot issues the same instructions; only the compute is
  // skipped past the end.
  if (n_ctx_steps > 0) {
    store_step(0, step_lim(0), st0);
    __syncthreads();
    auto body = [&](int i, bf16x8 (&ld)[4], bf16x8 (&nx)[4]) {
      load_ctx(i + 3, ld);
      if (i < n_ctx_steps) compute(i & 1, false, step_lim(i));
      store_step((i + 1) & 1, step_lim(min(i + 1, last)), nx);
      __syncthreads();
    };
    for (int i = 0; i < n_ctx_steps; i += 3) {
      body(i, st0, st1);
      body(i + 1, st1, st2);
      body(i + 2, st2, st0);
    }
  }

  // ---- merge the two key halves, then the partial (m, l, unnormalised O) of the rows ----
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (kh == 1) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) xo[wq][lane][dt * 4 + e] = o[dt][e];
    xm[wq][lane] = m;
    xl[wq][lane] = lsum;
  }
  __syncthreads();
  if (kh == 1) return;
  const float m1 = xm[wq][lane], l1 = xl[wq][lane];
  const float mt = fmaxf(m, m1);
  const float a0 = m == -INFINITY ? 0.f : exp2f(m - mt);
  const float a1 = m1 == -INFINITY ? 0.f : exp2f(m1 - mt);
  const size_t unit = ((size_t)b * a.Hkv + kvh) * a.n_rg + rg;
  float* dst = a.part + (unit * a.n_splits + s) * 64 * PSTRIDE + (size_t)(wq * 16 + r) * PSTRIDE;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    *(float4*)(dst + dt * 16 + g * 4) =
        make_float4(o[dt][0] * a0 + xo[wq][lane][dt * 4 + 0] * a1, o[dt][1] * a0 + xo[wq][lane][dt * 4 + 1] * a1,
                    o[dt][2] * a0 + xo[wq][lane][dt * 4 + 2] * a1, o[dt][3] * a0 + xo[wq][lane][dt * 4 + 3] * a1);
  if (g == 0) {
    dst[AD] = mt;
    dst[AD + 1] = lsum * a0 + l1 * a1;
  }
}


// Split merge as its own launch: 8 query rows per workgroup, 32 threads x 4 columns per
// row.  The splits' (m, l) of the 8 rows are read into LDS by all threads at once, the
// log-sum-exp weights are formed there, and each thread then sums its 4 columns over the
// splits with independent loads.
#define MERGE_MAX_SPLITS 512
#define MERGE_REG_SPLITS 32
__global__ __launch_bounds__(256) void attn_merge_bf16(AttnArgs a) {
  __shared__ float wsh[8][MERGE_MAX_SPLITS];
  __shared__ float lsh[8][MERGE_MAX_SPLITS];
  const int rl = threadIdx.x >> 5, t = threadIdx.x & 31;
  const int rho0 = blockIdx.x * 8;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int R = a.G * a.B, S = a.n_splits;
  const size_t ss = 64 * PSTRIDE;
  const int rho = rho0 + rl;
  // up to MERGE_REG_SPLITS splits: this thread's 4 columns of every split are loaded now,
  // together with the (m, l) of the workgroup's rows below, instead of after the weights
  // (one memory round trip less; the sum runs in the same split order either way)
  constexpr int SR = MERGE_REG_SPLITS;
  const int rho_c = min(rho, R - 1);
  const float* prc = a.part + (((size_t)b * a.Hkv + kvh) * a.n_rg + rho_c / 64) * S * ss +
                     (size_t)(rho_c % 64) * PSTRIDE + 4 * t;
  float4 xr[SR];
  if (S <= SR) {
#pragma unroll
    for (int sp = 0; sp < SR; ++sp) xr[sp] = *(const float4*)(prc + min(sp, S - 1) * ss);
  }
  // (m, l) of every (split, row) of this workgroup
  for (int idx = threadIdx.x; idx < S * 8; idx += 256) {
    const int sp = idx >> 3, row = idx & 7, rho = min(rho0 + row, R - 1);
    const size_t unit = ((size_t)b * a.Hkv + kvh) * a.n_rg + rho / 64;
    const float* pr = a.part + (unit * S + sp) * ss + (size_t)(rho % 64) * PSTRIDE;
    wsh[row][sp] = pr[AD];
    lsh[row][sp] = pr[AD + 1];
  }
  __syncthreads();
  // weights: the row's 32 threads split the splits, then combine through lane shuffles
  float ms = -INFINITY;
  for (int sp = t; sp < S; sp += 32) ms = fmaxf(ms, wsh[rl][sp]);
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) ms = fmaxf(ms, __shfl_xor(ms, o, 64));
  float lt = 0.f;
  for (int sp = t; sp < S; sp += 32) {
    const float mv = wsh[rl][sp];
    const float wgt = mv == -INFINITY ? 0.f : exp2f(mv - ms);
    lt += lsh[rl][sp] * wgt;
    wsh[rl][sp] = wgt;
  }
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) lt += __shfl_xor(lt, o, 64);
  __syncthreads();
  if (rho >= R) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (S <= SR) {
#pragma unroll
    for (int sp = 0; sp < SR; ++sp) {
      if (sp < S) {
        const float wgt = wsh[rl][sp];
        acc.x += xr[sp].x * wgt;
        acc.y += xr[sp].y * wgt;
        acc.z += xr[sp].z * wgt;
        acc.w += xr[sp].w * wgt;
      }
    }
  } else {
#pragma unroll 16
    for (int sp = 0; sp < S; ++sp) {
      const float wgt = wsh[rl][sp];
      const float4 x = *(const float4*)(prc + sp * ss);
      acc.x += x.x * wgt;
      acc.y += x.y * wgt;
      acc.z += x.z * wgt;
      acc.w += x.w * wgt;
    }
  }
  const float inv = 1.f / lt;
  const int gq = rho / a.B, j = rho % a.B;
  const int m = b * a.B + j, k = (kvh * a.G + gq) * AD + 4 * t;
  const float4 y = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (a.out_afrag == 2) {
    // 4 consecutive k of one lane: 8 bytes in each plane
    bf16* p = (bf16*)a.out + pfrag_off(m, k, (a.Hq * AD) >> 5);
    const bf16x4 hi = {(bf16)y.x, (bf16)y.y, (bf16)y.z, (bf16)y.w};
    const bf16x4 lo = {(bf16)(y.x - (float)hi[0]), (bf16)(y.y - (float)hi[1]), (bf16)(y.z - (float)hi[2]),
                       (bf16)(y.w - (float)hi[3])};
    *(bf16x4*)p = hi;
    *(bf16x4*)(p + 512) = lo;
  } else {
    float* out = a.out + (a.out_afrag ? afrag_off(m, k, (a.Hq * AD) >> 5) : (size_t)m * a.Hq * AD + k);
    *(float4*)out = y;
  }
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
static int attn_num_cus() {
  static int n = 0;
  if (!n) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    hipDeviceProp_t p;
    n = (hipGetDeviceProperties(&p, dev) == hipSuccess && p.multiProcessorCount > 0) ? p.multiProcessorCount : 256;
  }
  return n;
}

AttnPlan attn_plan(int dt, int batch, int Hkv, int G, int B, int ctx_cap, int n_layers, int d) {
  AttnPlan p;
  p.n_rg = (G * B + 63) / 64;
  // stream the context past the caches once the K/V of all layers (bf16) is well beyond
  // what the 256 MB last-level cache could keep from one call to the next
  p.kv_stream = (double)batch * Hkv * (double)(ctx_cap > 0 ? ctx_cap : 1) * d * 2 * 2 * n_layers >
                192.0 * (1 << 20);
  if (dt != BF16) {
    p.n_ctx_splits = 1;
    p.split_len = 0;
    return p;
  }
  const int cap = ctx_cap > 0 ? ctx_cap : 1;
  const int units = batch * Hkv * p.n_rg;
  // one workgroup per CU (register-bound): aim for one wave of workgroups over the chip,
  // with at least 192 keys (3 steps) in a split
  int want = attn_num_cus() / units;
  const int max_splits = (cap + 191) / 192;
  if (want > max_splits) want = max_splits;
  if (want < 1) want = 1;
  // planned split length: the capacity over `want` splits in whole pages, at least 192 keys
  // (the kernel then spreads each sequence's actual context evenly over the splits)
  int len = (cap + want - 1) / want;
  len = len <= 192 ? 192 : (len + 63) / 64 * 64;
  if (len > 64 * ATTN_MAX_SPLIT_PAGES) len = 64 * ATTN_MAX_SPLIT_PAGES;
  if ((cap + len - 1) / len > MERGE_MAX_SPLITS) len = (cap + MERGE_MAX_SPLITS - 1) / MERGE_MAX_SPLITS;
  len = (len + 63) / 64 * 64;
  p.split_len = len;
  p.n_ctx_splits = (cap + len - 1) / len;
  return p;
}

size_t attn_partial_floats(const AttnPlan& p, int batch, int Hkv, int d) {
  return (size_t)batch * Hkv * p.n_rg * p.n_ctx_splits * 64 * (d + 4);
}

hipError_t launch_attention(int dt, const AttnPlan& p, const float* q, const void* kblk,
                            const void* vblkT, const void* kblk_lo, const void* vblkT_lo,
                            const KvLayer& kv, int batch, int B, int Bp, int Hq, int Hkv, int d,
                            int causal, float* part, float* o, int o_afrag, hipStream_t st) {
  const int G = Hq / Hkv;
  if (dt == BF16) {
    AttnArgs a;
    a.q = q;
    a.kblk = (const bf16*)kblk;
    a.vblkT = (const bf16*)vblkT;
    a.kblk_lo = (const bf16*)kblk_lo;
    a.vblkT_lo = (const bf16*)vblkT_lo;
    if (!kblk_lo || !vblkT_lo) return hipErrorInvalidValue;
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
    a.n_splits = p.n_ctx_splits;
    a.split_len = p.split_len;
    a.n_rg = p.n_rg;
    a.causal = causal;
    a.scale_log2 = 1.4426950408889634f / sqrtf((float)d);
    a.part = part;
    a.out = o;
    a.out_afrag = o_afrag;
    // the split's page list and the merge's weights live in fixed LDS arrays
    if (p.split_len > 64 * ATTN_MAX_SPLIT_PAGES || p.n_ctx_splits > MERGE_MAX_SPLITS)
      return hipErrorInvalidValue;
    dim3 grid(p.n_ctx_splits, Hkv * p.n_rg, batch);
    if (p.kv_stream) hipLaunchKernelGGL(attn_splitk_bf16<true>, grid, dim3(ATTN_THREADS), 0, st, a);
    else hipLaunchKernelGGL(attn_splitk_bf16<false>, grid, dim3(ATTN_THREADS), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 g2((p.n_rg * 64 + 7) / 8, Hkv, batch);
    hipLaunchKernelGGL(attn_merge_bf16, g2, dim3(256), 0, st, a);
    return hipGetLastError();
  }
  AttnF32Args a;
  a.q = q;
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
  a.out = o;
  dim3 grid(B, Hq, batch);
  hipLaunchKernelGGL(attn_f32, grid, dim3(256), (size_t)(d + 256) * sizeof(float), st, a);
  return hipGetLastError();
}

}  // namespace dflash
