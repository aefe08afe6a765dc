// Weight-streaming GEMM for M <= 16 rows (one drafter block of one sequence, or a short
// injection): acc[m][n] = sum_k A[m][k] W[n][k] with optional A-side RMSNorm and a fused
// epilogue (epilogue.h).  W (bf16) is in B-fragment order and the float32 activations in
// A-fragment order (common.h), so every operand load of a wave is one contiguous 1 KB
// burst; activations enter the MFMAs as compensated (hi, lo) bf16 pairs.
#include "gemm_common.h"

namespace dflash {

// M <= 16: NW waves split K, one 32-wide step per MFMA (pair).
//  * ASTAT (many tiles, K <= 4096): one workgroup per CU walks the tiles; each wave keeps
//    its K-slice of the A rows for all of them, already multiplied by the RMSNorm gain and
//    split into (hi, lo) (rstd is applied in the epilogue): hi in registers, lo in LDS
//    (128 KB: the workgroup owns the CU), so the vector memory path carries only W: a wave
//    issues all of its W loads of a tile at once (CH steps, 1 KB each) and the next tile's
//    loads go out right after the MFMAs, in flight across the reduction.
//  * streamed (few tiles, or K > 4096): A and W are loaded together in chunks of CHS
//    steps; no LDS for A, so several workgroups share a CU and every tile is in flight.
//  * the K-split form further below (QKV, down): column groups over K ranges that meet in
//    the last-arriving workgroup.
// 8 waves of 512 threads leave each wave 256 registers, so the stationary A, a full tile
// of W in flight and the epilogue never spill.  Weights load through wload_k: streamed
// past the caches (non-temporal) except for gate/up.
#define GEMV_MAX_TILES 8   // tiles per workgroup whose epilogue is deferred (non-argmax kinds)

template <typename TA, int NW, bool NORM, bool ASTAT, int KIND>
__global__ __launch_bounds__(NW * 64) void gemm_gemv_bf16(GemmArgs ga) {
  constexpr bool TWO = AIsFloat<TA>::value;
  constexpr int CH = GEMV_CH;        // stationary steps per wave (K = 32 NW CH = 4096)
  constexpr int CHS = 8;             // streamed chunk
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int M = ga.M, N = ga.N, K = ga.K;
  const int KS = K >> 5;
  // steps per wave: K % (32 NW) == 0; the stationary form takes exactly K = 32 NW CH
  const int spw = ASTAT ? CH : KS / NW;
  const int ks0 = w * spw;
  const int n_tiles = (N + 15) >> 4;
  __shared__ f32x4 red[NW][64];
  __shared__ f32x4 done[GEMV_MAX_TILES][64];
  __shared__ float ss_red[NW][16];
  __shared__ float rstd[16];
  __shared__ bf16x8 alo[ASTAT && TWO ? NW : 1][ASTAT && TWO ? CH : 1][64];
  __shared__ bf16x8 gsh[ASTAT && NORM ? NW * 64 : 1];   // stationary form: the K norm gains
  // running argmax keys of wave 0's lanes (kept out of the main loop's registers)
  __shared__ unsigned long long bsh[KIND == EPI_ARGMAX ? 4 : 1][64];
  const bf16* gk = NORM ? (const bf16*)ga.norm_g + g * 8 : nullptr;
  // this lane's 8 A values of step ks (row r)
  auto load_a = [&](int ks, float v[8]) {
    if constexpr (TWO)
      afrag_load8((const float*)ga.A, 0, ks, KS, lane, v);
    else
      load8((const bf16*)ga.A + (size_t)min(r, M - 1) * ga.lda + (size_t)ks * 32 + g * 8, v);
  };
  int nbuf = 0;
  bool first = true;
  if (KIND == EPI_ARGMAX && w == 0)
#pragma unroll
    for (int i = 0; i < (KIND == EPI_ARGMAX ? 4 : 1); ++i) bsh[i][lane] = 0ull;

  bf16x8 ah[ASTAT ? CH : 1];
  // stationary form: one tile of W per wave in registers, reloaded step by step with the
  // next tile of the walk right after each step's MFMAs, so that about CH loads stay in
  // flight at every moment (a whole next tile is in flight across the reduction).  Past
  // the walk the reload is clamped to its last tile (an L2 hit), keeping every load
  // unconditional.  The first tile's loads go out before the A prologue (independent).
  bf16x8 wa[ASTAT ? CH : 1];
  // every step's load is issued unconditionally, so the compiler can count the loads and
  // never drains the ring with a full wait
  // (the steps of one tile are consecutive 1 KB fragments: one base address per tile)
  auto load_w = [&](bf16x8 (&wn)[ASTAT ? CH : 1], int t) {
    const bf16* p = wblock(ga.B, t, ks0, KS) + lane * 8;
#pragma unroll
    for (int s = 0; s < CH; ++s) wn[s] = wload_k<KIND>(p + (size_t)s * 512);
  };
  const int G = gridDim.x;
  const int bx = blockIdx.x;
  const int t_last = bx < n_tiles ? bx + (n_tiles - 1 - bx) / G * G : 0;
  if constexpr (ASTAT) {
    // The norm gains (K = 8 per thread) and every A step of this wave are loaded at once;
    // the first W tile goes out only when this wave's A has arrived.  W issued earlier
    // (independent of A) floods the memory system with every workgroup's first tile and
    // delays the A fetches by about twice their own latency.  The launch keeps
    // gridDim.x <= n_tiles.
    bf16x8 gl;
    if constexpr (NORM) gl = *(const bf16x8*)((const bf16*)ga.norm_g + threadIdx.x * 8);
    float av[CH][8];
#pragma unroll
    for (int s = 0; s < CH; ++s) load_a(ks0 + s, av[s]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NORM) {
      gsh[threadIdx.x] = gl;
      __syncthreads();
    }
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < CH; ++s) {
      const bf16x8 gv = NORM ? gsh[(ks0 + s) * 4 + g] : bf16x8{};
      bf16x8 lo;
      a_operand<NORM>(av[s], gv, &ss, ah[s], lo);
      if constexpr (TWO) alo[w][s][lane] = lo;
    }
    __builtin_amdgcn_sched_barrier(0);
    load_w(wa, blockIdx.x);
    __builtin_amdgcn_sched_barrier(0);
    if (NORM) {
      ss += __shfl_xor(ss, 16, 64);
      ss += __shfl_xor(ss, 32, 64);
      if (g == 0) ss_red[w][r] = ss;
      __syncthreads();
      if (threadIdx.x < 16) {
        float s = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) s += ss_red[ww][threadIdx.x];
        rstd[threadIdx.x] = 1.0f / sqrtf(s / (float)K + ga.eps);
      }
      __syncthreads();
    }
  }

  // reduction of a tile's 8 wave partials, then its epilogue (argmax) or a deferred slot
  auto finish = [&](int t, f32x4 acc, f32x4 acc2) {
    red[w][lane] = acc + acc2;
    __syncthreads();
    if (NORM && !ASTAT && first) {
      if (threadIdx.x < 16) {
        float s = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) s += ss_red[ww][threadIdx.x];
        rstd[threadIdx.x] = 1.0f / sqrtf(s / (float)K + ga.eps);
      }
      __syncthreads();
    }
    first = false;
    if (w == 0) {
      f32x4 s = red[0][lane];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) s += red[ww][lane];
      if constexpr (KIND == EPI_ARGMAX) {
        float v[4];
        unsigned long long best[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = NORM ? s[i] * rstd[g * 4 + i] : s[i];
          best[i] = bsh[i][lane];
        }
        tile_epilogue<bf16, KIND>(ga, g * 4, t * 16 + r, v, r, best);
#pragma unroll
        for (int i = 0; i < 4; ++i) bsh[i][lane] = best[i];
      } else {
        done[nbuf][lane] = s;   // epilogue deferred until the A registers are dead
      }
    }
    ++nbuf;
    __syncthreads();
  };

  if constexpr (ASTAT) {
    for (int t = blockIdx.x; t < n_tiles; t += G) {
      const int tn = min(t + G, t_last);
      const bf16* pn = wblock(ga.B, tn, ks0, KS) + lane * 8;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < CH; ++s) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[s], wa[s], acc, 0, 0, 0);
        if constexpr (TWO) acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[w][s][lane], wa[s], acc2, 0, 0, 0);
        wa[s] = wload_k<KIND>(pn + (size_t)s * 512);
      }
      finish(t, acc, acc2);
    }
  } else {
    for (int t = blockIdx.x; t < n_tiles; t += G) {
      const bf16* pt = wblock(ga.B, t, 0, KS) + lane * 8;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
      float ss = 0.f;
      for (int c0 = 0; c0 < spw; c0 += CHS) {
        // a chunk's weights, activations and gains loaded together, unconditionally (steps
        // past spw clamped to the last one, their activations zeroed)
        bf16x8 wf[CHS], gv[CHS];
        float av[CHS][8];
#pragma unroll
        for (int s = 0; s < CHS; ++s) {
          const int k = ks0 + min(c0 + s, spw - 1);
          wf[s] = wload_k<KIND>(pt + (size_t)k * 512);
          load_a(k, av[s]);
          if constexpr (NORM) gv[s] = *(const bf16x8*)(gk + (size_t)k * 32);
        }
#pragma unroll
        for (int s = 0; s < CHS; ++s) {
#pragma unroll
          for (int e = 0; e < 8; ++e) av[s][e] = c0 + s < spw ? av[s][e] : 0.f;
          bf16x8 hi, lo;
          a_operand<NORM>(av[s], gv[s], &ss, hi, lo);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, wf[s], acc, 0, 0, 0);
          if constexpr (TWO) acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, wf[s], acc2, 0, 0, 0);
        }
      }
      if (NORM && first) {
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        if (g == 0) ss_red[w][r] = ss;
      }
      finish(t, acc, acc2);
    }
  }
  if constexpr (KIND == EPI_DCONV) {
    // the convolution of the tile's 128 channels for every row, from the tile's 16
    // correction columns (two per 16-channel group) held in `done`, by all threads
    const EpiArgs& e = ga.e;
    const float* x = (const float*)ga.A;
    const bf16* base = (const bf16*)e.dconv_base;
    const int KS2 = K >> 5;
    for (int i = 0; i < nbuf; ++i) {
      const int t = blockIdx.x + i * gridDim.x;
      for (int q = threadIdx.x; q < 16 * 128; q += NW * 64) {
        const int m = q >> 7, c = t * 128 + (q & 127);
        if (m >= M || c >= K) continue;
        const int p = m % e.B == 0 ? m : m - 1;
        const int pair = 2 * ((c >> 4) - 8 * t);        // the channel group's two columns
        float k0 = done[i][(m >> 2) * 16 + pair][m & 3];
        float k1 = done[i][(m >> 2) * 16 + pair + 1][m & 3];
        float xr = x[afrag_off(m, c, KS2)], xp = x[afrag_off(p, c, KS2)];
        if constexpr (NORM) {
          const float gc = (float)((const bf16*)ga.norm_g)[c];
          k0 *= rstd[m];
          k1 *= rstd[m];
          xr *= rstd[m] * gc;
          xp *= rstd[p] * gc;
        }
        k0 += (float)base[c];
        k1 += (float)base[K + c];
        const float y = k0 * xr + k1 * xp;
        float* o = (float*)e.out + afrag_off(m, c, KS2);
        const float v = e.dconv_accumulate ? *o + y : y;
        *o = v;
        if (e.hdbg) e.hdbg[(size_t)m * K + c] = v;
      }
    }
  } else if constexpr (KIND != EPI_ARGMAX) {
    // every wave takes buffered tiles: the epilogues run in parallel, off the main loop's
    // register budget
    unsigned long long best[4];
    for (int i = w; i < nbuf; i += NW) {
      const f32x4 s = done[i][lane];
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = NORM ? s[e] * rstd[g * 4 + e] : s[e];
      tile_epilogue<bf16, KIND>(ga, g * 4, (blockIdx.x + i * gridDim.x) * 16 + r, v, r, best);
    }
  }
  if (KIND == EPI_ARGMAX && w == 0 && r == 0) {
#pragma unroll
    for (int i = 0; i < (KIND == EPI_ARGMAX ? 4 : 1); ++i) {
      const int row = g * 4 + i;
      const unsigned long long k = bsh[i][lane];
      if (row < M && k) atomicMax(&ga.e.keys[row], k);
    }
  }
  if constexpr (KIND == EPI_ARGMAX) {
    if (ga.e.ids_cnt) {
      // the draft ids (or the greedy acceptance), by the last workgroup to arrive: every
      // key update of a workgroup (device-coherent atomics) has completed before it counts
      // itself in
      __shared__ unsigned arrived;
      __builtin_amdgcn_s_waitcnt(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __syncthreads();
      if (threadIdx.x == 0)
        arrived = __hip_atomic_fetch_add(ga.e.ids_cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      if (arrived == gridDim.x - 1) {
        const int B = ga.e.ids_B;
        if (ga.e.ids_out) {
          const int n = (M / B) * (B - 1);
          for (int i = threadIdx.x; i < n; i += NW * 64) {
            const unsigned long long k = __hip_atomic_load(ga.e.keys + (i / (B - 1)) * B + i % (B - 1) + 1,
                                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ga.e.ids_out[i] = unpack_argmax_idx(k);
          }
        }
        if (ga.e.acc_tau)   // one wave per sequence
          for (int b = w; b < M / B; b += NW)
            accept_wave<true>(ga.e.keys, ga.e.acc_drafts, B, b, ga.e.acc_g, ga.e.acc_tau, ga.e.acc_bonus);
        if (threadIdx.x == 0) __hip_atomic_store(ga.e.ids_cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
// K-split M <= 16 GEMV.  Every 16-column tile needs the whole A, so one workgroup per tile
// re-reads all of A per tile.  Here a workgroup takes TW tiles (one column group) over one
// of S K ranges - A is read once per group, in S parts - and the splits meet without a
// grid-wide barrier or a release fence (which writes back the whole L2 of an XCD): each
// workgroup stores its partial tiles (and, with the A-side norm, its rows' partial sums of
// squares) with agent-scope stores, which are coherent across the XCDs' L2s once complete,
// waits for them to complete, then counts itself in on the group's counter; the workgroup
// that arrives last reads the S partials with agent-scope loads, sums them in split order
// (so the result does not depend on which one that is), applies rstd and runs the
// epilogue, then re-arms the counter for the next launch.  The counters start at zero
// (zeroed by the step's embedding kernel).
template <int TW, int NW, bool NORM, int KIND>
__global__ __launch_bounds__(NW * 64) void gemm_gemv_splitk_bf16(GemmArgs ga) {
  constexpr int CHS = 4;   // steps loaded together per wave
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int KS = ga.K >> 5;
  const int n_tiles = (ga.N + 15) >> 4, n_groups = (n_tiles + TW - 1) / TW;
  const int S = (int)gridDim.x / n_groups;          // the launcher makes gridDim.x = groups S
  const int grp = blockIdx.x % n_groups, sp = blockIdx.x / n_groups;
  const int spw = KS / (S * NW);                    // the launcher checks KS % (S NW) == 0
  const int ks0 = (sp * NW + w) * spw;
  const bf16* wp[TW];
#pragma unroll
  for (int j = 0; j < TW; ++j) wp[j] = wblock(ga.B, min(grp * TW + j, n_tiles - 1), 0, KS) + lane * 8;
  const bf16* gk = NORM ? (const bf16*)ga.norm_g + g * 8 : nullptr;
  f32x4 acc[TW], acc2[TW];
#pragma unroll
  for (int j = 0; j < TW; ++j) acc[j] = acc2[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  for (int c0 = 0; c0 < spw; c0 += CHS) {
    // a chunk's weights, activations and gains loaded together, unconditionally (steps
    // past spw clamped to the last one, their activations zeroed)
    bf16x8 wf[CHS][TW], gv[CHS];
    float av[CHS][8];
#pragma unroll
    for (int s = 0; s < CHS; ++s) {
      const int k = ks0 + min(c0 + s, spw - 1);
#pragma unroll
      for (int j = 0; j < TW; ++j) wf[s][j] = wload_k<KIND>(wp[j] + (size_t)k * 512);
      afrag_load8((const float*)ga.A, 0, k, KS, lane, av[s]);
      if constexpr (NORM) gv[s] = *(const bf16x8*)(gk + (size_t)k * 32);
    }
    // (left to itself the compiler waits for each step's loads right after issuing them)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < CHS; ++s) {
#pragma unroll
      for (int e = 0; e < 8; ++e) av[s][e] = c0 + s < spw ? av[s][e] : 0.f;
      bf16x8 hi, lo;
      a_operand<NORM>(av[s], gv[s], &ss, hi, lo);
#pragma unroll
      for (int j = 0; j < TW; ++j) {
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, wf[s][j], acc[j], 0, 0, 0);
        acc2[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, wf[s][j], acc2[j], 0, 0, 0);
      }
    }
  }
  // the split's partial tiles: wave j < TW sums tile j over the waves in wave order (and
  // wave TW the rows' sums of squares)
  __shared__ f32x4 red[NW][TW][64];
  __shared__ float ss_red[NORM ? NW : 1][16];
  __shared__ float rstd[16];
  __shared__ unsigned arrived;
#pragma unroll
  for (int j = 0; j < TW; ++j) red[w][j][lane] = acc[j] + acc2[j];
  if (NORM) {
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    if (g == 0) ss_red[w][r] = ss;
  }
  __syncthreads();
  const GemvSplitArgs& gs = ga.gsplit;
  const size_t slot = (size_t)sp * n_groups + grp;
  if (w < TW) {
    f32x4 p = red[0][w][lane];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) p += red[ww][w][lane];
    float* q = gs.part + ((slot * TW + w) * 64 + lane) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) __hip_atomic_store(q + e, p[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (NORM && w == TW && lane < 16) {
    float t = ss_red[0][lane];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) t += ss_red[ww][lane];
    __hip_atomic_store(gs.ss + slot * 16 + lane, t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // every partial store of this workgroup has completed before it counts itself in
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0)
    arrived = __hip_atomic_fetch_add(gs.cnt + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (arrived != (unsigned)(S - 1)) return;
  // the group's last workgroup: the S partials summed in split order, then the epilogue
  if (NORM) {
    if (threadIdx.x < 16) {
      float t = 0.f;
      for (int s = 0; s < S; ++s)
        t += __hip_atomic_load(gs.ss + ((size_t)s * n_groups + grp) * 16 + threadIdx.x, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      rstd[threadIdx.x] = 1.0f / sqrtf(t / (float)ga.K + ga.eps);
    }
    __syncthreads();
  }
  if (w < TW) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < S; ++s) {
      const float* q = gs.part + ((((size_t)s * n_groups + grp) * TW + w) * 64 + lane) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += __hip_atomic_load(q + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    float vv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) vv[e] = NORM ? v[e] * rstd[g * 4 + e] : v[e];
    unsigned long long best[4];
    tile_epilogue<bf16, KIND>(ga, g * 4, (grp * TW + w) * 16 + r, vv, r, best);
  }
  if (threadIdx.x == 0) __hip_atomic_store(gs.cnt + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int gemv_split_tiles(int max_n) { return (max_n + 15) / 16 + 3; }
size_t gemv_split_part_bytes(int max_n) { return (size_t)GEMV_SPLIT_MAX * gemv_split_tiles(max_n) * 1024; }
size_t gemv_split_ss_bytes(int max_n) { return (size_t)GEMV_SPLIT_MAX * gemv_split_tiles(max_n) * 64; }

#define GEMV_SPLIT_NW 8     // waves per workgroup of the K-split GEMV

// Which GEMVs take the K-split form (measured on the Qwen3-8B shapes, M = 16): QKV (the
// A-side norm; 384 tiles over 128 groups of 3, two splits: 20.2 -> 18.6 us, the
// stationary form's per-workgroup prologue of the whole normalised A slice gone) and the
// down projection (K = 12288: 27.7 -> 25.7 us).  Not O (K = 4096, no norm: the streamed
// 16-wave form has one chunk per wave already; 12.4 -> 14.0 us split), nor gate/up and the
// LM head (too many tiles for one resident grid).
template <bool NORM, int KIND>
constexpr bool gemv_split_kind() {
  return NORM ? KIND == EPI_QKV : (KIND == EPI_RESID || KIND == EPI_STORE_F32);
}

// Tile width and splits of the K-split GEMV for this shape (false when it does not apply):
// a grid resident at once (one 8-wave workgroup per CU: 3 waves per SIMD by registers)
// that keeps the most CUs busy, each wave with at least one 4-step chunk; among equals the
// widest column group (the least A traffic).  Without the norm only for K > 4096.
static bool gemv_split_plan(const GemmArgs& ga, int* tw, int* splits) {
  const GemvSplitArgs& gs = ga.gsplit;
  const int n_tiles = (ga.N + 15) / 16, KS = ga.K / 32;
  if (!gs.part || !gs.cnt || (ga.norm_g && !gs.ss) || ga.a_bf16 || ga.K % 32 || n_tiles + 3 > gs.max_tiles)
    return false;
  if (!ga.norm_g && ga.K <= 4096) return false;
  int best = 0;
  for (int t = 4; t >= 2; --t) {
    const int groups = (n_tiles + t - 1) / t;
    for (int S = GEMV_SPLIT_MAX; S >= 2; S /= 2)
      if (KS % (S * GEMV_SPLIT_NW) == 0 && KS / (S * GEMV_SPLIT_NW) >= 4 && groups * S <= num_cus() &&
          groups * S > best) {
        best = groups * S;
        *tw = t;
        *splits = S;
      }
  }
  return best > 0;
}

struct GemvLaunch {
  template <typename TA, bool NORM, int KIND>
  static hipError_t run(const GemmArgs& ga, hipStream_t st) {
    if constexpr (AIsPair<TA>::value) {
      return hipErrorInvalidValue;   // the GEMV splits its activations itself
    } else {
    const int n_tiles = (ga.N + 15) / 16;
    if constexpr (gemv_split_kind<NORM, KIND>() && AIsFloat<TA>::value) {
      int tw = 0, S = 0;
      if (gemv_split_plan(ga, &tw, &S)) {
        const dim3 grid(((n_tiles + tw - 1) / tw) * S), block(GEMV_SPLIT_NW * 64);
        switch (tw) {
          case 4: return launch1(gemm_gemv_splitk_bf16<4, GEMV_SPLIT_NW, NORM, KIND>, grid, block, st, ga);
          case 3: return launch1(gemm_gemv_splitk_bf16<3, GEMV_SPLIT_NW, NORM, KIND>, grid, block, st, ga);
          default: return launch1(gemm_gemv_splitk_bf16<2, GEMV_SPLIT_NW, NORM, KIND>, grid, block, st, ga);
        }
      }
    }
    // few tiles (up to one per CU) or K != 4096: one workgroup
    // per tile, A streamed with W, so that several workgroups may share a CU and every tile
    // is in flight at once; otherwise one workgroup per CU with the A slice stationary,
    // walking the tiles (the deferred epilogue buffer bounds the tiles per workgroup)
    if (n_tiles <= num_cus() || ga.K != 32 * GEMV_NW * GEMV_CH) {
      // 16 waves split K whenever it divides (one workgroup per tile, up to the 8-wave form's
      // grid): each wave's share is then one chunk in flight at K = 4096 (O), three at 12288
      // (down), instead of two and six - these launches are bound by their chain of load
      // round trips, not by bytes (O and down: 21.0 -> 20.2 us)
      if (ga.K % (32 * 16) == 0 && n_tiles <= 8 * num_cus())
        return launch1(gemm_gemv_bf16<TA, 16, NORM, false, KIND>, dim3(n_tiles), dim3(16 * 64), st, ga);
      int grid = n_tiles;
      if (grid > 8 * num_cus()) grid = 8 * num_cus();
      if (KIND != EPI_ARGMAX && grid * GEMV_MAX_TILES < n_tiles)
        grid = (n_tiles + GEMV_MAX_TILES - 1) / GEMV_MAX_TILES;
      return launch1(gemm_gemv_bf16<TA, GEMV_NW, NORM, false, KIND>, dim3(grid), dim3(GEMV_NW * 64), st, ga);
    } else {
      int grid = n_tiles < num_cus() ? n_tiles : num_cus();
      if (KIND != EPI_ARGMAX && grid * GEMV_MAX_TILES < n_tiles)
        grid = (n_tiles + GEMV_MAX_TILES - 1) / GEMV_MAX_TILES;
      return launch1(gemm_gemv_bf16<TA, GEMV_NW, NORM, true, KIND>, dim3(grid), dim3(GEMV_NW * 64), st, ga);
    }
    }
  }
};

// bf16 models, M <= 16, K a multiple of 32 * GEMV_NW (checked by launch_gemm)
hipError_t launch_gemv(const GemmArgs& ga, hipStream_t st) { return dispatch_gemm<GemvLaunch>(ga, st); }

// The convolution's correction GEMM with the convolution as its epilogue: the 16-wave
// streamed form, one workgroup per 16-column tile (128 channels).
bool gemv_dconv_supported(int M, int K) {
  const int n_tiles = (K / 8 + 15) / 16;
  return M >= 1 && M <= 16 && K % (32 * 16) == 0 && n_tiles * 4 <= num_cus();
}

hipError_t launch_gemv_dconv(const GemmArgs& ga, hipStream_t st) {
  if (ga.a_bf16 || ga.N * 8 != ga.K || !gemv_dconv_supported(ga.M, ga.K) || !ga.e.dconv_base ||
      !ga.e.out || ga.e.B < 1)
    return hipErrorInvalidValue;
  const int n_tiles = (ga.N + 15) / 16;
  if (ga.norm_g)
    return launch1(gemm_gemv_bf16<float, 16, true, false, EPI_DCONV>, dim3(n_tiles), dim3(16 * 64), st, ga);
  return launch1(gemm_gemv_bf16<float, 16, false, false, EPI_DCONV>, dim3(n_tiles), dim3(16 * 64), st, ga);
}

}  // namespace dflash
