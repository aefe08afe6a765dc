// DFlash 2 path selector ([DF] section 7.1, "Problem 1: Selection Headroom"): top-k
// candidates of every masked position, the bilinear pair scores
//   S_t(a, b) = U_t(b) + <A(a) * H(h_t), B(b)>
// and the greedy walk from the anchor.  The projections A, B (of the gathered candidate
// embeddings) and H (of the final hidden states) run as ordinary GEMMs between these
// launches; here:
//   1. topk_partial_kernel: the top-k keys of every 4096-id chunk of every logit row;
//   2. topk_merge_kernel:   the row's top-k over its chunks -> candidate ids, and the
//                           candidates' (and each anchor's) embedding rows gathered as the
//                           projection GEMM's A operand;
//   3. select_score_kernel: every pair score of every position in float32, in parallel;
//   4. select_walk_kernel:  the greedy walk over the scores.
// Keys are the packed (value, id) keys of the argmax epilogue: larger value first, equal
// values to the lower id.
#include "epilogue.h"

namespace dflash {

#define TOPK_MAX 16
#define TOPK_CHUNK 4096
#define TOPK_THREADS 256

// 64-bit DPP move (both halves with the same control): lane i reads the lane CTRL names
template <int CTRL>
DF_DEV unsigned long long dpp_u64(unsigned long long k) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)k, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(k >> 32), CTRL, 0xF, 0xF, false);
  return ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo;
}
DF_DEV unsigned long long umax_u64(unsigned long long a, unsigned long long b) { return a > b ? a : b; }
DF_DEV unsigned long long readlane_u64(unsigned long long k, int lane) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)k, lane);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(k >> 32), lane);
  return ((unsigned long long)hi << 32) | lo;
}

// the largest key of the wave, on every lane (the whole wave must be active): DPP within
// each row of 16 lanes (quad swaps 1 and 2, half-row mirror, row mirror), then the four
// rows' results read out as scalars - no LDS round trips
DF_DEV unsigned long long wave_max_u64(unsigned long long k) {
  k = umax_u64(k, dpp_u64<0xB1>(k));    // quad_perm [1, 0, 3, 2]
  k = umax_u64(k, dpp_u64<0x4E>(k));    // quad_perm [2, 3, 0, 1]
  k = umax_u64(k, dpp_u64<0x141>(k));   // row_half_mirror
  k = umax_u64(k, dpp_u64<0x140>(k));   // row_mirror
  return umax_u64(umax_u64(readlane_u64(k, 0), readlane_u64(k, 16)),
                  umax_u64(readlane_u64(k, 32), readlane_u64(k, 48)));
}

// k rounds over a wave's keys (the first n <= N per lane, n uniform over the wave): each
// round takes the largest remaining key of the wave and removes it from its lane.  Keys are
// distinct (the id is part of the key), a removed key is 0, and an exhausted wave yields 0.
template <int N>
DF_DEV void wave_topk(unsigned long long (&key)[N], int n, int k, unsigned long long* out) {
  for (int r = 0; r < k; ++r) {
    unsigned long long m = 0ull;
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (i < n) m = key[i] > m ? key[i] : m;
    const unsigned long long w = wave_max_u64(m);
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (i < n) key[i] = key[i] == w ? 0ull : key[i];
    if ((threadIdx.x & 63) == 0) out[r] = w;
  }
}

// Pruning before the rounds.  T = the k-th largest of the 64 lane maxima bounds the wave's
// top k from below (those k maxima are k distinct keys >= T), so the rounds need only the
// keys >= T - usually a little over k of the wave's N x 64.  They are compacted into one
// key per lane through LDS slots `cs` (64 per wave; the caller's barrier between the two
// halves makes them visible).  Step 1 returns the lane's candidates' first slot; step 2 runs
// the rounds over the compacted keys, or over all of them when T = 0 (fewer than k keys) or
// more than 64 keys tie at or above T.
template <int N>
DF_DEV void prune_stage(const unsigned long long (&key)[N], int k, unsigned long long* cs,
                        unsigned long long& T, int& total) {
  const int lane = threadIdx.x & 63;
  unsigned long long m = 0ull;
#pragma unroll
  for (int i = 0; i < N; ++i) m = key[i] > m ? key[i] : m;
  unsigned long long mm = m;
  T = 0ull;
  for (int r = 0; r < k; ++r) {
    const unsigned long long x = wave_max_u64(mm);
    mm = mm == x ? 0ull : mm;
    T = x;
  }
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) cnt += key[i] && key[i] >= T ? 1 : 0;
  int incl = cnt;   // inclusive prefix of the counts over the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  total = __shfl(incl, 63, 64);
  int pos = incl - cnt;
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (key[i] && key[i] >= T) {
      if (pos < 64) cs[pos] = key[i];
      ++pos;
    }
}
template <int N>
DF_DEV void prune_finish(unsigned long long (&key)[N], int k, const unsigned long long* cs,
                         unsigned long long T, int total, unsigned long long* out) {
  const int lane = threadIdx.x & 63;
  if (T != 0ull && total <= 64) {
    unsigned long long c[1] = {lane < total ? cs[lane] : 0ull};
    wave_topk<1>(c, 1, k, out);
  } else {
    wave_topk<N>(key, N, k, out);
  }
}

// grid (rows, chunks): chunk c of row `row` covers ids [c * clen, min(V, (c + 1) * clen)),
// clen <= TOPK_CHUNK; writes keys[(row * chunks + c) * TOPK_MAX + r], r < k.
__global__ __launch_bounds__(TOPK_THREADS) void topk_partial_kernel(const float* z, int V, int clen,
                                                                     int k,
                                                                     unsigned long long* keys) {
  constexpr int N = TOPK_CHUNK / TOPK_THREADS;
  __shared__ unsigned long long wk[TOPK_THREADS / 64][TOPK_MAX];
  __shared__ unsigned long long cs[TOPK_THREADS / 64][64];
  const int row = blockIdx.x, c = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float* zr = z + (size_t)row * V;
  const int v0 = c * clen, v1 = min(V, v0 + clen);
  unsigned long long key[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int v = v0 + threadIdx.x + i * TOPK_THREADS;
    const float x = zr[min(v, v1 - 1)];
    key[i] = v < v1 ? pack_argmax_key(x, v) : 0ull;
  }
  unsigned long long T;
  int total;
  prune_stage<N>(key, k, cs[w], T, total);
  __syncthreads();
  prune_finish<N>(key, k, cs[w], T, total, wk[w]);
  __syncthreads();
  if (w == 0) {
    // the 4 waves' lists (k <= 16 each, 64 keys) are one key per lane
    unsigned long long m[1];
    m[0] = lane < 4 * k ? wk[lane / k][lane % k] : 0ull;
    wave_topk<1>(m, 1, k, keys + ((size_t)row * gridDim.y + c) * TOPK_MAX);
  }
}

struct TopkMergeArgs {
  const unsigned long long* keys;   // [rows][chunks][TOPK_MAX]
  int chunks, k, B;                 // rows = batch * (B - 1)
  const void* embed;                // [V, D] model dtype
  int D, esz;
  const int32_t* anchor;            // [batch]
  int V;                            // vocabulary: an anchor outside [0, V) reads row 0
  int32_t* err;                     // device error word or NULL
  int32_t* cand;                    // [rows][TOPK_MAX] (workspace)
  int32_t* cand_out;                // [rows][k] or NULL
  void* gather;                     // [batch * (1 + (B - 1) k)][D] model dtype
};

// grid (rows, parts), 256 threads: wave 0 of every workgroup merges the row's chunk lists
// (one list per lane, chunks <= 64; the same result in each), then each of the row's `parts`
// workgroups copies its share of the candidates' embedding rows (and, at position 1, the
// anchor's) into the gather rows of the projection GEMM; part 0 writes the candidate ids.
__global__ __launch_bounds__(256) void topk_merge_kernel(TopkMergeArgs a) {
  __shared__ unsigned long long top[TOPK_MAX];
  __shared__ unsigned long long cs[64];
  const int row = blockIdx.x, lane = threadIdx.x & 63;
  const int b = row / (a.B - 1), t = row % (a.B - 1) + 1;
  // wave 0 merges (the other waves only pass the barriers)
  unsigned long long key[TOPK_MAX];
  unsigned long long T = 0ull;
  int ncand = 0;
  if (threadIdx.x < 64) {
    // unconditional loads (clamped to valid entries), masked afterwards
    const unsigned long long* src = a.keys + ((size_t)row * a.chunks + min(lane, a.chunks - 1)) * TOPK_MAX;
#pragma unroll
    for (int i = 0; i < TOPK_MAX; ++i) key[i] = src[i];
#pragma unroll
    for (int i = 0; i < TOPK_MAX; ++i) key[i] = lane < a.chunks && i < a.k ? key[i] : 0ull;
    prune_stage<TOPK_MAX>(key, a.k, cs, T, ncand);
  }
  __syncthreads();
  if (threadIdx.x < 64) prune_finish<TOPK_MAX>(key, a.k, cs, T, ncand, top);
  __syncthreads();
  if (blockIdx.y == 0 && (int)threadIdx.x < a.k) {
    const unsigned long long kk = top[threadIdx.x];
    const int id = kk ? unpack_argmax_idx(kk) : 0;   // fewer than k ids: id 0 (never when V >= k)
    a.cand[(size_t)row * TOPK_MAX + threadIdx.x] = id;
    if (a.cand_out) a.cand_out[(size_t)row * a.k + threadIdx.x] = id;
  }
  // gather: rows per sequence = 1 (anchor) + (B - 1) k
  const size_t rps = 1 + (size_t)(a.B - 1) * a.k;
  const size_t rb = (size_t)a.D * a.esz;   // bytes per row
  const size_t n16 = rb / 16;              // D * esz is a multiple of 16
  char* g = (char*)a.gather;
  const int nrow = a.k + (t == 1 ? 1 : 0);
  const int n16i = (int)n16, total = nrow * n16i;
  // an anchor id outside the vocabulary is read as row 0 and flagged (as the embedding does)
  int aid = a.anchor[b];
  if (aid < 0 || aid >= a.V) {
    if (threadIdx.x == 0 && t == 1) flag_error(a.err, DEVERR_TOKEN);
    aid = 0;
  }
  // this workgroup's share of the copies
  const int per = (total + gridDim.y - 1) / gridDim.y;
  const int p0 = blockIdx.y * per, p1 = min(total, p0 + per);
  // 8 independent 16-byte copies per thread in flight at a time (named registers: an array
  // here ends up in scratch)
  auto src = [&](int idx) {
    idx = min(idx, total - 1);
    const int j = idx / n16i;
    const int id = j < a.k ? unpack_argmax_idx(top[j]) : aid;
    return *(const uint4*)((const char*)a.embed + (size_t)id * rb + (size_t)(idx - j * n16i) * 16);
  };
  auto put = [&](int idx, const uint4& v) {
    if (idx >= p1) return;
    const int j = idx / n16i;
    const size_t drow = j < a.k ? b * rps + 1 + (size_t)(t - 1) * a.k + j : b * rps;
    *(uint4*)(g + drow * rb + (size_t)(idx - j * n16i) * 16) = v;
  };
  for (int i0 = p0 + threadIdx.x; i0 < p1; i0 += 256 * 8) {
    const uint4 v0 = src(i0), v1 = src(i0 + 256), v2 = src(i0 + 512), v3 = src(i0 + 768);
    const uint4 v4 = src(i0 + 1024), v5 = src(i0 + 1280), v6 = src(i0 + 1536), v7 = src(i0 + 1792);
    put(i0, v0);
    put(i0 + 256, v1);
    put(i0 + 512, v2);
    put(i0 + 768, v3);
    put(i0 + 1024, v4);
    put(i0 + 1280, v5);
    put(i0 + 1536, v6);
    put(i0 + 1792, v7);
  }
}

struct SelectArgs {
  const float* P;          // [batch * rps][2 r]: A(x) = columns 0 .. r-1, B(x) = r .. 2r-1
  const float* Hh;         // [batch * B][r]: H of every block row (row b*B + t)
  const float* logits;     // [batch * (B - 1)][V]
  const int32_t* cand;     // [batch * (B - 1)][TOPK_MAX]
  int B, k, r, V;
  float* S;                // [batch * (B - 1)][TOPK_MAX][TOPK_MAX]: S_t(pred p, cand j)
  int32_t* draft_ids;      // [batch][B - 1]
};

// grid (batch, B - 1), 256 threads = (predecessor p, candidate j) pairs of position t =
// blockIdx.y + 1, whose predecessors are the anchor (t = 1) or the k candidates of t - 1.
// Every position is scored independently (the scores need no pick).
#define WALK_MAX_R 512
__global__ __launch_bounds__(256) void select_score_kernel(SelectArgs a) {
  __shared__ float ah[TOPK_MAX][WALK_MAX_R + 4];   // A(pred) * H(h_t)
  __shared__ float bv[TOPK_MAX][WALK_MAX_R + 4];   // B(cand)
  const int b = blockIdx.x, t = blockIdx.y + 1, tid = threadIdx.x, r = a.r, k = a.k;
  const size_t rps = 1 + (size_t)(a.B - 1) * k;
  const float* Pb = a.P + (size_t)b * rps * 2 * r;
  const int np = t == 1 ? 1 : k;
  const float* hh = a.Hh + ((size_t)b * a.B + t) * r;
  for (int idx = tid; idx < np * r; idx += 256) {
    const int p = idx / r, c = idx % r;
    const size_t prow = t == 1 ? 0 : 1 + (size_t)(t - 2) * k + p;
    ah[p][c] = Pb[prow * 2 * r + c] * hh[c];
  }
  for (int idx = tid; idx < k * r; idx += 256) {
    const int j = idx / r, c = idx % r;
    bv[j][c] = Pb[(1 + (size_t)(t - 1) * k + j) * 2 * r + r + c];
  }
  const int row = b * (a.B - 1) + t - 1;
  const int p = tid / TOPK_MAX, j = tid % TOPK_MAX;
  const float u = j < k ? a.logits[(size_t)row * a.V + a.cand[(size_t)row * TOPK_MAX + j]] : 0.f;
  __syncthreads();
  if (p < np && j < k) {
    float s = 0.f;
    for (int c = 0; c < r; c += 4) {
      const float4 x = *(const float4*)&ah[p][c];
      const float4 y = *(const float4*)&bv[j][c];
      s = fmaf(x.x, y.x, s);
      s = fmaf(x.y, y.y, s);
      s = fmaf(x.z, y.z, s);
      s = fmaf(x.w, y.w, s);
    }
    a.S[((size_t)row * TOPK_MAX + p) * TOPK_MAX + j] = u + s;
  }
}

// grid (batch), 256 threads: the scores and candidate ids of the sequence into LDS, then the
// walk from the anchor: at each position the candidate of the largest score given the
// previous pick (ties to the lower id).
__global__ __launch_bounds__(256) void select_walk_kernel(SelectArgs a) {
  __shared__ float S[63 * TOPK_MAX * TOPK_MAX];
  __shared__ int32_t cid[63 * TOPK_MAX];
  const int b = blockIdx.x, n = a.B - 1, k = a.k;
  const size_t r0 = (size_t)b * n;
  const int total = n * TOPK_MAX * TOPK_MAX;
  // 8 independent loads per thread in flight at a time (entries no pick can read are
  // never written by the scoring kernel and are not used)
  for (int i0 = threadIdx.x; i0 < total; i0 += 256 * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = a.S[r0 * TOPK_MAX * TOPK_MAX + min(i0 + u * 256, total - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (i0 + u * 256 < total) S[i0 + u * 256] = v[u];
  }
  for (int i = threadIdx.x; i < n * TOPK_MAX; i += 256) cid[i] = a.cand[r0 * TOPK_MAX + i];
  __syncthreads();
  // the walk on wave 0: at each position lanes 0 .. k-1 hold the candidates' scores given
  // the previous pick; the largest (score, lower id) key wins
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int prev = 0;   // index of the predecessor among its position's rows
    for (int t = 0; t < n; ++t) {
      const int id = cid[t * TOPK_MAX + min(lane, k - 1)];
      const float x = S[(t * TOPK_MAX + prev) * TOPK_MAX + min(lane, k - 1)];
      const unsigned long long key = wave_max_u64(lane < k ? pack_argmax_key(x, id) : 0ull);
      const int best_id = unpack_argmax_idx(key);
      const unsigned long long hit = __ballot(lane < k && id == best_id);
      prev = (int)__builtin_ctzll(hit);
      if (lane == 0) a.draft_ids[r0 + t] = best_id;
    }
  }
}

hipError_t launch_topk(const float* logits, int rows, int V, int k, unsigned long long* keys,
                       int* chunks, hipStream_t st) {
  const int nch = std::min(SAMPLE_MAX_CHUNKS, std::max(1, (V + TOPK_CHUNK - 1) / TOPK_CHUNK));
  const int clen = (V + nch - 1) / nch;
  *chunks = nch;
  if (rows <= 0) return hipSuccess;
  if (k < 1 || k > TOPK_MAX || clen > TOPK_CHUNK) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_partial_kernel, dim3(rows, nch), dim3(TOPK_THREADS), 0, st, logits, V, clen, k,
                     keys);
  return hipGetLastError();
}

hipError_t launch_topk_merge(const unsigned long long* keys, int chunks, int k, int batch, int B,
                             const void* embed, int D, int esz, const int32_t* anchor, int V,
                             int32_t* err, int32_t* cand, int32_t* cand_out, void* gather,
                             hipStream_t st) {
  if (batch <= 0 || B < 2) return hipSuccess;
  if ((D * esz) % 16) return hipErrorInvalidValue;
  TopkMergeArgs a{keys, chunks, k, B, embed, D, esz, anchor, V, err, cand, cand_out, gather};
  // the gather (k or k + 1 embedding rows per row) over 4 workgroups per row
  hipLaunchKernelGGL(topk_merge_kernel, dim3(batch * (B - 1), 4), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_select(const float* P, const float* Hh, const float* logits, const int32_t* cand,
                         int batch, int B, int k, int r, int V, float* S, int32_t* draft_ids,
                         hipStream_t st) {
  if (batch <= 0 || B < 2) return hipSuccess;
  if (B > 64 || k < 1 || k > TOPK_MAX || r < 4 || r > WALK_MAX_R || r % 4) return hipErrorInvalidValue;
  SelectArgs a{P, Hh, logits, cand, B, k, r, V, S, draft_ids};
  hipLaunchKernelGGL(select_score_kernel, dim3(batch, B - 1), dim3(256), 0, st, a);
  hipLaunchKernelGGL(select_walk_kernel, dim3(batch), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dflash
