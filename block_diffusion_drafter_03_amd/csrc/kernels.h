// Internal launchers of libdflash (host side).  Every launcher only enqueues work on the
// given stream; shapes were validated by the caller (api.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dflash {

enum Dt { F32 = 0, BF16 = 1 };

// B operand of a GEMM: rows of W [N, K] (row stride ldb elements), possibly split into
// up to 8 equal row segments living at different addresses (one per draft layer when
// the injection GEMM covers every layer's K/V projection in one launch).
struct BSeg {
  const void* ptr[8];
  int seg_rows;   // rows per segment (N when nseg == 1)
  int nseg;
  int ldb;
};

// C[s][M][N] (float32; s < splits) = A[M, K] (row stride lda) x W^T.
int gemm_splits(int dt, int M, int N, int K);
hipError_t launch_gemm(int dt, const void* A, int lda, const BSeg& B, float* C, int M, int N,
                       int K, int splits, hipStream_t st);

// Paged-cache view of one layer.
struct KvLayer {
  void* k;                  // [num_pages, Hkv, 64, d]
  void* v;                  // [num_pages, Hkv, d, 64]
  const int32_t* block_table;
  const int32_t* seq_len;
  int max_pages, num_pages;
  int32_t* err;
};

struct AttnPlan {
  int n_ctx_splits;   // context splits (grid dimension, before the block split)
  int split_len;      // keys per context split (multiple of 128)
  int n_rg;           // 64-row groups of the G*B query rows of one KV head
};
AttnPlan attn_plan(int dt, int batch, int Hkv, int G, int B, int ctx_cap);
size_t attn_partial_floats(const AttnPlan& p, int batch, int Hkv, int d);

// o[M, Hq d] = softmax(q k^T / sqrt(d)) v over [context ; block] (causal inside the block
// when `causal`), one query row per (sequence, block position, head).
hipError_t launch_attention(int dt, const AttnPlan& p, const void* q, const void* kblk,
                            const void* vblkT, const KvLayer& kv, int batch, int B, int Bp,
                            int Hq, int Hkv, int d, int causal, float* part, void* o,
                            hipStream_t st);

// ---- row / elementwise kernels (elementwise.hip) ----
// h[r] = E[token(r)] (float32).  mode 0: token = j == 0 ? anchor[b] : mask_id; mode 1:
// token = ids[r].  hdbg (if not NULL) receives a copy.
hipError_t launch_embed(int dt, const int32_t* ids, const int32_t* anchor, int mode, int batch,
                        int B, int mask_id, const void* E, int V, int D, float* h, float* hdbg,
                        int32_t* err, hipStream_t st);

struct RowFin {
  const float* C;      // split partials [S][rows][N] (may be NULL: x = h)
  int S;
  size_t split_stride; // elements between splits
  int N;               // row width (== D)
  float* h;            // residual stream [rows, N] (NULL: x = sum of partials)
  int add_resid;       // x = h + sum(C) (else x = sum(C))
  int write_h;         // h = x
  float* hdbg;         // copy of x [rows, N] or NULL
  void* tap;           // tap output (model dtype) or NULL: tap[r * tap_ld + tap_col + c] = x
  int tap_ld, tap_col;
  const void* g;       // RMSNorm gain or NULL (no normalised output)
  void* u;             // normalised output (model dtype)
  int compact_B;       // 0: u row = r; else skip rows with r % B == 0 and write r - r/B - 1
  float eps;
};
hipError_t launch_row_finalize(int dt, const RowFin& f, int rows, hipStream_t st);

// q/k rotation + v transpose after the QKV projection.  Rows r = b*B + j at position
// seq_len[b] + j.  When `cache` is set the block's K/V are also written into it.
hipError_t launch_qkv_post(int dt, const float* C, int S, size_t split_stride, int batch, int B,
                           int Bp, int Hq, int Hkv, int d, double rope_base,
                           const int32_t* seq_len, void* q, void* kblk, void* vblkT,
                           const KvLayer* cache, hipStream_t st);

// act[m, j] = SiLU(g) * u with g = C[m, j], u = C[m, F + j] (summed over splits).
hipError_t launch_swiglu(int dt, const float* C, int S, size_t split_stride, int M, int F,
                         void* act, hipStream_t st);

// Injection scatter: C2[r] holds, per draft layer, [K (Hkv d) | V (Hkv d)]; K is rotated
// at the row's position and both are written into the layer's pages.
hipError_t launch_inject_scatter(int dt, const float* C2, int S, size_t split_stride, int rows,
                                 int L, int Hkv, int d, double rope_base,
                                 const int32_t* row_seq, const int32_t* row_pos, int pos_relative,
                                 void* const* kpools, void* const* vpools,
                                 const int32_t* block_table, const int32_t* seq_len,
                                 int max_pages, int num_pages, int batch, int32_t* err,
                                 hipStream_t st);

// ids[r] = argmax_v logits[r, v] (lowest index on ties).
hipError_t launch_argmax(const float* logits, int rows, int V, int32_t* ids, hipStream_t st);
hipError_t launch_accept(const int32_t* block_ids, const int32_t* g, int batch, int B,
                         int32_t* tau, int32_t* bonus, hipStream_t st);
hipError_t launch_commit(int32_t* seq_t, int32_t* seq_d, int32_t* err_t, int32_t* err_d,
                         const int32_t* tau, int batch, int B, hipStream_t st);

}  // namespace dflash
