// Internal launchers of libdflash (host side).  Every launcher only enqueues work on the
// given stream; shapes were validated by the caller (api.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dflash {

enum Dt { F32 = 0, BF16 = 1 };

// B operand of a GEMM: rows of W [N, K] (row stride ldb elements), possibly split into
// up to 8 equal row segments at different addresses (the injection GEMM covers every
// draft layer's K/V row block in one launch).
struct BSeg {
  const void* ptr[8];
  int seg_rows;   // rows per segment (N when nseg == 1)
  int nseg;
  int ldb;
};

// Activations (h, q, attention output, SwiGLU output, fused injection rows) are float32;
// K/V (block and cache) and tapped features are stored in the model dtype.  For bfloat16
// models the activations that feed GEMMs (h, attention output, SwiGLU output, fused
// injection rows) are kept in the MFMA A-fragment order of common.h (afrag = 1) and the
// weight matrices in the B-fragment order; float32 models keep both row-major.
enum EpiKind {
  EPI_STORE_F32 = 0,  // out[row*ldo + col] = acc (float)
  EPI_RESID,          // h += acc; optional hdbg / tap (model dtype) copies
  EPI_QKV,            // RoPE q, k; write q (float), k_blk, v_blk^T (and the block K/V into a cache)
  EPI_SWIGLU,         // act = SiLU(gate) * up (float)
  EPI_INJECT_KV,      // RoPE K, scatter K and V of every draft layer into the paged cache
  EPI_ARGMAX,         // per-row argmax (packed 64-bit atomic max); optional float logits
  EPI_DCONV           // DFlash 2 convolution from its correction coefficients (M <= 16 GEMV only)
};

struct EpiArgs {
  int kind;
  int afrag;      // 1: out / h / act are float32 in the A-fragment order (row stride ignored)
  int act_pair;   // EPI_SWIGLU: act holds compensated operand planes (bf16) instead
  // EPI_STORE_*
  void* out;
  int ldo;
  // EPI_RESID
  float* h;
  int ldh;
  float* hdbg;
  void* tap;
  int tap_ld, tap_col;
  // EPI_QKV / EPI_INJECT_KV geometry
  int B, Bp, Hq, Hkv, hd;
  const float2* rope;       // [M, hd/2] (cos, sin) of each row's position
  const int32_t* seq_len;
  float* q;
  void* kblk;
  void* vblkT;
  void* kblk_lo;            // bf16 models: low parts (x - bf16(x)) of k_blk / v_blk^T, zero
  void* vblkT_lo;           // when the block is written into a cache (verification)
  // paged cache: per-layer pools (EPI_QKV uses slot 0), block table, bounds
  void* kp[8];
  void* vp[8];
  const int32_t* block_table;
  int max_pages, num_pages, batch;
  int32_t* err;
  int has_cache;
  // EPI_INJECT_KV rows
  const int32_t* row_seq;
  const int32_t* row_pos;
  int pos_relative;
  int pos_limit;            // rows with row_pos outside [0, pos_limit) are skipped (flagged)
  // EPI_SWIGLU
  float* act;
  int F;
  // EPI_ARGMAX: keys[row] for every row; the optional float logits copy skips the first
  // row of every skipB-row block when skipB != 0 (the drafter's anchor rows)
  unsigned long long* keys;
  float* logits;
  int skipB;
  // and, when ids_cnt != NULL (taken by the M <= 16 GEMV only), work on the finished keys
  // by the launch's last workgroup (arrival counter ids_cnt, zero between launches), for
  // blocks of ids_B rows: the draft ids of the masked rows when ids_out != NULL
  // (ids_out[b (ids_B - 1) + j - 1] = argmax of row b ids_B + j, j >= 1), the greedy
  // acceptance of acc_drafts when acc_tau != NULL (acc_g, acc_tau, acc_bonus as
  // launch_accept writes them)
  int32_t* ids_out;
  unsigned* ids_cnt;
  int ids_B;
  const int32_t* acc_drafts;
  int32_t* acc_g;
  int32_t* acc_tau;
  int32_t* acc_bonus;
  // sampling instead of argmax: key = logit / temperature + Gumbel noise of draw (counter,
  // purpose 0, b = row / B, i = row % B, v = column)
  int sample;
  float temperature;
  unsigned long long seed;
  unsigned counter;
  // EPI_DCONV: the GEMM's outputs are the correction coefficients of a two-tap convolution
  // of its own A rows x (normalised by the A-side RMSNorm when there is one):
  // y[m][c] = (base[c] + acc[m][2(c/16)]) x[m][c] + (base[D + c] + acc[m][2(c/16) + 1]) x[p][c]
  // with p = m - 1 inside a B-row block (p = m for its first row); out (A-fragment order,
  // row length D = K) = y, or += y when dconv_accumulate; hdbg (row-major) gets the result
  const void* dconv_base;   // [2, D] (bf16)
  int dconv_accumulate;
};

// Scratch of the M > 16 GEMMs of bf16 models.
//  * K splits of the row-resident GEMM (gemm_rows.hip): raw partial accumulators of every
//    split in fragment order, [splits][16-row blocks][16-column tiles][256] floats, and
//    partial sums of squares [splits][row blocks * 16].  part == NULL: never split.
//  * pair: the float32 activations of one GEMM as compensated (hi, lo) bf16 planes with the
//    A-side RMSNorm folded in (pair_split), 4 bytes per element; NULL: the GEMM kernels
//    split the activations themselves.
struct SplitArgs {
  float* part;
  float* ss;
  size_t part_bytes;   // capacity of `part`
  int splits, mb_pad, nt_pad;
  void* pair;
  size_t pair_bytes;   // capacity of `pair`
};
#define ROWS_MAX_SPLITS 8
#define ROWS_MAX_NORM_K 16384          // A-side norm gains held in LDS
#define ROWS_SPLIT_BYTES ((size_t)32 << 20)

// Scratch of the K-split M <= 16 GEMV: each workgroup takes 2-4 16-column tiles over one
// of `splits` K ranges; the last of a column group's workgroups to arrive sums the partial
// tiles in split order and runs the epilogue.
#define GEMV_SPLIT_MAX 8
struct GemvSplitArgs {
  float* part;          // [splits][groups][tiles a group][64 lanes][4]: partial tiles
  float* ss;            // [splits][groups][16]: partial sums of squares (A-side norm)
  unsigned* cnt;        // [groups]: arrivals within the running launch; zero between launches
  int max_tiles;        // capacity: splits x groups x tiles a group <= GEMV_SPLIT_MAX max_tiles
};
// scratch for GEMMs of up to max_n columns: tile capacity and the bytes of part and ss
int gemv_split_tiles(int max_n);
size_t gemv_split_part_bytes(int max_n);
size_t gemv_split_ss_bytes(int max_n);

struct GemmArgs {
  const void* A;        // [M, K]: float32 activations (A-fragment order for bf16 models), or
                        // caller-supplied bf16 rows (row-major, stride lda) when a_bf16
  int a_bf16;
  int lda;
  BSeg B;               // bf16 models: segments of B-fragment-ordered weights (ldb ignored)
  int M, N, K;
  const void* norm_g;   // A-side RMSNorm gain [K] (model dtype) or NULL
  float eps;
  EpiArgs e;
  SplitArgs split;      // bf16 models, M > 16: K-split and operand scratch
  int a_pair;           // set by launch_gemm: A holds (hi, lo) planes (pair_split), no norm
  GemvSplitArgs gsplit; // bf16 models, M <= 16, no norm: K-split scratch (or none)
};
// split scratch bytes for GEMMs of up to `rows` rows and `max_n` columns: (part, ss)
size_t rows_split_bytes(int rows, int max_n);
size_t rows_split_ss_bytes(int rows);
// operand-plane scratch bytes for GEMMs of up to `rows` rows and `max_k` reduction length
size_t pair_plane_bytes(int rows, int max_k);

// acc = A x W^T over the full K, then the epilogue.
hipError_t launch_gemm(int dt, const GemmArgs& g, hipStream_t st);
// whether launch_gemm takes the M <= 16 GEMV for these arguments
bool gemm_takes_gemv(int dt, const GemmArgs& g);
// The DFlash 2 convolution fused into its correction GEMM (EPI_DCONV): bf16 models, M <= 16,
// N = K / 8 with K a multiple of 512 and at most one 16-column tile per four CUs.
bool gemv_dconv_supported(int M, int K);
hipError_t launch_gemv_dconv(const GemmArgs& g, hipStream_t st);

// Paged-cache view of one layer.
struct KvLayer {
  void* k;                  // [num_pages, Hkv, 64, d]
  void* v;                  // [num_pages, Hkv, d, 64]
  const int32_t* block_table;
  const int32_t* seq_len;
  int max_pages, num_pages, batch;
  int32_t* err;
};

struct AttnPlan {
  int n_ctx_splits;   // context splits (grid dimension, before the block split)
  int split_len;      // keys per context split (multiple of 64)
  int n_rg;           // 64-row groups of the G*B query rows of one KV head
  int kv_stream;      // context K/V loads carry the non-temporal hint
};
// n_layers, d: the model's layers and head size (the K/V footprint of all its layers decides
// whether the context is streamed past the caches)
AttnPlan attn_plan(int dt, int batch, int Hkv, int G, int B, int ctx_cap, int n_layers = 1, int d = 128);
size_t attn_partial_floats(const AttnPlan& p, int batch, int Hkv, int d);

// o[M, Hq d] = softmax(q k^T / sqrt(d)) v over [context ; block] (causal inside the block
// when `causal`), one query row per (sequence, block position, head).  `part` holds the
// per-split partials (attn_partial_floats floats).  bf16 models take the block's own K/V as
// (kblk + kblk_lo, vblkT + vblkT_lo).
hipError_t launch_attention(int dt, const AttnPlan& p, const float* q, const void* kblk,
                            const void* vblkT, const void* kblk_lo, const void* vblkT_lo,
                            const KvLayer& kv, int batch, int B, int Bp, int Hq, int Hkv, int d,
                            int causal, float* part, float* o, int o_afrag, hipStream_t st);
// o_afrag: 0 row-major float32, 1 A-fragment order, 2 compensated operand planes (bf16)

// ---- row kernels (elementwise.hip) ----
struct EmbedArgs {
  const int32_t* ids;       // mode 1: drafts [batch, B-1]
  const int32_t* anchor;    // [batch]
  int mode, batch, B, mask_id;
  const void* E;
  int V, D;
  float* h;
  int afrag;
  float* hdbg;
  unsigned long long* keys;
  int n_keys;
  int32_t* err;
  const int32_t* seq_len;   // rows sit at positions seq_len[b] + j
  int hd;
  double rope_base;
  float2* rope;             // [batch*B, hd/2] out
  unsigned* zero;           // [n_zero] counters zeroed for the step (K-split GEMV arrivals)
  int n_zero;
};
// h[r] = E[token(r)] (float32), r = b*B + j:
// token = anchor[b] for j == 0, else mask_id (mode 0) or ids[b*(B-1) + j-1] (mode 1).
// Also writes the rows' RoPE (cos, sin) table and zeroes the argmax keys and `zero`.
hipError_t launch_embed(int dt, const EmbedArgs& a, hipStream_t st);
// one read of n16 16-byte words at src (plain or non-temporal loads), 1024 workgroups, one
// 16-byte xor per workgroup to sink
hipError_t launch_probe_read(const void* src, size_t n16, int nontemporal, void* sink, hipStream_t st);

// RoPE (cos, sin) table of injection rows: position row_pos[r] (+ seq_len[row_seq[r]]).
hipError_t launch_rope_rows(const int32_t* row_seq, const int32_t* row_pos, int pos_relative,
                            const int32_t* seq_len, int batch, int rows, int hd, double base,
                            float2* rope, hipStream_t st);

// ids[b*(B-1) + j-1] = argmax index decoded from keys[b*B + j], j = 1 .. B-1.
hipError_t launch_unpack_ids(const unsigned long long* keys, int batch, int B, int32_t* ids,
                             hipStream_t st);
// g[b*B + j] = argmax of verify row j; tau, bonus of the longest accepted draft prefix.
hipError_t launch_accept(const unsigned long long* keys, const int32_t* drafts, int batch, int B,
                         int32_t* g, int32_t* tau, int32_t* bonus, hipStream_t st);
hipError_t launch_commit(int32_t* seq_t, int32_t* seq_d, int32_t* err_t, int32_t* err_d,
                         const int32_t* tau, int batch, int B, hipStream_t st);
// Rejection-sampling verification of every sequence's block at temperature T.  zt: target
// logits [batch, B, V]; zd: drafter logits of positions 1 .. B-1 [batch, B-1, V]; drafts
// [batch, B-1].  Writes tau[b] and next_token[b].  Scratch (workspace):
#define SAMPLE_MAX_CHUNKS 64
struct SampleWs {
  float2* part;              // [batch * (2B - 1)][chunks] (max, sum) partials
  float* lse;                // [batch * (2B - 1)] row log-sum-exps
  int32_t* acc;              // [batch] accepted prefix
  unsigned long long* keys;  // [batch][chunks] Gumbel-max keys
};
int sample_chunks(int V);   // vocabulary chunks per row, 1 .. SAMPLE_MAX_CHUNKS
hipError_t launch_verify_sampled(const float* zt, const float* zd, const int32_t* drafts, int batch,
                                 int B, int V, float temperature, unsigned long long seed,
                                 unsigned counter, const SampleWs& ws, int32_t* tau,
                                 int32_t* next_token, int32_t* err, hipStream_t st);

// DFlash 2 two-tap dynamic convolution of M block rows (B rows per sequence):
// out[r] (=, or += when accumulate) k0 * x_r + k1 * x_p, p = r - 1 (the sequence's first row:
// p = r), k_j[c] = base[j][c] + corr[r][2 (c / 16) + j].  With norm_g, x = RMSNorm(x; norm_g)
// (each row's own rstd).  x, out: float [M, D], A-fragment order when afrag, else row-major;
// hdbg: optional row-major copy of out after the add.
struct DconvArgs {
  const float* x;
  const void* norm_g;
  float eps;
  const float* corr;   // [M, D / 8] row-major
  const void* base;    // [2, D] (model dtype)
  int M, D, B, afrag, bf16, accumulate;
  float* out;
  float* hdbg;
};
hipError_t launch_dconv(const DconvArgs& a, hipStream_t st);

// DFlash 2 path selector (select.hip).  Top-k keys of every chunk of every logit row
// (keys [rows][chunks][16]; *chunks returns the chunk count), their merge into candidate
// ids with the gather of the candidates' and anchors' embedding rows, and the scoring walk.
hipError_t launch_topk(const float* logits, int rows, int V, int k, unsigned long long* keys,
                       int* chunks, hipStream_t st);
hipError_t launch_topk_merge(const unsigned long long* keys, int chunks, int k, int batch, int B,
                             const void* embed, int D, int esz, const int32_t* anchor, int V,
                             int32_t* err, int32_t* cand, int32_t* cand_out, void* gather,
                             hipStream_t st);
hipError_t launch_select(const float* P, const float* Hh, const float* logits, const int32_t* cand,
                         int batch, int B, int k, int r, int V, float* S, int32_t* draft_ids,
                         hipStream_t st);

}  // namespace dflash
