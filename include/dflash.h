/*
 * dflash.h - C ABI of libdflash: the DFlash drafter step and greedy block verification
 * on one AMD Instinct MI355X (gfx950).
 *
 * Pages the operations follow (cited by title and section):
 *   [DF]  "DFlash - Block Diffusion for Flash Speculative Decoding" (paper notes page)
 *   [TRY] "Trying "DFlash," a Diffusion-Model Approach to Parallel Draft-Token
 *         Generation, on Gemma" (llama.cpp experiment write-up)
 *
 * One decoding cycle is   draft_block -> verify_accept -> inject_ctx -> kv_commit
 * ([DF] section 4.5, "The Decoding Loop"): the drafter proposes B-1 tokens in one pass,
 * the target checks the whole block in one causal pass, the longest matching prefix plus
 * a bonus token is kept, and both KV caches advance by tau.
 *
 * Conventions for every call
 *  - Tensor arguments are DEVICE pointers owned by the caller.  The library never
 *    allocates or frees device memory and never synchronises the host: each call only
 *    enqueues kernels on `stream` (a hipStream_t; NULL = the null stream).  Outputs are
 *    valid once the stream reaches that point.
 *  - Host-side arguments (descriptors, pointer tables, sizes) are read during the call
 *    only and may be freed when it returns.
 *  - Return value: DFLASH_OK (0) or a negative dflash_status.  Argument, shape, dtype,
 *    capacity and workspace errors are detected on the host before anything is enqueued,
 *    so no cache or sequence length has been touched; DFLASH_E_HIP (a failed launch) may
 *    leave the call's earlier kernels enqueued.
 *  - Capacity is checked on the host against two host-side fields of dflash_kv:
 *    capacity_tokens (positions mapped for every sequence) and len_bound (an upper bound
 *    on every seq_len[b], kept by the caller and advanced by dflash_kv_commit), so a call
 *    that could write or read past the mapped pages returns DFLASH_E_CAPACITY instead of
 *    launching.
 *  - The workspace `ws` is scratch for the duration of the call's kernels: calls that may
 *    overlap on the device (different streams) need separate workspaces.  Its contents on
 *    entry do not matter: a draft or verify call clears the arrival counters its split
 *    GEMMs keep there in its first kernel.
 *  - Errors the host cannot see (an unmapped page, an out-of-range token id or tau) are
 *    detected on the device: the offending row or sequence is skipped and a bit is OR-ed
 *    into dflash_kv.error_flags (when that pointer is non-NULL).
 *  - Matrices are [out, in] (y = x W^T), two of them with their rows packed as described
 *    at DFLASH_W_QKV and DFLASH_W_GATE_UP.  float32 models pass them row-major.  bfloat16
 *    models pass every matrix except the token embedding (W_qkv, W_o, W_gate_up, W_down,
 *    lm_head, w_c) in the matrix-core fragment order: rows padded with zeros to a multiple
 *    of 16; element (n, k) of W [N, K] at
 *        ((n / 16 * (K / 32) + k / 32) * 64 + (k % 32) / 8 * 16 + n % 16) * 8 + k % 8,
 *    i.e. one contiguous 1 KB block per 16-row x 32-column tile, tiles row-major, which
 *    is the operand order of a 16x16x32 bf16 matrix instruction (lane l = 16 g + r holds
 *    row r, columns 8 g .. 8 g + 7).  The embedding stays row-major [vocab, hidden].
 *    Storage dtype (weights, caches, tapped features) is the model's dtype: float32 or
 *    bfloat16; logits and debug hidden states are always float32; ids are int32.  Between kernels the activations of a
 *    step live in the workspace in float32; a bfloat16 model's matrix units take them as
 *    a compensated pair of bfloat16 values (about 16 significant bits), so the result
 *    tracks a float32 evaluation over bfloat16 weights and caches.
 *  - Calls on distinct caches and streams may run concurrently; a model is immutable
 *    after creation.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DFLASH_OK = 0,
  DFLASH_E_ARG = -1,        /* NULL pointer, non-positive size, bad enum            */
  DFLASH_E_SHAPE = -2,      /* shape the kernels do not support, or inconsistent    */
  DFLASH_E_DTYPE = -3,      /* unknown dtype or mismatch between model and cache    */
  DFLASH_E_CAPACITY = -4,   /* the rows the call would touch pass capacity_tokens   */
  DFLASH_E_WORKSPACE = -5,  /* workspace NULL or smaller than dflash_workspace_bytes */
  DFLASH_E_HIP = -6         /* a HIP launch failed                                   */
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

/* Device-side error bits OR-ed into dflash_kv.error_flags. */
enum {
  DFLASH_DEVERR_PAGE = 1,   /* a row's page was unmapped (-1) or out of the pool      */
  DFLASH_DEVERR_TOKEN = 2,  /* a token id outside [0, vocab)                          */
  DFLASH_DEVERR_TAU = 4     /* kv_commit got tau outside [1, block]                   */
};

/* Per-layer weight table: layer_w[l * DFLASH_LAYER_TENSORS + slot]. */
enum {
  DFLASH_W_G_IN = 0,     /* [hidden]                 RMSNorm gain before attention       */
  DFLASH_W_QKV = 1,      /* [(Hq + 2 Hkv) d, hidden] rows: q heads, k heads, v heads;
                            within each q and k head the rows are rotary-interleaved:
                            packed row 2i = original row i, packed row 2i+1 = original
                            row i + d/2 (the two inputs of one rotate-half rotation sit
                            side by side); v heads are stored as they are               */
  DFLASH_W_O = 2,        /* [hidden, Hq d]           attention output projection          */
  DFLASH_W_G_POST = 3,   /* [hidden]                 RMSNorm gain before the FFN          */
  DFLASH_W_GATE_UP = 4,  /* [2 ffn, hidden]          rows interleaved: packed row 2j = gate
                            row j, packed row 2j+1 = up row j                           */
  DFLASH_W_DOWN = 5,     /* [hidden, ffn]            SwiGLU down projection               */
  DFLASH_LAYER_TENSORS = 6
};

/*
 * Model descriptor, for the drafter or the target.  A decoder layer is pre-norm:
 * h += Attn(RMSNorm(h)) W_o^T; h += (SiLU(u W_g^T) * (u W_u^T)) W_d^T with
 * u = RMSNorm(h); rotate-half RoPE on q and k.  The drafter shares the target's token
 * embedding and LM head ([DF] section 5.2, shared embedding and LM head).
 */
typedef struct dflash_model_desc {
  int32_t dtype;                /* dflash_dtype                                              */
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  float rms_eps;                /* RMSNorm epsilon                                            */
  float rope_base;              /* RoPE base; angles p * base^(-2i/d) evaluated in float64    */
  int32_t mask_token_id;        /* drafter: token placed at the B-1 masked positions          */
  int32_t n_taps;               /* drafter: k, the W_c input is k * hidden wide;
                                   target: number of tapped layers written to feats_out       */
  const int32_t* tap_layers;    /* target: host array [n_taps] of 0-indexed layers whose
                                   outputs are tapped, in concatenation order; drafter: NULL  */
  const void* embed;            /* [vocab, hidden]                                            */
  const void* lm_head;          /* [vocab, hidden]                                            */
  const void* final_norm;       /* [hidden]                                                   */
  const void* w_c;              /* drafter: fusion weight W_c [hidden, n_taps * hidden]       */
  const void* g_c;              /* drafter: gain of the RMSNorm after W_c [hidden]            */
  const void* const* layer_w;   /* host array [n_layers * DFLASH_LAYER_TENSORS]               */
  const void* const* dconv;     /* NULL, or a DFlash 2 drafter's two-tap convolutions: host
                                   array [n_layers * 8], see DFLASH_DCONV_* below            */
} dflash_model_desc;

/*
 * DFlash 2 two-tap dynamic convolution ([DF] section 7.1, "Problem 2: Suffix Decay"):
 * Conv(x)_t = k_{t,0} * x_t + k_{t,1} * x_{t-1}, depthwise, before and after each attention
 * and feed-forward sublayer; each coefficient is a base kernel plus a content-dependent
 * correction.  Readings: "before" acts on the sublayer's normalised input, "after" on its
 * output ahead of the residual add (h <- h + Conv_post(Sub(Conv_pre(RMSNorm(h))))); the
 * correction is linear in the convolution's input, one coefficient per tap per group of 16
 * channels: k_{t,j}[c] = base[j][c] + (x_t W_k^T)[2 (c / 16) + j]; the block's first row
 * (the anchor) reads itself, every later row its predecessor in the block.
 * dconv[l * 8 + 2 * conv] = base [2, hidden] (model dtype, row j = tap j) and
 * dconv[l * 8 + 2 * conv + 1] = W_k [hidden / 8, hidden] in the weight layout (row 2g + j =
 * tap j of channel group g), conv = DFLASH_DCONV_*.  Drafter only (no taps): hidden must be a
 * multiple of 128.
 */
enum {
  DFLASH_DCONV_PRE_ATTN = 0,
  DFLASH_DCONV_POST_ATTN = 1,
  DFLASH_DCONV_PRE_FFN = 2,
  DFLASH_DCONV_POST_FFN = 3
};

/*
 * Paged KV cache (the target's cache, or the drafter's own injected-context cache -
 * [TRY]: the drafter keeps an independent KV cache filled by injection).
 * Pages hold `page_size` consecutive positions of one sequence.  Per layer:
 *   K pool [num_pages, n_kv_heads, page_size, head_dim]   (K stored after RoPE)
 *   V pool [num_pages, n_kv_heads, head_dim, page_size]   (V stored transposed per page)
 * Position p of sequence b lives in page block_table[b * max_pages_per_seq + p / page_size]
 * at slot p % page_size.  seq_len[b] is the committed length n_b.
 *
 * Capacity ([DF] section 4.5: verification writes the block's K/V at n .. n+B-1 before
 * acceptance is known, so those positions must be mapped first).  The host cannot read
 * seq_len without a synchronisation, so the caller states two host-side bounds:
 *   capacity_tokens  positions 0 .. capacity_tokens-1 are mapped for every sequence
 *                    (0 <= capacity_tokens <= max_pages_per_seq * page_size);
 *   len_bound        an upper bound on every seq_len[b], set by the caller together with
 *                    seq_len; dflash_kv_commit adds `block` to it (tau <= block), and the
 *                    caller may lower it again after reading seq_len back.
 * draft_block needs len_bound <= capacity_tokens; verify_accept / verify_sampled and
 * kv_commit need len_bound + block <= capacity_tokens; inject_ctx needs its rows'
 * positions (pos_limit below) to fit.  Otherwise the call returns DFLASH_E_CAPACITY and
 * launches nothing.  The device checks every row again against the block table (a row
 * that still lands on an unmapped page is skipped and DFLASH_DEVERR_PAGE flagged).
 */
typedef struct dflash_kv {
  int32_t n_layers, n_kv_heads, head_dim;
  int32_t page_size;            /* must be 64                                                 */
  int32_t batch;                /* number of sequences                                        */
  int32_t max_pages_per_seq;    /* row length of block_table                                  */
  int32_t num_pages;            /* pages in each pool                                         */
  void* const* k_pool;          /* host array [n_layers] of device pointers                   */
  void* const* v_pool;          /* host array [n_layers] of device pointers                   */
  const int32_t* block_table;   /* device [batch, max_pages_per_seq]; -1 = unmapped          */
  int32_t* seq_len;             /* device [batch]                                             */
  int32_t* error_flags;         /* device [1] or NULL: DFLASH_DEVERR_* bits are OR-ed in      */
  int32_t capacity_tokens;      /* host: positions mapped for every sequence                  */
  int32_t len_bound;            /* host: upper bound on every seq_len[b]; kv_commit adds block */
} dflash_kv;

typedef struct dflash_model dflash_model;   /* opaque: shapes + non-owning weight pointers */

/* Validates the descriptor and copies it (host memory only).  Returns DFLASH_E_ARG,
 * _SHAPE or _DTYPE for descriptors the kernels cannot run.  bf16 models need
 * head_dim = 128, hidden and ffn multiples of 128, and n_q_heads a multiple of
 * n_kv_heads; float32 models need an even head_dim. */
int dflash_model_create(const dflash_model_desc* desc, dflash_model** out);
void dflash_model_destroy(dflash_model* model);

/* Human-readable name of a dflash_status. */
const char* dflash_status_str(int status);

/* Bytes of scratch workspace any call on `model` needs for `batch` sequences, blocks of
 * up to `block` tokens, cache capacity up to `max_ctx_tokens` positions per sequence,
 * and inject_ctx calls of up to `max_inject_rows` rows.  Returns 0 on bad arguments. */
size_t dflash_workspace_bytes(const dflash_model* model, int32_t batch, int32_t block,
                              int32_t max_ctx_tokens, int32_t max_inject_rows);

/*
 * KV injection ([DF] section 4.2 fusion equation and section 4.3 KV-injection equations):
 *   H_t = RMSNorm(feats W_c^T; g_c),  and for every draft layer i
 *   K_i = RoPE(H_t W_i^K^T, p),  V_i = H_t W_i^V^T,
 * written into the drafter's cache at position p of sequence row_seq[r] for each row r.
 * W_i^K, W_i^V are the k and v row blocks of layer i's DFLASH_W_QKV.
 *   feats    device [n_rows, n_taps * hidden] (model dtype): tapped target features.
 *   row_seq  device int32 [n_rows]: sequence of each row.
 *   row_pos  device int32 [n_rows]: position of each row, absolute when pos_relative = 0,
 *            else added to seq_len[row_seq[r]].
 *   pos_limit host int32: every row_pos[r] lies in [0, pos_limit).  The rows' positions
 *            then end before pos_limit (absolute) or len_bound + pos_limit (relative),
 *            which must not pass capacity_tokens (else DFLASH_E_CAPACITY, nothing
 *            launched).  A row outside [0, pos_limit) is skipped on the device and
 *            DFLASH_DEVERR_PAGE flagged.
 * seq_len is not changed (kv_commit advances it).  n_rows = 0 is a no-op (the row
 * arrays are then not read and may be NULL); n_rows < 0 or pos_limit < 1 is DFLASH_E_ARG.
 * A row whose sequence or position has no mapped page is skipped and DFLASH_DEVERR_PAGE
 * flagged.
 */
int dflash_inject_ctx(const dflash_model* draft, dflash_kv* draft_ctx, const void* feats,
                      int32_t n_rows, const int32_t* row_seq, const int32_t* row_pos,
                      int32_t pos_relative, int32_t pos_limit, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * One drafter step ([DF] section 4.4, parallel diffusion drafting; [TRY] appendix on the
 * drafter: mask-token queries and non-causal attention): the block
 * [anchor[b], mask x (block-1)] sits at positions seq_len[b] .. seq_len[b]+block-1, runs
 * through every draft layer in one pass with bidirectional attention over the injected
 * context and the whole block, and each masked position takes the argmax of its logits.
 *   anchor     device int32 [batch]
 *   draft_ids  device int32 [batch, block-1] (out)
 *   logits_dbg device float [batch, block-1, vocab] or NULL (out)
 *   hidden_dbg device float [n_layers+1, batch, block, hidden] or NULL (out): residual
 *              stream after the embedding and after each layer.
 * 1 <= block <= 64; the cache is only read (len_bound <= capacity_tokens).
 */
int dflash_draft_block(const dflash_model* draft, const dflash_kv* draft_ctx,
                       const int32_t* anchor, int32_t block, int32_t* draft_ids,
                       float* logits_dbg, float* hidden_dbg, void* ws, size_t ws_bytes,
                       void* stream);

/*
 * dflash_draft_block without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  It runs the same kernels as dflash_draft_block; their scratch lives in one
 * array of DFLASH_NOALLOC_SCRATCH_BYTES bytes compiled into the library, one copy per GPU,
 * held until the process ends.  Its device address is looked up once per device on the
 * first call made with that device current; nothing is allocated, then or later.
 *   Limit: the scratch the call needs (dflash_workspace_bytes(draft, batch, block,
 *   max_pages_per_seq * page_size, 0)) must fit DFLASH_NOALLOC_SCRATCH_BYTES, else
 *   DFLASH_E_WORKSPACE before any launch.  64 MiB holds e.g. a Qwen3-8B-shaped drafter
 *   step of 16 sequences x 16 rows over 8K-token caches.
 *   Sharing: every call on one GPU uses that GPU's single array, which keeps the last
 *   call's contents (the kernels initialise what they read).  Calls that may overlap on
 *   one GPU (different streams or threads) race on it: serialise them.
 * Other arguments, outputs and errors as dflash_draft_block.
 */
#define DFLASH_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int dflash_draft_block_noalloc(const dflash_model* draft, const dflash_kv* draft_ctx,
                               const int32_t* anchor, int32_t block, int32_t* draft_ids,
                               float* logits_dbg, float* hidden_dbg, void* stream);

/*
 * Block verification and greedy acceptance ([DF] section 4.5 steps 2-3; [TRY] Fig. 1:
 * the main model checks the block with causal attention in one parallel pass).
 * The target runs the block y = [x, d_1 .. d_{block-1}] (x = anchor[b], d = draft_ids[b])
 * at positions n = seq_len[b] .. n+block-1, causal inside the block with the whole cache
 * visible, and writes the block's K/V into the cache at those positions (tentatively:
 * only kv_commit makes them part of the sequence).  A prompt chunk is verified the same
 * way (its first token as anchor, the rest as drafts) to fill the cache.
 *   anchor        device int32 [batch]
 *   draft_ids     device int32 [batch, block-1] (may be NULL when block == 1)
 *   feats_out     device [batch, block, n_taps * hidden] (model dtype) or NULL (out):
 *                 outputs of the tapped layers, concatenated in tap order.
 *   target_argmax device int32 [batch, block] (out): g_j, greedy id after row j.
 *   tau, bonus    device int32 [batch] (out): a = leading j with d_j == g_{j-1},
 *                 tau = a + 1 in [1, block], bonus = g_a (the next anchor).
 *   logits_dbg    device float [batch, block, vocab] or NULL; hidden_dbg as in draft_block.
 * The cache must map positions up to seq_len[b] + block - 1: len_bound + block <=
 * capacity_tokens, else DFLASH_E_CAPACITY before any launch.
 */
int dflash_verify_accept(const dflash_model* target, dflash_kv* target_kv,
                         const int32_t* anchor, const int32_t* draft_ids, int32_t block,
                         void* feats_out, int32_t* target_argmax, int32_t* tau, int32_t* bonus,
                         float* logits_dbg, float* hidden_dbg, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * Sampling: temperature-T drafting and lossless rejection-sampling verification ([DF]
 * section 6.2, sampling at temperature 1; the DFlash 2 notes, section 7.2, name lossless
 * rejection sampling as the verifier).  The pages give no more detail; the rule is the
 * standard speculative-sampling one:
 *   * the drafter samples each masked position i = 1 .. block-1 from q_i = softmax(z_i / T);
 *   * the target's row j gives p_j = softmax(z^t_j / T); draft d_i is accepted while
 *     u_i < p_{i-1}(d_i) / q_i(d_i); a = the accepted prefix, tau = a + 1;
 *   * the emitted token (the next anchor) is drawn from norm(max(0, p_a - q_{a+1})) after a
 *     rejection, else from p_{block-1}.
 * Random numbers: draw number index + 1 of a splitmix64 stream seeded with `seed` (Vigna's
 * mixing function over the Weyl sequence of step 0x9E3779B97F4A7C15), index =
 * (((counter * 4 + purpose) * 4096 + b) * 128 + i) * 262144 + v, u = ((r >> 41) + 1/2) / 2^23;
 * purpose 0 = drafter noise (position i, id v), 1 = acceptance uniform (position i), 2 = noise
 * of the emitted token (target row a, id v).  Samples use the Gumbel-max identity: argmax of
 * x + G, G = -log(-log(u)), in float32.  A cycle passes the same (seed, counter) to both
 * calls and a new counter to the next cycle.  batch <= 4096, vocab <= 262144, 0 <= counter
 * < 2^25, temperature > 0, 2 <= block <= 64; the workspace is dflash_workspace_bytes'.
 *
 * dflash_draft_block_sampled: as dflash_draft_block, with the ids drawn as above.
 *   draft_logits device float [batch, block-1, vocab] (out, required): the drafter's logits
 *                of positions 1 .. block-1 (its proposal distribution, read by the verifier).
 * dflash_verify_sampled: as dflash_verify_accept (same target pass, cache writes and taps),
 * then the rejection rule.
 *   draft_logits  device float [batch, block-1, vocab] (in): from the drafting call.
 *   target_logits device float [batch, block, vocab] (out, required): the target's logits.
 *   tau           device int32 [batch] (out): a + 1.
 *   next_token    device int32 [batch] (out): the emitted token.
 * A draft id outside [0, vocab) counts as rejected and flags DFLASH_DEVERR_TOKEN.
 */
int dflash_draft_block_sampled(const dflash_model* draft, const dflash_kv* draft_ctx,
                               const int32_t* anchor, int32_t block, float temperature,
                               uint64_t seed, int32_t counter, int32_t* draft_ids,
                               float* draft_logits, void* ws, size_t ws_bytes, void* stream);
int dflash_verify_sampled(const dflash_model* target, dflash_kv* target_kv,
                          const int32_t* anchor, const int32_t* draft_ids,
                          const float* draft_logits, int32_t block, float temperature,
                          uint64_t seed, int32_t counter, void* feats_out, float* target_logits,
                          int32_t* tau, int32_t* next_token, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * DFlash 2 path selector ([DF] section 7.1, "Problem 1: Selection Headroom"): the drafter
 * keeps the top_k candidates of each masked position and scores every adjacent pair
 * (predecessor a, candidate b) as S_t(a, b) = U_t(b) + <A(a) * H(h_t), B(b)>; a greedy walk
 * from the anchor over the scores picks the drafts.  Readings (the page names the pieces,
 * not their inputs): U_t(b) = the raw logit z_t(b); A(a) = E[a] W_A and B(b) = E[b] W_B with
 * E the shared embedding; H(h_t) = RMSNorm(h_t; final norm) W_H with h_t the drafter's final
 * hidden state (the LM head's input); position 1's predecessor is the anchor, position t's
 * the candidate chosen at t - 1; candidates are the top_k logits (ties to the lower id), and
 * the walk's ties go to the lower id.  All scoring is in float32.
 *
 * dflash_selector: caller-owned weights in the drafter's dtype and weight layout (the
 * B-fragment order for bfloat16 models, row-major for float32 ones), K = hidden:
 *   w_ab  [2 * rank, hidden]: rows 0 .. rank-1 are W_A^T, rows rank .. 2 rank - 1 W_B^T.
 *   w_h   [rank, hidden]: W_H^T.
 *   rank  multiple of 16 in [16, 512] (the page's selector uses 256); top_k in [1, 16].
 *
 * dflash_selector_workspace_bytes: scratch of the selection (a second workspace, beside the
 * step workspace of dflash_workspace_bytes); 0 on invalid arguments.
 *
 * dflash_draft_block_select: the drafter pass of dflash_draft_block, then the selector.
 *   draft_ids     device int32 [batch, block-1] (out): the walk's picks.
 *   draft_logits  device float [batch, block-1, vocab] (out, required): the drafter's logits
 *                 of positions 1 .. block-1.
 *   candidates    device int32 [batch, block-1, top_k] (out) or NULL: each position's
 *                 candidates in descending logit.
 *   ws / sel_ws   the step workspace and the selector scratch.
 * 2 <= block <= 64; batch * (1 + (block - 1) * top_k) <= 2^20.
 */
typedef struct dflash_selector {
  const void* w_ab;
  const void* w_h;
  int32_t rank;
  int32_t top_k;
} dflash_selector;

size_t dflash_selector_workspace_bytes(const dflash_model* draft, const dflash_selector* sel,
                                       int32_t batch, int32_t block);
int dflash_draft_block_select(const dflash_model* draft, const dflash_kv* draft_ctx,
                              const int32_t* anchor, int32_t block, const dflash_selector* sel,
                              int32_t* draft_ids, float* draft_logits, int32_t* candidates,
                              void* ws, size_t ws_bytes, void* sel_ws, size_t sel_ws_bytes,
                              void* stream);

/*
 * Commit / rollback ([DF] section 4.5: accepted tokens are appended, the cycle repeats
 * from the updated context): seq_len[b] += tau[b] in the target cache and in the drafter
 * context (either may be NULL).  Rows written beyond the new length by verify_accept or
 * inject_ctx are left in place and are overwritten by later calls: rollback is a length
 * truncation.  tau outside [1, block] is clamped and flagged DFLASH_DEVERR_TAU.  Each
 * given cache needs len_bound + block <= capacity_tokens (else DFLASH_E_CAPACITY, nothing
 * changed); on success its len_bound grows by block.
 */
int dflash_kv_commit(dflash_kv* target_kv, dflash_kv* draft_ctx, const int32_t* tau,
                     int32_t block, void* stream);

/*
 * Measurement hook (benchmarks only; not thread-safe).  dflash_timing_arm(kernel, n)
 * makes the library record a HIP event pair on the launching stream around each of the
 * next n launches of one kernel class (events created with hipEventDisableSystemFence, so
 * that recording them flushes no caches); dflash_timing_read(ms, n) waits for those events,
 * writes each launch's duration in milliseconds, disarms, and returns the number of
 * launches recorded (or a negative dflash_status).  Events are host-side HIP objects;
 * no device memory is allocated.
 */
typedef enum {
  DFLASH_KERNEL_LM_HEAD = 0,      /* LM-head GEMM of draft_block / verify_accept          */
  DFLASH_KERNEL_GEMM_QKV = 1,
  DFLASH_KERNEL_GEMM_O = 2,
  DFLASH_KERNEL_GEMM_GATE_UP = 3,
  DFLASH_KERNEL_GEMM_DOWN = 4,
  DFLASH_KERNEL_ATTENTION = 5,    /* split-K attention + split merge                      */
  DFLASH_KERNEL_INJECT_FUSE = 6,  /* feats W_c^T GEMM of inject_ctx                       */
  DFLASH_KERNEL_INJECT_KV = 7,    /* H_t [W^K; W^V]^T GEMM of inject_ctx                   */
  DFLASH_KERNEL_COUNT = 8
} dflash_kernel_id;
int dflash_timing_arm(int32_t kernel, int32_t capacity);
int dflash_timing_read(float* ms, int32_t capacity);

/*
 * Measurement utility (benchmarks only): reads `bytes` (a multiple of 16) of device memory
 * at `src` once, on `stream`, with plain loads (nontemporal == 0) or with the non-temporal
 * hint that the weight streams use (nontemporal != 0), and writes one 16-byte value per
 * workgroup (1024 workgroups) to the device memory at `sink` (at least 16 KiB) so that the
 * loads are kept.  A read of known size in each load form calibrates the hardware read
 * counters for kernels that use that form.  Returns DFLASH_E_ARG on NULL pointers or a size
 * that is not a multiple of 16, DFLASH_E_HIP when the launch fails.
 */
int dflash_probe_read(const void* src, size_t bytes, int32_t nontemporal, void* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
