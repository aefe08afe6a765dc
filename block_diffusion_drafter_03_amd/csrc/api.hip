// libdflash C ABI: argument validation, workspace layout and launch sequencing.
// The operations are specified in include/dflash.h.
//
// Activations stay float32 between launches (the bf16 MFMAs take them as compensated
// hi/lo pairs); K/V and tapped features are written in the model dtype.  For bfloat16
// models the GEMM inputs (h, attention output, SwiGLU output, fused injection rows) live in
// the MFMA A-fragment order, their row count padded to a multiple of 16.
//
// One decoder layer of up to 16 rows is six launches (the norms, RoPE, SwiGLU and residual
// adds are fused into them):
//   QKV GEMM   A = h, RMSNorm(g_in) applied on the A side; epilogue: RoPE,
//              q / k_blk / v_blk^T (and, for verification, the block K/V into the cache)
//   attention  split-K over [context ; block], then the log-sum-exp merge of the splits
//   O GEMM     epilogue: h += o W_o^T
//   GATE/UP    A = h, RMSNorm(g_post) on the A side; epilogue: SiLU(gate) * up
//   DOWN GEMM  epilogue: h += act W_d^T (+ tapped-feature / debug copies)
// and the LM head is one GEMM with RMSNorm(g_f) on the A side and an argmax epilogue.
// Beyond 16 rows a GEMM with an A-side norm first splits its rows into operand planes
// (pair_split), and the K-split GEMMs add a reduce launch.
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/dflash.h"
#include "kernels.h"

using namespace dflash;

struct dflash_model {
  dflash_model_desc d;
  std::vector<const void*> layer_w;
  std::vector<int32_t> taps;
  std::vector<const void*> dconv;   // empty, or [n_layers * 8] (DFlash 2 convolutions)
};

namespace {

const size_t kAlign = 256;
inline size_t al(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline size_t esz(int dt) { return dt == DFLASH_BF16 ? 2 : 4; }
inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Bump allocator over the caller's workspace (offsets only; nothing is allocated).
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base((char*)b) {}
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off += al(bytes);
    return p;
  }
};

inline const void* W(const dflash_model* m, int l, int slot) {
  return m->layer_w[(size_t)l * DFLASH_LAYER_TENSORS + slot];
}

// Scratch of one draft / verify step for `batch` sequences of `B` rows.
struct StepWs {
  float* h;
  float* q;
  void* kblk;
  void* vblkT;
  void* kblk_lo;      // bf16 models: the low parts of the block's own K / V^T
  void* vblkT_lo;
  float* part;
  float* o;
  float* act;
  unsigned long long* keys;
  float2* rope;
  SampleWs smp;       // sampling verification scratch
  float* xa;          // DFlash 2 convolutions: a convolution's input or output [Mp, D]
  float* dk;          // and its correction coefficients [M, D / 8]
  SplitArgs split;    // K-split scratch of the M > 16 GEMMs
  GemvSplitArgs gsplit;  // K-split scratch of the M <= 16 O and down GEMVs
  AttnPlan plan;
};

// K-split and operand-plane scratch for GEMMs of `rows` rows whose column count is at most
// max_n and reduction length at most max_k (bf16 models with more than 16 rows; otherwise
// none)
SplitArgs carve_split(Carve& cv, int dt, int rows, int max_n, int max_k) {
  SplitArgs s;
  memset(&s, 0, sizeof(s));
  const bool use = dt == DFLASH_BF16 && rows > 16;
  s.part_bytes = use ? rows_split_bytes(rows, max_n) : 0;
  s.part = (float*)cv.take(s.part_bytes);
  s.ss = (float*)cv.take(use ? rows_split_ss_bytes(rows) : 0);
  s.pair_bytes = use ? pair_plane_bytes(rows, max_k) : 0;
  s.pair = cv.take(s.pair_bytes);
  if (!use) s.part = nullptr, s.pair = nullptr;
  return s;
}

size_t step_ws(const dflash_model* m, int batch, int B, int ctx_cap, void* base, StepWs* w) {
  const dflash_model_desc& d = m->d;
  const int dt = d.dtype, M = batch * B, Mp = round_up(M, 16), Bp = round_up(B, 32);
  const int D = d.hidden, Hq = d.n_q_heads, Hkv = d.n_kv_heads, hd = d.head_dim;
  StepWs t;
  t.plan = attn_plan(dt, batch, Hkv, Hq / Hkv, B, ctx_cap, d.n_layers, hd);
  Carve cv(base);
  t.h = (float*)cv.take((size_t)Mp * D * 4);
  t.q = (float*)cv.take((size_t)M * Hq * hd * 4);
  t.kblk = cv.take((size_t)M * Hkv * hd * esz(dt));
  t.vblkT = cv.take((size_t)batch * Hkv * hd * Bp * esz(dt));
  t.kblk_lo = cv.take(dt == DFLASH_BF16 ? (size_t)M * Hkv * hd * 2 : 0);
  t.vblkT_lo = cv.take(dt == DFLASH_BF16 ? (size_t)batch * Hkv * hd * Bp * 2 : 0);
  t.part = (float*)cv.take(dt == DFLASH_BF16 ? attn_partial_floats(t.plan, batch, Hkv, hd) * 4 : 0);
  t.o = (float*)cv.take((size_t)Mp * Hq * hd * 4);
  t.act = (float*)cv.take((size_t)Mp * d.ffn * 4);
  t.keys = (unsigned long long*)cv.take((size_t)M * 8);
  t.rope = (float2*)cv.take((size_t)M * (hd / 2) * sizeof(float2));
  const size_t srows = (size_t)batch * (2 * B - 1);
  t.smp.part = (float2*)cv.take(srows * SAMPLE_MAX_CHUNKS * sizeof(float2));
  t.smp.lse = (float*)cv.take(srows * 4);
  t.smp.acc = (int32_t*)cv.take((size_t)batch * 4);
  t.smp.keys = (unsigned long long*)cv.take((size_t)batch * SAMPLE_MAX_CHUNKS * 8);
  const bool dc = !m->dconv.empty();
  t.xa = (float*)cv.take(dc ? (size_t)Mp * D * 4 : 0);
  t.dk = (float*)cv.take(dc ? (size_t)M * (D / 8) * 4 : 0);
  const int max_k = std::max(std::max(D, Hq * hd), d.ffn);
  t.split = carve_split(cv, dt, M, (Hq + 2 * Hkv) * hd > D ? (Hq + 2 * Hkv) * hd : D, max_k);
  memset(&t.gsplit, 0, sizeof(t.gsplit));
  if (dt == DFLASH_BF16 && M <= 16) {   // the M <= 16 GEMVs of the layers: N <= max(D, Nqkv)
    const int max_n = std::max(D, (Hq + 2 * Hkv) * hd);
    t.gsplit.max_tiles = gemv_split_tiles(max_n);
    t.gsplit.part = (float*)cv.take(gemv_split_part_bytes(max_n));
    t.gsplit.ss = (float*)cv.take(gemv_split_ss_bytes(max_n));
    // (one more counter: the LM head's draft-id decode)
    t.gsplit.cnt = (unsigned*)cv.take((size_t)(t.gsplit.max_tiles + 1) * 4);
  }
  if (w) *w = t;
  return cv.off;
}

size_t inject_ws(const dflash_model* m, int rows, void* base, float** x, float2** rope,
                 SplitArgs* split = nullptr) {
  Carve cv(base);
  float* p = (float*)cv.take((size_t)round_up(rows, 16) * m->d.hidden * 4);
  float2* r = (float2*)cv.take((size_t)rows * (m->d.head_dim / 2) * sizeof(float2));
  const SplitArgs s = carve_split(cv, m->d.dtype, rows, m->d.hidden, m->d.hidden);
  if (x) *x = p;
  if (rope) *rope = r;
  if (split) *split = s;
  return cv.off;
}

EmbedArgs embed_args(const dflash_model* m, const dflash_kv* kv, const StepWs& w, int mode,
                     const int32_t* ids, const int32_t* anchor, int B, float* hidden_dbg) {
  const dflash_model_desc& d = m->d;
  EmbedArgs a;
  memset(&a, 0, sizeof(a));
  a.ids = ids;
  a.anchor = anchor;
  a.mode = mode;
  a.batch = kv->batch;
  a.B = B;
  a.mask_id = d.mask_token_id;
  a.E = d.embed;
  a.V = d.vocab;
  a.D = d.hidden;
  a.h = w.h;
  a.afrag = d.dtype == DFLASH_BF16;
  a.hdbg = hidden_dbg;
  a.keys = w.keys;
  a.n_keys = kv->batch * B;
  a.err = kv->error_flags;
  a.seq_len = kv->seq_len;
  a.hd = d.head_dim;
  a.zero = w.gsplit.cnt;
  a.n_zero = w.gsplit.cnt ? w.gsplit.max_tiles + 1 : 0;
  a.rope_base = d.rope_base;
  a.rope = w.rope;
  return a;
}

int check_kv(const dflash_model* m, const dflash_kv* kv) {
  if (!kv || !kv->k_pool || !kv->v_pool || !kv->block_table || !kv->seq_len) return DFLASH_E_ARG;
  if (kv->batch < 1 || kv->max_pages_per_seq < 1 || kv->num_pages < 1) return DFLASH_E_ARG;
  if (kv->page_size != 64) return DFLASH_E_SHAPE;
  if (kv->n_layers != m->d.n_layers || kv->n_kv_heads != m->d.n_kv_heads ||
      kv->head_dim != m->d.head_dim)
    return DFLASH_E_SHAPE;
  for (int l = 0; l < kv->n_layers; ++l)
    if (!kv->k_pool[l] || !kv->v_pool[l]) return DFLASH_E_ARG;
  if (kv->capacity_tokens < 0 || kv->len_bound < 0 ||
      (int64_t)kv->capacity_tokens > (int64_t)kv->max_pages_per_seq * kv->page_size)
    return DFLASH_E_ARG;
  return DFLASH_OK;
}

// Host-side capacity rule: the positions a call touches end before `end` (exclusive),
// which must not pass the positions mapped for every sequence.
int check_capacity(const dflash_kv* kv, int64_t end) {
  return end > (int64_t)kv->capacity_tokens ? DFLASH_E_CAPACITY : DFLASH_OK;
}

KvLayer layer_view(const dflash_kv* kv, int l) {
  KvLayer v;
  v.k = kv->k_pool[l];
  v.v = kv->v_pool[l];
  v.block_table = kv->block_table;
  v.seq_len = kv->seq_len;
  v.max_pages = kv->max_pages_per_seq;
  v.num_pages = kv->num_pages;
  v.batch = kv->batch;
  v.err = kv->error_flags;
  return v;
}

#define HIPCHK(x)                              \
  do {                                         \
    if ((x) != hipSuccess) return DFLASH_E_HIP; \
  } while (0)

// ---- measurement hook: event pairs around the launches of one kernel class ----
struct TimingState {
  int kernel = -1;
  int capacity = 0;
  int count = 0;
  std::vector<hipEvent_t> ev;   // 2 per launch
};
TimingState g_timing;

// event pair of the next launch of `kernel` when that class is armed, else -1
int timing_slot(int kernel) {
  if (g_timing.kernel == kernel && g_timing.count < g_timing.capacity) return g_timing.count++;
  return -1;
}
// events recorded around the launches of one kernel class; created without the
// system-scope fence (hipEventDisableSystemFence), so that recording them writes back and
// invalidates no caches and the pair brackets the kernels with the least added time
struct Timed {
  hipStream_t st;
  int slot;
  Timed(int kernel, hipStream_t s) : st(s), slot(timing_slot(kernel)) {
    if (slot >= 0) (void)hipEventRecord(g_timing.ev[2 * slot], st);
  }
  ~Timed() {
    if (slot >= 0) (void)hipEventRecord(g_timing.ev[2 * slot + 1], st);
  }
};

BSeg one_seg(const void* p, int rows, int ldb) {
  BSeg b;
  memset(&b, 0, sizeof(b));
  b.ptr[0] = p;
  b.seg_rows = rows;
  b.nseg = 1;
  b.ldb = ldb;
  return b;
}

GemmArgs gemm_args(const void* A, int lda, const BSeg& B, int M, int N, int K, const void* norm_g,
                   float eps, int kind) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.A = A;
  g.lda = lda;
  g.B = B;
  g.M = M;
  g.N = N;
  g.K = K;
  g.norm_g = norm_g;
  g.eps = eps;
  g.e.kind = kind;
  return g;
}

int run_gemm(int kernel_class, int dt, const GemmArgs& g, hipStream_t st) {
  Timed t(kernel_class, st);
  HIPCHK(launch_gemm(dt, g, st));
  return DFLASH_OK;
}

// The decoder stack shared by the drafter (bidirectional block, no cache writes) and the
// target (causal block, block K/V written into the cache, taps copied out).  On entry h
// holds the embedded block; on exit it holds the last layer's output.
int run_layers(const dflash_model* m, const dflash_kv* kv, int batch, int B, const StepWs& w,
               int causal, int write_cache, void* feats_out, float* hidden_dbg, hipStream_t st) {
  const dflash_model_desc& d = m->d;
  const int dt = d.dtype, M = batch * B, Bp = round_up(B, 32);
  const int D = d.hidden, Hq = d.n_q_heads, Hkv = d.n_kv_heads, hd = d.head_dim, F = d.ffn;
  const int Nqkv = (Hq + 2 * Hkv) * hd;
  const float eps = d.rms_eps;
  const int afrag = dt == DFLASH_BF16;
  // bf16 models beyond 16 rows: attention and SwiGLU write their outputs as compensated
  // operand planes, which the O and down GEMMs take as they are
  const int pairs = dt == DFLASH_BF16 && M > 16;
  const bool dc = !m->dconv.empty();
  if (dc && feats_out) return DFLASH_E_ARG;   // the convolutions belong to a drafter
  // DFlash 2 convolution `c` of layer l: its correction GEMM, then the convolution itself.
  // pre: w.xa = Conv(RMSNorm(h; g_norm)); post: h += Conv(w.xa) (+ the hidden_dbg copy).
  auto conv = [&](int l, int c, const void* g_norm, bool post, float* hdbg) -> int {
    const float* x = post ? w.xa : w.h;
    if (dt == DFLASH_BF16 && gemv_dconv_supported(M, D)) {
      // one launch: the correction GEMV with the convolution as its epilogue
      GemmArgs g = gemm_args(x, D, one_seg(m->dconv[l * 8 + 2 * c + 1], D / 8, D), M, D / 8, D,
                             g_norm, eps, EPI_DCONV);
      g.e.out = post ? w.h : w.xa;
      g.e.afrag = 1;
      g.e.B = B;
      g.e.hdbg = hdbg;
      g.e.dconv_base = m->dconv[l * 8 + 2 * c];
      g.e.dconv_accumulate = post;
      HIPCHK(launch_gemv_dconv(g, st));
      return DFLASH_OK;
    }
    GemmArgs g = gemm_args(x, D, one_seg(m->dconv[l * 8 + 2 * c + 1], D / 8, D), M, D / 8, D,
                           g_norm, eps, EPI_STORE_F32);
    g.e.out = w.dk;
    g.e.ldo = D / 8;
    HIPCHK(launch_gemm(dt, g, st));
    DconvArgs a;
    a.x = x;
    a.norm_g = g_norm;
    a.eps = eps;
    a.corr = w.dk;
    a.base = m->dconv[l * 8 + 2 * c];
    a.M = M;
    a.D = D;
    a.B = B;
    a.afrag = afrag;
    a.bf16 = dt == DFLASH_BF16;
    a.accumulate = post;
    a.out = post ? w.h : w.xa;
    a.hdbg = hdbg;
    HIPCHK(launch_dconv(a, st));
    return DFLASH_OK;
  };
  for (int l = 0; l < d.n_layers; ++l) {
    const KvLayer kvl = layer_view(kv, l);
    if (dc)
      if (int s = conv(l, DFLASH_DCONV_PRE_ATTN, W(m, l, DFLASH_W_G_IN), false, nullptr)) return s;
    {  // QKV projection with RMSNorm(g_in) on the A side (or of the convolved input);
       // RoPE / layout epilogue
      GemmArgs g = gemm_args(dc ? w.xa : w.h, D, one_seg(W(m, l, DFLASH_W_QKV), Nqkv, D), M, Nqkv, D,
                             dc ? nullptr : W(m, l, DFLASH_W_G_IN), eps, EPI_QKV);
      EpiArgs& e = g.e;
      e.B = B;
      e.Bp = Bp;
      e.Hq = Hq;
      e.Hkv = Hkv;
      e.hd = hd;
      e.rope = w.rope;
      e.seq_len = kv->seq_len;
      e.q = w.q;
      e.kblk = w.kblk;
      e.vblkT = w.vblkT;
      e.kblk_lo = w.kblk_lo;
      e.vblkT_lo = w.vblkT_lo;
      e.has_cache = write_cache;
      e.kp[0] = kvl.k;
      e.vp[0] = kvl.v;
      e.block_table = kv->block_table;
      e.max_pages = kv->max_pages_per_seq;
      e.num_pages = kv->num_pages;
      e.batch = kv->batch;
      e.err = kv->error_flags;
      g.split = w.split;
      g.gsplit = w.gsplit;
      if (int s = run_gemm(DFLASH_KERNEL_GEMM_QKV, dt, g, st)) return s;
    }
    {
      Timed t(DFLASH_KERNEL_ATTENTION, st);
      HIPCHK(launch_attention(dt, w.plan, w.q, w.kblk, w.vblkT, w.kblk_lo, w.vblkT_lo, kvl, batch,
                              B, Bp, Hq, Hkv, hd, causal, w.part, w.o, pairs ? 2 : afrag, st));
    }
    {  // O projection + residual (with the convolutions: the output, convolved below)
      GemmArgs g = gemm_args(w.o, Hq * hd, one_seg(W(m, l, DFLASH_W_O), D, Hq * hd), M, D,
                             Hq * hd, nullptr, eps, dc ? EPI_STORE_F32 : EPI_RESID);
      g.a_pair = pairs;
      g.e.h = w.h;
      g.e.ldh = D;
      g.e.out = w.xa;
      g.e.ldo = D;
      g.e.afrag = afrag;
      g.split = w.split;
      g.gsplit = w.gsplit;
      if (int s = run_gemm(DFLASH_KERNEL_GEMM_O, dt, g, st)) return s;
    }
    if (dc) {
      if (int s = conv(l, DFLASH_DCONV_POST_ATTN, nullptr, true, nullptr)) return s;
      if (int s = conv(l, DFLASH_DCONV_PRE_FFN, W(m, l, DFLASH_W_G_POST), false, nullptr)) return s;
    }
    {  // gate/up with RMSNorm(g_post) on the A side (or of the convolved input); SwiGLU
      GemmArgs g = gemm_args(dc ? w.xa : w.h, D, one_seg(W(m, l, DFLASH_W_GATE_UP), 2 * F, D), M,
                             2 * F, D, dc ? nullptr : W(m, l, DFLASH_W_G_POST), eps, EPI_SWIGLU);
      g.e.act = w.act;
      g.e.F = F;
      g.e.afrag = afrag;
      g.e.act_pair = pairs;
      g.split = w.split;
      if (int s = run_gemm(DFLASH_KERNEL_GEMM_GATE_UP, dt, g, st)) return s;
    }
    float* hdbg_l = hidden_dbg ? hidden_dbg + (size_t)(l + 1) * M * D : nullptr;
    {  // down projection + residual (+ tap / debug copies; with the convolutions: the output,
       // convolved below)
      GemmArgs g = gemm_args(w.act, F, one_seg(W(m, l, DFLASH_W_DOWN), D, F), M, D, F, nullptr, eps,
                             dc ? EPI_STORE_F32 : EPI_RESID);
      g.a_pair = pairs;
      g.e.h = w.h;
      g.e.ldh = D;
      g.e.out = w.xa;
      g.e.ldo = D;
      g.e.afrag = afrag;
      g.e.hdbg = dc ? nullptr : hdbg_l;
      if (feats_out) {
        for (size_t t = 0; t < m->taps.size(); ++t)
          if (m->taps[t] == l) {
            g.e.tap = feats_out;
            g.e.tap_ld = (int)m->taps.size() * D;
            g.e.tap_col = (int)t * D;
          }
      }
      g.split = w.split;
      g.gsplit = w.gsplit;
      if (int s = run_gemm(DFLASH_KERNEL_GEMM_DOWN, dt, g, st)) return s;
    }
    if (dc)
      if (int s = conv(l, DFLASH_DCONV_POST_FFN, nullptr, true, hdbg_l)) return s;
  }
  return DFLASH_OK;
}

// LM head with RMSNorm(g_f) on the A side and the argmax epilogue over every row of h
// (argmax keys per row; the optional logits copy leaves out each block's anchor row when
// skipB != 0).
// Sampling parameters of the drafter's LM head (temperature <= 0: argmax)
struct Sampling {
  float temperature = 0.f;
  unsigned long long seed = 0;
  unsigned counter = 0;
};

// With draft_ids (drafter) or acc (verifier) the M <= 16 GEMV also decodes the draft ids
// or runs the greedy acceptance (its last workgroup); *done tells whether it did.
struct AcceptOut {
  const int32_t* drafts;
  int32_t *g, *tau, *bonus;
};
int run_lm_head(const dflash_model* m, const StepWs& w, int rows, int skipB, float* logits,
                hipStream_t st, int B = 0, const Sampling& smp = Sampling(), int32_t* draft_ids = nullptr,
                bool* ids_done = nullptr, const AcceptOut* acc = nullptr) {
  const dflash_model_desc& d = m->d;
  GemmArgs g = gemm_args(w.h, d.hidden, one_seg(d.lm_head, d.vocab, d.hidden), rows, d.vocab,
                         d.hidden, d.final_norm, d.rms_eps, EPI_ARGMAX);
  g.e.keys = w.keys;
  g.e.logits = logits;
  g.e.skipB = skipB;
  g.split = w.split;
  if (smp.temperature > 0.f) {
    g.e.sample = 1;
    g.e.temperature = smp.temperature;
    g.e.seed = smp.seed;
    g.e.counter = smp.counter;
    g.e.B = B;
  }
  // the M <= 16 GEMV decodes the draft ids (or accepts) itself, saving a launch
  const bool fold = (draft_ids || acc) && B > 1 && B <= 64 && w.gsplit.cnt && gemm_takes_gemv(d.dtype, g);
  if (fold) {
    g.e.ids_out = draft_ids;
    g.e.ids_cnt = w.gsplit.cnt + w.gsplit.max_tiles;
    g.e.ids_B = B;
    if (acc) {
      g.e.acc_drafts = acc->drafts;
      g.e.acc_g = acc->g;
      g.e.acc_tau = acc->tau;
      g.e.acc_bonus = acc->bonus;
    }
  }
  if (ids_done) *ids_done = fold;
  return run_gemm(DFLASH_KERNEL_LM_HEAD, d.dtype, g, st);
}

int validate_model(const dflash_model_desc* d) {
  if (!d) return DFLASH_E_ARG;
  if (d->dtype != DFLASH_F32 && d->dtype != DFLASH_BF16) return DFLASH_E_DTYPE;
  if (d->n_layers < 1 || d->hidden < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 ||
      d->head_dim < 2 || d->ffn < 1 || d->vocab < 2)
    return DFLASH_E_ARG;
  if (!d->embed || !d->lm_head || !d->final_norm || !d->layer_w) return DFLASH_E_ARG;
  if (d->n_q_heads % d->n_kv_heads) return DFLASH_E_SHAPE;
  if (d->head_dim % 2) return DFLASH_E_SHAPE;
  if (d->n_layers > 8 && d->w_c) return DFLASH_E_SHAPE;   // injection GEMM covers <= 8 layers
  if (d->n_taps < 0 || (d->n_taps > 0 && d->tap_layers == nullptr && !d->w_c)) return DFLASH_E_ARG;
  if (d->w_c && (!d->g_c || d->n_taps < 1)) return DFLASH_E_ARG;
  if (d->mask_token_id < 0 || d->mask_token_id >= d->vocab) return DFLASH_E_ARG;
  if (!(d->rms_eps >= 0.f) || !(d->rope_base > 0.f)) return DFLASH_E_ARG;
  if (d->dtype == DFLASH_BF16) {
    if (d->head_dim != 128) return DFLASH_E_SHAPE;
    if (d->hidden % 128 || d->ffn % 128) return DFLASH_E_SHAPE;
  } else {
    if (d->hidden % 16 || d->ffn % 16 || (d->n_q_heads * d->head_dim) % 16) return DFLASH_E_SHAPE;
    if (d->head_dim > 512) return DFLASH_E_SHAPE;
  }
  for (int i = 0; i < d->n_layers * DFLASH_LAYER_TENSORS; ++i)
    if (!d->layer_w[i]) return DFLASH_E_ARG;
  if (d->tap_layers)
    for (int t = 0; t < d->n_taps; ++t)
      if (d->tap_layers[t] < 0 || d->tap_layers[t] >= d->n_layers) return DFLASH_E_ARG;
  if (d->dconv) {
    if (d->tap_layers || d->hidden % 128) return DFLASH_E_SHAPE;   // drafter only
    for (int i = 0; i < d->n_layers * 8; ++i)
      if (!d->dconv[i]) return DFLASH_E_ARG;
  }
  return DFLASH_OK;
}

// Path-selector scratch: H of every block row, chunk top-k keys, candidate ids, the gathered
// embedding rows (anchor, then position-major candidates, per sequence) and their [A | B]
// projections.
struct SelWs {
  float* hh;
  unsigned long long* keys;
  int32_t* cand;
  void* gather;
  float* P;
  float* S;
  SplitArgs split;    // K-split scratch of the projection GEMMs
};

size_t sel_ws(const dflash_model* m, const dflash_selector* s, int batch, int B, void* base,
              SelWs* w) {
  const int D = m->d.hidden, r = s->rank, k = s->top_k;
  const size_t rows = (size_t)batch * (B - 1);
  const size_t msel = (size_t)batch * (1 + (size_t)(B - 1) * k);
  Carve cv(base);
  SelWs t;
  t.hh = (float*)cv.take((size_t)batch * B * r * 4);
  t.keys = (unsigned long long*)cv.take(rows * SAMPLE_MAX_CHUNKS * 16 * 8);
  t.cand = (int32_t*)cv.take(rows * 16 * 4);
  t.gather = cv.take(msel * D * esz(m->d.dtype));
  t.P = (float*)cv.take(msel * 2 * r * 4);
  t.S = (float*)cv.take(rows * 16 * 16 * 4);
  // K splits of the projection GEMMs (the [A | B] one has msel rows)
  t.split = carve_split(cv, m->d.dtype, (int)msel, 2 * r, D);
  if (w) *w = t;
  return cv.off;
}

int check_selector(const dflash_model* m, const dflash_selector* s) {
  if (!m || !s || !s->w_ab || !s->w_h) return DFLASH_E_ARG;
  if (s->rank < 16 || s->rank > 512 || s->rank % 16) return DFLASH_E_SHAPE;
  if (s->top_k < 1 || s->top_k > 16 || s->top_k > m->d.vocab) return DFLASH_E_SHAPE;
  return DFLASH_OK;
}

}  // namespace

// Scratch of dflash_draft_block_noalloc: one array per GPU, part of the library's code
// object.  Host code must not use the symbol itself as a device address (in host code it
// names a host-side stand-in): the address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) char scratch[DFLASH_NOALLOC_SCRATCH_BYTES];

namespace {
#define NOALLOC_MAX_DEVICES 64
std::mutex g_scratch_mu;
void* g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};

// device address of the current device's scratch (looked up once per device)
int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) return DFLASH_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DFLASH_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DFLASH_OK;
}
}  // namespace

extern "C" {

const char* dflash_status_str(int s) {
  switch (s) {
    case DFLASH_OK: return "DFLASH_OK";
    case DFLASH_E_ARG: return "DFLASH_E_ARG: invalid argument";
    case DFLASH_E_SHAPE: return "DFLASH_E_SHAPE: unsupported or inconsistent shape";
    case DFLASH_E_DTYPE: return "DFLASH_E_DTYPE: unsupported or mismatched dtype";
    case DFLASH_E_CAPACITY: return "DFLASH_E_CAPACITY: cache too small";
    case DFLASH_E_WORKSPACE: return "DFLASH_E_WORKSPACE: workspace too small";
    case DFLASH_E_HIP: return "DFLASH_E_HIP: HIP launch failed";
    default: return "unknown dflash status";
  }
}

int dflash_model_create(const dflash_model_desc* desc, dflash_model** out) {
  if (!out) return DFLASH_E_ARG;
  *out = nullptr;
  const int v = validate_model(desc);
  if (v != DFLASH_OK) return v;
  dflash_model* m = new (std::nothrow) dflash_model;
  if (!m) return DFLASH_E_ARG;
  m->d = *desc;
  m->layer_w.assign(desc->layer_w, desc->layer_w + (size_t)desc->n_layers * DFLASH_LAYER_TENSORS);
  if (desc->tap_layers) m->taps.assign(desc->tap_layers, desc->tap_layers + desc->n_taps);
  if (desc->dconv) m->dconv.assign(desc->dconv, desc->dconv + (size_t)desc->n_layers * 8);
  m->d.layer_w = nullptr;
  m->d.tap_layers = nullptr;
  m->d.dconv = nullptr;
  *out = m;
  return DFLASH_OK;
}

void dflash_model_destroy(dflash_model* m) { delete m; }

size_t dflash_workspace_bytes(const dflash_model* m, int32_t batch, int32_t block,
                              int32_t max_ctx_tokens, int32_t max_inject_rows) {
  if (!m || batch < 1 || block < 1 || block > 64 || max_ctx_tokens < 0 || max_inject_rows < 0)
    return 0;
  size_t s = step_ws(m, batch, block, max_ctx_tokens, nullptr, nullptr);
  if (max_inject_rows > 0 && m->d.w_c) {
    const size_t i = inject_ws(m, max_inject_rows, nullptr, nullptr, nullptr);
    if (i > s) s = i;
  }
  return s;
}

int dflash_inject_ctx(const dflash_model* m, dflash_kv* kv, const void* feats, int32_t n_rows,
                      const int32_t* row_seq, const int32_t* row_pos, int32_t pos_relative,
                      int32_t pos_limit, void* ws, size_t ws_bytes, void* stream) {
  if (!m || n_rows < 0 || pos_limit < 1) return DFLASH_E_ARG;
  if (!m->d.w_c) return DFLASH_E_ARG;
  int e = check_kv(m, kv);
  if (e) return e;
  e = check_capacity(kv, (pos_relative ? (int64_t)kv->len_bound : 0) + pos_limit);
  if (e) return e;
  if (n_rows == 0) return DFLASH_OK;   // nothing to inject (the row arrays may be empty)
  if (!feats || !row_seq || !row_pos) return DFLASH_E_ARG;
  float* x = nullptr;
  float2* rope = nullptr;
  SplitArgs split;
  const size_t need = inject_ws(m, n_rows, ws, &x, &rope, &split);
  if (!ws || ws_bytes < need) return DFLASH_E_WORKSPACE;
  const dflash_model_desc& d = m->d;
  const int dt = d.dtype, D = d.hidden, L = d.n_layers, Hkv = d.n_kv_heads, hd = d.head_dim;
  const int Kc = d.n_taps * D, N2 = L * 2 * Hkv * hd;
  hipStream_t st = (hipStream_t)stream;
  {  // x = feats W_c^T (float32)
    GemmArgs g = gemm_args(feats, Kc, one_seg(d.w_c, D, Kc), n_rows, D, Kc, nullptr, d.rms_eps,
                           EPI_STORE_F32);
    g.a_bf16 = dt == DFLASH_BF16;
    g.e.afrag = dt == DFLASH_BF16;
    g.e.out = x;
    g.e.ldo = D;
    g.split = split;
    if (int s = run_gemm(DFLASH_KERNEL_INJECT_FUSE, dt, g, st)) return s;
  }
  HIPCHK(launch_rope_rows(row_seq, row_pos, pos_relative, kv->seq_len, kv->batch, n_rows, hd,
                          d.rope_base, rope, st));
  {  // H_t = RMSNorm(x; g_c) on the A side; one GEMM over every layer's [W^K; W^V] rows;
     // epilogue: RoPE(K) and the page scatter of K and V
    BSeg b;
    memset(&b, 0, sizeof(b));
    for (int l = 0; l < L; ++l)
      b.ptr[l] = (const char*)W(m, l, DFLASH_W_QKV) + (size_t)d.n_q_heads * hd * D * esz(dt);
    b.seg_rows = 2 * Hkv * hd;
    b.nseg = L;
    b.ldb = D;
    GemmArgs g = gemm_args(x, D, b, n_rows, N2, D, d.g_c, d.rms_eps, EPI_INJECT_KV);
    EpiArgs& ep = g.e;
    ep.Hkv = Hkv;
    ep.hd = hd;
    ep.rope = rope;
    ep.seq_len = kv->seq_len;
    for (int l = 0; l < L; ++l) {
      ep.kp[l] = kv->k_pool[l];
      ep.vp[l] = kv->v_pool[l];
    }
    ep.block_table = kv->block_table;
    ep.max_pages = kv->max_pages_per_seq;
    ep.num_pages = kv->num_pages;
    ep.batch = kv->batch;
    ep.err = kv->error_flags;
    ep.row_seq = row_seq;
    ep.row_pos = row_pos;
    ep.pos_relative = pos_relative;
    ep.pos_limit = pos_limit;
    g.split = split;
    if (int s = run_gemm(DFLASH_KERNEL_INJECT_KV, dt, g, st)) return s;
  }
  return DFLASH_OK;
}

static int draft_block_impl(const dflash_model* m, const dflash_kv* kv, const int32_t* anchor,
                            int32_t block, int32_t* draft_ids, float* logits_dbg, float* hidden_dbg,
                            void* ws, size_t ws_bytes, void* stream, const Sampling& smp) {
  if (!m || !anchor || !draft_ids) return DFLASH_E_ARG;
  if (block < 1 || block > 64) return DFLASH_E_SHAPE;
  int e = check_kv(m, kv);
  if (e) return e;
  e = check_capacity(kv, kv->len_bound);   // the context is read, nothing is written
  if (e) return e;
  const dflash_model_desc& d = m->d;
  const int batch = kv->batch, B = block, M = batch * B;
  StepWs w;
  const size_t need = step_ws(m, batch, B, kv->max_pages_per_seq * 64, ws, &w);
  if (!ws || ws_bytes < need) return DFLASH_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  HIPCHK(launch_embed(d.dtype, embed_args(m, kv, w, 0, nullptr, anchor, B, hidden_dbg), st));
  e = run_layers(m, kv, batch, B, w, /*causal=*/0, /*write_cache=*/0, nullptr, hidden_dbg, st);
  if (e) return e;
  if (B == 1) return DFLASH_OK;   // a block of one has no masked position to draft
  bool ids_done = false;
  e = run_lm_head(m, w, M, B, logits_dbg, st, B, smp, draft_ids, &ids_done);
  if (e) return e;
  if (!ids_done) HIPCHK(launch_unpack_ids(w.keys, batch, B, draft_ids, st));
  return DFLASH_OK;
}

int dflash_draft_block(const dflash_model* m, const dflash_kv* kv, const int32_t* anchor,
                       int32_t block, int32_t* draft_ids, float* logits_dbg, float* hidden_dbg,
                       void* ws, size_t ws_bytes, void* stream) {
  return draft_block_impl(m, kv, anchor, block, draft_ids, logits_dbg, hidden_dbg, ws, ws_bytes,
                          stream, Sampling());
}

int dflash_draft_block_noalloc(const dflash_model* m, const dflash_kv* kv, const int32_t* anchor,
                               int32_t block, int32_t* draft_ids, float* logits_dbg,
                               float* hidden_dbg, void* stream) {
  if (!m || !anchor || !draft_ids) return DFLASH_E_ARG;
  if (block < 1 || block > 64) return DFLASH_E_SHAPE;
  int e = check_kv(m, kv);
  if (e) return e;
  const size_t need = step_ws(m, kv->batch, block, kv->max_pages_per_seq * 64, nullptr, nullptr);
  if (need > DFLASH_NOALLOC_SCRATCH_BYTES) return DFLASH_E_WORKSPACE;
  void* ws = nullptr;
  e = scratch_for_current_device(&ws);
  if (e) return e;
  return draft_block_impl(m, kv, anchor, block, draft_ids, logits_dbg, hidden_dbg, ws, need, stream,
                          Sampling());
}

int dflash_draft_block_sampled(const dflash_model* m, const dflash_kv* kv, const int32_t* anchor,
                               int32_t block, float temperature, uint64_t seed, int32_t counter,
                               int32_t* draft_ids, float* draft_logits, void* ws, size_t ws_bytes,
                               void* stream) {
  if (!(temperature > 0.f) || counter < 0 || !draft_logits) return DFLASH_E_ARG;
  if (block < 2) return DFLASH_E_SHAPE;
  if (kv && kv->batch > 4096) return DFLASH_E_SHAPE;   // the generator's sequence field
  if (m && m->d.vocab > 262144) return DFLASH_E_SHAPE;  // and its vocabulary field
  Sampling smp;
  smp.temperature = temperature;
  smp.seed = seed;
  smp.counter = (unsigned)counter;
  return draft_block_impl(m, kv, anchor, block, draft_ids, draft_logits, nullptr, ws, ws_bytes,
                          stream, smp);
}

size_t dflash_selector_workspace_bytes(const dflash_model* m, const dflash_selector* sel,
                                       int32_t batch, int32_t block) {
  if (check_selector(m, sel) || batch < 1 || block < 2 || block > 64) return 0;
  return sel_ws(m, sel, batch, block, nullptr, nullptr);
}

int dflash_draft_block_select(const dflash_model* m, const dflash_kv* kv, const int32_t* anchor,
                              int32_t block, const dflash_selector* sel, int32_t* draft_ids,
                              float* draft_logits, int32_t* candidates, void* ws, size_t ws_bytes,
                              void* sws, size_t sws_bytes, void* stream) {
  if (!m || !anchor || !draft_ids || !draft_logits) return DFLASH_E_ARG;
  if (block < 2 || block > 64) return DFLASH_E_SHAPE;
  int e = check_selector(m, sel);
  if (e) return e;
  e = check_kv(m, kv);
  if (e) return e;
  const dflash_model_desc& d = m->d;
  const int dt = d.dtype, batch = kv->batch, B = block, D = d.hidden, V = d.vocab;
  const int r = sel->rank, k = sel->top_k;
  if ((size_t)batch * (1 + (size_t)(B - 1) * k) > ((size_t)1 << 20)) return DFLASH_E_SHAPE;
  SelWs sw;
  const size_t need = sel_ws(m, sel, batch, B, sws, &sw);
  if (!sws || sws_bytes < need) return DFLASH_E_WORKSPACE;
  // the drafter pass and its LM head (logits of positions 1 .. B-1)
  e = draft_block_impl(m, kv, anchor, block, draft_ids, draft_logits, nullptr, ws, ws_bytes,
                       stream, Sampling());
  if (e) return e;
  StepWs w;
  step_ws(m, batch, B, kv->max_pages_per_seq * 64, ws, &w);
  hipStream_t st = (hipStream_t)stream;
  {  // H(h_t) of every block row: the final RMSNorm on the A side, then W_H
    GemmArgs g = gemm_args(w.h, D, one_seg(sel->w_h, r, D), batch * B, r, D, d.final_norm,
                           d.rms_eps, EPI_STORE_F32);
    g.e.out = sw.hh;
    g.e.ldo = r;
    HIPCHK(launch_gemm(dt, g, st));
  }
  int chunks = 1;
  HIPCHK(launch_topk(draft_logits, batch * (B - 1), V, k, sw.keys, &chunks, st));
  HIPCHK(launch_topk_merge(sw.keys, chunks, k, batch, B, d.embed, D, (int)esz(dt), anchor, V,
                           kv->error_flags, sw.cand, candidates, sw.gather, st));
  {  // [A | B] of the gathered embedding rows
    const int msel = batch * (1 + (B - 1) * k);
    GemmArgs g = gemm_args(sw.gather, D, one_seg(sel->w_ab, 2 * r, D), msel, 2 * r, D, nullptr,
                           d.rms_eps, EPI_STORE_F32);
    g.a_bf16 = dt == DFLASH_BF16;
    g.e.out = sw.P;
    g.e.ldo = 2 * r;
    g.split = sw.split;
    HIPCHK(launch_gemm(dt, g, st));
  }
  HIPCHK(launch_select(sw.P, sw.hh, draft_logits, sw.cand, batch, B, k, r, V, sw.S, draft_ids, st));
  return DFLASH_OK;
}

int dflash_verify_accept(const dflash_model* m, dflash_kv* kv, const int32_t* anchor,
                         const int32_t* draft_ids, int32_t block, void* feats_out,
                         int32_t* target_argmax, int32_t* tau, int32_t* bonus, float* logits_dbg,
                         float* hidden_dbg, void* ws, size_t ws_bytes, void* stream) {
  if (!m || !anchor || !target_argmax || !tau || !bonus) return DFLASH_E_ARG;
  if (block < 1 || block > 64) return DFLASH_E_SHAPE;
  if (block > 1 && !draft_ids) return DFLASH_E_ARG;
  int e = check_kv(m, kv);
  if (e) return e;
  e = check_capacity(kv, (int64_t)kv->len_bound + block);   // the block's K/V are written
  if (e) return e;
  if (feats_out && m->taps.empty()) return DFLASH_E_ARG;
  const dflash_model_desc& d = m->d;
  const int batch = kv->batch, B = block, M = batch * B;
  StepWs w;
  const size_t need = step_ws(m, batch, B, kv->max_pages_per_seq * 64, ws, &w);
  if (!ws || ws_bytes < need) return DFLASH_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  HIPCHK(launch_embed(d.dtype, embed_args(m, kv, w, 1, draft_ids, anchor, B, hidden_dbg), st));
  e = run_layers(m, kv, batch, B, w, /*causal=*/1, /*write_cache=*/1, feats_out, hidden_dbg, st);
  if (e) return e;
  const AcceptOut acc{draft_ids, target_argmax, tau, bonus};
  bool accepted = false;
  e = run_lm_head(m, w, M, 0, logits_dbg, st, B, Sampling(), nullptr, &accepted, &acc);
  if (e) return e;
  if (!accepted) HIPCHK(launch_accept(w.keys, draft_ids, batch, B, target_argmax, tau, bonus, st));
  return DFLASH_OK;
}

int dflash_verify_sampled(const dflash_model* m, dflash_kv* kv, const int32_t* anchor,
                          const int32_t* draft_ids, const float* draft_logits, int32_t block,
                          float temperature, uint64_t seed, int32_t counter, void* feats_out,
                          float* target_logits, int32_t* tau, int32_t* next_token, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!m || !anchor || !draft_ids || !draft_logits || !target_logits || !tau || !next_token)
    return DFLASH_E_ARG;
  if (!(temperature > 0.f) || counter < 0) return DFLASH_E_ARG;
  if (block < 2 || block > 64) return DFLASH_E_SHAPE;
  int e = check_kv(m, kv);
  if (e) return e;
  e = check_capacity(kv, (int64_t)kv->len_bound + block);   // the block's K/V are written
  if (e) return e;
  if (kv->batch > 4096 || m->d.vocab > 262144) return DFLASH_E_SHAPE;
  if (feats_out && m->taps.empty()) return DFLASH_E_ARG;
  const dflash_model_desc& d = m->d;
  const int batch = kv->batch, B = block, M = batch * B, V = d.vocab;
  StepWs w;
  const size_t need = step_ws(m, batch, B, kv->max_pages_per_seq * 64, ws, &w);
  if (!ws || ws_bytes < need) return DFLASH_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  HIPCHK(launch_embed(d.dtype, embed_args(m, kv, w, 1, draft_ids, anchor, B, nullptr), st));
  e = run_layers(m, kv, batch, B, w, /*causal=*/1, /*write_cache=*/1, feats_out, nullptr, st);
  if (e) return e;
  e = run_lm_head(m, w, M, 0, target_logits, st);
  if (e) return e;
  HIPCHK(launch_verify_sampled(target_logits, draft_logits, draft_ids, batch, B, V, temperature,
                               seed, (unsigned)counter, w.smp, tau, next_token, kv->error_flags,
                               st));
  return DFLASH_OK;
}

int dflash_kv_commit(dflash_kv* tkv, dflash_kv* dkv, const int32_t* tau, int32_t block,
                     void* stream) {
  if (!tau || (!tkv && !dkv)) return DFLASH_E_ARG;
  if (block < 1 || block > 64) return DFLASH_E_SHAPE;
  if (tkv && (!tkv->seq_len || tkv->batch < 1)) return DFLASH_E_ARG;
  if (dkv && (!dkv->seq_len || dkv->batch < 1)) return DFLASH_E_ARG;
  if (tkv && dkv && tkv->batch != dkv->batch) return DFLASH_E_SHAPE;
  for (const dflash_kv* kv : {(const dflash_kv*)tkv, (const dflash_kv*)dkv}) {
    if (!kv) continue;
    if (kv->capacity_tokens < 0 || kv->len_bound < 0) return DFLASH_E_ARG;
    if (int e = check_capacity(kv, (int64_t)kv->len_bound + block)) return e;
  }
  const int batch = tkv ? tkv->batch : dkv->batch;
  HIPCHK(launch_commit(tkv ? tkv->seq_len : nullptr, dkv ? dkv->seq_len : nullptr,
                       tkv ? tkv->error_flags : nullptr, dkv ? dkv->error_flags : nullptr, tau,
                       batch, block, (hipStream_t)stream));
  // tau <= block: the host-side bounds stay upper bounds of the new lengths
  if (tkv) tkv->len_bound += block;
  if (dkv) dkv->len_bound += block;
  return DFLASH_OK;
}

int dflash_timing_arm(int32_t kernel, int32_t capacity) {
  if (kernel < 0 || kernel >= DFLASH_KERNEL_COUNT || capacity < 1) return DFLASH_E_ARG;
  for (hipEvent_t e : g_timing.ev) (void)hipEventDestroy(e);
  g_timing.ev.assign(2 * (size_t)capacity, nullptr);
  for (auto& e : g_timing.ev)
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return DFLASH_E_HIP;
  g_timing.kernel = kernel;
  g_timing.capacity = capacity;
  g_timing.count = 0;
  return DFLASH_OK;
}

int dflash_probe_read(const void* src, size_t bytes, int32_t nontemporal, void* sink, void* stream) {
  if (!src || !sink || bytes % 16) return DFLASH_E_ARG;
  HIPCHK(launch_probe_read(src, bytes / 16, nontemporal, sink, (hipStream_t)stream));
  return DFLASH_OK;
}

int dflash_timing_read(float* ms, int32_t capacity) {
  if (!ms || capacity < 0) return DFLASH_E_ARG;
  const int n = g_timing.count < capacity ? g_timing.count : capacity;
  for (int i = 0; i < n; ++i) {
    if (hipEventSynchronize(g_timing.ev[2 * i + 1]) != hipSuccess) return DFLASH_E_HIP;
    if (hipEventElapsedTime(&ms[i], g_timing.ev[2 * i], g_timing.ev[2 * i + 1]) != hipSuccess)
      return DFLASH_E_HIP;
  }
  g_timing.kernel = -1;
  return n;
}

}  // extern "C"
