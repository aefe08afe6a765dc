// libdflash C ABI: argument validation, workspace layout and launch sequencing.
// The operations are specified in include/dflash.h.
#include <string.h>

#include <new>
#include <vector>

#include "../../include/dflash.h"
#include "kernels.h"

using namespace dflash;

struct dflash_model {
  dflash_model_desc d;
  std::vector<const void*> layer_w;
  std::vector<int32_t> taps;
};

namespace {

const size_t kAlign = 256;
inline size_t al(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline size_t esz(int dt) { return dt == DFLASH_BF16 ? 2 : 4; }

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

inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Scratch of one draft / verify step for `batch` sequences of `B` rows.
struct StepWs {
  float* h;
  void* u;
  float* C;
  void* q;
  void* kblk;
  void* vblkT;
  float* part;
  void* o;
  void* act;
  float* logits;
  int32_t* ids;
  AttnPlan plan;
  int Cs_max;   // max split count over the layer GEMMs
};

size_t step_ws(const dflash_model* m, int batch, int B, int ctx_cap, void* base, StepWs* w) {
  const dflash_model_desc& d = m->d;
  const int dt = d.dtype, M = batch * B, Bp = round_up(B, 32);
  const int D = d.hidden, Hq = d.n_q_heads, Hkv = d.n_kv_heads, hd = d.head_dim;
  const int Nqkv = (Hq + 2 * Hkv) * hd;
  size_t cmax = 0;
  int smax = 1;
  const int shapes[4][2] = {{Nqkv, D}, {D, Hq * hd}, {2 * d.ffn, D}, {D, d.ffn}};
  for (auto& s : shapes) {
    const int sp = gemm_splits(dt, M, s[0], s[1]);
    if (sp > smax) smax = sp;
    const size_t c = (size_t)sp * M * s[0];
    if (c > cmax) cmax = c;
  }
  StepWs t;
  t.plan = attn_plan(dt, batch, Hkv, Hq / Hkv, B, ctx_cap);
  t.Cs_max = smax;
  Carve cv(base);
  t.h = (float*)cv.take((size_t)M * D * 4);
  t.u = cv.take((size_t)M * D * esz(dt));
  t.C = (float*)cv.take(cmax * 4);
  t.q = cv.take((size_t)M * Hq * hd * esz(dt));
  t.kblk = cv.take((size_t)M * Hkv * hd * esz(dt));
  t.vblkT = cv.take((size_t)batch * Hkv * hd * Bp * esz(dt));
  t.part = (float*)cv.take(attn_partial_floats(t.plan, batch, Hkv, hd) * 4);
  t.o = cv.take((size_t)M * Hq * hd * esz(dt));
  t.act = cv.take((size_t)M * d.ffn * esz(dt));
  t.logits = (float*)cv.take((size_t)M * d.vocab * 4);
  t.ids = (int32_t*)cv.take((size_t)M * 4);
  if (w) *w = t;
  return cv.off;
}

struct InjWs {
  float* C1;
  void* Ht;
  float* C2;
  int S1, S2;
};

size_t inject_ws(const dflash_model* m, int rows, void* base, InjWs* w) {
  const dflash_model_desc& d = m->d;
  const int dt = d.dtype, D = d.hidden;
  const int N2 = d.n_layers * 2 * d.n_kv_heads * d.head_dim;
  InjWs t;
  t.S1 = gemm_splits(dt, rows, D, d.n_taps * D);
  t.S2 = gemm_splits(dt, rows, N2, D);
  Carve cv(base);
  t.C1 = (float*)cv.take((size_t)t.S1 * rows * D * 4);
  t.Ht = cv.take((size_t)rows * D * esz(dt));
  t.C2 = (float*)cv.take((size_t)t.S2 * rows * N2 * 4);
  if (w) *w = t;
  return cv.off;
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
  return DFLASH_OK;
}

KvLayer layer_view(const dflash_kv* kv, int l) {
  KvLayer v;
  v.k = kv->k_pool[l];
  v.v = kv->v_pool[l];
  v.block_table = kv->block_table;
  v.seq_len = kv->seq_len;
  v.max_pages = kv->max_pages_per_seq;
  v.num_pages = kv->num_pages;
  v.err = kv->error_flags;
  return v;
}

#define HIPCHK(x)                              \
  do {                                         \
    if ((x) != hipSuccess) return DFLASH_E_HIP; \
  } while (0)

BSeg one_seg(const void* p, int rows, int ldb) {
  BSeg b;
  memset(&b, 0, sizeof(b));
  b.ptr[0] = p;
  b.seg_rows = rows;
  b.nseg = 1;
  b.ldb = ldb;
  return b;
}

// The decoder stack shared by the drafter (bidirectional block, no cache writes) and the
// target (causal block, block K/V written into the cache, taps copied out).
int run_layers(const dflash_model* m, const dflash_kv* kv, int batch, int B, const StepWs& w,
               int causal, int write_cache, void* feats_out, float* hidden_dbg,
               const void* final_gain, int compact_final, hipStream_t st) {
  const dflash_model_desc& d = m->d;
  const int dt = d.dtype, M = batch * B, Bp = round_up(B, 32);
  const int D = d.hidden, Hq = d.n_q_heads, Hkv = d.n_kv_heads, hd = d.head_dim, F = d.ffn;
  const int Nqkv = (Hq + 2 * Hkv) * hd;
  const size_t es = esz(dt);
  (void)es;
  // u = RMSNorm(h, g_in[0])
  {
    RowFin f{};
    f.h = w.h;
    f.add_resid = 1;
    f.N = D;
    f.g = W(m, 0, DFLASH_W_G_IN);
    f.u = w.u;
    f.eps = d.rms_eps;
    HIPCHK(launch_row_finalize(dt, f, M, st));
  }
  for (int l = 0; l < d.n_layers; ++l) {
    const KvLayer kvl = layer_view(kv, l);
    // QKV projection, rotation, (verify) cache write
    int S = gemm_splits(dt, M, Nqkv, D);
    HIPCHK(launch_gemm(dt, w.u, D, one_seg(W(m, l, DFLASH_W_QKV), Nqkv, D), w.C, M, Nqkv, D, S, st));
    HIPCHK(launch_qkv_post(dt, w.C, S, (size_t)M * Nqkv, batch, B, Bp, Hq, Hkv, hd, d.rope_base,
                           kv->seq_len, w.q, w.kblk, w.vblkT, write_cache ? &kvl : nullptr, st));
    // attention over [context ; block]
    HIPCHK(launch_attention(dt, w.plan, w.q, w.kblk, w.vblkT, kvl, batch, B, Bp, Hq, Hkv, hd,
                            causal, w.part, w.o, st));
    // O projection + residual, then u = RMSNorm(h, g_post)
    S = gemm_splits(dt, M, D, Hq * hd);
    HIPCHK(launch_gemm(dt, w.o, Hq * hd, one_seg(W(m, l, DFLASH_W_O), D, Hq * hd), w.C, M, D, Hq * hd, S, st));
    {
      RowFin f{};
      f.C = w.C;
      f.S = S;
      f.split_stride = (size_t)M * D;
      f.N = D;
      f.h = w.h;
      f.add_resid = 1;
      f.write_h = 1;
      f.g = W(m, l, DFLASH_W_G_POST);
      f.u = w.u;
      f.eps = d.rms_eps;
      HIPCHK(launch_row_finalize(dt, f, M, st));
    }
    // SwiGLU FFN + residual, then the next layer's (or the final) RMSNorm
    S = gemm_splits(dt, M, 2 * F, D);
    HIPCHK(launch_gemm(dt, w.u, D, one_seg(W(m, l, DFLASH_W_GATE_UP), 2 * F, D), w.C, M, 2 * F, D, S, st));
    HIPCHK(launch_swiglu(dt, w.C, S, (size_t)M * 2 * F, M, F, w.act, st));
    S = gemm_splits(dt, M, D, F);
    HIPCHK(launch_gemm(dt, w.act, F, one_seg(W(m, l, DFLASH_W_DOWN), D, F), w.C, M, D, F, S, st));
    {
      RowFin f{};
      f.C = w.C;
      f.S = S;
      f.split_stride = (size_t)M * D;
      f.N = D;
      f.h = w.h;
      f.add_resid = 1;
      f.write_h = 1;
      f.hdbg = hidden_dbg ? hidden_dbg + (size_t)(l + 1) * M * D : nullptr;
      if (feats_out) {
        for (size_t t = 0; t < m->taps.size(); ++t)
          if (m->taps[t] == l) {
            f.tap = feats_out;
            f.tap_ld = (int)m->taps.size() * D;
            f.tap_col = (int)t * D;
          }
      }
      const bool last = (l + 1 == d.n_layers);
      f.g = last ? final_gain : W(m, l + 1, DFLASH_W_G_IN);
      f.u = w.u;
      f.compact_B = (last && compact_final) ? B : 0;
      f.eps = d.rms_eps;
      HIPCHK(launch_row_finalize(dt, f, M, st));
    }
  }
  return DFLASH_OK;
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
  m->d.layer_w = nullptr;
  m->d.tap_layers = nullptr;
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
    const size_t i = inject_ws(m, max_inject_rows, nullptr, nullptr);
    if (i > s) s = i;
  }
  return s;
}

int dflash_inject_ctx(const dflash_model* m, dflash_kv* kv, const void* feats, int32_t n_rows,
                      const int32_t* row_seq, const int32_t* row_pos, int32_t pos_relative,
                      void* ws, size_t ws_bytes, void* stream) {
  if (!m || !feats || !row_seq || !row_pos || n_rows < 1) return DFLASH_E_ARG;
  if (!m->d.w_c) return DFLASH_E_ARG;
  int e = check_kv(m, kv);
  if (e) return e;
  InjWs w;
  const size_t need = inject_ws(m, n_rows, ws, &w);
  if (!ws || ws_bytes < need) return DFLASH_E_WORKSPACE;
  const dflash_model_desc& d = m->d;
  const int dt = d.dtype, D = d.hidden, L = d.n_layers, Hkv = d.n_kv_heads, hd = d.head_dim;
  const int Kc = d.n_taps * D, N2 = L * 2 * Hkv * hd;
  hipStream_t st = (hipStream_t)stream;
  // H_t = RMSNorm(feats W_c^T; g_c)
  HIPCHK(launch_gemm(dt, feats, Kc, one_seg(d.w_c, D, Kc), w.C1, n_rows, D, Kc, w.S1, st));
  {
    RowFin f{};
    f.C = w.C1;
    f.S = w.S1;
    f.split_stride = (size_t)n_rows * D;
    f.N = D;
    f.g = d.g_c;
    f.u = w.Ht;
    f.eps = d.rms_eps;
    HIPCHK(launch_row_finalize(dt, f, n_rows, st));
  }
  // one GEMM over every draft layer's [W^K; W^V] row block, then RoPE(K) + page scatter
  BSeg b;
  memset(&b, 0, sizeof(b));
  for (int l = 0; l < L; ++l)
    b.ptr[l] = (const char*)W(m, l, DFLASH_W_QKV) + (size_t)d.n_q_heads * hd * D * esz(dt);
  b.seg_rows = 2 * Hkv * hd;
  b.nseg = L;
  b.ldb = D;
  HIPCHK(launch_gemm(dt, w.Ht, D, b, w.C2, n_rows, N2, D, w.S2, st));
  HIPCHK(launch_inject_scatter(dt, w.C2, w.S2, (size_t)n_rows * N2, n_rows, L, Hkv, hd, d.rope_base,
                               row_seq, row_pos, pos_relative, kv->k_pool, kv->v_pool,
                               kv->block_table, kv->seq_len, kv->max_pages_per_seq, kv->num_pages,
                               kv->batch, kv->error_flags, st));
  return DFLASH_OK;
}

int dflash_draft_block(const dflash_model* m, const dflash_kv* kv, const int32_t* anchor,
                       int32_t block, int32_t* draft_ids, float* logits_dbg, float* hidden_dbg,
                       void* ws, size_t ws_bytes, void* stream) {
  if (!m || !anchor || !draft_ids) return DFLASH_E_ARG;
  if (block < 1 || block > 64) return DFLASH_E_SHAPE;
  int e = check_kv(m, kv);
  if (e) return e;
  const dflash_model_desc& d = m->d;
  const int batch = kv->batch, B = block, M = batch * B;
  StepWs w;
  const size_t need = step_ws(m, batch, B, kv->max_pages_per_seq * 64, ws, &w);
  if (!ws || ws_bytes < need) return DFLASH_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int dt = d.dtype, D = d.hidden;
  HIPCHK(launch_embed(dt, nullptr, anchor, 0, batch, B, d.mask_token_id, d.embed, d.vocab, D, w.h,
                      hidden_dbg, kv->error_flags, st));
  e = run_layers(m, kv, batch, B, w, /*causal=*/0, /*write_cache=*/0, nullptr, hidden_dbg,
                 d.final_norm, /*compact_final=*/1, st);
  if (e) return e;
  if (B == 1) return DFLASH_OK;   // a block of one has no masked position to draft
  // LM head over the B-1 masked rows, argmax per row
  const int Mp = batch * (B - 1);
  float* logits = logits_dbg ? logits_dbg : w.logits;
  HIPCHK(launch_gemm(dt, w.u, D, one_seg(d.lm_head, d.vocab, D), logits, Mp, d.vocab, D, 1, st));
  HIPCHK(launch_argmax(logits, Mp, d.vocab, draft_ids, st));
  (void)M;
  return DFLASH_OK;
}

int dflash_verify_accept(const dflash_model* m, dflash_kv* kv, const int32_t* block_ids,
                         int32_t block, void* feats_out, int32_t* target_argmax, int32_t* tau,
                         int32_t* bonus, float* logits_dbg, float* hidden_dbg, void* ws,
                         size_t ws_bytes, void* stream) {
  if (!m || !block_ids || !target_argmax || !tau || !bonus) return DFLASH_E_ARG;
  if (block < 1 || block > 64) return DFLASH_E_SHAPE;
  int e = check_kv(m, kv);
  if (e) return e;
  if (feats_out && m->taps.empty()) return DFLASH_E_ARG;
  const dflash_model_desc& d = m->d;
  const int batch = kv->batch, B = block, M = batch * B;
  StepWs w;
  const size_t need = step_ws(m, batch, B, kv->max_pages_per_seq * 64, ws, &w);
  if (!ws || ws_bytes < need) return DFLASH_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int dt = d.dtype, D = d.hidden;
  HIPCHK(launch_embed(dt, block_ids, nullptr, 1, batch, B, d.mask_token_id, d.embed, d.vocab, D,
                      w.h, hidden_dbg, kv->error_flags, st));
  e = run_layers(m, kv, batch, B, w, /*causal=*/1, /*write_cache=*/1, feats_out, hidden_dbg,
                 d.final_norm, /*compact_final=*/0, st);
  if (e) return e;
  float* logits = logits_dbg ? logits_dbg : w.logits;
  HIPCHK(launch_gemm(dt, w.u, D, one_seg(d.lm_head, d.vocab, D), logits, M, d.vocab, D, 1, st));
  HIPCHK(launch_argmax(logits, M, d.vocab, target_argmax, st));
  HIPCHK(launch_accept(block_ids, target_argmax, batch, B, tau, bonus, st));
  return DFLASH_OK;
}

int dflash_kv_commit(dflash_kv* tkv, dflash_kv* dkv, const int32_t* tau, int32_t block,
                     void* stream) {
  if (!tau || (!tkv && !dkv)) return DFLASH_E_ARG;
  if (block < 1 || block > 64) return DFLASH_E_SHAPE;
  if (tkv && (!tkv->seq_len || tkv->batch < 1)) return DFLASH_E_ARG;
  if (dkv && (!dkv->seq_len || dkv->batch < 1)) return DFLASH_E_ARG;
  if (tkv && dkv && tkv->batch != dkv->batch) return DFLASH_E_SHAPE;
  const int batch = tkv ? tkv->batch : dkv->batch;
  HIPCHK(launch_commit(tkv ? tkv->seq_len : nullptr, dkv ? dkv->seq_len : nullptr,
                       tkv ? tkv->error_flags : nullptr, dkv ? dkv->error_flags : nullptr, tau,
                       batch, block, (hipStream_t)stream));
  return DFLASH_OK;
}

}  // extern "C"
