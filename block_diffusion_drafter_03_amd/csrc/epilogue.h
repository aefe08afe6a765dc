// Fused GEMM epilogues shared by the MFMA and VALU GEMM kernels.
//
// A GEMM computes acc[m][n] = sum_k A[m][k] W[n][k] over the FULL K inside one workgroup,
// so every epilogue sees final values.  Optional A-side RMSNorm (norm_g != NULL): the
// kernel accumulates sum_k A[m][k]^2 of the raw rows while loading them, multiplies the
// operand by the gain, and scales acc by rstd[m] = 1/sqrt(mean_k A^2 + eps) here, so
// RMSNorm(x) W^T never needs a separate pass over x.
//
// Packed weight row order that makes every pair-wise epilogue local to a pair of adjacent
// output columns (2i, 2i+1) (bfloat16 models then store the matrices in B-fragment order):
//   * q and k heads of DFLASH_W_QKV are stored rotary-interleaved: packed row 2i of a head
//     is original row i and packed row 2i+1 is original row i + d/2, so the two inputs of
//     one rotate-half rotation land in columns 2i, 2i+1 (v heads are stored plainly);
//   * DFLASH_W_GATE_UP rows are interleaved: packed row 2j = gate row j, 2j+1 = up row j.
#pragma once
#include "common.h"
#include "kernels.h"

namespace dflash {

DF_DEV unsigned long long pack_argmax_key(float v, int idx) {
  unsigned u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // order-preserving map of the float
  return ((unsigned long long)u << 32) | (unsigned)(0xFFFFFFFFu - (unsigned)idx);  // ties: lowest idx
}
DF_DEV int unpack_argmax_idx(unsigned long long key) {
  return (int)(0xFFFFFFFFu - (unsigned)(key & 0xFFFFFFFFull));
}

// Greedy acceptance of sequence b by one wavefront (B <= 64): lane j decodes g_j, the
// target's argmax after row j, from its packed key; lane j >= 1 compares draft d_j with
// g_{j-1} (its neighbour's id); a ballot of the mismatches gives the leading run of matches
// a by a bit scan; tau = a + 1 and bonus = g_a.  AGENT: the keys are read with agent-scope
// loads (they were updated by other workgroups of the same launch).
template <bool AGENT>
DF_DEV void accept_wave(const unsigned long long* keys, const int32_t* drafts, int B, int b, int32_t* g,
                        int32_t* tau, int32_t* bonus) {
  const int j = threadIdx.x & 63;
  unsigned long long k = 0ull;
  if (j < B)
    k = AGENT ? __hip_atomic_load(keys + (size_t)b * B + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
              : keys[(size_t)b * B + j];
  const int gj = j < B ? unpack_argmax_idx(k) : -1;
  if (j < B) g[(size_t)b * B + j] = gj;
  const int gprev = __shfl_up(gj, 1, 64);
  const bool miss = j >= 1 && j < B && drafts[(size_t)b * (B - 1) + j - 1] != gprev;
  const unsigned long long mask = __ballot(miss);
  // drafts 1 .. a match, draft a + 1 (if any) does not: a = (lowest mismatching lane) - 1
  const int a = mask ? __ffsll((long long)mask) - 2 : B - 1;
  const int ga = __shfl(gj, a, 64);
  if (j == 0) {
    tau[b] = a + 1;
    bonus[b] = ga;
  }
}

template <typename T, int KIND>
DF_DEV void epi_elem(const EpiArgs& e, int row, int col, float v) {
  switch (KIND) {
    case EPI_STORE_F32:
      ((float*)e.out)[e.afrag ? afrag_off(row, col, e.ldo >> 5) : (size_t)row * e.ldo + col] = v;
      break;
    case EPI_RESID: {
      const size_t i = (size_t)row * e.ldh + col;
      const size_t ih = e.afrag ? afrag_off(row, col, e.ldh >> 5) : i;
      const float x = e.h[ih] + v;
      e.h[ih] = x;
      if (e.hdbg) e.hdbg[i] = x;
      if (e.tap) ((T*)e.tap)[(size_t)row * e.tap_ld + e.tap_col + col] = from_f<T>(x);
      break;
    }
    default:
      break;
  }
}

// cache slot of position `pos` of sequence `b`; returns false (and flags) when unmapped
DF_DEV bool cache_slot(const EpiArgs& e, int b, int pos, int* page) {
  const int pg = pos >> 6;
  int p = -1;
  if (b >= 0 && b < e.batch && pos >= 0 && pg < e.max_pages) p = e.block_table[(size_t)b * e.max_pages + pg];
  if (p < 0 || p >= e.num_pages) {
    flag_error(e.err, DEVERR_PAGE);
    return false;
  }
  *page = p;
  return true;
}

// (v0, v1) = acc[row][col], acc[row][col + 1] with col even.
template <typename T, int KIND>
DF_DEV void epi_pair(const EpiArgs& e, int row, int col, float v0, float v1) {
  switch (KIND) {
    case EPI_SWIGLU: {
      const int c = col >> 1;
      const float y = v0 / (1.f + expf(-v0)) * v1;
      if (e.act_pair) store_pair((bf16*)e.act, pfrag_off(row, c, e.F >> 5), y);
      else e.act[e.afrag ? afrag_off(row, c, e.F >> 5) : (size_t)row * e.F + c] = y;
      break;
    }
    case EPI_QKV: {
      const int b = row / e.B, j = row - (row / e.B) * e.B;
      const int pos = e.seq_len[b] + j;
      const int hd = e.hd, head = col / hd, el = col - head * hd;
      int page = -1;
      const bool cache = e.has_cache && head >= e.Hq && cache_slot(e, b, pos, &page);
      const int slot = pos & 63;
      if (head < e.Hq + e.Hkv) {
        const int i = el >> 1;
        const float2 cs = e.rope[(size_t)row * (hd >> 1) + i];
        const float y1 = v0 * cs.x - v1 * cs.y, y2 = v1 * cs.x + v0 * cs.y;
        if (head < e.Hq) {
          float* dst = e.q + (size_t)row * e.Hq * hd + (size_t)head * hd;
          dst[i] = y1;
          dst[i + hd / 2] = y2;
        } else {
          const int kh = head - e.Hq;
          const size_t o = (size_t)row * e.Hkv * hd + (size_t)kh * hd;
          T* dst = (T*)e.kblk + o;
          const T k1 = from_f<T>(y1), k2 = from_f<T>(y2);
          dst[i] = k1;
          dst[i + hd / 2] = k2;
          if constexpr (sizeof(T) == 2) {   // low parts: zero when the rows are stored
            bf16* lo = (bf16*)e.kblk_lo + o;
            lo[i] = e.has_cache ? (bf16)0.f : (bf16)(y1 - (float)k1);
            lo[i + hd / 2] = e.has_cache ? (bf16)0.f : (bf16)(y2 - (float)k2);
          }
          if (cache) {
            T* kc = (T*)e.kp[0] + (((size_t)page * e.Hkv + kh) * 64 + slot) * hd;
            kc[i] = from_f<T>(y1);
            kc[i + hd / 2] = from_f<T>(y2);
          }
        }
      } else {
        const int vh = head - e.Hq - e.Hkv;
        const size_t o = ((size_t)(b * e.Hkv + vh) * hd + el) * e.Bp + j;
        T* vt = (T*)e.vblkT + o;
        const T u0 = from_f<T>(v0), u1 = from_f<T>(v1);
        vt[0] = u0;
        vt[e.Bp] = u1;
        if constexpr (sizeof(T) == 2) {
          bf16* lo = (bf16*)e.vblkT_lo + o;
          lo[0] = e.has_cache ? (bf16)0.f : (bf16)(v0 - (float)u0);
          lo[e.Bp] = e.has_cache ? (bf16)0.f : (bf16)(v1 - (float)u1);
        }
        if (cache) {
          T* vc = (T*)e.vp[0] + (((size_t)page * e.Hkv + vh) * hd + el) * 64 + slot;
          vc[0] = from_f<T>(v0);
          vc[64] = from_f<T>(v1);
        }
      }
      break;
    }
    case EPI_INJECT_KV: {
      const int b = e.row_seq[row];
      const int rp = e.row_pos[row];
      if (rp < 0 || rp >= e.pos_limit) {   // outside the range the host checked
        flag_error(e.err, DEVERR_PAGE);
        break;
      }
      const int pos = rp + ((e.pos_relative && b >= 0 && b < e.batch) ? e.seq_len[b] : 0);
      int page;
      if (!cache_slot(e, b, pos, &page)) break;
      const int slot = pos & 63, hd = e.hd;
      const int per_layer = 2 * e.Hkv * hd;
      const int l = col / per_layer, c = col - l * per_layer;
      if (c < e.Hkv * hd) {
        const int kh = c / hd, el = c - kh * hd, i = el >> 1;
        const float2 cs = e.rope[(size_t)row * (hd >> 1) + i];
        T* kc = (T*)pick8(e.kp, l) + (((size_t)page * e.Hkv + kh) * 64 + slot) * hd;
        kc[i] = from_f<T>(v0 * cs.x - v1 * cs.y);
        kc[i + hd / 2] = from_f<T>(v1 * cs.x + v0 * cs.y);
      } else {
        const int cv = c - e.Hkv * hd, vh = cv / hd, el = cv - vh * hd;
        T* vc = (T*)pick8(e.vp, l) + (((size_t)page * e.Hkv + vh) * hd + el) * 64 + slot;
        vc[0] = from_f<T>(v0);
        vc[64] = from_f<T>(v1);
      }
      break;
    }
    default:
      break;
  }
}

__host__ __device__ constexpr bool epi_is_pair(int kind) {
  return kind == EPI_SWIGLU || kind == EPI_QKV || kind == EPI_INJECT_KV;
}

}  // namespace dflash
