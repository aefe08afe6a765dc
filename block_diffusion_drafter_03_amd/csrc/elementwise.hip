// Row kernels of the drafter / verifier step that are not GEMM epilogues: the block
// embedding, argmax decoding, greedy acceptance and the commit of sequence lengths.
#include "common.h"
#include "kernels.h"

namespace dflash {

// ---------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(EmbedArgs a) {
  const int B = a.B, D = a.D;
  const int row = blockIdx.x, b = row / B, j = row % B;
  // mode 0: [anchor, mask ...]; mode 1: [anchor, drafts ...] with ids = drafts [batch, B-1]
  int tok = j == 0 ? a.anchor[b] : (a.mode == 0 ? a.mask_id : a.ids[(size_t)b * (B - 1) + j - 1]);
  if (tok < 0 || tok >= a.V) {
    if (threadIdx.x == 0) flag_error(a.err, DEVERR_TOKEN);
    tok = 0;
  }
  const T* e = (const T*)a.E + (size_t)tok * D;
  for (int c = threadIdx.x; c < D; c += 256) {
    const float x = to_f(e[c]);
    a.h[a.afrag ? afrag_off(row, c, D >> 5) : (size_t)row * D + c] = x;
    if (a.hdbg) a.hdbg[(size_t)row * D + c] = x;
  }
  // RoPE angles of this row's position (float64, rounded to float32)
  const int pos = a.seq_len[b] + j;
  for (int i = threadIdx.x; i < a.hd / 2; i += 256) {
    float c, s;
    rope_cs(pos, i, a.hd, a.rope_base, &c, &s);
    a.rope[(size_t)row * (a.hd / 2) + i] = make_float2(c, s);
  }
  // arm this call's argmax keys
  if (row == 0)
    for (int i = threadIdx.x; i < a.n_keys; i += 256) a.keys[i] = 0ull;
}

hipError_t launch_embed(int dt, const EmbedArgs& a, hipStream_t st) {
  const int rows = a.batch * a.B;
  if (dt == BF16)
    hipLaunchKernelGGL(embed_kernel<bf16>, dim3(rows), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(rows), dim3(256), 0, st, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(64) void rope_rows_kernel(const int32_t* row_seq, const int32_t* row_pos,
                                                       int pos_relative, const int32_t* seq_len,
                                                       int batch, int hd, double base, float2* rope) {
  const int row = blockIdx.x;
  const int b = row_seq[row];
  const int pos = row_pos[row] + ((pos_relative && b >= 0 && b < batch) ? seq_len[b] : 0);
  for (int i = threadIdx.x; i < hd / 2; i += 64) {
    float c, s;
    rope_cs(pos, i, hd, base, &c, &s);
    rope[(size_t)row * (hd / 2) + i] = make_float2(c, s);
  }
}

hipError_t launch_rope_rows(const int32_t* row_seq, const int32_t* row_pos, int pos_relative,
                            const int32_t* seq_len, int batch, int rows, int hd, double base,
                            float2* rope, hipStream_t st) {
  hipLaunchKernelGGL(rope_rows_kernel, dim3(rows), dim3(64), 0, st, row_seq, row_pos, pos_relative,
                     seq_len, batch, hd, base, rope);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
DF_DEV int key_index(unsigned long long k) { return (int)(0xFFFFFFFFu - (unsigned)(k & 0xFFFFFFFFull)); }

// draft ids of the masked rows j = 1 .. B-1 of every block (the anchor rows' argmax is unused)
__global__ void unpack_ids_kernel(const unsigned long long* keys, int n, int B, int32_t* ids) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) ids[i] = key_index(keys[(i / (B - 1)) * B + i % (B - 1) + 1]);
}

hipError_t launch_unpack_ids(const unsigned long long* keys, int batch, int B, int32_t* ids,
                             hipStream_t st) {
  const int n = batch * (B - 1);
  hipLaunchKernelGGL(unpack_ids_kernel, dim3((n + 255) / 256), dim3(256), 0, st, keys, n, B, ids);
  return hipGetLastError();
}

// g = argmax of every verify row; a = leading drafts that equal the target's choice at
// the previous row; tau = a + 1; bonus = g_a.
__global__ void accept_kernel(const unsigned long long* keys, const int32_t* drafts, int batch,
                              int B, int32_t* g, int32_t* tau, int32_t* bonus) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  for (int j = 0; j < B; ++j) g[(size_t)b * B + j] = key_index(keys[(size_t)b * B + j]);
  int a = 0;
  while (a < B - 1 && drafts[(size_t)b * (B - 1) + a] == key_index(keys[(size_t)b * B + a])) ++a;
  tau[b] = a + 1;
  bonus[b] = key_index(keys[(size_t)b * B + a]);
}

hipError_t launch_accept(const unsigned long long* keys, const int32_t* drafts, int batch, int B,
                         int32_t* g, int32_t* tau, int32_t* bonus, hipStream_t st) {
  hipLaunchKernelGGL(accept_kernel, dim3((batch + 63) / 64), dim3(64), 0, st, keys, drafts, batch,
                     B, g, tau, bonus);
  return hipGetLastError();
}

__global__ void commit_kernel(int32_t* seq_t, int32_t* seq_d, int32_t* err_t, int32_t* err_d,
                              const int32_t* tau, int batch, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= batch) return;
  int t = tau[b];
  if (t < 1 || t > B) {
    flag_error(err_t, DEVERR_TAU);
    flag_error(err_d, DEVERR_TAU);
    t = t < 1 ? 1 : B;
  }
  if (seq_t) seq_t[b] += t;
  if (seq_d) seq_d[b] += t;
}

hipError_t launch_commit(int32_t* seq_t, int32_t* seq_d, int32_t* err_t, int32_t* err_d,
                         const int32_t* tau, int batch, int B, hipStream_t st) {
  hipLaunchKernelGGL(commit_kernel, dim3((batch + 63) / 64), dim3(64), 0, st, seq_t, seq_d, err_t,
                     err_d, tau, batch, B);
  return hipGetLastError();
}

}  // namespace dflash
