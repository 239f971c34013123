// Cross-split merge: out = sum_i 2^{(m_i - M)c} o_i / sum_i 2^{(m_i - M)c} l_i, M = max_i m_i,
// taken over the splits of one (row, q-head) in increasing split order.  The merge order is
// fixed, so the result is reproducible run to run (no float atomics: sparkinfer server
// README, "Determinism").  One wave per (query row, q-head); each lane owns D/64 dims.
#include "common.h"
#include "kernels.h"

namespace kvp {

template <typename E, int D>
__global__ __launch_bounds__(64) void attn_reduce_kernel(AttnArgs a) {
  constexpr int DPL = D / 64;
  const int lane = threadIdx.x;
  const int s = blockIdx.z, hh = blockIdx.y, i = blockIdx.x;
  int L, T;
  seq_lens(a, s, L, T);
  if (i >= T) return;
  const int grow = wave_prefix_total(a.q_lens, s) + i;
  if (grow >= a.total_q) return;
  const int p = L - T + i;
  const int ns = min(a.max_splits, p / a.split_tokens + 1);
  const size_t slot0 = ((size_t)grow * a.num_q_heads + hh) * a.max_splits;
  const float c = a.scale_log2;

  float M = -INFINITY;
  for (int k = lane; k < ns; k += 64) M = fmaxf(M, a.part_ml[2 * (slot0 + k)]);
  M = xrow_max(row_max(M));

  float acc[DPL] = {};
  float den = 0.f;
  for (int k = 0; k < ns; ++k) {
    const float m = a.part_ml[2 * (slot0 + k)];
    const float l = a.part_ml[2 * (slot0 + k) + 1];
    const float w = fast_exp2((m - M) * c);
    den = fmaf(w, l, den);
    const float* op = a.part_o + (slot0 + k) * D + lane * DPL;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = fmaf(w, op[e], acc[e]);
  }
  const float inv = 1.f / den;
  const size_t ob = ((size_t)grow * a.num_q_heads + hh) * D + lane * DPL;
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    if constexpr (sizeof(E) == 2)
      reinterpret_cast<uint16_t*>(a.out)[ob + e] = (uint16_t)f32_to_bf16_bits(acc[e] * inv);
    else
      reinterpret_cast<float*>(a.out)[ob + e] = acc[e] * inv;
  }
}

hipError_t launch_attn_reduce(const AttnArgs& a, int elt_bytes, int head_dim, int max_q_len,
                              hipStream_t st) {
  dim3 grid(max_q_len, a.num_q_heads, a.num_seqs);
  if (elt_bytes == 2) {
    if (head_dim == 128) attn_reduce_kernel<uint16_t, 128><<<grid, 64, 0, st>>>(a);
    else attn_reduce_kernel<uint16_t, 64><<<grid, 64, 0, st>>>(a);
  } else {
    if (head_dim == 128) attn_reduce_kernel<float, 128><<<grid, 64, 0, st>>>(a);
    else attn_reduce_kernel<float, 64><<<grid, 64, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace kvp
