// Cross-split merge: out = sum_i 2^{(m_i - M)c} o_i / sum_i 2^{(m_i - M)c} l_i, M = max_i m_i,
// over the splits of one (row, q-head).  Every partial's contribution is summed in a fixed
// order, so the result is reproducible run to run (no float atomics: sparkinfer server README,
// "Determinism").  Rows whose keys all fall in split 0 were finished by the attention kernel.
//
// One 256-thread workgroup per (row of the partial buffers, q-head); the row's sequence is
// found from the per-sequence counts of split-K tokens.  The weights 2^{(m_i - M)c} are computed
// once into LDS; then thread t accumulates dims 4*(t % (D/4)) .. +4 over splits
// t / (D/4), + 256/(D/4), ..., so each pass over the partials reads whole rows of D floats
// with 16-byte loads; the split groups are summed in LDS in a fixed order at the end.
#include "common.h"
#include "kernels.h"

namespace kvp {

namespace {
constexpr int RT = 256;            // threads per workgroup
constexpr int WMAX = 4096;         // split weights held in LDS per pass
}  // namespace

template <typename E, int D>
__global__ __launch_bounds__(256) void attn_reduce_kernel(AttnArgs a) {
  constexpr int DQ = D / 4;        // float4 columns
  constexpr int SG = RT / DQ;      // split groups
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = blockIdx.x, hh = blockIdx.y;
  int s, i, q_start;
  if (!find_split_row(a, r, s, i, q_start)) return;
  int L, T;
  seq_lens(a, s, L, T);
  int Lv, vs1, vshift;
  seq_vlayout(a, L, T, Lv, vs1, vshift);  // the splits cut the sequence's virtual key positions
  const int p = virt_key(L - T + i, vs1, vshift);
  const int ns = min(a.max_splits, p / seq_split(a, Lv) + 1);
  if (ns <= 1) return;
  const int grow = q_start + i;
  if (grow >= a.total_q) return;
  const size_t slot0 = ((size_t)r * a.num_q_heads + hh) * a.max_splits;
  const float c = a.scale_log2;

  __shared__ float s_w[WMAX];
  __shared__ float s_red[RT / 64];
  __shared__ floatx4 s_acc[SG][DQ];

  // M = max_i m_i
  float M = -INFINITY;
  for (int k = tid; k < ns; k += RT) M = fmaxf(M, a.part_ml[2 * (slot0 + k)]);
  M = xrow_max(row_max(M));
  if (lane == 0) s_red[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  __syncthreads();

  const int dq = tid % DQ, sg = tid / DQ;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int k0 = 0; k0 < ns; k0 += WMAX) {
    const int kn = min(ns - k0, WMAX);
    for (int k = tid; k < kn; k += RT) {
      const float m = a.part_ml[2 * (slot0 + k0 + k)];
      const float w = fast_exp2((m - M) * c);
      s_w[k] = w;
      den = fmaf(w, a.part_ml[2 * (slot0 + k0 + k) + 1], den);
    }
    __syncthreads();
    const floatx4* po = reinterpret_cast<const floatx4*>(a.part_o + (slot0 + k0) * D) + dq;
    int k = sg;
#pragma unroll 4
    for (; k < kn; k += SG) acc += s_w[k] * po[(size_t)k * DQ];
    __syncthreads();
  }
  s_acc[sg][dq] = acc;
  den = xrow_sum(row_sum(den));
  if (lane == 0) s_red[wave] = den;
  __syncthreads();
  if (tid < DQ) {
    floatx4 v = s_acc[0][tid];
#pragma unroll
    for (int g2 = 1; g2 < SG; ++g2) v += s_acc[g2][tid];
    const float inv = 1.f / ((s_red[0] + s_red[1]) + (s_red[2] + s_red[3]));
    v *= inv;
    const size_t ob = ((size_t)grow * a.num_q_heads + hh) * D + 4 * tid;
    if constexpr (sizeof(E) == 2) {
      const uint32_t w0 = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
      const uint32_t w1 = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + ob) = make_uint2(w0, w1);
    } else {
      *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(a.out) + ob) = v;
    }
  }
}

hipError_t launch_attn_reduce(const AttnArgs& a, int elt_bytes, int head_dim, hipStream_t st) {
  if (a.part_rows <= 0) return hipSuccess;
  dim3 grid(a.part_rows, a.num_q_heads);
  if (elt_bytes == 2) {
    if (head_dim == 128) attn_reduce_kernel<uint16_t, 128><<<grid, RT, 0, st>>>(a);
    else attn_reduce_kernel<uint16_t, 64><<<grid, RT, 0, st>>>(a);
  } else {
    if (head_dim == 128) attn_reduce_kernel<float, 128><<<grid, RT, 0, st>>>(a);
    else attn_reduce_kernel<float, 64><<<grid, RT, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace kvp
