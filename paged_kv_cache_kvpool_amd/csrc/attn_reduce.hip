// Cross-split merge: out = sum_i 2^{(m_i - M)c} o_i / sum_i 2^{(m_i - M)c} l_i, M = max_i m_i,
// over the splits of one (row, q-head).  Every partial's contribution is summed in a fixed
// order, so the result is reproducible run to run (no float atomics: sparkinfer server README,
// "Determinism").  Rows whose keys all fall in split 0 were finished by the attention kernel.
//
// One 256-thread workgroup per (row of the partial buffers, q-head); the row's sequence is
// found from the per-sequence counts of split-K tokens.  Thread t owns dims 4 (t % (D/4)) .. +4
// and the splits t / (D/4), + 256/(D/4), ...; it merges them in split order with a running max
// (each partial's m, l and o loaded together, so the loads of all its splits are independent
// and go out at once: one memory round trip), and the split groups are merged in LDS in a fixed
// order at the end.
#include "common.h"
#include "kernels.h"

namespace kvp {

namespace {
constexpr int RT = 256;  // threads per workgroup
}  // namespace

// The merge of partial row r for q-head hh (one workgroup).
template <typename E, int D>
__device__ __forceinline__ void reduce_split_row(const AttnArgs& a, int r, int hh) {
  constexpr int DQ = D / 4;    // float4 columns
  constexpr int SG = RT / DQ;  // split groups
  const int tid = threadIdx.x;
  int s, i, q_start, L, T;
  if (!find_split_row(a, r, s, i, q_start, L, T)) return;
  int Lv, vs1, vshift;
  seq_vlayout(a, L, T, Lv, vs1, vshift);  // the splits cut the sequence's virtual key positions
  const int p = virt_key(L - T + i, vs1, vshift);
  const int ns = min(a.max_splits, p / seq_split(a, Lv, T, vshift > 0) + 1);
  if (ns <= 1) return;
  const int grow = q_start + i;
  if (grow >= a.total_q) return;
  const size_t slot0 = ((size_t)r * a.num_q_heads + hh) * a.max_splits;
  const float c = a.scale_log2;

  __shared__ float s_m[SG], s_l[SG];
  __shared__ floatx4 s_acc[SG][DQ];

  // Running merge over this thread's splits, in split order: mt is the largest m seen so far
  // (-inf before any split with a key), lt and acc the sums scaled to it.  A split with no key
  // for this row (m = -inf, l = 0, o = 0) contributes nothing.  Splits go in batches of 8 whose
  // loads are all issued before any is used (indices clamped, no branches around them).
  const int dq = tid % DQ, sg = tid / DQ;
  float mt = -INFINITY, lt = 0.f;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  const float2* pml = reinterpret_cast<const float2*>(a.part_ml) + slot0;
  const floatx4* po = reinterpret_cast<const floatx4*>(a.part_o + slot0 * D) + dq;
  constexpr int NB = 8;
  for (int k0 = sg; k0 < ns; k0 += NB * SG) {
    float2 ml[NB];
    floatx4 ok[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int k = min(k0 + u * SG, ns - 1);
      ml[u] = pml[k];
      ok[u] = po[(size_t)k * DQ];
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const bool has = k0 + u * SG < ns && ml[u].x != -INFINITY;
      const float mn = has ? fmaxf(mt, ml[u].x) : mt;
      const float sc = mn == mt ? 1.f : fast_exp2((mt - mn) * c);  // 0 while mt is -inf
      const float w = has ? fast_exp2((ml[u].x - mn) * c) : 0.f;
      acc = acc * sc + w * ok[u];
      lt = fmaf(w, ml[u].y, lt * sc);
      mt = mn;
    }
  }
  s_acc[sg][dq] = acc;
  if (dq == 0) {
    s_m[sg] = mt;
    s_l[sg] = lt;
  }
  __syncthreads();
  if (tid < DQ) {
    float M = s_m[0];
#pragma unroll
    for (int g2 = 1; g2 < SG; ++g2) M = fmaxf(M, s_m[g2]);
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
#pragma unroll
    for (int g2 = 0; g2 < SG; ++g2) {
      const float mg = s_m[g2];
      const float w = mg == -INFINITY ? 0.f : fast_exp2((mg - M) * c);
      v += w * s_acc[g2][tid];
      den = fmaf(w, s_l[g2], den);
    }
    v *= 1.f / den;
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

template <typename E, int D>
__global__ __launch_bounds__(256) void attn_reduce_kernel(AttnArgs a) {
  reduce_split_row<E, D>(a, blockIdx.x, blockIdx.y);
}

// ---- prefill key ranges ----------------------------------------------------------------
// Sequence s of query token grow (q_lens prefix sums, 64 sequences per step), the token's index
// i in it and the sequence's lengths.  False past the last token.
__device__ __forceinline__ bool find_token(const AttnArgs& a, int grow, int& s, int& i, int& L,
                                           int& T) {
  const int lane = threadIdx.x & (WAVE - 1);
  int qbase = 0;
  for (int base = 0; base < a.num_seqs; base += WAVE) {
    const int j = base + lane;
    int Lj = 0, Tj = 0, q = 0;
    if (j < a.num_seqs) {
      const int ql = a.q_lens[j];
      Lj = min(max(a.ctx_lens[j], 0), a.max_blocks_per_seq * a.block_size);
      Tj = min(max(ql, 0), Lj);
      q = max(0, ql);
    }
    const int qin = wave_incl_scan(q);
    const int tot = __builtin_amdgcn_readlane(qin, WAVE - 1);
    const int g = grow - qbase;
    if (g < tot) {
      const int k = __builtin_popcountll(__builtin_amdgcn_ballot_w64(qin <= g));
      s = base + k;
      i = g - (__builtin_amdgcn_readlane(qin, k) - __builtin_amdgcn_readlane(q, k));
      L = __builtin_amdgcn_readlane(Lj, k);
      T = __builtin_amdgcn_readlane(Tj, k);
      return true;
    }
    qbase += tot;
  }
  return false;
}

// Merge of the pf_ksplit (= KR) key-range partials of the prefill rows of one query token:
// out = sum_k 2^{m_k - M} o_k / sum_k 2^{m_k - M} l_k, M = max_k m_k (m in exp2 units), summed
// in range order.  Grid (token, slice group): thread t of workgroup y takes the (q-head, 4 dims)
// slice 256 y + t and loads its KR partials at once; tokens of split-K sequences leave at once.
constexpr int kMaxKSplit = 8;
template <typename E, int D, int KR>
__device__ __forceinline__ void merge_prefill_token(const AttnArgs& a, int grow, int y) {
  constexpr int DQ = D / 4;
  const int Hq = a.num_q_heads;
  const int u = y * RT + threadIdx.x;  // (q-head, 4-dim) slice
  const bool slice = u < Hq * DQ;
  const int hh = slice ? u / DQ : 0, dq = u % DQ;
  // The token's partials are requested before its metadata (their slots depend on the token
  // and slice alone, inside the buffer for every token < total_q), so the two reads overlap; a
  // token the prefill kernel did not compute leaves them unused.  (Every lane stays for the
  // token search, whose wave scans need the whole wave.)
  const size_t slot0 = ((size_t)grow * Hq + hh) * KR;
  const float2* pml = reinterpret_cast<const float2*>(a.pf_part_ml) + slot0;
  const floatx4* po = reinterpret_cast<const floatx4*>(a.pf_part_o) + slot0 * DQ + dq;
  float2 ml[KR];
  floatx4 ok[KR];
  if (slice) {
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      ml[k] = pml[k];
      ok[k] = po[(size_t)k * DQ];
    }
  }
  int s, i, L, T;
  if (!find_token(a, grow, s, i, L, T)) return;
  if (T <= a.split_q_max || i >= T) return;  // not a row the prefill kernel computed
  if (!slice) return;
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < KR; ++k) M = fmaxf(M, ml[k].x);
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    if (ml[k].x == -INFINITY) continue;  // an empty range adds nothing
    const float w = fast_exp2(ml[k].x - M);
    acc += w * ok[k];
    den = fmaf(w, ml[k].y, den);
  }
  const floatx4 v = acc * (1.f / den);
  const size_t ob = ((size_t)grow * Hq + hh) * D + 4 * dq;
  if constexpr (sizeof(E) == 2) {
    const uint32_t w0 = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
    const uint32_t w1 = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + ob) = make_uint2(w0, w1);
  } else {
    *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(a.out) + ob) = v;
  }
}

template <typename E, int D, int KR>
__global__ __launch_bounds__(256) void attn_reduce_prefill_kernel(AttnArgs a) {
  merge_prefill_token<E, D, KR>(a, blockIdx.x, blockIdx.y);
}

// Both merges in one launch (a call with split-K rows and prefill key ranges): workgroups
// [0, part_rows * Hq) merge split-K rows as attn_reduce_kernel, the rest merge prefill tokens as
// attn_reduce_prefill_kernel (block-uniform choice; the two sets touch disjoint rows of out).
template <typename E, int D, int KR>
__global__ __launch_bounds__(256) void attn_reduce_both_kernel(AttnArgs a, int pf_groups) {
  const int nsplit = a.part_rows * a.num_q_heads;
  const int b = blockIdx.x;
  if (b < nsplit) {
    reduce_split_row<E, D>(a, b / a.num_q_heads, b % a.num_q_heads);
  } else {
    const int c = b - nsplit;
    merge_prefill_token<E, D, KR>(a, c / pf_groups, c % pf_groups);
  }
}

template <typename E, int D, int KR>
hipError_t launch_reduce_pf(const AttnArgs& a, bool both, hipStream_t st) {
  if constexpr (KR > kMaxKSplit) {
    return hipErrorInvalidConfiguration;
  } else if (a.pf_ksplit != KR) {
    return launch_reduce_pf<E, D, KR + 1>(a, both, st);
  } else {
    const int groups = (a.num_q_heads * (D / 4) + RT - 1) / RT;
    if (both) {
      const long long wgs = (long long)a.part_rows * a.num_q_heads + (long long)a.total_q * groups;
      if (wgs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
      attn_reduce_both_kernel<E, D, KR><<<(unsigned)wgs, RT, 0, st>>>(a, groups);
    } else {
      const dim3 grid(a.total_q, groups);
      attn_reduce_prefill_kernel<E, D, KR><<<grid, RT, 0, st>>>(a);
    }
    return hipGetLastError();
  }
}

hipError_t launch_attn_reduce_prefill(const AttnArgs& a, int elt_bytes, int head_dim, bool both,
                                      hipStream_t st) {
  if (a.pf_ksplit <= 1 || a.total_q <= 0) return both ? launch_attn_reduce(a, elt_bytes, head_dim, st) : hipSuccess;
  if (a.pf_ksplit > kMaxKSplit) return hipErrorInvalidConfiguration;
  both = both && a.part_rows > 0;
  if (elt_bytes == 2)
    return head_dim == 128 ? launch_reduce_pf<uint16_t, 128, 2>(a, both, st) : launch_reduce_pf<uint16_t, 64, 2>(a, both, st);
  return head_dim == 128 ? launch_reduce_pf<float, 128, 2>(a, both, st) : launch_reduce_pf<float, 64, 2>(a, both, st);
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
