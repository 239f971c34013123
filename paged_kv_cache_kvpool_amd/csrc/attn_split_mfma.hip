// Split-K (flash-decoding) paged attention on the gfx950 matrix cores, bf16 K/V.
//
// Serves single-token decode of a batch (NInfer serving doc, "Execution behavior") and the
// verification of 1 + k draft tokens (sparkinfer server README, "Serve Qwen3.8 with DSpark"):
// few query rows per KV head against a long paged context.  The context of each sequence is
// cut into splits of a fixed number of keys that depend only on that sequence's length, and
// each wave reduces one split to a partial (max, sum, unnormalised output); the reduce kernel
// merges them in split order, so there are no float atomics (sparkinfer server README,
// "Determinism": the decode path has none).
//
// One wave handles up to 16*NT query rows (row = token * G + head-in-group, so the G q-heads
// that share a KV head are computed together from one read of K/V).  Per 32-key chunk:
//   S^T[key][row] = K[key][:] . Q[row][:]        2 x (D/32) v_mfma_f32_16x16x32_bf16 per N-tile
//   online softmax on the fp32 scores (exp2 with scale*log2e folded in)
//   O^T[dim][row] += V^T[dim][key] . P^T[key][row]   D/16 MFMAs per N-tile
// The A operands come straight from the pool: a K tile is stored as 16-byte dim chunks of 16
// tokens and a V tile dims-major, so every lane loads one 16-byte run and each load
// instruction covers whole 64-byte segments.  Keys inside a chunk are assigned to the K
// operand's rows in the order pi(m) = 8*(m/4) + 4*half + m%4, which makes the score tile's
// output layout (lane = row, 4 consecutive entries per lane group) equal to the P^T operand
// layout of the PV product, so P never leaves registers.
#include "common.h"
#include "kernels.h"

namespace kvp {

namespace {

__device__ __forceinline__ bf16x8 load16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace

template <int D, int NT>
__global__ __launch_bounds__(64) void attn_split_mfma_kernel(AttnArgs a) {
  constexpr int KK = D / 32;  // 32-dim steps of the score product
  constexpr int MT = D / 16;  // 16-dim tiles of the output
  const int lane = threadIdx.x;
  const int n = lane & 15, g = lane >> 4;
  const int s = blockIdx.z, kvh = blockIdx.y;
  const int rt = blockIdx.x % a.row_tiles, sp = blockIdx.x / a.row_tiles;
  int L, T;
  seq_lens(a, s, L, T);
  const int G = a.group;
  const int rows = T * G;
  const int r0 = rt * 16 * NT;
  if (r0 >= rows) return;
  const int p_last = L - T + (min(r0 + 16 * NT, rows) - 1) / G;
  int kb = 0, ke = min(L, p_last + 1);
  if (a.split_mode) {
    kb = sp * a.split_tokens;
    ke = min(ke, kb + a.split_tokens);
  }
  if (kb >= ke) return;
  const int q_start = wave_prefix_total(a.q_lens, s);
  const int Hq = a.num_q_heads;

  // Q^T as the B operand: lane (n, g) holds row n of N-tile nt, dims 32*kk + 8*g .. +8.
  bf16x8 qb[NT][KK];
  int prow[NT];
  int grow[NT], ghead[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = r0 + 16 * nt + n;
    const int i = r / G;
    grow[nt] = q_start + i;
    ghead[nt] = kvh * G + r % G;
    const bool valid = r < rows && grow[nt] < a.total_q;
    prow[nt] = valid ? L - T + i : -1;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) +
                         ((size_t)(valid ? grow[nt] : 0) * Hq + (valid ? ghead[nt] : 0)) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      bf16x8 z = {};
      qb[nt][kk] = valid ? load16(qp + 32 * kk + 8 * g) : z;
    }
  }

  float m_run[NT], l_run[NT];
  floatx4 o[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const int32_t* tbl = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  const uint16_t* kl = reinterpret_cast<const uint16_t*>(a.k_layer);
  const uint16_t* vl = reinterpret_cast<const uint16_t*>(a.v_layer);
  const float c = a.scale_log2;
  // K operand row m of half h reads key pi(m) = 8*(m/4) + 4*h + m%4 of the 32-key chunk.
  const int key_lo = 8 * (n >> 2) + (n & 3);

  for (int c0 = kb; c0 < ke; c0 += 32) {
    size_t toff[2];
    bool tv[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int pos = c0 + 16 * t;
      tv[t] = pos < ke;
      toff[t] = tv[t] ? tile_offset(tbl, pos, kvh, a.block_size, a.num_blocks, a.num_kv_heads, D)
                      : 0;
    }
    bf16x8 ka[2][KK];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int key = key_lo + 4 * h;
      const int t = key >> 4, tok = key & 15;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        bf16x8 z = {};
        ka[h][kk] = tv[t] ? load16(kl + toff[t] + ((4 * kk + g) * 16 + tok) * 8) : z;
      }
    }
    bf16x8 va[MT];
    {
      const int t = g >> 1;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        bf16x8 z = {};
        va[mt] = tv[t] ? load16(vl + toff[t] + (16 * mt + n) * 16 + 8 * (g & 1)) : z;
      }
    }
    if (c0 + 32 > ke) {
      // Last chunk: slots at or past ke may hold anything (NaN included); zero their V so
      // that p = 0 really contributes nothing.
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (c0 + 8 * g + j >= ke) va[mt][j] = (__bf16)0.f;
    }

#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      floatx4 sc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) acc = mfma16(ka[h][kk], qb[nt][kk], acc);
        sc[h] = acc;
      }
      // This lane now holds row n's scores for keys c0 + 8*g + j, j = 4*h + i.
      float sv[8];
      float cmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = c0 + 8 * g + j;
        const float x = sc[j >> 2][j & 3];
        sv[j] = (key < ke && key <= prow[nt]) ? x : -INFINITY;
        cmax = fmaxf(cmax, sv[j]);
      }
      cmax = xrow_max(cmax);
      const float m_new = fmaxf(m_run[nt], cmax);
      const bool none = (m_new == -INFINITY);
      const float alpha = none ? 1.f : fast_exp2((m_run[nt] - m_new) * c);
      const float msub = none ? 0.f : m_new * c;
      uint32_t pk[4];
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float p0 = round_to_bf16(fast_exp2(sv[j] * c - msub));
        const float p1 = round_to_bf16(fast_exp2(sv[j + 1] * c - msub));
        psum += p0 + p1;
        pk[j >> 1] = pack_exact_bf16(p0, p1);
      }
      l_run[nt] = l_run[nt] * alpha + psum;
      m_run[nt] = m_new;
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[nt][mt] = mfma16(va[mt], pb, o[nt][mt] * alpha);
    }
  }

  // Row n's sum is spread over the 4 lane groups; the max is already uniform across them.
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float lt = xrow_sum(l_run[nt]);
    if (prow[nt] < kb) continue;  // padding row, or a row that sees no key of this split
    const size_t rh = (size_t)grow[nt] * Hq + ghead[nt];
    if (a.split_mode) {
      const size_t slot = rh * a.max_splits + sp;
      if (g == 0) {
        a.part_ml[2 * slot] = m_run[nt];
        a.part_ml[2 * slot + 1] = lt;
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        *reinterpret_cast<floatx4*>(a.part_o + slot * D + 16 * mt + 4 * g) = o[nt][mt];
    } else {
      const float inv = 1.f / lt;
      uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + rh * D;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const floatx4 v = o[nt][mt] * inv;
        const uint32_t w0 = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
        const uint32_t w1 = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
        *reinterpret_cast<uint2*>(op + 16 * mt + 4 * g) = make_uint2(w0, w1);
      }
    }
  }
}

hipError_t launch_attn_split_mfma(const AttnArgs& a, int head_dim, int rows_per_tile,
                                  int grid_x, hipStream_t st) {
  dim3 grid(grid_x, a.num_kv_heads, a.num_seqs);
  if (head_dim == 128) {
    if (rows_per_tile <= 16) attn_split_mfma_kernel<128, 1><<<grid, 64, 0, st>>>(a);
    else attn_split_mfma_kernel<128, 2><<<grid, 64, 0, st>>>(a);
  } else {
    if (rows_per_tile <= 16) attn_split_mfma_kernel<64, 1><<<grid, 64, 0, st>>>(a);
    else attn_split_mfma_kernel<64, 2><<<grid, 64, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace kvp
