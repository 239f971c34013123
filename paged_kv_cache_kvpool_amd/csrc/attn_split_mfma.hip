// Split-K (flash-decoding) paged attention on the gfx950 matrix cores, bf16 K/V.
//
// Serves single-token decode of a batch (NInfer serving doc, "Execution behavior") and the
// verification of 1 + k draft tokens (sparkinfer server README, "Serve Qwen3.8 with DSpark"):
// few query rows per KV head against a long paged context.  Each sequence's context is cut
// into splits of a fixed number of keys (so the cut depends only on that sequence's length)
// and one workgroup reduces one split to a partial (max, sum, unnormalised output); the
// reduce kernel merges splits in split order, so there are no float atomics (sparkinfer
// server README, "Determinism": the decode path has none).  A row whose keys all fall in split
// 0 is finished here and skips the reduce.
//
// Workgroup = 4 waves over one (row tile of <= 16*NT rows, split, KV head, sequence).  Rows are
// (token, head-in-group) pairs, so the G q-heads sharing a KV head use one read of K/V.  Each
// wave takes a contiguous quarter of the split and walks it in 32-key chunks:
//   S^T[key][row] = K[key][:] . Q[row][:]          2 x (D/32) v_mfma_f32_16x16x32_bf16 / N-tile
//   online softmax on the fp32 scores (exp2, scale*log2e folded in)
//   O^T[dim][row] += V^T[dim][key] . P^T[key][row]  D/16 MFMAs per N-tile
// Memory: the A operands load straight from the pool (K tiles are 16-byte dim chunks of 16
// tokens, V tiles are dims-major), every byte of a tile read once, and every load instruction
// reads one tile from a wave-uniform base: 1 KiB contiguous for K, 512 bytes for V.  Loads are
// double-buffered: chunk i+1 is in flight while chunk i is computed (32 KiB per wave), and the
// block ids of the wave's tiles are read once into lanes and broadcast with v_readlane, so no
// table read sits between a chunk and its data.  Score tile h of a chunk is pool tile h, so a
// lane of the score output holds keys 4*g .. 4*g+3 of both tiles for its row; the PV product
// takes exactly those 8 keys as its k-slice (V^T rows read as two 8-byte runs), so P stays in
// registers.  The 4 waves' partials merge through LDS at the end.
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

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int D>
struct Chunk {
  bf16x8 k[2][D / 32];  // K operand of score tile h (= pool tile h of the chunk)
  u32x2 v[2][D / 16];   // V^T operand halves: keys 4g..4g+3 of pool tile 0 and of tile 1
};

}  // namespace

// NW: waves per workgroup sharing one split (their partials merge through LDS); NW == 1 gives
// one independent wave per split, which the dispatcher balances at the finest grain.
// RELOAD: the wave's span may exceed 128 tiles (calls without splits), so block ids are
// reloaded every 128 tiles.  Without it (split mode, span <= 2048 keys per wave) they are read
// once, and no load in the chunk loop can force a wait on the chunks in flight.
template <int D, int NT, bool RELOAD, int NW>
__global__ __launch_bounds__(64 * NW) void attn_split_mfma_kernel(AttnArgs a) {
  constexpr int KK = D / 32;  // 32-dim steps of the score product
  constexpr int MT = D / 16;  // 16-dim tiles of the output
  // The wave index is uniform within a wave: say so, so that every per-wave bound below lives
  // in scalar registers and the chunk loop is a scalar loop.
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int split = seq_split(a, L);
  int kb = 0, ke = min(L, p_last + 1);
  if (a.split_mode) {
    kb = sp * split;
    ke = min(ke, kb + split);
  }
  if (kb >= ke) return;

  // This wave's keys: a contiguous, 32-aligned quarter of [kb, ke).
  const int span = (ke - kb + NW * 32 - 1) / (NW * 32) * 32;
  const int wb = kb + wave * span;
  const int we = min(ke, wb + span);
  const int nch = wb < we ? (we - wb + 31) >> 5 : 0;
  const int ntile = wb < we ? (we - wb + 15) >> 4 : 0;
  const int tile0 = wb >> 4;

  const int32_t* tbl = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  const uint16_t* kl = reinterpret_cast<const uint16_t*>(a.k_layer);
  const uint16_t* vl = reinterpret_cast<const uint16_t*>(a.v_layer);
  const int bmask = a.block_size - 1;

  // Lane i of ids[k] holds the block id of the wave's tile tb + 64*k + i (128 tiles per batch).
  int tb = 0;
  auto load_id = [&](int base) -> int {
    // Unconditional load with the index clamped into the sequence's own blocks (ke >= 1).
    const int ti = min(base + lane, max(ntile - 1, 0));
    return tbl[(min((tile0 + ti) << 4, ke - 1)) >> a.block_shift];
  };
  int ids0 = load_id(0), ids1 = load_id(64);
  auto tile_off = [&](int ti) -> size_t {
    ti = min(ti, ntile - 1);  // past the end: re-read the last tile (a cache hit; masked out)
    if (RELOAD && ti - tb >= 128) {
      tb = ti & ~127;
      ids0 = load_id(tb);
      ids1 = load_id(tb + 64);
    }
    const int r = ti - tb;
    const int blk = r < 64 ? __builtin_amdgcn_readlane(ids0, r) : __builtin_amdgcn_readlane(ids1, r - 64);
    const int sub = (((tile0 + ti) << 4) & bmask) >> 4;
    return block_tile_offset(blk, sub, kvh, a.block_shift, a.num_blocks, a.num_kv_heads, D);
  };
  auto load_chunk = [&](Chunk<D>& c, int ci) {
    const size_t o0 = tile_off(2 * ci), o1 = tile_off(2 * ci + 1);
    const uint16_t* kt[2] = {kl + o0, kl + o1};
    const uint16_t* vt[2] = {vl + o0, vl + o1};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) c.k[h][kk] = load16(kt[h] + ((4 * kk + g) * 16 + n) * 8);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        c.v[h][mt] = *reinterpret_cast<const u32x2*>(vt[h] + (16 * mt + n) * 16 + 4 * g);
    }
  };

  // The q_lens prefix sum waits on its loads (and the block ids): do it before any chunk is in
  // flight, so that the chunk loop only ever waits for the chunk it computes.
  const int q_start = wave_prefix_total(a.q_lens, s);
  // vmcnt(0) on every path (encoding: vmcnt 0, expcnt 7, lgkmcnt 15), so the compiler knows the
  // block ids have arrived and never waits for them inside the chunk loop.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  Chunk<D> bufA, bufB;
  if (nch) load_chunk(bufA, 0);

  // Q^T as the B operand: lane (n, g) holds row n of N-tile nt, dims 32*kk + 8*g .. +8.
  const int Hq = a.num_q_heads;
  bf16x8 qb[NT][KK];
  int prow[NT];
  size_t rh[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = r0 + 16 * nt + n;
    const int i = r / G;
    const int grow = q_start + i;
    const bool valid = r < rows && grow < a.total_q;
    prow[nt] = valid ? L - T + i : -1;
    rh[nt] = valid ? (size_t)grow * Hq + kvh * G + r % G : 0;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + rh[nt] * D;
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
  const float c = a.scale_log2;

  auto compute = [&](Chunk<D>& ch, int ci) {
    const int c0 = wb + 32 * ci;
    if (c0 + 32 > we) {
      // Last chunk: slots at or past `we` may hold anything (NaN included); zero their V so
      // that p = 0 really contributes nothing.
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (c0 + 16 * h + 4 * g + j >= we) {
              const uint32_t w = ch.v[h][mt][j >> 1];
              ch.v[h][mt][j >> 1] = (j & 1) ? (w & 0x0000ffffu) : (w & 0xffff0000u);
            }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      floatx4 sc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) acc = mfma16(ch.k[h][kk], qb[nt][kk], acc);
        sc[h] = acc;
      }
      // This lane now holds row n's scores for keys c0 + 16*h + 4*g + i (j = 4*h + i).
      float sv[8];
      float cmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = c0 + 16 * (j >> 2) + 4 * g + (j & 3);
        sv[j] = (key < we && key <= prow[nt]) ? sc[j >> 2][j & 3] : -INFINITY;
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
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 va = __builtin_bit_cast(
            bf16x8, u32x4{ch.v[0][mt][0], ch.v[0][mt][1], ch.v[1][mt][0], ch.v[1][mt][1]});
        o[nt][mt] = mfma16(va, pb, o[nt][mt] * alpha);
      }
    }
  };

  // Double-buffered walk: the loads of chunk i+1 are issued before chunk i is computed.  Loads
  // past the last chunk re-read it (cache hits) so that no branch sits between issue and use.
  for (int ci = 0; ci < nch; ci += 2) {
    load_chunk(bufB, min(ci + 1, nch - 1));
    compute(bufA, ci);
    load_chunk(bufA, min(ci + 2, nch - 1));
    if (ci + 1 < nch) compute(bufB, ci + 1);
  }

  if constexpr (NW == 1) {
    // One wave per split: finish straight from registers.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float lt = xrow_sum(l_run[nt]);
      if (prow[nt] < kb) continue;  // padding row, or a row that sees no key of this split
      const bool final_here = !a.split_mode || prow[nt] < split;
      if (final_here) {
        const float inv = 1.f / lt;
        uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + rh[nt] * D;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const floatx4 v = o[nt][mt] * inv;
          const uint32_t w0 = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
          const uint32_t w1 = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
          *reinterpret_cast<uint2*>(op + 16 * mt + 4 * g) = make_uint2(w0, w1);
        }
      } else {
        const size_t slot = rh[nt] * a.max_splits + sp;
        if (g == 0) {
          a.part_ml[2 * slot] = m_run[nt];
          a.part_ml[2 * slot + 1] = lt;
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          *reinterpret_cast<floatx4*>(a.part_o + slot * D + 16 * mt + 4 * g) = o[nt][mt];
      }
    }
    return;
  }

  // ---- merge the NW waves (rows are the same, keys differ) --------------------------------
  __shared__ float s_m[NW][NT][16], s_l[NW][NT][16];
  __shared__ floatx4 s_o[NW][MT][64];
  float lw[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    lw[nt] = xrow_sum(l_run[nt]);
    if (g == 0) {
      s_m[wave][nt][n] = m_run[nt];
      s_l[wave][nt][n] = lw[nt];
    }
  }
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][nt][n]);
    float Lsum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = s_m[w][nt][n];
      Lsum += mw == -INFINITY ? 0.f : s_l[w][nt][n] * fast_exp2((mw - M) * c);
    }
    const float myscale = m_run[nt] == -INFINITY ? 0.f : fast_exp2((m_run[nt] - M) * c);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) s_o[wave][mt][lane] = o[nt][mt] * myscale;
    __syncthreads();
    const bool row_ok = prow[nt] >= kb;  // a real row that sees a key of this split
    const bool final_here = !a.split_mode || prow[nt] < split;
    if (row_ok) {
      if (final_here) {
        const float inv = 1.f / Lsum;
        uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + rh[nt] * D;
        for (int mt = wave; mt < MT; mt += NW) {
          floatx4 v = s_o[0][mt][lane];
#pragma unroll
          for (int w = 1; w < NW; ++w) v += s_o[w][mt][lane];
          v *= inv;
          const uint32_t w0 = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
          const uint32_t w1 = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
          *reinterpret_cast<uint2*>(op + 16 * mt + 4 * g) = make_uint2(w0, w1);
        }
      } else {
        const size_t slot = rh[nt] * a.max_splits + sp;
        if (wave == 0 && g == 0) {
          a.part_ml[2 * slot] = M;
          a.part_ml[2 * slot + 1] = Lsum;
        }
        for (int mt = wave; mt < MT; mt += NW) {
          floatx4 v = s_o[0][mt][lane];
#pragma unroll
          for (int w = 1; w < NW; ++w) v += s_o[w][mt][lane];
          *reinterpret_cast<floatx4*>(a.part_o + slot * D + 16 * mt + 4 * g) = v;
        }
      }
    }
    __syncthreads();
  }
}

hipError_t launch_attn_split_mfma(const AttnArgs& a, int head_dim, int rows_per_tile,
                                  int grid_x, hipStream_t st) {
  dim3 grid(grid_x, a.num_kv_heads, a.num_seqs);
  // One wave per split (splits of at most 2048 keys); longer fixed splits and calls without
  // splits use 4 waves per workgroup.
  const bool one_wave = a.split_mode && a.split_tokens <= 2048;
  const bool reload = !a.split_mode || a.split_tokens > 8192;
#define KVP_SPLIT_LAUNCH(D, NT)                                                         \
  (one_wave ? attn_split_mfma_kernel<D, NT, false, 1><<<grid, 64, 0, st>>>(a)           \
   : reload ? attn_split_mfma_kernel<D, NT, true, 4><<<grid, 256, 0, st>>>(a)           \
            : attn_split_mfma_kernel<D, NT, false, 4><<<grid, 256, 0, st>>>(a))
  if (head_dim == 128) {
    if (rows_per_tile <= 16) KVP_SPLIT_LAUNCH(128, 1);
    else KVP_SPLIT_LAUNCH(128, 2);
  } else {
    if (rows_per_tile <= 16) KVP_SPLIT_LAUNCH(64, 1);
    else KVP_SPLIT_LAUNCH(64, 2);
  }
#undef KVP_SPLIT_LAUNCH
  return hipGetLastError();
}

}  // namespace kvp
