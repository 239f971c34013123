// Prefill attention over a paged pool on the gfx950 matrix cores, bf16 K/V: the uncached
// suffix of each sequence (many query rows) against its cached prefix plus itself, causal
// (sparkinfer server README, "Automatic prefix cache": only the suffix is prefilled, over the
// shared prefix blocks; "Request isolation & continuous batching": prefill in chunks).
//
// Workgroup = 4 waves over one row tile of one (sequence, KV head); a wave owns 16*NTW rows
// (row = token * G + head-in-group, so every row of a workgroup reads the same K/V).  K/V are
// walked in tiles of 64 keys = 4 pool tiles, each streamed verbatim from the pool into LDS with
// global_load_lds (no register staging; the pool's tile layout is already the order the matrix
// cores read: K as 16-byte dim chunks of 16 tokens, V dims-major) through 3 LDS stages: tiles
// j+1 and j+2 are in flight while tile j is computed; one vmcnt wait and one barrier per tile.
// Per wave and tile:
//   S^T[key][row] = K . Q^T   4 key tiles x NTW row tiles x D/32 v_mfma_f32_16x16x32_bf16,
//                             each K operand (one conflict-free ds_read_b128) feeding NTW MFMAs
//   causal mask only on tiles that reach past the wave's first row; online softmax in fp32
//   O^T[dim][row] += V^T . P^T   2 key halves x D/16 dim tiles x NTW; P never leaves registers
//                             (a lane of the score tile already holds the 8 keys the PV k-slice
//                             needs: keys 4g..4g+3 of two pool tiles)
// The logical workgroup order is remapped so that the row tiles of one (sequence, KV head) run
// on the same XCD (workgroups are dealt to the 8 XCDs round-robin) and share its L2.
#include "common.h"
#include "kernels.h"

namespace kvp {

namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

constexpr int NXCD = 8;

// 16 bytes per lane from gbase + voff into LDS at lds_addr + 16*lane (global_load_lds_dwordx4,
// scalar base + per-lane offset).  Issued as inline asm so that the compiler's wait insertion
// never ties these loads to LDS reads of other stages or to reused address registers: the
// kernel waits for them itself (vmcnt) before the barrier that publishes a stage.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(gbase), "s"(lds_addr)
               : "memory", "m0");
}

template <typename P>
__device__ __forceinline__ uint32_t lds_address(P* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)(p));
}

// Workgroup id -> logical index such that the ids an XCD receives (id % 8 == x) map to one
// contiguous logical range.  A bijection on [0, n).
__device__ __forceinline__ int xcd_logical(int id, int n) {
  const int x = id % NXCD, k = id / NXCD;
  const int q = n / NXCD, r = n % NXCD;
  return x < r ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

}  // namespace

template <int D, int NTW>
__global__ __launch_bounds__(256) void attn_prefill_mfma_kernel(AttnArgs a) {
  constexpr int KK = D / 32;           // 32-dim steps of the score product
  constexpr int MT = D / 16;           // 16-dim tiles of the output
  constexpr int ROWS_W = 16 * NTW;     // rows per wave
  constexpr int ROWS_WG = 4 * ROWS_W;  // rows per workgroup
  constexpr int TE = 16 * D;           // elements of one pool tile (K or V)
  constexpr int TQ = TE * 2 / 1024;    // 1 KiB wave loads per pool tile
  constexpr int NST = 3;               // LDS stages: tile j computed while j+1, j+2 arrive
  constexpr int IDS = 1024;            // block ids of pool tiles held in LDS
  // One array per LDS stage ([K0..K3, V0..V3] each): with every access naming its array, the
  // compiler can tell the stage being computed from the ones the DMA is filling, and does not
  // wait for those loads before reading.
  __shared__ __attribute__((aligned(16))) uint16_t lds0[8][TE];
  __shared__ __attribute__((aligned(16))) uint16_t lds1[8][TE];
  __shared__ __attribute__((aligned(16))) uint16_t lds2[8][TE];
  __shared__ int s_ids[IDS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int logical = xcd_logical(blockIdx.x, gridDim.x);
  const int rt = logical % a.row_tiles;
  const int pair = logical / a.row_tiles;
  const int s = pair / a.num_kv_heads, kvh = pair % a.num_kv_heads;
  int L, T;
  seq_lens(a, s, L, T);
  const int G = a.group;
  const int rows = T * G;
  const int r0 = rt * ROWS_WG;
  if (r0 >= rows) return;
  const int ke = min(L, L - T + (min(r0 + ROWS_WG, rows) - 1) / G + 1);  // keys the WG needs
  const int ntiles = (ke + 63) >> 6;
  const int npt = (ke + 15) >> 4;  // pool tiles the WG reads
  const int rw0 = r0 + wave * ROWS_W;
  const int kew = rw0 < rows ? min(L, L - T + (min(rw0 + ROWS_W, rows) - 1) / G + 1) : 0;
  const int pw0 = L - T + rw0 / G;  // keys <= pw0 are visible to every row of this wave

  const int32_t* tbl = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  const char* kbase = reinterpret_cast<const char*>(a.k_layer);
  const char* vbase = reinterpret_cast<const char*>(a.v_layer);
  const int bmask = a.block_size - 1;

  // Block ids of pool tiles [ids0, ids0 + IDS) of this sequence, in LDS.
  int ids0 = 0;
  auto load_ids = [&](int base) {
    for (int i = tid; i < IDS; i += 256) {
      const int pt = min(base + i, npt - 1);
      s_ids[i] = tbl[(pt << 4) >> a.block_shift];
    }
  };
  load_ids(0);
  __syncthreads();

  // ---- K/V staging: wave w streams pool tiles 2w and 2w+1 of [K0..K3, V0..V3] of a 64-key
  // tile straight into LDS (global_load_lds: lane l's 16 bytes land at base + 16*l).  Pool tiles
  // past the context re-read the last one; those keys are masked and their V zeroed.
  const uint32_t lane_off = 16u * lane;
  auto fetch = [&](int j, uint16_t (&stage)[8][TE]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int slot = 2 * wave + u;        // 0..3: K tiles, 4..7: V tiles
      const int pt = min(4 * j + (slot & 3), npt - 1);
      const int blk = s_ids[pt - ids0];
      const size_t off = block_tile_offset(blk, ((pt << 4) & bmask) >> 4, kvh, a.block_shift,
                                           a.num_blocks, a.num_kv_heads, D) * 2;
      // wave-uniform base (scalar registers) + a fixed per-lane offset
      const char* base = (slot < 4 ? kbase : vbase) + off;
      const uint32_t dst = lds_address(stage[slot]);
#pragma unroll
      for (int q = 0; q < TQ; ++q) dma16(base + 1024 * q, lane_off, dst + 1024 * q);
    }
  };
  fetch(0, lds0);
  if (ntiles > 1) fetch(1, lds1);

  // ---- Q^T operands and per-row state ----------------------------------------------------
  const int q_start = wave_prefix_total(a.q_lens, s);
  const int Hq = a.num_q_heads;
  bf16x8 qb[NTW][KK];
  int prow[NTW];
  size_t rh[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int r = rw0 + 16 * nt + n;
    const int i = r / G;
    const int grow = q_start + i;
    const bool valid = r < rows && grow < a.total_q;
    prow[nt] = valid ? L - T + i : -1;
    rh[nt] = valid ? (size_t)grow * Hq + kvh * G + r % G : 0;
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + rh[nt] * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      qb[nt][kk] = __builtin_bit_cast(
          bf16x8, valid ? *reinterpret_cast<const u32x4*>(qp + 32 * kk + 8 * g) : z);
    }
  }
  // m_run: running row max (raw score units); o: O^T accumulators; osum: the same product
  // with a ones tile in place of V^T, i.e. the row sum of the very bf16 P values that feed o
  // (rescaled together with o).
  float m_run[NTW];
  floatx4 o[NTW][MT], osum[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    m_run[nt] = -INFINITY;
    osum[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  const float c = a.scale_log2;

  // Tile 0 must have landed (the prologue's own waits may already have drained more).
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  // Attention of this wave's rows against one 64-key tile held in LDS (K tiles at kt, V^T tiles
  // at vt, 4 pool tiles each), in two halves of 32 keys (pool tiles 2h and 2h+1).  `edge`: the
  // tile reaches past the wave's first row (causal diagonal) or past the context.
  auto tile = [&](const uint16_t* kt, const uint16_t* vt, int k0, bool edge) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kh = k0 + 32 * h;
      // ---- S^T = K Q^T over keys kh .. kh+31 -------------------------------------------------
      floatx4 sc[2][NTW];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) sc[t][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 ka = __builtin_bit_cast(
              bf16x8,
              *reinterpret_cast<const u32x4*>(kt + (2 * h + t) * TE + ((4 * kk + g) * 16 + n) * 8));
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) sc[t][nt] = mfma16(ka, qb[nt][kk], sc[t][nt]);
        }
      }
      // lane (n, g) holds row n's scores for keys kh + 16*t + 4*g + i
      uint32_t vkeep[2][2] = {{~0u, ~0u}, {~0u, ~0u}};  // V words to keep (slots < L)
      if (edge) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kh + 16 * t + 4 * g + i;
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
              if (key > prow[nt] || key >= L) sc[t][nt][i] = -INFINITY;
            if (key >= L) vkeep[t][i >> 1] &= (i & 1) ? 0x0000ffffu : 0xffff0000u;
          }
        }
      }
      // ---- online softmax (lazy: the running max moves only when a row's max grows by more
      // than 2^8 in exp2 units, so P stays <= 256 and the rescale is rare) ------------------
      bf16x8 pb[NTW];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        float cmax = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) cmax = fmaxf(cmax, sc[t][nt][i]);
        cmax = xrow_max(cmax);
        const bool grow = (cmax - m_run[nt]) * c > 8.f;  // false for NaN (both -inf)
        const float m_new = grow ? cmax : m_run[nt];
        if (__builtin_amdgcn_ballot_w64(grow)) {
          const float alpha = grow ? fast_exp2((m_run[nt] - m_new) * c) : 1.f;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) o[nt][mt] *= alpha;
          osum[nt] *= alpha;
        }
        m_run[nt] = m_new;
        const float msub = m_new == -INFINITY ? 0.f : m_new * c;
        uint32_t pk[4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; i += 2)
            pk[2 * t + (i >> 1)] = cvt_pk_bf16(fast_exp2(sc[t][nt][i] * c - msub),
                                               fast_exp2(sc[t][nt][i + 1] * c - msub));
        pb[nt] = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
      }
      // ---- O^T += V^T P^T (and the ones tile for the row sums) ------------------------------
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x2 v0 = *reinterpret_cast<const u32x2*>(vt + (2 * h) * TE + (16 * mt + n) * 16 + 4 * g);
        const u32x2 v1 = *reinterpret_cast<const u32x2*>(vt + (2 * h + 1) * TE + (16 * mt + n) * 16 + 4 * g);
        const bf16x8 va = __builtin_bit_cast(
            bf16x8, u32x4{v0[0] & vkeep[0][0], v0[1] & vkeep[0][1], v1[0] & vkeep[1][0],
                          v1[1] & vkeep[1][1]});
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) o[nt][mt] = mfma16(va, pb[nt], o[nt][mt]);
      }
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) osum[nt] = mfma16(ones, pb[nt], osum[nt]);
    }
  };

  // One 64-key tile: compute tile j from `cur` while tile j+2 streams into `nxt2`.
  auto step = [&](int j, uint16_t (&cur)[8][TE], uint16_t (&nxt2)[8][TE]) {
    // refill the id cache every IDS pool tiles (rare: only past 16K keys)
    if (4 * (j + 2) + 3 - ids0 >= IDS && 4 * (j + 2) < npt) {
      __builtin_amdgcn_s_waitcnt(0x0F70);
      __syncthreads();
      ids0 = 4 * (j + 2);
      load_ids(ids0);
      __syncthreads();
    }
    fetch(min(j + 2, ntiles - 1), nxt2);
    const int k0 = 64 * j;
    if (k0 < kew) {
      // Tiles that reach past the wave's first row (causal diagonal) or past the context take
      // the masked path; all others run branch-free.
      tile(cur[0], cur[4], k0, k0 + 63 > pw0 || k0 + 64 > L);
    }
    // tile j+1 (issued one iteration ago) has landed once at most the 2*TQ loads of tile j+2
    // are outstanding; every wave's share of it is visible after the barrier
    __builtin_amdgcn_s_waitcnt(TQ == 4 ? 0x0F78 : 0x0F74);
    barrier_no_fence();
  };
  for (int j = 0; j < ntiles; j += NST) {
    step(j, lds0, lds2);
    if (j + 1 < ntiles) step(j + 1, lds1, lds0);
    if (j + 2 < ntiles) step(j + 2, lds2, lds1);
  }

  // ---- normalise and store ---------------------------------------------------------------
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    if (prow[nt] < 0) continue;
    const float inv = 1.f / osum[nt][0];
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + rh[nt] * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const floatx4 v = o[nt][mt] * inv;
      const uint32_t w0 = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
      const uint32_t w1 = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
      *reinterpret_cast<uint2*>(op + 16 * mt + 4 * g) = make_uint2(w0, w1);
    }
  }
}

int prefill_rows_per_wave_choice(int rows_per_pair, int pairs, int num_cus) {
  // Makespan model: one workgroup per CU at a time (the kernel runs at occupancy 1); pick the
  // rows per wave (16*NTW) that minimises rounds x rows per workgroup, preferring larger tiles
  // (more K/V reuse) on ties.
  int best = 5;
  double best_cost = 1e300;
  for (int ntw = 5; ntw >= 2; --ntw) {
    const int rows_wg = 64 * ntw;
    const long long wgs = (long long)pairs * ((rows_per_pair + rows_wg - 1) / rows_wg);
    const long long rounds = (wgs + num_cus - 1) / num_cus;
    const double cost = (double)rounds * rows_wg;
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = ntw;
    }
  }
  return best;
}

hipError_t launch_attn_prefill_mfma(const AttnArgs& a, int head_dim, int ntw, hipStream_t st) {
  dim3 grid(a.row_tiles * a.num_kv_heads * a.num_seqs);
#define KVP_PREFILL(D, NTW) attn_prefill_mfma_kernel<D, NTW><<<grid, 256, 0, st>>>(a)
  if (head_dim == 128) {
    switch (ntw) {
      case 2: KVP_PREFILL(128, 2); break;
      case 3: KVP_PREFILL(128, 3); break;
      case 4: KVP_PREFILL(128, 4); break;
      default: KVP_PREFILL(128, 5); break;
    }
  } else {
    switch (ntw) {
      case 2: KVP_PREFILL(64, 2); break;
      case 3: KVP_PREFILL(64, 3); break;
      case 4: KVP_PREFILL(64, 4); break;
      default: KVP_PREFILL(64, 5); break;
    }
  }
#undef KVP_PREFILL
  return hipGetLastError();
}

}  // namespace kvp
