// Split-K paged attention on the vector ALUs (fp32 and bf16 K/V).
//
// The fp32 path of every call, and an alternative bf16 decode path.  Same work split as the
// matrix-core kernel: one workgroup per (row tile, split, KV head, sequence), partials merged
// by the reduce kernel in fixed split order (no float atomics: sparkinfer server README,
// "Determinism").  Sequences with more than split_q_max query tokens make one pass (split 0
// only) in the same launch.  A workgroup is one wave, except for single-row tiles (one q-head
// per KV head, decode), where 4 waves take contiguous quarters of the split's tiles and merge
// through LDS in wave order, so that a lone short decode is not one wave's walk.
//
// Per 16-token tile a wave reads K and V with contiguous 1 KiB wave loads (16 bytes per lane),
// the tiles' block ids 64 at a time; single-row waves stream the tiles through a ring of
// register buffers (the loads of later tiles in flight while one is computed).  With the pool's
// tile layout, lane l of K load j holds dim chunk 4*j + l/16 of token l%16, so each lane forms
// partial dot products over its chunks and two cross-row swaps (v_permlane32_swap /
// v_permlane16_swap) finish them: every lane then holds the full score of token l%16.  The tile
// max uses DPP within rows of 16 lanes.  For V (stored dims-major), lane l of load j holds X
// consecutive tokens of one dim, so the probabilities are exchanged through LDS once per tile
// and each lane accumulates its dims; the few lanes that share a dim are summed with DPP at the
// end of the split.  bf16 products use v_dot2_f32_bf16 on packed pairs, with P rounded to bf16
// (the same rounded P feeds numerator and denominator).
#include "common.h"
#include "kernels.h"

namespace kvp {

namespace {

template <typename E>
struct VecTraits;

template <>
struct VecTraits<float> {
  static constexpr int X = 4;
};
template <>
struct VecTraits<uint16_t> {
  static constexpr int X = 8;
};

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

}  // namespace

// Waves per workgroup: single-row waves (one query row per (sequence, KV head): no grouped
// heads) split their split's tiles over 4 waves, merged through LDS in wave order, so that a
// lone short decode is not one wave's walk; other instances run one wave per workgroup.
template <int ROWS>
constexpr int vec_waves() { return ROWS == 1 ? 4 : 1; }

template <typename E, int D, int ROWS>
__global__ __launch_bounds__(64 * vec_waves<ROWS>()) void attn_vec_kernel(AttnArgs a) {
  constexpr bool BF = sizeof(E) == 2;
  constexpr int X = VecTraits<E>::X;       // elements per 16 bytes
  constexpr int NL = TILE * D * (int)sizeof(E) / 1024;  // 16-byte loads per lane per tile
  constexpr int LPD = (int)sizeof(E);      // lanes sharing one V^T row (one dim)
  constexpr int QW = BF ? X / 2 : X;       // q words per lane per load slot
  constexpr int NWV = vec_waves<ROWS>();
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int s = blockIdx.z, kvh = blockIdx.y;
  const int rt = blockIdx.x % a.row_tiles, sp = blockIdx.x / a.row_tiles;
  int L, T;
  seq_lens(a, s, L, T);
  const int G = a.group;
  const int rows = T * G;
  const int r0 = rt * ROWS;
  if (r0 >= rows) return;
  const int p_last = L - T + (min(r0 + ROWS, rows) - 1) / G;
  // Split-K sequences (q_len <= split_q_max) cut their keys into splits; longer query blocks
  // make one pass over all their keys, in split slot 0.
  const bool split_k = T <= a.split_q_max;
  if (!split_k && sp > 0) return;
  const int split = split_k ? seq_split(a, L, T, false) : L;
  const int kb = split_k ? sp * split : 0;
  const int ke = min(min(L, p_last + 1), kb + split);
  if (kb >= ke) return;
  int q_start, p_start;
  seq_starts(a, s, q_start, p_start);
  const int Hq = a.num_q_heads;

  // q[r][j][w]: the dims of chunk 4*j + g (fp32 values, or packed bf16 pairs).
  uint32_t q[ROWS][NL][QW];
  int prow[ROWS];
  size_t rh[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const int rr = r0 + r;
    const int i = rr / G;
    const int grow = q_start + i;
    const bool valid = rr < rows && grow < a.total_q;
    prow[r] = valid ? L - T + i : -1;
    rh[r] = valid ? (size_t)grow * Hq + kvh * G + rr % G : 0;
    const E* qp = reinterpret_cast<const E*>(a.q) + rh[r] * D;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      u32x4 w = valid ? *reinterpret_cast<const u32x4*>(qp + (4 * j + g) * X) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < QW; ++e) q[r][j][e] = w[e];
    }
  }

  float m_run[ROWS], l_run[ROWS], o[ROWS][NL];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
#pragma unroll
    for (int j = 0; j < NL; ++j) o[r][j] = 0.f;
  }

  __shared__ float sp_lds[NWV][ROWS][TILE];
  const int32_t* tbl = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  const E* kl = reinterpret_cast<const E*>(a.k_layer);
  const E* vl = reinterpret_cast<const E*>(a.v_layer);
  const float c = a.scale_log2;
  const int tok0 = X * (lane % LPD);  // first token of this lane's V run

  // The split's tiles go through a ring of RN register buffers: the loads of tile i + RN - 1 are
  // issued before tile i is computed, so RN - 1 tiles are in flight behind the one computed.
  // Block ids come 64 tiles at a time (lane l: tile tb + l), read with readlane; tiles past the
  // split's last re-read it (never computed).
  // Single-row waves (no grouped heads) only: with more rows the registers q and o hold leave
  // room for no ring without cutting the waves a SIMD runs at once, which large batches need
  // more (bf16 decode of 4 rows per wave measured 130 -> 141 us with two buffers).  RN = 1: no
  // lookahead (the block ids still come ahead, so a tile waits for one memory latency).
  constexpr int RN = ROWS == 1 ? (NL <= 4 ? 4 : 2) : 1;
  // this wave's tiles of the split: [wt0, wt0 + ntl) (a contiguous share; possibly none)
  const int ntl_all = (ke - kb + TILE - 1) / TILE;
  const int wq = (ntl_all + NWV - 1) / NWV;
  const int wt0 = min(wave * wq, ntl_all);
  const int ntl = min(ntl_all - wt0, wq);  // tiles of this wave, counted from wt0
  const int bshift = a.block_shift;
  const int last_bi = (ke - 1) >> bshift;
  int tb = 0;
  auto load_ids = [&](int base) -> int {
    return tbl[min((kb + TILE * (wt0 + base + lane)) >> bshift, last_bi)];
  };
  int ids = load_ids(0);
  struct VTile {
    u32x4 k[NL], v[NL];
  };
  auto load_tile = [&](VTile& b, int ti) {
    ti = min(ti, ntl - 1);
    if (ti - tb >= WAVE) {  // wave-uniform: the next 64 tiles' block ids
      tb = ti & ~(WAVE - 1);
      ids = load_ids(tb);
    }
    const int blk = __builtin_amdgcn_readlane(ids, ti - tb);
    const int t0 = kb + TILE * (wt0 + ti);
    const size_t toff = block_tile_offset(blk, (t0 & (a.block_size - 1)) / TILE, kvh, bshift,
                                          a.num_blocks, a.num_kv_heads, D);
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      b.k[j] = *reinterpret_cast<const u32x4*>(kl + toff + (size_t)(1024 * j + 16 * lane) / sizeof(E));
      b.v[j] = *reinterpret_cast<const u32x4*>(vl + toff + (size_t)(1024 * j + 16 * lane) / sizeof(E));
    }
  };

  auto compute = [&](VTile& b, int ti) {
    const int t0 = kb + TILE * (wt0 + ti);
    u32x4 (&kw)[NL] = b.k;
    u32x4 (&vw)[NL] = b.v;
    const bool tail = t0 + TILE > ke;
    if (tail) {
      // V slots at or past ke may hold NaN: zero them (their p is 0).
#pragma unroll
      for (int j = 0; j < NL; ++j)
#pragma unroll
        for (int e = 0; e < X; ++e)
          if (t0 + tok0 + e >= ke) {
            if constexpr (BF) {
              const uint32_t wd = vw[j][e >> 1];
              vw[j][e >> 1] = (e & 1) ? (wd & 0x0000ffffu) : (wd & 0xffff0000u);
            } else {
              vw[j][e] = 0u;
            }
          }
    }
    const int key = t0 + n;
    float p[ROWS], alpha[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        if constexpr (BF) {
#pragma unroll
          for (int w = 0; w < QW; ++w) acc = dot2(kw[j][w], q[r][j][w], acc);
        } else {
#pragma unroll
          for (int e = 0; e < X; ++e)
            acc = fmaf(__uint_as_float(kw[j][e]), __uint_as_float(q[r][j][e]), acc);
        }
      }
      float sc = xrow_sum(acc);
      sc = (key < ke && key <= prow[r]) ? sc : -INFINITY;
      const float m_new = fmaxf(m_run[r], row_max(sc));
      const bool none = (m_new == -INFINITY);
      alpha[r] = none ? 1.f : fast_exp2((m_run[r] - m_new) * c);
      float pr = fast_exp2(sc * c - (none ? 0.f : m_new * c));
      if constexpr (BF) pr = round_to_bf16(pr);
      p[r] = pr;
      l_run[r] = l_run[r] * alpha[r] + pr;
      m_run[r] = m_new;
    }
    // P goes to the lanes that hold each V run through the wave's own LDS slice.  A wave's LDS
    // operations are performed in order, so no barrier is needed between the last tile's reads,
    // these writes and the reads below (a barrier would also wait for the ring's loads).
    if (g == 0) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) sp_lds[wave][r][n] = p[r];
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      float pv[X];
#pragma unroll
      for (int e = 0; e < X; ++e) pv[e] = sp_lds[wave][r][tok0 + e];
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        float acc = o[r][j] * alpha[r];
        if constexpr (BF) {
#pragma unroll
          for (int w = 0; w < X / 2; ++w)
            acc = dot2(vw[j][w], pack_exact_bf16(pv[2 * w], pv[2 * w + 1]), acc);
        } else {
#pragma unroll
          for (int e = 0; e < X; ++e) acc = fmaf(pv[e], __uint_as_float(vw[j][e]), acc);
        }
        o[r][j] = acc;
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  VTile rb[RN];
  if (ntl > 0) {  // wave-uniform
#pragma unroll
    for (int j = 0; j + 1 < RN; ++j) load_tile(rb[j], j);
  }
  for (int ti = 0; ti < ntl; ti += RN) {
    bool done = false;
#pragma unroll
    for (int j = 0; j < RN; ++j) {
      load_tile(rb[(j + RN - 1) % RN], ti + j + RN - 1);
      compute(rb[j], ti + j);
      if (ti + j + 1 >= ntl) {
        done = true;
        break;
      }
    }
    if (done) break;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the ring's re-reads past the end

  // Each lane's l_run counts its own token (identical across the 4 row groups).
  float lts[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    lts[r] = row_sum(l_run[r]);
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      float v = o[r][j];
      v += dpp<DPP_XOR1>(v);
      if constexpr (LPD == 4) v += dpp<DPP_XOR2>(v);
      o[r][j] = v;
    }
  }
  if constexpr (NWV > 1) {
    // The waves' (max, sum, O) merged in wave order by wave 0 (a wave without keys has max
    // -inf and weighs 0), which then stores as a single wave would.
    static_assert(ROWS == 1, "multi-wave workgroups hold one row");
    __shared__ float s_m[NWV], s_l[NWV];
    __shared__ float s_o[NWV][NL][WAVE];
    if (lane == 0) {
      s_m[wave] = m_run[0];
      s_l[wave] = lts[0];
    }
#pragma unroll
    for (int j = 0; j < NL; ++j) s_o[wave][j][lane] = o[0][j];
    __syncthreads();
    if (wave != 0) return;
    float M = s_m[0];
#pragma unroll
    for (int w = 1; w < NWV; ++w) M = fmaxf(M, s_m[w]);
    float lsum = 0.f, ov[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) ov[j] = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const float mw = s_m[w];
      const float wt = mw == -INFINITY ? 0.f : fast_exp2((mw - M) * c);
      lsum = __builtin_fmaf(wt, s_l[w], lsum);
#pragma unroll
      for (int j = 0; j < NL; ++j) ov[j] = __builtin_fmaf(wt, s_o[w][j][lane], ov[j]);
    }
    m_run[0] = M;
    lts[0] = lsum;
#pragma unroll
    for (int j = 0; j < NL; ++j) o[0][j] = ov[j];
  }
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    const float lt = lts[r];
    if (prow[r] < kb) continue;
    // Rows whose keys all lie in split 0 are finished here (the reduce skips them).
    if (prow[r] >= split) {
      const size_t prh = rh[r] + (size_t)(((long long)p_start - q_start) * Hq);  // partial row
      if (prh >= (size_t)a.part_rows * Hq) continue;
      const size_t slot = prh * a.max_splits + sp;
      if (lane == 0) {
        a.part_ml[2 * slot] = m_run[r];
        a.part_ml[2 * slot + 1] = lt;
      }
      if (lane % LPD == 0) {
#pragma unroll
        for (int j = 0; j < NL; ++j) a.part_o[slot * D + (64 * j + lane) / LPD] = o[r][j];
      }
    } else if (lane % LPD == 0) {
      const float inv = 1.f / lt;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int d = (64 * j + lane) / LPD;
        if constexpr (BF)
          reinterpret_cast<uint16_t*>(a.out)[rh[r] * D + d] =
              (uint16_t)f32_to_bf16_bits(o[r][j] * inv);
        else
          reinterpret_cast<float*>(a.out)[rh[r] * D + d] = o[r][j] * inv;
      }
    }
  }
}

template <typename E, int D>
static void launch_rows(const AttnArgs& a, int rows, dim3 grid, hipStream_t st) {
  if (rows <= 1) attn_vec_kernel<E, D, 1><<<grid, 64 * vec_waves<1>(), 0, st>>>(a);
  else if (rows <= 2) attn_vec_kernel<E, D, 2><<<grid, 64, 0, st>>>(a);
  else if (rows <= 4) attn_vec_kernel<E, D, 4><<<grid, 64, 0, st>>>(a);
  else if (rows <= 5) attn_vec_kernel<E, D, 5><<<grid, 64, 0, st>>>(a);
  else attn_vec_kernel<E, D, 8><<<grid, 64, 0, st>>>(a);
}

hipError_t launch_attn_vec(const AttnArgs& a, int elt_bytes, int head_dim, int rows_per_tile,
                           int grid_x, hipStream_t st) {
  dim3 grid(grid_x, a.num_kv_heads, a.num_seqs);
  if (elt_bytes == 4) {
    if (head_dim == 128) launch_rows<float, 128>(a, rows_per_tile, grid, st);
    else launch_rows<float, 64>(a, rows_per_tile, grid, st);
  } else {
    if (head_dim == 128) launch_rows<uint16_t, 128>(a, rows_per_tile, grid, st);
    else launch_rows<uint16_t, 64>(a, rows_per_tile, grid, st);
  }
  return hipGetLastError();
}

}  // namespace kvp
