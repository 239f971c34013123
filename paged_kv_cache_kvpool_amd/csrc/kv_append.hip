// KV append (scatter of new tokens' K/V rows into their pool blocks) and block copy.
//
// Append writes the K/V of the tokens being processed into the sequence's own blocks, so a
// prefix hit only adds the uncached suffix to the pool (sparkinfer server README, "Automatic
// prefix cache").  Block copy duplicates whole blocks for copy-on-write of a shared prefix
// block (same section: blocks are shared, not copied).  Both are bit copies.
#include "common.h"
#include "kernels.h"

namespace kvp {

// One workgroup per (16-token tile touched by the new tokens, KV head, sequence).  K chunks
// are copied 16 bytes at a time; V is transposed through LDS so that full 16-byte runs of the
// dims-major tile are written whole and partial runs element by element (slots of the tile
// that are not being appended keep their bits).
template <typename E>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  constexpr int X = 16 / sizeof(E);
  const int s = blockIdx.z, h = blockIdx.y;
  const int D = a.head_dim;
  const int cap = a.max_blocks_per_seq * a.block_size;
  const int L = min(max(a.ctx_lens[s], 0), cap);
  const int T = min(max(a.q_lens[s], 0), L);
  if (T == 0) return;
  const int p0 = L - T;
  const int tile_start = (p0 / TILE + (int)blockIdx.x) * TILE;
  if (tile_start >= L) return;
  const int lo = max(p0, tile_start), hi = min(L, tile_start + TILE);
  const int q_start = wave_prefix_total(a.q_lens, s);

  const int32_t* row_tbl = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  const size_t toff = tile_offset(row_tbl, tile_start, h, a.block_size, a.num_blocks,
                                  a.num_kv_heads, D);
  E* kt = reinterpret_cast<E*>(a.k_layer) + toff;
  E* vt = reinterpret_cast<E*>(a.v_layer) + toff;
  const E* kn = reinterpret_cast<const E*>(a.k_new);
  const E* vn = reinterpret_cast<const E*>(a.v_new);
  const int nchunk = D / X;

  __shared__ E sv[TILE * 128];  // V rows of this tile's new tokens, [t][d]
  for (int u = threadIdx.x; u < TILE * nchunk; u += blockDim.x) {
    const int c = u / TILE, t = u % TILE;
    const int p = tile_start + t;
    if (p < lo || p >= hi) continue;
    const int row = q_start + (p - p0);
    if (row >= a.total_q) continue;
    const size_t src = ((size_t)row * a.num_kv_heads + h) * D + c * X;
    *reinterpret_cast<u32x4*>(kt + (c * TILE + t) * X) =
        *reinterpret_cast<const u32x4*>(kn + src);
    *reinterpret_cast<u32x4*>(sv + t * D + c * X) = *reinterpret_cast<const u32x4*>(vn + src);
  }
  __syncthreads();
  // V^T tile row d holds the 16 tokens of dim d; a 16-byte run covers X consecutive tokens.
  constexpr int RUNS = TILE / X;
  for (int u = threadIdx.x; u < D * RUNS; u += blockDim.x) {
    const int d = u / RUNS, r = u % RUNS;
    const int t0 = r * X;
    bool whole = true;
    for (int e = 0; e < X; ++e) {
      const int p = tile_start + t0 + e;
      const int row = q_start + (p - p0);
      whole = whole && p >= lo && p < hi && row < a.total_q;
    }
    if (whole) {
      E run[X];
      for (int e = 0; e < X; ++e) run[e] = sv[(t0 + e) * D + d];
      *reinterpret_cast<u32x4*>(vt + d * TILE + t0) = *reinterpret_cast<const u32x4*>(run);
    } else {
      for (int e = 0; e < X; ++e) {
        const int p = tile_start + t0 + e;
        const int row = q_start + (p - p0);
        if (p >= lo && p < hi && row < a.total_q) vt[d * TILE + t0 + e] = sv[(t0 + e) * D + d];
      }
    }
  }
}

// int8 pools: each new (token, KV head) row is quantised and stored by store_row_i8 (common.h),
// one wave per row of the workgroup's 16-token tile.
template <int E>
__global__ __launch_bounds__(256) void append_i8_kernel(AppendArgs a) {
  constexpr int D = 64 * E;
  const int s = blockIdx.z, h = blockIdx.y;
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x >> 6;
  const int cap = a.max_blocks_per_seq * a.block_size;
  const int L = min(max(a.ctx_lens[s], 0), cap);
  const int T = min(max(a.q_lens[s], 0), L);
  if (T == 0) return;
  const int p0 = L - T;
  const int tile_start = (p0 / TILE + (int)blockIdx.x) * TILE;
  if (tile_start >= L) return;
  const int lo = max(p0, tile_start), hi = min(L, tile_start + TILE);
  const int q_start = wave_prefix_total(a.q_lens, s);
  const int32_t* row_tbl = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  const size_t toff = tile_offset(row_tbl, tile_start, h, a.block_size, a.num_blocks,
                                  a.num_kv_heads, D);  // bytes: one byte per element
  int8_t* kt = reinterpret_cast<int8_t*>(a.k_layer) + toff;
  int8_t* vt = reinterpret_cast<int8_t*>(a.v_layer) + toff;
  float* ks = a.k_scale_layer + toff / D;  // the tile's 16 token scales
  float* vs = a.v_scale_layer + toff / D;
  const uint16_t* kn = reinterpret_cast<const uint16_t*>(a.k_new);
  const uint16_t* vn = reinterpret_cast<const uint16_t*>(a.v_new);
  // This wave's rows (positions lo + wave, + 4, ...: at most 4 of the tile's 16): every row's
  // values are loaded before any is quantised, so the wave waits for memory once.
  float kx[4][E], vx[4][E];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = lo + wave + 4 * i;
    const int row = q_start + (p - p0);
    if (p < hi && row < a.total_q) {  // wave-uniform
      const size_t src = ((size_t)row * a.num_kv_heads + h) * D;
      load_row<E>(kn + src, kx[i]);
      load_row<E>(vn + src, vx[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = lo + wave + 4 * i;
    const int row = q_start + (p - p0);
    if (p < hi && row < a.total_q) store_row_i8<E>(kt, vt, ks, vs, kx[i], vx[i], p - tile_start);
  }
}

// grid (n, num_layers, 2 or 4): blockIdx.z picks K or V codes, then (int8 pools) K or V
// scales; 16-byte copies of one block of one layer.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyArgs a) {
  const int i = blockIdx.x, layer = blockIdx.y, z = blockIdx.z;
  const int src = a.src[i], dst = a.dst[i];
  if ((unsigned)src >= (unsigned)a.num_blocks || (unsigned)dst >= (unsigned)a.num_blocks) return;
  const size_t bb = z < 2 ? a.block_bytes : a.block_scale_bytes;
  char* base = reinterpret_cast<char*>(z == 0 ? a.k : z == 1 ? a.v : z == 2 ? a.k_scale : a.v_scale);
  const size_t layer_off = (size_t)layer * a.num_blocks * bb;
  const u32x4* from = reinterpret_cast<const u32x4*>(base + layer_off + (size_t)src * bb);
  u32x4* to = reinterpret_cast<u32x4*>(base + layer_off + (size_t)dst * bb);
  const int n16 = (int)(bb / 16);
  for (int u = threadIdx.x; u < n16; u += blockDim.x) to[u] = from[u];
}

hipError_t launch_append(const AppendArgs& a, int elt_bytes, int max_q_len, hipStream_t st) {
  const int tiles = (max_q_len + TILE - 1) / TILE + 1;
  dim3 grid(tiles, a.num_kv_heads, a.num_seqs);
  if (elt_bytes == 1) {
    if (a.head_dim == 128)
      append_i8_kernel<2><<<grid, 256, 0, st>>>(a);
    else
      append_i8_kernel<1><<<grid, 256, 0, st>>>(a);
  } else if (elt_bytes == 2) {
    append_kernel<uint16_t><<<grid, 256, 0, st>>>(a);
  } else {
    append_kernel<uint32_t><<<grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyArgs& a, int n, int num_layers, hipStream_t st) {
  dim3 grid(n, num_layers, a.k_scale ? 4 : 2);
  copy_blocks_kernel<<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvp
