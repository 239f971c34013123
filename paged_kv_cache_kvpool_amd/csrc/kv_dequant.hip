// Prefill over an int8 pool: the K/V tiles of the prefill-class sequences (q_len > split_q_max)
// are dequantized to bf16 (code times its token's scale, rounded to nearest even) into a
// workspace pool that the bf16 prefill kernel then reads.  The copy costs one extra pass over
// HBM; the alternative, converting the codes in the prefill kernel's LDS stages (its int8
// path, used when the workspace has no room for the copy), gives the same bits but adds vector
// work that the prefill kernel cannot hide behind its matrix work, and measured slower.
// (int8 KV storage: NInfer serving doc, "Server options", --kv-dtype int8; sparkinfer server
// README, "Env", SPARKINFER_KV_INT8.)
//
// The workspace pool has 16-token blocks; prefill sequence i (the i-th prefill-class sequence
// of the call) owns blocks i*mpb .. i*mpb + mpb - 1, and block j of it holds the sequence's
// tokens 16j .. 16j+15 (bf16 layout: K [d/8][t][d%8], V [d][t] per KV head).  Its block table
// row is written alongside.  One workgroup of 256 threads per (prefill sequence, KV head, group
// of kTiles 16-token tiles): its threads issue the loads of all its tiles before converting any,
// so the metadata and block-table round trips are paid once per group; the grid may exceed the
// groups there are (extra workgroups exit).
#include "common.h"
#include "kernels.h"

namespace kvp {

namespace {

constexpr int kTiles = 4;  // 16-token tiles per workgroup
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Prefill sequence, its index among the prefill-class sequences, KV head and tile group of flat
// workgroup n, where sequence i holds Hkv * ceil(ceil(L / 16) / kTiles) workgroups.  False past
// the last.
__device__ __forceinline__ bool find_dequant_tile(const AttnArgs& a, int n, int& s, int& i, int& h,
                                                  int& tile) {
  const int lane = threadIdx.x & (WAVE - 1);
  int wbase = 0, ibase = 0;
  for (int base = 0; base < a.num_seqs; base += WAVE) {
    const int j = base + lane;
    int cnt = 0, pf = 0;
    if (j < a.num_seqs) {
      int L, T;
      seq_lens(a, j, L, T);
      pf = T > a.split_q_max ? 1 : 0;
      cnt = pf * a.num_kv_heads * ((((L + 15) >> 4) + kTiles - 1) / kTiles);
    }
    const int win = wave_incl_scan(cnt);
    const int pin = wave_incl_scan(pf);
    const int wtot = __builtin_amdgcn_readlane(win, WAVE - 1);
    const int nn = n - wbase;
    if (nn < wtot) {
      const int k = __builtin_popcountll(__builtin_amdgcn_ballot_w64(win <= nn));
      s = base + k;
      i = ibase + __builtin_amdgcn_readlane(pin, k) - 1;
      const int within = nn - (__builtin_amdgcn_readlane(win, k) - __builtin_amdgcn_readlane(cnt, k));
      const int tiles = __builtin_amdgcn_readlane(cnt, k) / a.num_kv_heads;
      h = within / tiles;
      tile = within - h * tiles;
      return true;
    }
    wbase += wtot;
    ibase += __builtin_amdgcn_readlane(pin, WAVE - 1);
  }
  return false;
}

template <int D>
__global__ __launch_bounds__(256) void dequant_prefill_kernel(AttnArgs a, DequantOut o) {
  int s, i, h, grp;
  if (!find_dequant_tile(a, blockIdx.x, s, i, h, grp)) return;
  if (i >= o.max_seqs) return;  // beyond the workspace geometry
  int L, T;
  seq_lens(a, s, L, T);
  const int tile0 = grp * kTiles;
  // tiles of this group that exist and fit the workspace (workgroup-uniform)
  const int nt = min(kTiles, min((L + 15) >> 4, o.blocks_per_seq) - tile0);
  if (nt <= 0) return;
  const int tid = threadIdx.x;
  const int32_t* tbl = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  const int pb0 = i * o.blocks_per_seq + tile0;  // workspace block of the group's first tile
  if (h == 0 && tid < nt) o.tables[(size_t)s * o.blocks_per_seq + tile0 + tid] = pb0 + tid;
  size_t src[kTiles];  // byte offset of each tile in the int8 layer
#pragma unroll
  for (int u = 0; u < kTiles; ++u) {
    const int pos = 16 * (tile0 + min(u, nt - 1));
    int blk = tbl[pos >> a.block_shift];
    blk = ((unsigned)blk < (unsigned)a.num_blocks) ? blk : 0;
    src[u] = block_tile_offset(blk, (pos & (a.block_size - 1)) >> 4, h, a.block_shift,
                               a.num_blocks, a.num_kv_heads, D);
  }
  const int8_t* k8 = reinterpret_cast<const int8_t*>(a.k_layer);
  const int8_t* v8 = reinterpret_cast<const int8_t*>(a.v_layer);
  auto dst = [&](int u) { return ((size_t)(pb0 + u) * a.num_kv_heads + h) * 16 * D; };  // bf16
  if (tid < D) {
    // K: 16-dim chunk c of token t -> bf16 chunks 2c and 2c+1 of the token
    const int c = tid >> 4, t = tid & 15;
    u32x4 w[kTiles];
    float sc[kTiles];
#pragma unroll
    for (int u = 0; u < kTiles; ++u) {  // every load first (tiles past nt repeat the last one)
      w[u] = *reinterpret_cast<const u32x4*>(k8 + src[u] + (c * 16 + t) * 16);
      sc[u] = a.k_scale_layer[src[u] / D + t];
    }
#pragma unroll
    for (int u = 0; u < kTiles; ++u) {
      if (u >= nt) break;
      uint32_t r[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t x = w[u][e >> 1] >> (16 * (e & 1));
        r[e] = cvt_pk_bf16((float)(int8_t)(x & 0xff) * sc[u], (float)(int8_t)((x >> 8) & 0xff) * sc[u]);
      }
      uint16_t* kd = o.k + dst(u);
      *reinterpret_cast<u32x4*>(kd + ((2 * c) * 16 + t) * 8) = u32x4{r[0], r[1], r[2], r[3]};
      *reinterpret_cast<u32x4*>(kd + ((2 * c + 1) * 16 + t) * 8) = u32x4{r[4], r[5], r[6], r[7]};
    }
  }
  // V: the tile's codes ([t/4][d%16][d/16][t%4], 16 D bytes) are read by D threads with one
  // contiguous 16-byte load each, converted, and transposed through LDS into the bf16 rows
  // [d][t] that the threads then store 32 bytes each (contiguous as well).  Thread j's 16 bytes
  // are entries 4j .. 4j+3 of (token group tg, d%16, d/16), each the 4 tokens of group tg for one
  // dim; all four share tg (D entries per group), so one float4 of scales serves them.
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[kTiles][D * 16];
  const int j = tid - D;
  const bool vthr = tid >= D && tid < 2 * D;  // workgroup-uniform per wave (D is a multiple of 64)
  if (vthr) {
    u32x4 x[kTiles];
    floatx4 s4[kTiles];
    const int tg = (4 * j) / D;
#pragma unroll
    for (int u = 0; u < kTiles; ++u) {  // every load first (tiles past nt repeat the last one)
      x[u] = *reinterpret_cast<const u32x4*>(v8 + src[u] + 16 * j);
      s4[u] = *reinterpret_cast<const floatx4*>(a.v_scale_layer + src[u] / D + 4 * tg);
    }
#pragma unroll
    for (int u = 0; u < kTiles; ++u) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = 4 * j + q;
        const int d = 16 * (e % (D / 16)) + (e / (D / 16)) % 16;
        const uint32_t xx = x[u][q];
        const uint32_t r0 = cvt_pk_bf16((float)(int8_t)(xx & 0xff) * s4[u][0],
                                        (float)(int8_t)((xx >> 8) & 0xff) * s4[u][1]);
        const uint32_t r1 = cvt_pk_bf16((float)(int8_t)((xx >> 16) & 0xff) * s4[u][2],
                                        (float)(int8_t)(xx >> 24) * s4[u][3]);
        *reinterpret_cast<u32x2*>(&vt_lds[u][d * 16 + 4 * tg]) = u32x2{r0, r1};
      }
    }
  }
  __syncthreads();
  if (vthr) {
    const int d = j;
#pragma unroll
    for (int u = 0; u < kTiles; ++u) {
      if (u >= nt) break;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(&vt_lds[u][d * 16]);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(&vt_lds[u][d * 16 + 8]);
      uint16_t* vd = o.v + dst(u) + d * 16;
      *reinterpret_cast<u32x4*>(vd) = lo;
      *reinterpret_cast<u32x4*>(vd + 8) = hi;
    }
  }
}

}  // namespace

hipError_t launch_dequant_prefill(const AttnArgs& a, const DequantOut& o, int head_dim,
                                  hipStream_t st) {
  // at least the (prefill sequence, KV head, tile group) count there can be
  const long long wgs = (long long)o.max_seqs * a.num_kv_heads * ((o.blocks_per_seq + kTiles - 1) / kTiles);
  if (wgs <= 0) return hipSuccess;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (head_dim == 128)
    dequant_prefill_kernel<128><<<(unsigned)wgs, 256, 0, st>>>(a, o);
  else
    dequant_prefill_kernel<64><<<(unsigned)wgs, 256, 0, st>>>(a, o);
  return hipGetLastError();
}

}  // namespace kvp
