// Prefill over an int8 pool: the K/V tiles of the prefill-class sequences (q_len > split_q_max)
// are dequantized to bf16 (code times its token's scale, rounded to nearest even) into a
// workspace pool that the bf16 prefill kernel then reads.  Prefill is bound by the matrix
// cores and reads each key once per workgroup from LDS, so a converted copy costs one extra
// pass over HBM, while converting inside its inner loop would cost VALU work it has none of.
// (int8 KV storage: NInfer serving doc, "Server options", --kv-dtype int8; sparkinfer server
// README, "Env", SPARKINFER_KV_INT8.)
//
// The workspace pool has 16-token blocks; prefill sequence i (the i-th prefill-class sequence
// of the call) owns blocks i*mpb .. i*mpb + mpb - 1, and block j of it holds the sequence's
// tokens 16j .. 16j+15 (bf16 layout: K [d/8][t][d%8], V [d][t] per KV head).  Its block table
// row is written alongside.  One workgroup of 256 threads per (prefill sequence, KV head,
// 16-token tile); the grid may exceed the tiles there are (extra workgroups exit).
#include "common.h"
#include "kernels.h"

namespace kvp {

namespace {

// Prefill sequence, its index among the prefill-class sequences, KV head and tile of flat
// workgroup n, where sequence i holds Hkv * ceil(L / 16) workgroups.  False past the last.
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
      cnt = pf * a.num_kv_heads * ((L + 15) >> 4);
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
  int s, i, h, tile;
  if (!find_dequant_tile(a, blockIdx.x, s, i, h, tile)) return;
  if (i >= o.max_seqs || tile >= o.blocks_per_seq) return;  // beyond the workspace geometry
  const int tid = threadIdx.x;
  const int32_t* tbl = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  const int pos = 16 * tile;
  int blk = tbl[pos >> a.block_shift];
  blk = ((unsigned)blk < (unsigned)a.num_blocks) ? blk : 0;
  const size_t src = block_tile_offset(blk, (pos & (a.block_size - 1)) >> 4, h, a.block_shift,
                                       a.num_blocks, a.num_kv_heads, D);  // bytes
  const int pb = i * o.blocks_per_seq + tile;  // workspace block
  const size_t dst = ((size_t)pb * a.num_kv_heads + h) * 16 * D;  // bf16 elements
  if (h == 0 && tid == 0) o.tables[(size_t)s * o.blocks_per_seq + tile] = pb;
  const int8_t* k8 = reinterpret_cast<const int8_t*>(a.k_layer) + src;
  const int8_t* v8 = reinterpret_cast<const int8_t*>(a.v_layer) + src;
  const float* ks = a.k_scale_layer + src / D;
  const float* vs = a.v_scale_layer + src / D;
  if (tid < D) {
    // K: 16-dim chunk c of token t -> bf16 chunks 2c and 2c+1 of the token
    const int c = tid >> 4, t = tid & 15;
    const u32x4 w = *reinterpret_cast<const u32x4*>(k8 + (c * 16 + t) * 16);
    const float sc = ks[t];
    uint32_t r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t x = w[e >> 1] >> (16 * (e & 1));
      r[e] = cvt_pk_bf16((float)(int8_t)(x & 0xff) * sc, (float)(int8_t)((x >> 8) & 0xff) * sc);
    }
    uint16_t* kd = o.k + dst;
    *reinterpret_cast<u32x4*>(kd + ((2 * c) * 16 + t) * 8) = u32x4{r[0], r[1], r[2], r[3]};
    *reinterpret_cast<u32x4*>(kd + ((2 * c + 1) * 16 + t) * 8) = u32x4{r[4], r[5], r[6], r[7]};
  } else if (tid < 2 * D) {
    // V: dim d, its 16 tokens (4 groups of 4 codes) -> one bf16 row of 16 tokens
    const int d = tid - D;
    uint32_t r[8];
#pragma unroll
    for (int tg = 0; tg < 4; ++tg) {
      const uint32_t x = *reinterpret_cast<const uint32_t*>(v8 + ((tg * 16 + (d & 15)) * (D / 16) + (d >> 4)) * 4);
      const floatx4 sv = *reinterpret_cast<const floatx4*>(vs + 4 * tg);
      r[2 * tg] = cvt_pk_bf16((float)(int8_t)(x & 0xff) * sv[0], (float)(int8_t)((x >> 8) & 0xff) * sv[1]);
      r[2 * tg + 1] = cvt_pk_bf16((float)(int8_t)((x >> 16) & 0xff) * sv[2], (float)(int8_t)(x >> 24) * sv[3]);
    }
    uint16_t* vd = o.v + dst + d * 16;
    *reinterpret_cast<u32x4*>(vd) = u32x4{r[0], r[1], r[2], r[3]};
    *reinterpret_cast<u32x4*>(vd + 8) = u32x4{r[4], r[5], r[6], r[7]};
  }
}

}  // namespace

hipError_t launch_dequant_prefill(const AttnArgs& a, const DequantOut& o, int head_dim,
                                  long long wgs, hipStream_t st) {
  if (wgs <= 0) return hipSuccess;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (head_dim == 128)
    dequant_prefill_kernel<128><<<(unsigned)wgs, 256, 0, st>>>(a, o);
  else
    dequant_prefill_kernel<64><<<(unsigned)wgs, 256, 0, st>>>(a, o);
  return hipGetLastError();
}

}  // namespace kvp
