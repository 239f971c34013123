// Device helpers shared by the gfx950 kernels: bf16 bit handling, wave64 cross-lane
// reductions, pool tile addressing and the kernel argument block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int TILE = 16;        // tokens per layout tile
constexpr int WAVE = 64;
constexpr float LOG2E = 1.4426950408889634f;

// ---- bf16 <-> fp32 --------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> nearest-even bf16, result in the low 16 bits (finite and inf inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
// fp32 value of the nearest-even bf16 of f.
__device__ __forceinline__ float round_to_bf16(float f) {
  return __uint_as_float(f32_to_bf16_bits(f) << 16);
}
// Two floats -> packed nearest-even bf16 pair (lo in bits 0..15): v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const floatx2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
// Two floats that are already exact bf16 values -> packed pair (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_exact_bf16(float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// ---- wave64 cross-lane ----------------------------------------------------------------
// DPP controls (within a row of 16 lanes): quad_perm xor1 / xor2, row_ror 4 / 8.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_ROR4 = 0x124, DPP_ROR8 = 0x128;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Lane-pair views used for butterflies across rows: op(x[l], x[l ^ 16]) and op(x[l], x[l ^ 32]).
__device__ __forceinline__ void swap16(float x, float& a, float& b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float x, float& a, float& b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Reductions over the 4 rows of the wave (lanes l, l^16, l^32, l^48), result in every lane.
__device__ __forceinline__ float xrow_sum(float x) {
  float a, b;
  swap32(x, a, b);
  x = a + b;
  swap16(x, a, b);
  return a + b;
}
__device__ __forceinline__ float xrow_max(float x) {
  float a, b;
  swap32(x, a, b);
  x = fmaxf(a, b);
  swap16(x, a, b);
  return fmaxf(a, b);
}
// Reductions within each row of 16 lanes, result in every lane of the row.
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<DPP_ROR8>(x);
  x += dpp<DPP_ROR4>(x);
  x += dpp<DPP_XOR2>(x);
  x += dpp<DPP_XOR1>(x);
  return x;
}
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, dpp<DPP_ROR8>(x));
  x = fmaxf(x, dpp<DPP_ROR4>(x));
  x = fmaxf(x, dpp<DPP_XOR2>(x));
  x = fmaxf(x, dpp<DPP_XOR1>(x));
  return x;
}

// Integer reductions over the wave (exact at any size), result in every lane.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int wave_sum_i(int x) {
  x += dpp_i<DPP_ROR8>(x);
  x += dpp_i<DPP_ROR4>(x);
  x += dpp_i<DPP_XOR2>(x);
  x += dpp_i<DPP_XOR1>(x);
  auto r = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
  x = (int)(r[0] + r[1]);
  r = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
  return (int)(r[0] + r[1]);
}

// Inclusive prefix sum over the wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    const int t = __shfl_up(v, d);
    if (lane >= d) v += t;
  }
  return v;
}

// Sum of v[0 .. n) over the wave (negative entries count 0), every lane gets it.
__device__ __forceinline__ int wave_prefix_total(const int32_t* v, int n) {
  const int lane = threadIdx.x & (WAVE - 1);
  int acc = 0;
  for (int base = 0; base < n; base += WAVE)  // uniform trip count
    acc += (base + lane < n) ? max(0, v[base + lane]) : 0;
  return wave_sum_i(acc);
}

// Workgroup barrier without a memory fence.  __syncthreads() also waits for every outstanding
// vector memory operation (vmcnt(0)), which would drain LDS-DMA loads still meant to be in
// flight; callers of this one have already waited for what must be visible (an explicit vmcnt
// wait for LDS-DMA data, ds_read results before their use).  The empty asm statements keep the
// compiler from moving memory operations across the barrier.
__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// exp2 that maps -inf to 0 without a branch (hardware v_exp_f32 already does).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- kernel arguments -------------------------------------------------------------------
struct AttnArgs {
  const void* q;            // [total_q][Hq][D]
  void* out;                // [total_q][Hq][D]
  const void* k_layer;      // pool K storage of the selected layer
  const void* v_layer;
  const int32_t* block_tables;
  const int32_t* ctx_lens;
  const int32_t* q_lens;
  const float* k_scale_layer;  // int8 pools: the layer's [blocks][Hkv][block_size] scales
  const float* v_scale_layer;
  float* part_o;            // [part_rows][Hq][max_splits][D]  split-K partial outputs
  float* part_ml;           // [part_rows][Hq][max_splits][2]  their (max, sum) pairs
  int32_t num_seqs, total_q, num_q_heads, num_kv_heads, group, block_size, num_blocks;
  int32_t block_shift;      // log2(block_size)
  int32_t max_blocks_per_seq;
  int32_t split_tokens;     // split-K path: keys per split if > 0, else the per-length rule
  int32_t max_splits;       // splits per partial row in the workspace
  int32_t row_tiles;        // split-K and vector kernels: row tiles per (sequence, kv head)
  int32_t split_q_max;      // sequences with q_len <= split_q_max take the split-K path
  int32_t split_rows_lo;    // split-K kernels: only sequences with lo < q_len * group <= hi
  int32_t split_rows_hi;    // (a call may run its short and long sequences in two launches)
  int32_t part_rows;        // rows of the partial buffers (query tokens of the split-K path)
  int32_t pf_rblk;          // prefill kernel: 32-row blocks per workgroup
  // Prefill key splits (pf_ksplit > 1): each row tile's keys are cut into pf_ksplit ranges of
  // whole 64-key tiles, reduced by separate workgroups into partials [total_q][Hq][pf_ksplit]
  // ([D] outputs, (max, sum) pairs) that attn_reduce_prefill merges in range order.
  int32_t pf_ksplit;
  float* pf_part_o;
  float* pf_part_ml;
  // Sink + window sparsity (split-K path; off when sparse_window == 0): a query row at position
  // p with p + 1 >= sparse_min reads only keys j < sparse_sink or j > p - sparse_window.
  int32_t sparse_sink, sparse_window, sparse_min;
  float scale_log2;         // softmax scale * log2(e)
  // Fused append (kvattn_append_forward; split-K calls only): the new tokens' rows
  // [total_q][Hkv][D] (bf16), written into the pool by the split-K item whose keys hold them
  // before it reads them; null otherwise.
  const void* k_new;
  const void* v_new;
};

// Keys per split of a sequence with L (virtual) keys and T query rows on the split-K path: a
// fixed count if the caller set one, else ceil(L/128) rounded up to a multiple of 32 and clamped
// to [lo, 2048] with lo = split_floor(...).  That gives at most 128 splits up to 262144 keys (so
// one long sequence's splits fit the GPU in one pass, with no sliver of a split left over).  The
// split depends on the sequence and the pool alone, so its reduction order does too.
//
// The floor: 512 keys when the sequence's rows per KV head (T times the group size) fit one
// 16-row tile and its keys have no sparse gap (gapped: vshift > 0); otherwise 352 on bf16 / fp32
// pools and 256 on int8 pools, and 256 for a gapped walk.  Measured (step time, one MI355X):
//  - short single-tile sequences come in batches, where the wider floor halves their items and
//    partials (32 decode sequences of 1-8K keys 4% faster in bf16, 8% in int8 at 512 than 256);
//  - a verification of 1 + 3 drafts over 32K keys (two 16-row tiles per KV head) takes 41.0 us at
//    288-key splits, 37.8 at 352, 37.9 at 384 and 43.0 at 512 on a bf16 pool; on an int8 pool,
//    whose chunks are half the bytes, 40.6 at 288 and 42.2 at 352;
//  - a sparse walk of one window has few items, which bound its latency (two 4K-key windows:
//    14 -> 20 us with the 512 floor).
// Shared by the kernels (per sequence: its rows per KV head, whether its keys have a sparse gap)
// and the host (for a whole call: the largest rows per KV head of its split-K sequences and
// whether any may be gapped; the result is the smallest floor of the call), so the host's
// decision to skip the reduce launch (no sequence can have a second split) always agrees with the
// kernels' splits.
__host__ __device__ __forceinline__ int split_floor(int rows_per_kv_head, bool gapped, bool int8) {
  if (gapped) return 256;
  if (rows_per_kv_head <= 16) return 512;
  return int8 ? 256 : 352;
}
// k_scale_layer is set exactly for int8 pools.
__device__ __forceinline__ int seq_split(const AttnArgs& a, int L, int T, bool gapped) {
  if (a.split_tokens > 0) return a.split_tokens;
  const int per = (L >> 7) + ((L & 127) != 0);  // ceil(L / 128) without overflow
  const int lo = split_floor(T * a.group, gapped, a.k_scale_layer != nullptr);
  return min(max((per + 31) & ~31, lo), 2048);
}

// Key layout of a split-K sequence (L keys, T query rows) under sink + window sparsity.  When
// every row of the sequence is past the threshold (L - T + 1 >= sparse_min), no row reads the
// keys between the sink and the first row's window, so the walk skips them: virtual key
// positions [0, vs1) are real positions [0, vs1) and virtual v >= vs1 is real v + vshift, with
// vs1 = the sink rounded up to 32 keys and vs1 + vshift = the first row's window start rounded
// down to 32 keys (so a 32-key chunk never straddles the gap).  Keys that the walk still reads
// but a row must not see are masked by position.  Lv: virtual keys.  Without sparsity, or when
// there is no gap, the layout is the identity (vs1 = vshift = 0, Lv = L).
__device__ __forceinline__ void seq_vlayout(const AttnArgs& a, int L, int T, int& Lv, int& vs1,
                                            int& vshift) {
  Lv = L;
  vs1 = 0;
  vshift = 0;
  if (a.sparse_window > 0 && T > 0 && L - T + 1 >= a.sparse_min) {
    const int s1 = (min(a.sparse_sink, L) + 31) & ~31;
    const int w0 = max(0, L - T + 1 - a.sparse_window) & ~31;
    if (w0 > s1) {
      vs1 = s1;
      vshift = w0 - s1;
      Lv = L - vshift;
    }
  }
}
// Real position of virtual key v, and virtual position of a real key that the walk reads.
__device__ __forceinline__ int real_key(int v, int vs1, int vshift) {
  return v >= vs1 ? v + vshift : v;
}
__device__ __forceinline__ int virt_key(int p, int vs1, int vshift) {
  return p >= vs1 + vshift ? p - vshift : p;
}

// Clamped per-sequence lengths (bad metadata must never index out of bounds).
__device__ __forceinline__ void seq_lens(const AttnArgs& a, int s, int& L, int& T) {
  int cap = a.max_blocks_per_seq * a.block_size;
  L = min(max(a.ctx_lens[s], 0), cap);
  T = min(max(a.q_lens[s], 0), L);
}

// Query tokens the split-K path holds for sequence s: its q_len if that is at most split_q_max
// (decode and verification), else 0 (its rows make one pass in the prefill kernel).  The class
// depends on the sequence alone, so a sequence's rows take the same path in any batch.
__device__ __forceinline__ int split_rows_of(const AttnArgs& a, int s) {
  int L, T;
  seq_lens(a, s, L, T);
  return T <= a.split_q_max ? T : 0;
}

// First rows of sequence s: in q / out (the raw q_lens of the sequences before it, as the
// packing counts them) and in the partial buffers (the split-K tokens of the sequences before
// it).  Every lane gets both.
__device__ __forceinline__ void seq_starts(const AttnArgs& a, int s, int& q_start, int& p_start) {
  const int lane = threadIdx.x & (WAVE - 1);
  int qa = 0, pa = 0;
  for (int base = 0; base < s; base += WAVE) {  // uniform trip count
    const int j = base + lane;
    if (j < s) {
      qa += max(0, a.q_lens[j]);
      pa += split_rows_of(a, j);
    }
  }
  q_start = wave_sum_i(qa);
  p_start = wave_sum_i(pa);
}

// Sequence s and query row i of partial row r (the split-K tokens of the call, numbered in
// sequence order), and the sequence's first row in q / out.  False if r is past the last one.
// Wave-uniform; the whole wave must be active.
__device__ __forceinline__ bool find_split_row(const AttnArgs& a, int r, int& s, int& i,
                                               int& q_start, int& L, int& T) {
  const int lane = threadIdx.x & (WAVE - 1);
  int pbase = 0, qbase = 0;
  for (int base = 0; base < a.num_seqs; base += WAVE) {
    const int j = base + lane;
    int Lj = 0, Tj = 0, q = 0;
    if (j < a.num_seqs) {  // seq_lens(a, j, Lj, Tj), reading q_lens[j] once
      const int ql = a.q_lens[j];
      Lj = min(max(a.ctx_lens[j], 0), a.max_blocks_per_seq * a.block_size);
      Tj = min(max(ql, 0), Lj);
      q = max(0, ql);
    }
    const int pr = Tj <= a.split_q_max ? Tj : 0;  // split_rows_of(a, j)
    const int pin = wave_incl_scan(pr);
    const int qin = wave_incl_scan(q);
    const int ptot = __builtin_amdgcn_readlane(pin, WAVE - 1);
    const int rr = r - pbase;
    if (rr < ptot) {
      // Inclusive counts are nondecreasing: the row's sequence is the first lane past rr.
      const int k = __builtin_popcountll(__builtin_amdgcn_ballot_w64(pin <= rr));
      s = base + k;
      i = rr - (__builtin_amdgcn_readlane(pin, k) - __builtin_amdgcn_readlane(pr, k));
      q_start = qbase + __builtin_amdgcn_readlane(qin, k) - __builtin_amdgcn_readlane(q, k);
      L = __builtin_amdgcn_readlane(Lj, k);
      T = __builtin_amdgcn_readlane(Tj, k);
      return true;
    }
    pbase += ptot;
    qbase += __builtin_amdgcn_readlane(qin, WAVE - 1);
  }
  return false;
}
__device__ __forceinline__ bool find_split_row(const AttnArgs& a, int r, int& s, int& i,
                                               int& q_start) {
  int L, T;
  return find_split_row(a, r, s, i, q_start, L, T);
}

// Element offset of the 16-token tile holding logical position `pos` of sequence s for KV head
// h, within one layer.  Block ids outside [0, num_blocks) are clamped to 0.
__device__ __forceinline__ size_t tile_offset(const int32_t* table_row, int pos, int h,
                                              int block_size, int num_blocks, int num_kv_heads,
                                              int head_dim) {
  int bi = pos / block_size;
  int blk = table_row[bi];
  blk = ((unsigned)blk < (unsigned)num_blocks) ? blk : 0;
  int sub = (pos % block_size) / TILE;
  size_t tile = ((size_t)blk * num_kv_heads + h) * (size_t)(block_size / TILE) + sub;
  return tile * (size_t)(TILE * head_dim);
}

// Element offset of tile `sub` of block `blk` for KV head h within one layer (blk clamped).
__device__ __forceinline__ size_t block_tile_offset(int blk, int sub, int h, int block_shift,
                                                    int num_blocks, int num_kv_heads,
                                                    int head_dim) {
  blk = ((unsigned)blk < (unsigned)num_blocks) ? blk : 0;
  const size_t tile = (((size_t)blk * num_kv_heads + h) << (block_shift - 4)) + sub;
  return tile * (size_t)(TILE * head_dim);
}

// int8 pool (sparkinfer server README, "Env", SPARKINFER_KV_INT8; NInfer serving doc, "Server
// options", --kv-dtype int8): each new (token, KV head) row of bf16 values is quantised with
// one fp32 scale s = absmax / 127 and codes q = rint(x / s) (correctly rounded division, ties
// to even), clamped to +-127; a zero row gets s = 0 and codes 0.  Tile layouts (16 tokens):
//   K: [d / 16][t % 16][d % 16]                      (16-byte chunks of 16 dims)
//   V: [(t % 16) / 4][d % 16][d / 16][t % 4]         (the 4 keys of a dim group side by side)
// One wave per (token, KV head) row: lane l holds dims E*l .. E*l + E - 1 (E = head_dim / 64),
// the absolute max comes from a wave reduction, and codes are stored byte by byte (K) / to
// their scattered V slots.  The append kernel and the 32-row split-K kernel's fused append both
// store rows through store_row_i8, so their bits are the same.
__device__ __forceinline__ float wave_max_f(float v) {
  // across the 4 rows of 16 lanes (permlane swaps), then within each row (DPP): no LDS trips
  return row_max(xrow_max(v));
}

// A row's E bf16 values of this lane (dims E*lane ..), as floats.
template <int E>
__device__ __forceinline__ void load_row(const uint16_t* src, float (&x)[E]) {
  const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = __uint_as_float((uint32_t)src[E * lane + e] << 16);
}

template <int E>
__device__ __forceinline__ void quantise_vals(const float (&x)[E], float (&q)[E], float& scale) {
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) m = fmaxf(m, fabsf(x[e]));
  m = wave_max_f(m);
  scale = __fdiv_rn(m, 127.f);
#pragma unroll
  for (int e = 0; e < E; ++e)
    q[e] = scale > 0.f ? fminf(fmaxf(rintf(__fdiv_rn(x[e], scale)), -127.f), 127.f) : 0.f;
}

// Quantises the K and V values kx / vx of one (token, KV head) row (head_dim 64 E, this lane's
// dims) and stores the codes and scales at token slot tt of a 16-token tile (kt, vt: the tile's
// codes; ks, vs: its 16 scales).  The whole wave takes part (wave reductions).
template <int E>
__device__ __forceinline__ void store_row_i8(int8_t* kt, int8_t* vt, float* ks, float* vs,
                                             const float (&kx)[E], const float (&vx)[E], int tt) {
  constexpr int D = 64 * E;
  const int lane = threadIdx.x & (WAVE - 1);
  float qk[E], qv[E], sk, sv;
  quantise_vals<E>(kx, qk, sk);
  quantise_vals<E>(vx, qv, sv);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int d = E * lane + e;
    kt[(d >> 4) * 256 + tt * 16 + (d & 15)] = (int8_t)(int)qk[e];
    vt[(((tt >> 2) * 16 + (d & 15)) * (D / 16) + (d >> 4)) * 4 + (tt & 3)] = (int8_t)(int)qv[e];
  }
  if (lane == 0) {
    ks[tt] = sk;
    vs[tt] = sv;
  }
}

// The same from the bf16 rows krow / vrow in memory.
template <int E>
__device__ __forceinline__ void append_row_i8(int8_t* kt, int8_t* vt, float* ks, float* vs,
                                              const uint16_t* krow, const uint16_t* vrow, int tt) {
  float kx[E], vx[E];
  load_row<E>(krow, kx);
  load_row<E>(vrow, vx);
  store_row_i8<E>(kt, vt, ks, vs, kx, vx, tt);
}

}  // namespace kvp
