// Split-K (flash-decoding) paged attention on the gfx950 matrix cores, bf16 K/V.
//
// Serves single-token decode of a batch (NInfer serving doc, "Execution behavior") and the
// verification of 1 + k draft tokens (sparkinfer server README, "Serve Qwen3.8 with DSpark"):
// few query rows per KV head against a long paged context.  Each sequence's context is cut
// into splits whose size depends on that sequence's length alone, and one wave reduces one
// item, (split, KV head, row tile of <= 16*NT rows), to a partial (max, sum, unnormalised
// output); the reduce kernel merges splits in split order, so there are no float atomics
// (sparkinfer server README, "Determinism": the decode path has none).  A row whose keys all
// fall in split 0 is finished here and skips the reduce.
//
// Scheduling: persistent waves.  The grid holds as many one-wave workgroups as the GPU keeps
// resident at once, W, and wave w takes items w, w + W, w + 2W, ... (a fixed round robin, no
// atomics).  Items are numbered sequence by sequence and found from prefix sums of per-sequence
// item counts held one sequence per lane.  While a wave streams one item, the block ids of its
// next item are already in registers, so it moves from the last chunk of one item to the loads
// of the next with no metadata round trip.  Which wave computes an item never changes that
// item's result.
//
// Only sequences whose q_len is at most split_q_max are served here; longer query blocks of
// the same call (a prefill chunk batched with decode rows) are left to the prefill kernel.
// Partials are stored at the row's index among the split-K tokens of the call.
//
// Per item, rows are (token, head-in-group) pairs, so the G q-heads sharing a KV head use one
// read of K/V, walked in 32-key chunks:
//   S^T[key][row] = K[key][:] . Q[row][:]          2 x (D/32) v_mfma_f32_16x16x32_bf16 / N-tile
//   online softmax on the fp32 scores (exp2, scale*log2e folded in)
//   O^T[dim][row] += V^T[dim][key] . P^T[key][row]  D/16 MFMAs per N-tile
// Memory: the A operands load straight from the pool (K tiles are 16-byte dim chunks of 16
// tokens, V tiles are dims-major), every byte of a tile read once, and every load instruction
// reads one tile from a wave-uniform base: 1 KiB contiguous for K, 512 bytes for V.  Loads are
// double-buffered: chunk i+1 is in flight while chunk i is computed (32 KiB per wave), and the
// block ids of the item's tiles are read once into lanes and broadcast with v_readlane, so no
// table read sits between a chunk and its data.  Score tile h of a chunk is pool tile h, so a
// lane of the score output holds keys 4*g .. 4*g+3 of both tiles for its row; the PV product
// takes exactly those 8 keys as its k-slice (V^T rows read as two 8-byte runs), so P stays in
// registers.
//
// Forced splits longer than 2048 keys (a test and tuning knob) run a non-persistent variant:
// 4 waves share one split and merge their partials through LDS.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace kvp {

namespace {

__device__ __forceinline__ bf16x8 load16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Pool reads are streamed: each K/V byte is read once per call (a whole GQA group shares the
// wave), so the loads carry the nontemporal hint, which measurably raises the rate at which
// random 4 KiB tiles come in from HBM over plain loads.
__device__ __forceinline__ bf16x8 stream16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}
__device__ __forceinline__ u32x2 stream8(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

// Buffer resource over `bytes` bytes at p (raw, no stride): loads at offsets past `bytes` return
// zero without touching memory, so a load that must be issued but is not needed fetches nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}
constexpr int kBufNT = 2;  // buffer load cache policy: nontemporal (streamed once)

typedef int int4v __attribute__((ext_vector_type(4)));
// 16x16x64 int8 product with int32 accumulation (exact).  The k order inside a lane does not
// matter as long as A and B use the same one: lane (n, g) holds 16 consecutive dims of row /
// column n, the group g of each 64-dim step.
__device__ __forceinline__ int4v mfma16_i8(int4v a, int4v b, int4v c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D, bool I8>
struct Chunk {
  bf16x8 k[2][D / 32];  // K operand of score tile h (= pool tile h of the chunk)
  u32x2 v[2][D / 16];   // V^T operand halves: keys 4g..4g+3 of pool tile 0 and of tile 1
};

// int8 pool (tile layouts: K [d/16][t%16][d%16], V [(t%16)/4][d%16][d/16][t%4], one fp32 scale
// per token): lane (n, g) loads K chunks 4m+g (16 dims) of key n for m < D/64 (16 bytes each,
// two score k-steps per chunk), its V run (dims n, n+16, ... for keys 4g..4g+3: D/4 bytes) and
// the K and V scales of keys 4g..4g+3 of each pool tile.
template <int D>
struct Chunk<D, true> {
  u32x4 k[2][D / 64];
  u32x4 v[2][D / 64];
  floatx4 ks[2], vs[2];
};

// 8 int8 codes (two dwords) -> 8 bf16 values (exact: |code| <= 127).
__device__ __forceinline__ bf16x8 i8x8_to_bf16(uint32_t lo, uint32_t hi) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t x = i ? hi : lo;
    w[2 * i] = cvt_pk_bf16((float)(int8_t)(x & 0xff), (float)(int8_t)((x >> 8) & 0xff));
    w[2 * i + 1] = cvt_pk_bf16((float)(int8_t)((x >> 16) & 0xff), (float)(int8_t)(x >> 24));
  }
  return __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
}

// One work item: split `sp` of sequence s for KV head kvh and row tile rt.
struct Item {
  int s, kvh, rt, sp;
  int L, T;     // keys of the sequence, query rows (tokens) of the sequence
  int q_start;  // index of the sequence's first query token in q / out
  int p_start;  // its first row in the partial buffers
  int kb, ke;   // the item's keys [kb, ke): its split, cut at its last row's position + 1
                // (virtual key positions: see seq_vlayout)
  int split;    // keys per split of this sequence
  int vs1, vshift;  // the sequence's sparse key layout (identity when dense)
  int wlo_max;      // sparse rows see keys > p - window: the largest such p - window of the
                    // item's rows, or -1 when no row of the item is sparse
};

// Key range of an item; false if no row of the item sees a key of its split.
template <int NT>
__device__ __forceinline__ bool item_keys(const AttnArgs& a, Item& it) {
  it.vs1 = it.vshift = 0;
  it.wlo_max = -1;
  if (it.T > a.split_q_max) return false;  // a prefill-class sequence
  const int rows = it.T * a.group;
  if (rows <= a.split_rows_lo || rows > a.split_rows_hi) return false;  // another launch's
  const int r0 = it.rt * 16 * NT;
  if (r0 >= rows) return false;
  const int p_last = it.L - it.T + (min(r0 + 16 * NT, rows) - 1) / a.group;
  int Lv;
  seq_vlayout(a, it.L, it.T, Lv, it.vs1, it.vshift);
  it.wlo_max = (a.sparse_window > 0 && p_last + 1 >= a.sparse_min) ? p_last - a.sparse_window : -1;
  it.split = seq_split(a, Lv, it.T, it.vshift > 0);
  it.kb = it.sp * it.split;
  it.ke = min(min(Lv, virt_key(p_last, it.vs1, it.vshift) + 1), it.kb + it.split);
  return it.kb < it.ke;
}

// Block id of tile (wb/16 + base + lane) of sequence s, the tile index clamped into the wave's
// ntile tiles and the position into the item's keys (ke >= 1), so the read is always in the
// sequence's own table row.  wb, ke: virtual key positions of the layout (vs1, vshift).
__device__ __forceinline__ int tile_block_id(const AttnArgs& a, int s, int wb, int ntile, int ke,
                                             int base, int vs1, int vshift) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int32_t* tbl = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  const int ti = min(base + lane, max(ntile - 1, 0));
  return tbl[real_key(min(((wb >> 4) + ti) << 4, ke - 1), vs1, vshift) >> a.block_shift];
}

// Element offset of tile ti (clamped to the walk's ntile tiles) of a walk starting at tile
// tile0, whose block ids for tiles tb .. tb + 127 are in ids0 / ids1 (lane i: tile tb + i / 64 +
// i).  The tile past the end gets the last tile's address (loaded, never computed).
template <int D>
__device__ __forceinline__ size_t walk_tile_off(const AttnArgs& a, int kvh, int tile0, int ntile,
                                                int vs1, int vshift, int ids0, int ids1, int tb,
                                                int ti) {
  ti = min(ti, ntile - 1);
  const int r = ti - tb;
  const int blk = r < 64 ? __builtin_amdgcn_readlane(ids0, r) : __builtin_amdgcn_readlane(ids1, r - 64);
  const int sub = (real_key((tile0 + ti) << 4, vs1, vshift) & (a.block_size - 1)) >> 4;
  return block_tile_offset(blk, sub, kvh, a.block_shift, a.num_blocks, a.num_kv_heads, D);
}

// bf16 pool: the K and V operands of one 32-key chunk, pool tiles at element offsets o0, o1.
template <int D>
__device__ __forceinline__ void load_chunk_bf16(const AttnArgs& a, Chunk<D, false>& c, size_t o0,
                                                size_t o1) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int n = lane & 15, g = lane >> 4;
  const uint16_t* kl = reinterpret_cast<const uint16_t*>(a.k_layer);
  const uint16_t* vl = reinterpret_cast<const uint16_t*>(a.v_layer);
  const uint16_t* kt[2] = {kl + o0, kl + o1};
  const uint16_t* vt[2] = {vl + o0, vl + o1};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) c.k[h][kk] = stream16(kt[h] + ((4 * kk + g) * 16 + n) * 8);
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) c.v[h][mt] = stream8(vt[h] + (16 * mt + n) * 16 + 4 * g);
  }
}

// Row r0 + 16 nt + n of an item (n = lane % 16): its index in q / out and whether it exists.
__device__ __forceinline__ bool item_row(const AttnArgs& a, const Item& it, int r, size_t& rh) {
  const int G = a.group;
  const int i = r / G;
  const int grow = it.q_start + i;
  const bool valid = r < it.T * G && grow < a.total_q;
  rh = valid ? (size_t)grow * a.num_q_heads + it.kvh * G + r % G : 0;
  return valid;
}

// Q^T of an item's rows as the B operand of the score product: lane (n, g) holds row n of N-tile
// nt, dims 32 kk + 8 g .. +8 (int8 pools: dims 16 (4 (kk / 2) + g) + 8 (kk % 2) .. +8, the order
// of the K codes it meets); zero for rows that do not exist.
template <int D, int NT, bool I8>
__device__ __forceinline__ void load_q(const AttnArgs& a, const Item& it, bf16x8 (&qb)[NT][D / 32]) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    size_t rh;
    const bool valid = item_row(a, it, it.rt * 16 * NT + 16 * nt + n, rh);
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + rh * D;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      bf16x8 z = {};
      const int d0 = I8 ? 16 * (4 * (kk >> 1) + g) + 8 * (kk & 1) : 32 * kk + 8 * g;
      qb[nt][kk] = valid ? load16(qp + d0) : z;
    }
  }
}

// Reduces the keys [wb, we) of item `it` for one wave.  ids0/ids1: lane i holds the block id of
// the wave's tile i / 64 + i (from tile_block_id).  NW: waves sharing the item, whose partials
// merge through LDS (NW == 1: the wave finishes the item from registers).  RELOAD: the wave's
// keys may span more than 128 tiles, so block ids are reloaded every 128 tiles; without it no
// load in the chunk loop can force a wait on the chunks in flight.
// keys: false for an item none of whose rows sees a key of its split (one wave per item only):
// then nothing is computed or stored.  end_walk() (bf16 walks): called on every path once every
// load of the walk has been consumed, before the stores (see attn_split_persist_kernel).
template <int D, int NT, bool RELOAD, int NW, bool I8, typename EndWalk>
__device__ __forceinline__ void run_item(const AttnArgs& a, const Item& it, bool keys, int wave,
                                         int wb, int we, int ids0, int ids1, EndWalk&& end_walk) {
  constexpr int KK = D / 32;  // 32-dim steps of the score product
  constexpr int MT = D / 16;  // 16-dim tiles of the output
  const int lane = threadIdx.x & (WAVE - 1);
  const int n = lane & 15, g = lane >> 4;
  const int s = it.s, kvh = it.kvh, sp = it.sp, L = it.L, T = it.T, q_start = it.q_start;
  const int kb = it.kb, split = it.split;
  const int G = a.group;
  const int rows = T * G;
  const int r0 = it.rt * 16 * NT;
  const int nch = keys && wb < we ? (we - wb + 31) >> 5 : 0;
  const int ntile = keys && wb < we ? (we - wb + 15) >> 4 : 0;
  const int tile0 = wb >> 4;
  const uint16_t* kl = reinterpret_cast<const uint16_t*>(a.k_layer);
  const uint16_t* vl = reinterpret_cast<const uint16_t*>(a.v_layer);
  const int bmask = a.block_size - 1;

  int tb = 0;
  auto tile_off = [&](int ti) -> size_t {
    ti = min(ti, ntile - 1);  // past the end: the last tile's address (never computed)
    if (RELOAD && ti - tb >= 128) {
      tb = ti & ~127;
      ids0 = tile_block_id(a, s, wb, ntile, it.ke, tb, it.vs1, it.vshift);
      ids1 = tile_block_id(a, s, wb, ntile, it.ke, tb + 64, it.vs1, it.vshift);
    }
    return walk_tile_off<D>(a, kvh, tile0, ntile, it.vs1, it.vshift, ids0, ids1, tb, ti);
  };
  // Fused append (kvattn_append_forward): the new tokens whose keys fall in this item's range
  // are written for its KV head (the same bits as the append kernel: bf16 rows copied, int8 rows
  // quantised by append_row_i8) just before the loads of the first chunk that holds one, so
  // the walk's earlier chunks never queue behind the stores.  The wave's later loads of those
  // bytes see them without a wait: a wave's vector memory operations to one address are
  // performed in order (the compiler relies on the same for any thread's store-then-load); the
  // empty asm only keeps the compiler from moving loads above the stores.  Items of other row
  // tiles of the same split write the same bytes.
  // (int8 pools: 32-row tiles only; in the 16-row int8 kernel, at two waves per SIMD, the code
  // would cost registers the walk needs, and such calls append with the append kernel.)
  // New tokens are the last T real positions; under sparsity they sit past the layout's gap
  // (the window always holds them), so their virtual positions are contiguous too.
  const int p_new = L - T;
  const int v_new = virt_key(p_new, it.vs1, it.vshift);  // virtual position of the first
  const int v_end = v_new + T;
  const int c_new = ((!I8 || NT == 2) && NW == 1 && a.k_new != nullptr && nch > 0 && v_new < we &&
                     v_end > wb)
                        ? (max(v_new, wb) - wb) >> 5 : -1;  // wave-uniform
  auto append_new = [&]() {
    const uint16_t* kn = reinterpret_cast<const uint16_t*>(a.k_new);
    const uint16_t* vn = reinterpret_cast<const uint16_t*>(a.v_new);
    for (int vp = max(v_new, wb); vp < min(v_end, we); ++vp) {
      const int p = p_new + (vp - v_new);  // real position
      const int row = q_start + (p - p_new);
      if (row >= a.total_q) continue;
      const size_t off = tile_off((vp >> 4) - tile0);  // elements of the pool tile
      const int tt = p & 15;
      const size_t src = ((size_t)row * a.num_kv_heads + kvh) * D;
      if constexpr (!I8) {
        uint16_t* kt = const_cast<uint16_t*>(kl) + off;
        uint16_t* vt = const_cast<uint16_t*>(vl) + off;
        if (lane < D / 8)  // K: 8-dim chunk `lane` of the token
          *reinterpret_cast<u32x4*>(kt + (lane * 16 + tt) * 8) =
              *reinterpret_cast<const u32x4*>(kn + src + 8 * lane);
#pragma unroll
        for (int d = lane; d < D; d += WAVE) vt[d * 16 + tt] = vn[src + d];  // V^T: dim d, slot tt
      } else {
        // int8 pools (32-row tiles): quantised and stored as the append kernel does
        int8_t* kt = const_cast<int8_t*>(reinterpret_cast<const int8_t*>(a.k_layer)) + off;
        int8_t* vt = const_cast<int8_t*>(reinterpret_cast<const int8_t*>(a.v_layer)) + off;
        append_row_i8<D / 64>(kt, vt, const_cast<float*>(a.k_scale_layer) + off / D,
                              const_cast<float*>(a.v_scale_layer) + off / D, kn + src, vn + src, tt);
      }
    }
    asm volatile("" ::: "memory");
  };

  auto load_chunk = [&](Chunk<D, I8>& c, int ci) {
    if constexpr (!I8 || NT == 2) {
      if (ci == c_new) append_new();  // wave-uniform; once, before the chunk's own loads
    }
    const size_t o0 = tile_off(2 * ci), o1 = tile_off(2 * ci + 1);
    if constexpr (I8) {
      // Byte offsets here (tile index = offset / (16 D)).  Buffer loads over the tile: a tile
      // past the walk (the ring runs up to three chunks ahead of the last one) gets a zero-size
      // resource, so its loads are issued but fetch nothing.
      const int8_t* k8 = reinterpret_cast<const int8_t*>(a.k_layer);
      const int8_t* v8 = reinterpret_cast<const int8_t*>(a.v_layer);
      const size_t oo[2] = {o0, o1};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bool live = 2 * ci + h < ntile;  // wave-uniform
        const auto rk = tile_rsrc(k8 + oo[h], live ? 16 * D : 0);
        const auto rv = tile_rsrc(v8 + oo[h], live ? 16 * D : 0);
#pragma unroll
        for (int m = 0; m < D / 64; ++m) {
          c.k[h][m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, ((4 * m + g) * 16 + n) * 16, 0, kBufNT));
          c.v[h][m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, (g * 16 + n) * (D / 4) + 16 * m, 0, kBufNT));
        }
        // the 16 K and V scales of the tile; lane (n, g) takes those of keys 4g .. 4g+3
        const auto rks = tile_rsrc(a.k_scale_layer + oo[h] / D, live ? 64 : 0);
        const auto rvs = tile_rsrc(a.v_scale_layer + oo[h] / D, live ? 64 : 0);
        c.ks[h] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rks, 16 * g, 0, 0));
        c.vs[h] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rvs, 16 * g, 0, 0));
      }
    } else {
      load_chunk_bf16<D>(a, c, o0, o1);
    }
  };

  // int8: a ring of RN chunks, RN - 1 in flight while one is computed.  16-row tiles: three,
  // at two waves per SIMD (250 registers); 32-row tiles: four, at one wave per SIMD (a chunk
  // is half the bytes, so the lone wave needs more of them in flight).  Measured on batched
  // decode: ring of three at two waves per SIMD 71 us, ring of four at one wave 81 us, ring of
  // six at one wave 90 us (each item ends with RN - 1 chunks of zero-size loads).  The ring is
  // filled right after the Q loads, before Q is converted, so that the wait for Q has the ring
  // in flight behind it and never waits for it.  bf16: two buffers, chunk i+1 in flight while
  // chunk i is computed (a ring measured slower there).
  constexpr bool RING = I8;
  constexpr int RN = NT == 1 ? 3 : 4;
  Chunk<D, I8> bufA, bufB;
  Chunk<D, I8> rb[RING ? RN : 1];
  if (!RING && nch) load_chunk(bufA, 0);

  // Q^T as the B operand: lane (n, g) holds row n of N-tile nt, dims 32*kk + 8*g .. +8 (int8
  // pools: dims 16*(4*(kk/2) + g) + 8*(kk%2) .. +8, the order of the K chunks it meets).
  const int Hq = a.num_q_heads;
  bf16x8 qb[NT][KK];
  load_q<D, NT, I8>(a, it, qb);
  if constexpr (RING) {
    // Unconditional (a wave without keys has ntile = 0: zero-size loads that fetch nothing), so
    // the compiler's count of loads in flight is exact at the wait for Q.
#pragma unroll
    for (int j = 0; j + 1 < RN; ++j) load_chunk(rb[j], j);
  }
  int prow[NT];   // the row's real key position (-1: padding row)
  int vprow[NT];  // its virtual position in the sequence's key layout
  int wlo[NT];    // sparse row: keys <= wlo (and >= the sink) are not seen; else -1
  size_t rh[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = r0 + 16 * nt + n;
    const bool valid = item_row(a, it, r, rh[nt]);
    prow[nt] = valid ? L - T + r / G : -1;
    vprow[nt] = virt_key(prow[nt], it.vs1, it.vshift);
    wlo[nt] = (valid && a.sparse_window > 0 && prow[nt] + 1 >= a.sparse_min)
                  ? prow[nt] - a.sparse_window : -1;
  }

  // int8 pools: the q row as a 15-bit fixed-point value with a per-row power-of-two scale,
  // q ~ (256 hi + lo) * qs with hi in [-64, 64] and lo in [-128, 127], so that q.k of the int8
  // codes is two exact int8 products (scores then carry a relative error of about 2^-15 of the
  // row's largest |q|, far below the bf16 rounding of P).  Lane (n, g) holds dims
  // 16 (4 m + g) .. + 16 of row n for 64-dim step m, in the order of its K codes.
  int4v qhi[I8 ? NT : 1][I8 ? D / 64 : 1], qlo[I8 ? NT : 1][I8 ? D / 64 : 1];
  float qs[NT];
  if constexpr (I8) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float qm = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) qm = fmaxf(qm, fabsf((float)qb[nt][kk][e]));
      qm = xrow_max(qm);  // the row's lanes n, n + 16, n + 32, n + 48
      int ex = 0;
      (void)frexpf(qm, &ex);  // qm < 2^ex
      const int sh = qm > 0.f ? 14 - ex : 0;
      qs[nt] = qm > 0.f ? __builtin_amdgcn_ldexpf(1.f, -sh) : 0.f;
#pragma unroll
      for (int m = 0; m < D / 64; ++m) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          uint32_t hv = 0, lv = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int j = 4 * w4 + b;  // dim 16 (4 m + g) + j
            const float x = (float)qb[nt][2 * m + (j >> 3)][j & 7];
            const int q16 = (int)rintf(__builtin_amdgcn_ldexpf(x, sh));  // |q16| <= 2^14
            const int lo = ((q16 + 128) & 255) - 128;
            const int hi = (q16 - lo) >> 8;
            hv |= (uint32_t)(hi & 255) << (8 * b);
            lv |= (uint32_t)(lo & 255) << (8 * b);
          }
          hw[w4] = hv;
          lw[w4] = lv;
        }
        qhi[nt][m] = int4v{(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3]};
        qlo[nt][m] = int4v{(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3]};
      }
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

  auto compute = [&](Chunk<D, I8>& ch, int ci) {
    const int c0 = wb + 32 * ci;  // virtual position of the chunk's first key
    const int rc0 = real_key(c0, it.vs1, it.vshift);
    // the sparse mask can remove a key of this chunk (wave-uniform)
    const bool smask = rc0 <= it.wlo_max && rc0 + 32 > a.sparse_sink;
    // int8: the V scales of slots at or past `we` (never written: may hold anything) zeroed so
    // that p * scale stays 0; with two N-tiles the V^T operands are converted once for both
    auto v_i8 = [&](int mt) {
      return i8x8_to_bf16(ch.v[0][mt >> 2][mt & 3], ch.v[1][mt >> 2][mt & 3]);
    };
    bf16x8 va8[NT > 1 ? MT : 1];
    if constexpr (I8) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (c0 + 16 * h + 4 * g + j >= we) ch.vs[h][j] = 0.f;
      if constexpr (NT > 1) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) va8[mt] = v_i8(mt);
      }
    } else if (c0 + 32 > we) {
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
        if constexpr (I8) {
          // exact int32 dot products of the codes with the two halves of the fixed-point q
          int4v ah = {0, 0, 0, 0}, al = {0, 0, 0, 0};
#pragma unroll
          for (int m = 0; m < D / 64; ++m) {
            const int4v ka = __builtin_bit_cast(int4v, ch.k[h][m]);
            ah = mfma16_i8(ka, qhi[nt][m], ah);
            al = mfma16_i8(ka, qlo[nt][m], al);
          }
          const floatx4 ksq = ch.ks[h] * qs[nt];  // key 4g + i of tile h: K scale times q scale
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[h][i] = (float)(ah[i] * 256 + al[i]) * ksq[i];
        } else {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) acc = mfma16(ch.k[h][kk], qb[nt][kk], acc);
          sc[h] = acc;
        }
      }
      // This lane now holds row n's scores for keys c0 + 16*h + 4*g + i (j = 4*h + i).
      float sv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int off = 16 * (j >> 2) + 4 * g + (j & 3);
        sv[j] = (c0 + off < we && rc0 + off <= prow[nt]) ? sc[j >> 2][j & 3] : -INFINITY;
      }
      if (smask) {  // sink + window: keys past the sink and at or before p - window are unseen
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int rk = rc0 + 16 * (j >> 2) + 4 * g + (j & 3);
          if (rk >= a.sparse_sink && rk <= wlo[nt]) sv[j] = -INFINITY;
        }
      }
      float cmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) cmax = fmaxf(cmax, sv[j]);
      cmax = xrow_max(cmax);
      // Lazy rescaling: the row's reference max moves only when the chunk's max exceeds it by
      // more than 8 in exp2 units (so p <= 2^8), and o and l are rescaled only in a chunk where
      // some row's reference moved; otherwise alpha = 1 and the rescale is skipped.
      const bool grow = (cmax - m_run[nt]) * c > 8.f;  // also true for the first finite max
      const float m_new = grow ? cmax : m_run[nt];
      const float msub = m_new == -INFINITY ? 0.f : m_new * c;
      const bool rescale = __builtin_amdgcn_ballot_w64(grow) != 0;  // wave-uniform
      const float alpha = grow ? fast_exp2((m_run[nt] - m_new) * c) : 1.f;
      uint32_t pk[4];
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        if constexpr (I8) {
          // P times the V scale of its key goes to the PV product; the row sum takes P alone
          const float p0 = fast_exp2(sv[j] * c - msub), p1 = fast_exp2(sv[j + 1] * c - msub);
          psum += p0 + p1;
          pk[j >> 1] = cvt_pk_bf16(p0 * ch.vs[j >> 2][j & 3], p1 * ch.vs[j >> 2][(j & 3) + 1]);
        } else {
          const float p0 = round_to_bf16(fast_exp2(sv[j] * c - msub));
          const float p1 = round_to_bf16(fast_exp2(sv[j + 1] * c - msub));
          psum += p0 + p1;
          pk[j >> 1] = pack_exact_bf16(p0, p1);
        }
      }
      m_run[nt] = m_new;
      if (rescale) {
        l_run[nt] *= alpha;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) o[nt][mt] *= alpha;
      }
      l_run[nt] += psum;
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        bf16x8 va;
        if constexpr (I8) {
          if constexpr (NT > 1) va = va8[mt];
          else va = v_i8(mt);
        } else {
          va = __builtin_bit_cast(
              bf16x8, u32x4{ch.v[0][mt][0], ch.v[0][mt][1], ch.v[1][mt][0], ch.v[1][mt][1]});
        }
        o[nt][mt] = mfma16(va, pb, o[nt][mt]);
      }
    }
  };

  if constexpr (RING) {
    // Chunk ci sits in rb[ci % RN]; chunk ci + RN - 1 goes into the slot chunk ci - 1 left,
    // before chunk ci is computed.  Loads past the last chunk are issued with zero-size buffer
    // resources (nothing is fetched) and never computed, so every load is unconditional and the
    // waits before each compute are static.
    if (nch) {
      for (int ci = 0;; ci += RN) {
        bool done = false;
#pragma unroll
        for (int j = 0; j < RN; ++j) {
          load_chunk(rb[(j + RN - 1) % RN], ci + j + RN - 1);
          compute(rb[j], ci + j);
          if (ci + j + 1 >= nch) {
            done = true;
            break;
          }
        }
        if (done) break;
      }
    }
    // Only the ring's loads past the end (zero-size) may be outstanding: as in the bf16 walk
    // below, this lets the next item start without waiting for its ids behind the stores.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    end_walk();
  } else {
    // Double-buffered walk: the loads of chunk i+1 are issued before chunk i is computed.  The
    // last one or two chunks are peeled off, so that no load is left in flight after the walk
    // (the registers it would land in are reused right after).
    int ci = 0;
    for (; ci + 2 < nch; ci += 2) {
      load_chunk(bufB, ci + 1);
      compute(bufA, ci);
      load_chunk(bufA, ci + 2);
      compute(bufB, ci + 1);
    }
    if (ci + 1 < nch) {
      load_chunk(bufB, ci + 1);
      compute(bufA, ci);
      compute(bufB, ci + 1);
    } else if (ci < nch) {
      compute(bufA, ci);
    }
    // Every load of the walk has been consumed.  With 32-row tiles, saying so here and having
    // end_walk read the next item's block ids (loaded before this item's chunks) tells the
    // compiler they have arrived, so the next item does not wait for them, and behind them for
    // the stores below, before its first loads.
    if constexpr (NT == 2) __builtin_amdgcn_s_waitcnt(0x0F70);
    end_walk();
  }
  if (!keys) return;  // wave-uniform

  // Adds to a row's output index (q_start + i) * Hq + head to give its partial row index
  // (p_start + i) * Hq + head (modulo 2^64: the sum is never negative).
  const size_t pofs = (size_t)(((long long)it.p_start - q_start) * Hq);
  if constexpr (NW == 1) {
    // One wave per split: finish straight from registers.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float lt = xrow_sum(l_run[nt]);
      if (vprow[nt] < kb) continue;  // padding row, or a row that sees no key of this split
      const bool final_here = vprow[nt] < split;
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
        const size_t prh = rh[nt] + pofs;  // (p_start + i) * Hq + head
        if (prh >= (size_t)a.part_rows * Hq) continue;
        const size_t slot = prh * a.max_splits + sp;
        if (g == 0) {
          a.part_ml[2 * slot] = m_run[nt];
          a.part_ml[2 * slot + 1] = lt;
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          *reinterpret_cast<floatx4*>(a.part_o + slot * D + 16 * mt + 4 * g) = o[nt][mt];
      }
    }
  } else {
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
      const bool row_ok = vprow[nt] >= kb;  // a real row that sees a key of this split
      const bool final_here = vprow[nt] < split;
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
        } else if (rh[nt] + pofs < (size_t)a.part_rows * Hq) {
          const size_t slot = (rh[nt] + pofs) * a.max_splits + sp;
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
}

// ---- persistent scheduling ----------------------------------------------------------------

// Items of one sequence: splits x KV heads x row tiles, bounded by the launch's workspace
// geometry (max_splits, row_tiles) whatever the device metadata says.
template <int NT>
__device__ __forceinline__ int seq_items(const AttnArgs& a, int L, int T) {
  if (T <= 0 || T > a.split_q_max) return 0;  // no rows, or a prefill-class sequence
  if (T * a.group <= a.split_rows_lo || T * a.group > a.split_rows_hi) return 0;  // another launch's
  int Lv, vs1, vshift;
  seq_vlayout(a, L, T, Lv, vs1, vshift);
  const int split = seq_split(a, Lv, T, vshift > 0);
  const int ns = min(Lv / split + (Lv % split != 0), a.max_splits);
  const int rts = min((T * a.group + 16 * NT - 1) / (16 * NT), a.row_tiles);
  return ns * a.num_kv_heads * rts;
}

// The item table of 64 consecutive sequences, sequence base + i in lane i.
struct SeqGroup {
  int base;       // first sequence of the group
  int item_base;  // items of the sequences before the group
  int q_base;     // query tokens of the sequences before the group
  int p_base;     // split-K tokens (partial rows) of the sequences before the group
  int items;      // items of the group
  int q_total;    // query tokens of the group
  int p_total;    // split-K tokens of the group
  int incl;       // lane: items of sequences base .. base + lane
  int L, T, qx;   // lane: its lengths and the query tokens of the group's sequences before it
  int px;         // lane: split-K tokens of the group's sequences before it
};

template <int NT>
__device__ __forceinline__ void load_group(const AttnArgs& a, SeqGroup& gp, int base) {
  const int lane = threadIdx.x & (WAVE - 1);
  const int s = base + lane;
  const int sc = min(s, a.num_seqs - 1);
  int L, T;
  seq_lens(a, sc, L, T);
  int q = max(0, a.q_lens[sc]);  // row offsets count the raw q_lens, like the other kernels
  if (s >= a.num_seqs) L = T = q = 0;
  gp.base = base;
  gp.incl = wave_incl_scan(seq_items<NT>(a, L, T));
  const int qi = wave_incl_scan(q);
  gp.qx = qi - q;
  const int pr = T <= a.split_q_max ? T : 0;
  const int pi = wave_incl_scan(pr);
  gp.px = pi - pr;
  gp.p_total = __builtin_amdgcn_readlane(pi, WAVE - 1);
  gp.L = L;
  gp.T = T;
  gp.items = __builtin_amdgcn_readlane(gp.incl, WAVE - 1);
  gp.q_total = __builtin_amdgcn_readlane(qi, WAVE - 1);
}

// Decodes ticket t (wave-uniform) into an item; false once t is past the last item.  Within a
// sequence the KV head varies fastest, then the row tile, then the split.
template <int NT>
__device__ __forceinline__ bool find_item(const AttnArgs& a, SeqGroup& gp, int t, Item& it) {
  if (t < gp.item_base) {  // tickets of a wave normally increase; restart the scan if not
    gp.item_base = 0;
    gp.q_base = 0;
    gp.p_base = 0;
    load_group<NT>(a, gp, 0);
  }
  while (t - gp.item_base >= gp.items) {
    if (gp.base + WAVE >= a.num_seqs) return false;
    gp.item_base += gp.items;
    gp.q_base += gp.q_total;
    gp.p_base += gp.p_total;
    load_group<NT>(a, gp, gp.base + WAVE);
  }
  const int r_in = t - gp.item_base;
  const int j = __builtin_popcountll(__builtin_amdgcn_ballot_w64(gp.incl <= r_in));
  int r = r_in - (j ? __builtin_amdgcn_readlane(gp.incl, j - 1) : 0);
  it.s = gp.base + j;
  it.L = __builtin_amdgcn_readlane(gp.L, j);
  it.T = __builtin_amdgcn_readlane(gp.T, j);
  it.q_start = gp.q_base + __builtin_amdgcn_readlane(gp.qx, j);
  it.p_start = gp.p_base + __builtin_amdgcn_readlane(gp.px, j);
  const int rts = min((it.T * a.group + 16 * NT - 1) / (16 * NT), a.row_tiles);
  it.kvh = r % a.num_kv_heads;
  r /= a.num_kv_heads;
  it.rt = r % rts;
  it.sp = r / rts;
  return true;
}

}  // namespace

// Wave w of W takes items w, w + W, w + 2W, ... in increasing order.  W is what the GPU holds at
// once, so all waves start together; a wave's next item is known in advance, and its block ids
// are loaded before the current item's chunks.  (Holding the next item's first chunk in
// registers across an item's end does not fit the 256 registers of two waves per SIMD: the
// compiler spills.)
// Two waves per SIMD for 16-row tiles (NT = 1, up to 256 registers), one for 32-row tiles.
template <int D, int NT, bool I8>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(NT == 1 ? 2 : 1)))
void attn_split_persist_kernel(AttnArgs a) {
  const int W = gridDim.x;
  SeqGroup gp;
  gp.item_base = 0;
  gp.q_base = 0;
  gp.p_base = 0;
  load_group<NT>(a, gp, 0);
  Item cur;
  int t = blockIdx.x;
  bool have = find_item<NT>(a, gp, t, cur);
  bool cur_keys = have && item_keys<NT>(a, cur);
  int ids0 = 0, ids1 = 0;
  if (have) {
    const int nt = (cur.ke - cur.kb + 15) >> 4;
    ids0 = tile_block_id(a, cur.s, cur.kb, nt, cur.ke, 0, cur.vs1, cur.vshift);
    ids1 = tile_block_id(a, cur.s, cur.kb, nt, cur.ke, 64, cur.vs1, cur.vshift);
  }
  // Block ids at item starts (32-row tiles).  The compiler tracks loads per register and, where
  // paths merge, assumes the worst: the ids copied in at the loop's end look outstanding at the
  // next item's first block-id read, which then waits for every older memory operation, the
  // next item's own id loads and the last item's stores included (a full memory latency per
  // item).  Waiting for the first item's ids here and marking the next item's ids as arrived
  // at the end of each walk (run_item) removes that wait: verification of 4 drafts over 32K
  // keys, one item per wave, measured 34.7 -> 32 us.  With 16-row tiles (two waves per SIMD,
  // where the other wave covers the wait) the same change measured about 1% slower, so it is
  // left out there.
  if constexpr (NT == 2 || I8) {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("" ::"v"(ids0), "v"(ids1));
  }
  while (have) {
    t += W;
    Item nxt = cur;
    const bool nhave = t < (1 << 30) && find_item<NT>(a, gp, t, nxt);
    const bool nkeys = nhave && item_keys<NT>(a, nxt);
    // Unconditional loads (the current item's ids again when there is no next item), so that
    // no branch around a load makes the chunk loop wait for these.
    const int ps = nhave ? nxt.s : cur.s;
    const int pb = nhave ? nxt.kb : cur.kb;
    const int pe = nhave ? nxt.ke : cur.ke;
    const int pv1 = nhave ? nxt.vs1 : cur.vs1;
    const int pvs = nhave ? nxt.vshift : cur.vshift;
    const int pt = (pe - pb + 15) >> 4;
    const int nid0 = tile_block_id(a, ps, pb, pt, pe, 0, pv1, pvs);
    const int nid1 = tile_block_id(a, ps, pb, pt, pe, 64, pv1, pvs);
    run_item<D, NT, false, 1, I8>(a, cur, cur_keys, 0, cur.kb, cur.ke, ids0, ids1, [&]() {
      if constexpr (NT == 2 || I8) asm volatile("" ::"v"(nid0), "v"(nid1));
    });
    if (!nhave) break;
    cur = nxt;
    cur_keys = nkeys;
    ids0 = nid0;
    ids1 = nid1;
  }
}

// Forced splits longer than 2048 keys: one workgroup of 4 waves per item, on the grid
// x = (KV head, sequence, row tile) with the KV head fastest, y = split.
template <int D, int NT, bool RELOAD, bool I8>
__global__ __launch_bounds__(256) void attn_split_mfma_kernel(AttnArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Item it;
  it.kvh = blockIdx.x % a.num_kv_heads;
  const int pair = blockIdx.x / a.num_kv_heads;
  it.s = pair % a.num_seqs;
  it.rt = pair / a.num_seqs;
  it.sp = blockIdx.y;
  seq_lens(a, it.s, it.L, it.T);
  if (!item_keys<NT>(a, it)) return;
  // This wave's keys: a contiguous, 32-aligned quarter of [kb, ke).
  const int span = (it.ke - it.kb + 4 * 32 - 1) / (4 * 32) * 32;
  const int wb = it.kb + wave * span;
  const int we = min(it.ke, wb + span);
  const int ntile = wb < we ? (we - wb + 15) >> 4 : 0;
  const int ids0 = tile_block_id(a, it.s, wb, ntile, it.ke, 0, it.vs1, it.vshift);
  const int ids1 = tile_block_id(a, it.s, wb, ntile, it.ke, 64, it.vs1, it.vshift);
  seq_starts(a, it.s, it.q_start, it.p_start);
  // vmcnt(0) (encoding: vmcnt 0, expcnt 7, lgkmcnt 15), so the compiler knows the block ids
  // have arrived and never waits for them inside the chunk loop.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  run_item<D, NT, RELOAD, 4, I8>(a, it, true, wave, wb, we, ids0, ids1, []() {});
}

namespace {

// Workgroups of the persistent kernel the GPU holds at once (per CU, from the occupancy API).
template <int D, int NT, bool I8>
int persist_blocks_per_cu() {
  static const int n = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &b, reinterpret_cast<const void*>(&attn_split_persist_kernel<D, NT, I8>), 64, 0) != hipSuccess)
      return 0;
    return b;
  }();
  return n;
}

template <int D, int NT, bool I8>
hipError_t launch_split(const AttnArgs& a, int splits, int num_cus, hipStream_t st) {
  const bool persistent = a.split_tokens <= 2048;
  if (persistent) {
    const int per_cu = persist_blocks_per_cu<D, NT, I8>();
    if (per_cu <= 0) return hipErrorInvalidConfiguration;
    const long long items = (long long)a.num_seqs * a.num_kv_heads * a.row_tiles * splits;
    const long long waves = std::min<long long>(items, (long long)per_cu * std::max(num_cus, 1));
    attn_split_persist_kernel<D, NT, I8><<<(unsigned)waves, 64, 0, st>>>(a);
  } else {
    if (splits > 65535) return hipErrorInvalidConfiguration;
    const dim3 grid(a.num_kv_heads * a.num_seqs * a.row_tiles, splits, 1);
    if (a.split_tokens > 8192)
      attn_split_mfma_kernel<D, NT, true, I8><<<grid, 256, 0, st>>>(a);
    else
      attn_split_mfma_kernel<D, NT, false, I8><<<grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

template <bool I8>
hipError_t launch_split_dt(const AttnArgs& a, int head_dim, int rows_per_tile, int splits,
                           int num_cus, hipStream_t st) {
  if (head_dim == 128)
    return rows_per_tile <= 16 ? launch_split<128, 1, I8>(a, splits, num_cus, st)
                               : launch_split<128, 2, I8>(a, splits, num_cus, st);
  return rows_per_tile <= 16 ? launch_split<64, 1, I8>(a, splits, num_cus, st)
                             : launch_split<64, 2, I8>(a, splits, num_cus, st);
}

}  // namespace

hipError_t launch_attn_split_mfma(const AttnArgs& a, int head_dim, int rows_per_tile, int splits,
                                  int num_cus, bool int8_kv, hipStream_t st) {
  return int8_kv ? launch_split_dt<true>(a, head_dim, rows_per_tile, splits, num_cus, st)
                 : launch_split_dt<false>(a, head_dim, rows_per_tile, splits, num_cus, st);
}

}  // namespace kvp
