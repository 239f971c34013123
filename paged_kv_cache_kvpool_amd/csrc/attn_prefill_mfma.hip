// Prefill attention over a paged pool on the gfx950 matrix cores, bf16 K/V: the uncached
// suffix of each sequence (many query rows) against its cached prefix plus itself, causal
// (sparkinfer server README, "Automatic prefix cache": only the suffix is prefilled, over the
// shared prefix blocks; "Request isolation & continuous batching": prefill in chunks).
//
// Workgroup = W waves (4..12) over one row tile of one (sequence, KV head); a wave owns 32 rows
// (row = token * G + head-in-group, so every row of a workgroup reads the same K/V), the row
// blocks of a (sequence, KV head) dealt to its workgroups strided.  K/V are
// walked in tiles of 64 keys = 4 pool tiles, each streamed verbatim from the pool into LDS with
// global_load_lds (no register staging; the pool's tile layout is the order the matrix cores
// read) through a ring of 4 LDS stages: while tile j is computed, tile j+1 is ready, j+2 is
// landing and j+3 is being issued; one vmcnt wait and one barrier per tile.  (int8 pools whose
// bf16 copy does not fit the workspace: the codes and per-token scales stream into 3 int8
// stages, 3 bf16 stages hold the converted tiles; see the staging code.)  Each 64-key tile is
// two 32-key blocks; per wave and
// block, on v_mfma_f32_32x32x16_bf16 (the 32x32 shape runs at twice the rate of 16x16x32 on
// gfx950):
//   S^T[key][row] = K . Q^T      D/16 MFMAs, K rows read from LDS in a key order (bits 2 and 3
//                                of the key index swapped) that leaves each lane holding, for
//                                its row, exactly the 8 + 8 keys the PV step takes as its
//                                k-slices, so P goes from the score registers to the PV operand
//                                with a convert and nothing else
//   causal mask only on blocks that reach past the wave's first row or the context (V slots
//   past the context are zeroed in LDS once, in the last tile); online softmax in fp32 with
//   exp2 and a lazily raised running max; row sums on the VALU
//   O^T[dim][row] += V^T . P^T   2 k-steps x D/32 MFMAs
// The logical workgroup order is remapped so that the row tiles of one (sequence, KV head) run
// on the same XCD (workgroups are dealt to the 8 XCDs round-robin) and share its L2.
// When the row tiles alone leave CUs idle (a single prefill chunk, or one beside decode rows),
// each row tile's keys are cut into pf_ksplit ranges of whole 64-key tiles, one workgroup per
// range; such a workgroup stores its rows' unnormalised partials, merged in range order by
// attn_reduce_prefill (as split-K decode merges its splits).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace kvp {

namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

constexpr int NXCD = 8;

// One pool tile (NQ KiB) from gbase + voff into LDS at lds_addr: NQ global_load_lds_dwordx4
// with instruction offsets 0, 1024, ... (the offset advances the global and the LDS address
// alike; lane l's 16 bytes of piece q land at lds_addr + 1024*q + 16*l), one M0 write per tile.
// Issued as inline asm so that the compiler's wait insertion never ties these loads to LDS
// reads of other stages or to reused address registers: the kernel waits for them itself
// (vmcnt) before the barrier that publishes a stage.  The base and the LDS address are
// wave-uniform by construction; readfirstlane makes that explicit so that they always live in
// scalar registers, as the instruction requires.
template <int NQ>
__device__ __forceinline__ void dma_tile(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  // (readfirstlane returns a signed int: widen through uint32_t, never sign-extend the low word)
  const uint64_t g = reinterpret_cast<uint64_t>(gbase);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)g);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(g >> 32));
  const uint64_t gs = ((uint64_t)hi << 32) | (uint64_t)lo;
  const uint32_t ls = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr);
  static_assert(NQ == 1 || NQ == 2 || NQ == 4, "pool tiles of 1, 2 or 4 KiB");
  if constexpr (NQ == 1)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(reinterpret_cast<const void*>(gs)), "s"(ls)
                 : "memory", "m0");
  else if constexpr (NQ == 4)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1\n\t"
                 "global_load_lds_dwordx4 %0, %1 offset:1024\n\t"
                 "global_load_lds_dwordx4 %0, %1 offset:2048\n\t"
                 "global_load_lds_dwordx4 %0, %1 offset:3072"
                 :
                 : "v"(voff), "s"(reinterpret_cast<const void*>(gs)), "s"(ls)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1\n\t"
                 "global_load_lds_dwordx4 %0, %1 offset:1024"
                 :
                 : "v"(voff), "s"(reinterpret_cast<const void*>(gs)), "s"(ls)
                 : "memory", "m0");
}

// int8 pools: 64 dwords, lane l's from gbase + voff (voff per lane), into LDS at lds_addr + 4*l
// (one global_load_lds_dword, issued like dma_tile).  Used for the 16 per-token scales of a pool
// tile (voff = 4 * (lane % 16): four copies).
__device__ __forceinline__ void dma_dwords(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  const uint64_t g = reinterpret_cast<uint64_t>(gbase);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)g);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(g >> 32));
  const uint64_t gs = ((uint64_t)hi << 32) | (uint64_t)lo;
  const uint32_t ls = (uint32_t)__builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(reinterpret_cast<const void*>(gs)), "s"(ls)
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

// vmcnt(n) for the n DMA pieces a wave may have issued for the stage after next (0..8).
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
    case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F78); break;
  }
}

// Row tiles of one (sequence, KV head) pair of a prefill-class sequence (q_len > split_q_max):
// its 32-row blocks dealt to workgroups of R row blocks each; 0 for a sequence of the split-K
// path.
__device__ __forceinline__ int seq_row_tiles(const AttnArgs& a, int T, int R) {
  if (T <= a.split_q_max) return 0;
  const int nblk = (min(T, a.total_q) * a.group + 31) >> 5;  // T <= total_q for valid metadata
  return (nblk + R - 1) / R;
}

// Workgroups are numbered sequence by sequence: a prefill-class sequence holds num_kv_heads *
// row tiles of them, in (KV head, row tile) order.  Total number of them (every lane).
__device__ __forceinline__ int prefill_wg_total(const AttnArgs& a, int R) {
  const int lane = threadIdx.x & (WAVE - 1);
  int acc = 0;
  for (int base = 0; base < a.num_seqs; base += WAVE) {  // uniform trip count
    const int j = base + lane;
    if (j < a.num_seqs) {
      int L, T;
      seq_lens(a, j, L, T);
      acc += seq_row_tiles(a, T, R) * a.num_kv_heads;
    }
  }
  return wave_sum_i(acc);
}

// Sequence, KV head and row tile of workgroup n (in the numbering above), the sequence's row
// tiles and the index of its first query token in q / out.  Wave-uniform; the whole wave must be
// active.
__device__ __forceinline__ void find_prefill_tile(const AttnArgs& a, int n, int R, int& s,
                                                  int& kvh, int& rt, int& rts, int& q_start) {
  const int lane = threadIdx.x & (WAVE - 1);
  int wbase = 0, qbase = 0;
  s = kvh = rt = q_start = 0;
  rts = 1;
  for (int base = 0; base < a.num_seqs; base += WAVE) {
    const int j = base + lane;
    int r = 0, q = 0;
    if (j < a.num_seqs) {
      int L, T;
      seq_lens(a, j, L, T);
      r = seq_row_tiles(a, T, R);
      q = max(0, a.q_lens[j]);
    }
    const int wg = r * a.num_kv_heads;
    const int win = wave_incl_scan(wg);
    const int qin = wave_incl_scan(q);
    const int wtot = __builtin_amdgcn_readlane(win, WAVE - 1);
    const int nn = n - wbase;
    if (nn < wtot) {
      // Inclusive counts are nondecreasing: the workgroup's sequence is the first lane past nn.
      const int k = __builtin_popcountll(__builtin_amdgcn_ballot_w64(win <= nn));
      s = base + k;
      const int within = nn - (__builtin_amdgcn_readlane(win, k) - __builtin_amdgcn_readlane(wg, k));
      rts = __builtin_amdgcn_readlane(r, k);
      kvh = within / rts;
      rt = within - kvh * rts;
      q_start = qbase + __builtin_amdgcn_readlane(qin, k) - __builtin_amdgcn_readlane(q, k);
      return;
    }
    wbase += wtot;
    qbase += __builtin_amdgcn_readlane(qin, WAVE - 1);
  }
}

}  // namespace

// Issue order of one finish (the softmax and P.V of a 32-key block beside the score product of
// the next), as chunks of at most one MFMA each.  MFMA u < D/16 is k-step u of the next block's
// score product; u = D/16 + (D/32) j + mb is k-step j of P.V for output dims 32mb .. +32, which
// needs the P packs 4j .. 4j+3.  -1: a chunk without MFMA.  Operand loads run two MFMAs ahead.
// The softmax of a score pair is two stages: exp2 (with its scale-and-subtract FMA) in one
// chunk, the bf16 pack and the row-sum adds in a later one, so that no chunk's vector work waits
// on the latency of its own exp2.
template <int D> struct PfSched;
template <> struct PfSched<128> {
  static constexpr int N = 16;
  // MFMA of each chunk (all 16 chunks carry one): score k-steps 0-4, then P.V k-step 0 (u 8-11)
  // interleaved with score k-steps 5-7, then P.V k-step 1 (u 12-15)
  static constexpr int kOp[16] = {0, 1, 2, 3, 4, 8, 5, 9, 6, 10, 7, 11, 12, 13, 14, 15};
  // exp2 stage of each pair, and its pack stage a chunk later: packs 0-3 are made by chunk 4,
  // before P.V k-step 0 starts (chunk 5); packs 4-7 by chunk 11, before P.V k-step 1 (chunk 12)
  static constexpr int kExp[16] = {0, 1, 2, 3, 4, -1, 5, -1, 6, -1, 7, -1, -1, -1, -1, -1};
  static constexpr int kPack[16] = {-1, 0, 1, 2, 3, 4, -1, 5, -1, 6, -1, 7, -1, -1, -1, -1};
  static constexpr int op(int ci) { return kOp[ci]; }
  static constexpr int exp_pair(int ci) { return kExp[ci]; }
  static constexpr int pack_pair(int ci) { return kPack[ci]; }
  static constexpr int slot(int ci) { return ci; }
  static constexpr int next_load(int ci) { return ci + 2 < N ? ci + 2 : -1; }
  static constexpr int slot_of_load(int ci) { return ci; }
  // part of the next block's lane-local row max made beside the last P.V MFMAs (its last score
  // MFMA is issued in chunk 10, so its result is ready by then)
  static constexpr int kMax[16] = {-1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, 0, 1, 2};
  static constexpr int max_part(int ci) { return kMax[ci]; }
};
template <> struct PfSched<64> {
  static constexpr int N = 10;
  static constexpr int kOp[10] = {0, 1, 2, 3, 4, 5, -1, -1, 6, 7};
  static constexpr int kExp[10] = {0, 1, 2, 3, 4, 5, 6, 7, -1, -1};
  // MFMA chunks in order, and each chunk's index among them (operand slot)
  static constexpr int kMf[8] = {0, 1, 2, 3, 4, 5, 8, 9};
  static constexpr int kSlot[10] = {0, 1, 2, 3, 4, 5, 0, 0, 6, 7};
  static constexpr int op(int ci) { return kOp[ci]; }
  static constexpr int exp_pair(int ci) { return kExp[ci]; }
  static constexpr int pack_pair(int ci) { return kExp[ci]; }  // both stages in one chunk
  static constexpr int slot(int ci) { return kSlot[ci]; }
  // the chunk whose operand the MFMA of chunk ci loads: the MFMA two places later
  static constexpr int next_load(int ci) { return kSlot[ci] + 2 < 8 ? kMf[kSlot[ci] + 2] : -1; }
  static constexpr int slot_of_load(int ci) { return kSlot[ci]; }
  // the row max is made after the chunks
  static constexpr int max_part(int) { return -1; }
};

// Up to 12 waves per workgroup, 3 per SIMD: at most 168 registers per wave.
// I8: an int8 pool (codes and per-token fp32 scales), converted to bf16 in LDS (see the staging
// notes below).
template <int D, bool I8>
__global__ __launch_bounds__(768) __attribute__((amdgpu_waves_per_eu(3)))
void attn_prefill_mfma_kernel(AttnArgs a) {
  constexpr int KS = D / 16;          // 16-dim k-steps of the score product
  constexpr int MB = D / 32;          // 32-dim blocks of the output
  constexpr int TE = 16 * D;          // elements of one pool tile (K or V)
  constexpr int TQ = TE * (I8 ? 1 : 2) / 1024;  // 1 KiB DMA pieces per pool tile
  constexpr int IDS = 1024;           // block ids of pool tiles held in LDS
  // One array per LDS stage ([K0..K3, V0..V3] each): with every access naming its array, the
  // compiler can tell the stage being computed from the ones the DMA is filling, and does not
  // wait for those loads before reading.  bf16 pools: four bf16 stages.  int8 pools: three bf16
  // stages plus three int8 stages (the codes of a 64-key tile and the 16 scales of each of its
  // pool tiles, four times over: 64 floats); 154 KiB at D = 128.
  __shared__ __attribute__((aligned(16))) uint16_t lds0[8][TE];
  __shared__ __attribute__((aligned(16))) uint16_t lds1[8][TE];
  __shared__ __attribute__((aligned(16))) uint16_t lds2[8][TE];
  __shared__ __attribute__((aligned(16))) uint16_t lds3[I8 ? 1 : 8][I8 ? 8 : TE];
  __shared__ __attribute__((aligned(16))) uint8_t q8a[I8 ? 8 : 1][I8 ? TE : 16];
  __shared__ __attribute__((aligned(16))) uint8_t q8b[I8 ? 8 : 1][I8 ? TE : 16];
  __shared__ __attribute__((aligned(16))) uint8_t q8c[I8 ? 8 : 1][I8 ? TE : 16];
  __shared__ __attribute__((aligned(16))) float sca[I8 ? 8 : 1][64];
  __shared__ __attribute__((aligned(16))) float scb[I8 ? 8 : 1][64];
  __shared__ __attribute__((aligned(16))) float scc[I8 ? 8 : 1][64];
  __shared__ __attribute__((aligned(16))) int s_ids[IDS];

  const int W = blockDim.x >> 6;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, h = lane >> 5;  // MFMA column (query row of the wave) and half
  // The grid may exceed the workgroups there are (the host sized it from bounds); the ones
  // there are get ids [0, n) and are remapped over the XCDs, the rest leave at once.
  // R row blocks per workgroup, W/2 <= R <= W: the first F = 2R - W waves own one block each,
  // the other W - F waves pair up on the remaining blocks, the two waves of a pair taking the
  // even and the odd 32-key blocks (merged at the end).  Waves w, w+4, w+8 share a SIMD, so
  // with W = 12 and R = 10 every SIMD carries 2.5 blocks.
  const int R = a.pf_rblk;
  const int F = 2 * R - W;
  const bool half = wave >= F;
  const int rb = half ? F + ((wave - F) >> 1) : wave;  // the wave's row block in the workgroup
  const int par = half ? ((wave - F) & 1) : 0;          // half waves: parity of their blocks
  const int NKR = a.pf_ksplit;  // key ranges per row tile
  // The workgroup's key range kj, sequence s, KV head, row tile rt (of rts), first query row and
  // lengths.  logical = key range * n_base + row tile (n_base: row tiles of every (sequence, KV
  // head)): the row tiles of one key range of a (sequence, KV head) stay next to each other, on
  // one XCD.  (Wave-uniform values from divisions come out of vector registers: readfirstlane
  // keeps them in scalar ones, as the register budget of three waves per SIMD needs.)
  int kj, s, kvh, rt, rts, q_start, L, T;
  if (a.num_seqs <= WAVE) {
    // one read of the metadata (a sequence per lane) serves the count, the lookup and the
    // lengths: no dependent re-reads before the block ids
    int Lj = 0, Tj = 0, r = 0, q = 0;
    if (lane < a.num_seqs) {
      seq_lens(a, lane, Lj, Tj);
      r = seq_row_tiles(a, Tj, R);
      q = max(0, a.q_lens[lane]);
    }
    const int wg = r * a.num_kv_heads;
    const int win = wave_incl_scan(wg);
    const int qin = wave_incl_scan(q);
    const int n_base = __builtin_amdgcn_readlane(win, WAVE - 1);
    const int n_wg = n_base * NKR;
    if ((int)blockIdx.x >= n_wg) return;
    const int logical = xcd_logical(blockIdx.x, n_wg);
    kj = __builtin_amdgcn_readfirstlane(logical / n_base);
    const int nn = logical - kj * n_base;
    const int k = __builtin_popcountll(__builtin_amdgcn_ballot_w64(win <= nn));
    s = k;
    rts = __builtin_amdgcn_readlane(r, k);
    const int within = nn - (__builtin_amdgcn_readlane(win, k) - __builtin_amdgcn_readlane(wg, k));
    kvh = __builtin_amdgcn_readfirstlane(within / rts);
    rt = within - kvh * rts;
    q_start = __builtin_amdgcn_readlane(qin, k) - __builtin_amdgcn_readlane(q, k);
    L = __builtin_amdgcn_readlane(Lj, k);
    T = __builtin_amdgcn_readlane(Tj, k);
  } else {
    const int n_base = prefill_wg_total(a, R);
    const int n_wg = n_base * NKR;
    if ((int)blockIdx.x >= n_wg) return;
    const int logical = xcd_logical(blockIdx.x, n_wg);
    kj = __builtin_amdgcn_readfirstlane(logical / n_base);
    find_prefill_tile(a, logical - kj * n_base, R, s, kvh, rt, rts, q_start);
    seq_lens(a, s, L, T);
  }
  // wave-uniform: kept in scalar registers so the per-block edge tests stay on the SALU
  L = __builtin_amdgcn_readfirstlane(L);
  T = __builtin_amdgcn_readfirstlane(T);
  const int G = a.group;
  const int rows = T * G;
  // Row blocks of 32 rows are dealt to the workgroups of a (sequence, KV head) strided: row
  // block k of row tile rt is block rt + rts * k of the pair.  Every workgroup then holds early
  // and late rows alike, so under the causal mask all of them carry about the same work.
  const int nblk = (rows + 31) >> 5;
  if (rt >= nblk) return;
  const int last_blk = rt + rts * min(R - 1, (nblk - 1 - rt) / rts);
  const int ke = __builtin_amdgcn_readfirstlane(
      min(L, L - T + (min(32 * last_blk + 32, rows) - 1) / G + 1));  // keys the WG needs
  const int ntiles = (ke + 63) >> 6;
  const int npt = (ke + 15) >> 4;  // pool tiles the WG reads
  // This workgroup's 64-key tiles [jt0, jt1): key range kj of the sequence's tiles (the same cut
  // for every row tile), within the tiles the workgroup needs.  An empty range still stores
  // (empty) partials for its rows.
  const int tpk = __builtin_amdgcn_readfirstlane((((L + 63) >> 6) + NKR - 1) / NKR);
  const int jt0 = __builtin_amdgcn_readfirstlane(min(kj * tpk, ntiles));
  const int jt1 = __builtin_amdgcn_readfirstlane(min(jt0 + tpk, ntiles));
  const int rw0 = 32 * (rt + rts * rb);
  // the wave's keys end at the last key its rows see, and at the range's end
  const int kew = __builtin_amdgcn_readfirstlane(
      rw0 < rows ? min(64 * jt1, min(L, L - T + (min(rw0 + 32, rows) - 1) / G + 1)) : 0);
  const int pw0 = __builtin_amdgcn_readfirstlane(L - T + rw0 / G);  // keys <= pw0: visible to every row of the wave

  const int32_t* tbl = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  const char* kbase = reinterpret_cast<const char*>(a.k_layer);
  const char* vbase = reinterpret_cast<const char*>(a.v_layer);
  const int bmask = a.block_size - 1;

  // Block ids of pool tiles [ids0, ids0 + IDS) of this sequence, in LDS.
  auto load_ids = [&](int base) {
    for (int i = tid; i < IDS; i += blockDim.x) {
      const int pt = min(base + i, npt - 1);
      s_ids[i] = tbl[(pt << 4) >> a.block_shift];
    }
  };
  // Fetches are clamped into [jb, jlast] (for an empty range: its base tile, never computed).
  const int jb = __builtin_amdgcn_readfirstlane(min(jt0, ntiles - 1));
  const int jlast = __builtin_amdgcn_readfirstlane(max(min(jt1, ntiles) - 1, jb));
  int ids0 = 4 * jb;

  // Q^T operands: the B operand of k-step k, lane (col, h) holding dims 16k + 8h .. +8 of the
  // wave's row col.  Its loads go out right behind the first block-id loads (the ids are
  // written to LDS only after both are in flight), so reading the workgroup's Q overlaps the id
  // round trip.
  const int Hq = a.num_q_heads;
  const int r = rw0 + col;
  const int qi = r / G;
  const bool valid = r < rows && q_start + qi < a.total_q;
  const int prow = valid ? L - T + qi : -1;  // the row's position (keys <= prow are visible)
  // the row's index in q / out (recomputed for the store rather than held through the loop)
  auto row_index = [&]() -> size_t { return valid ? (size_t)(q_start + qi) * Hq + kvh * G + r % G : 0; };
  bf16x8 qb[KS];
  {
    constexpr int IDU = IDS / 256;  // ids per thread at most (at least 4 waves)
    int idv[IDU];
    // (loads unconditional, indices clamped, so that the waits before the LDS writes can count
    // them: slot i >= IDS re-reads slot IDS - 1, an invalid row reads row 0 and drops it)
#pragma unroll
    for (int u = 0; u < IDU; ++u) {
      const int i = min(tid + u * (int)blockDim.x, IDS - 1);
      idv[u] = tbl[(min(ids0 + i, npt - 1) << 4) >> a.block_shift];
    }
    const size_t rh = row_index();
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + rh * D + 8 * h;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      const u32x4 v = *reinterpret_cast<const u32x4*>(qp + 16 * k);
      qb[k] = __builtin_bit_cast(bf16x8, valid ? v : z);
    }
#pragma unroll
    for (int u = 0; u < IDU; ++u) {
      const int i = tid + u * (int)blockDim.x;
      if (i < IDS) s_ids[i] = idv[u];
    }
  }
  // the id writes are done before the barrier publishes them (no fence: the Q loads stay in
  // flight)
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  barrier_no_fence();

  // ---- K/V staging: the 8 pool tiles of a stage ([K0..K3, V0..V3] of a 64-key tile) are dealt
  // round-robin to the issuing waves, each streamed straight into LDS (global_load_lds: lane
  // l's 16 bytes land at base + 16*l).  Pool tiles past the context re-read the last one;
  // those keys are masked and their V zeroed.
  // The 4 block ids a stage needs (pool tiles 4j .. 4j+3, already clamped in the cache) are
  // read from the cache with one ds_read_b128 just before the issue (by the issuing waves only)
  // and moved to scalar registers, where the addresses are computed; holding them in vector
  // registers across a step would cost registers the compute loop needs.
  typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
  // The DMA issue goes to the waves with slack: with four or more half waves beside whole-block
  // waves, to waves 0-3, the oldest wave of each SIMD (the issue arbiter favours the oldest
  // wave, so these reach each tile's barrier first and wait there longest; the half waves, the
  // youngest, come last), else to the waves of the least loaded SIMDs (waves are placed on the 4
  // SIMDs round-robin, so with W % 4 != 0 the SIMDs holding wave indices >= W % 4 mod 4 carry
  // one wave less).  Fewer than 4 such waves would make the issue itself the bottleneck: then
  // all waves issue.
  const int wrem = W & 3;
  const bool by_half = F > 0 && W - F >= 4;
  const bool split = !by_half && wrem != 0 && (W >> 2) * (4 - wrem) >= 4;
  const int nissue = by_half ? 4 : split ? (W >> 2) * (4 - wrem) : W;  // waves that issue DMA
  const int issue_rank = by_half ? (wave < 4 ? wave : -1)
                         : !split ? wave
                         : (wave & 3) >= wrem ? (wave >> 2) * (4 - wrem) + (wave & 3) - wrem : -1;
  const uint32_t lane_off = 16u * lane;
  // pool tiles a wave streams per 64-key tile (at most 2: nissue >= 4), and its DMA
  // instructions per 64-key tile (int8: one more per pool tile, for its scales)
  const int my_slots = issue_rank < 0 ? 0 : (8 - issue_rank + nissue - 1) / nissue;
  const int my_pieces = my_slots * (TQ + (I8 ? 1 : 0));
  auto read_ids = [&](int j) -> i32x4 { return *reinterpret_cast<const i32x4*>(&s_ids[4 * j - ids0]); };
  // int8 staging, per lane: byte offset of its scale (token lane % 16) in a pool tile's 16
  // scales (the DMA offset of the scale loads)
  const uint32_t sc_off = 4u * (lane & 15);
  // Tile j into `stage` (bf16: a bf16 stage; int8: an int8 stage, the scales of pool tile slot s
  // into scales[s]).
  auto fetch = [&](int j, const i32x4& ids, auto&& stage, auto&& scales) {
    if (issue_rank < 0) return;  // wave-uniform
    int blk[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) blk[t] = __builtin_amdgcn_readfirstlane(ids[t]);
    for (int slot = issue_rank; slot >= 0 && slot < 8; slot += nissue) {  // 0..3: K, 4..7: V
      const int t = slot & 3;
      const int pt = min(4 * j + t, npt - 1);
      const int b = t == 0 ? blk[0] : t == 1 ? blk[1] : t == 2 ? blk[2] : blk[3];
      const size_t off = block_tile_offset(b, ((pt << 4) & bmask) >> 4, kvh, a.block_shift,
                                           a.num_blocks, a.num_kv_heads, D);  // elements
      dma_tile<TQ>((slot < 4 ? kbase : vbase) + off * (I8 ? 1 : 2), lane_off, lds_address(stage[slot]));
      if constexpr (I8)
        dma_dwords((slot < 4 ? a.k_scale_layer : a.v_scale_layer) + off / D, sc_off,
                   lds_address(&scales[slot][0]));
    }
  };
  // int8 pools: 64-key tile jf from an int8 stage (published by a barrier) into the bf16 stage
  // st.  Each value is code * scale rounded once to the nearest-even bf16 (computed as
  // fma(code + 128, s, -128 s): the exact product, rounded once, as the fp32 product), and keys
  // at or past the context get scale 0, so their K and V are exactly 0 (whatever the pool holds
  // there).  The tile is cut into units of 16 codes per lane (K: the 16-byte rows lane + 64 m of
  // a pool tile; V: token group pair m of a pool tile, D = 128; at D = 64 a pool tile is one
  // unit), dealt round-robin to the waves, the half waves first (they carry half the matrix
  // work), so that the conversion's vector work is spread over every SIMD and wave.  Per-lane
  // offsets are derived from a lane id read afresh (volatile: not hoisted out of the tile loop),
  // so they hold no registers through the rest of the step.
  //   K [d/16][t][d%16] -> [d/8][t][d%8]: lane takes row lane + 64 m (token lane % 16, dims
  //     16 (lane / 16 + 4 m) ..).
  //   V [t/4][d%16][d/16][t%4] -> [d][t]: lane (dlo = lane % 16, r = lane / 16) takes dims
  //     16 (dh0 + kk) + dlo, kk < 4, for the 4 tokens of group tg0 + m.
  constexpr int UPS = D / 64;  // units per pool tile
  const int conv_rank = half ? wave - F : (W - F) + wave;  // the waves' order for the deal
  auto convert = [&](int jf, auto&& qs, auto&& scs, uint16_t (&st)[8][TE]) {
    if constexpr (I8) {
      uint32_t ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      const uint32_t lsc = 4u * (ln & 15);
      const int v_tg0 = D == 128 ? 2 * (int)(ln >> 5) : (int)(ln >> 4);
      const int v_dh0 = D == 128 ? 4 * (int)((ln >> 4) & 1) : 0;
      const uint32_t k_src = 16u * ln;
      const uint32_t k_dst = 512u * (ln >> 4) + 16u * (ln & 15);
      const uint32_t v_src = (uint32_t)(((v_tg0 * 16 + (int)(ln & 15)) * (D / 16) + v_dh0) * 4);
      const uint32_t v_dst = (uint32_t)(((16 * v_dh0 + (int)(ln & 15)) * 16 + 4 * v_tg0) * 2);
      for (int u = conv_rank; u < 8 * UPS; u += W) {  // wave-uniform
        const int slot = u / UPS, m = u % UPS;
        const char* src = reinterpret_cast<const char*>(qs[slot]);
        const char* scl = reinterpret_cast<const char*>(scs[slot]);
        char* dst = reinterpret_cast<char*>(st[slot]);
        const int rem = L - (64 * jf + 16 * (slot & 3));  // keys of the pool tile in the context
        if (slot < 4) {
          const float sv = (int)(ln & 15) < rem ? *reinterpret_cast<const float*>(scl + lsc) : 0.f;
          const float nb = -128.f * sv;
          const u32x4 w = *reinterpret_cast<const u32x4*>(src + k_src + 1024 * m);
          uint32_t r[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t x = w[e] ^ 0x80808080u;  // code + 128 in each byte
            r[2 * e] = cvt_pk_bf16(__builtin_fmaf((float)(x & 0xffu), sv, nb),
                                   __builtin_fmaf((float)((x >> 8) & 0xffu), sv, nb));
            r[2 * e + 1] = cvt_pk_bf16(__builtin_fmaf((float)((x >> 16) & 0xffu), sv, nb),
                                       __builtin_fmaf((float)(x >> 24), sv, nb));
          }
          // chunks 2c and 2c + 1 of the token (c = lane / 16 + 4 m): 16 tokens * 16 bytes apart
          *reinterpret_cast<u32x4*>(dst + k_dst + 2048 * m) = u32x4{r[0], r[1], r[2], r[3]};
          *reinterpret_cast<u32x4*>(dst + k_dst + 2048 * m + 256) = u32x4{r[4], r[5], r[6], r[7]};
        } else {
          const int tg = v_tg0 + m;
          const u32x4 x = *reinterpret_cast<const u32x4*>(src + v_src + m * 16 * D / 4);
          const floatx4 s4 = *reinterpret_cast<const floatx4*>(scl + 16 * tg);
          float sv[4], nb[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            sv[e] = 4 * tg + e < rem ? s4[e] : 0.f;
            nb[e] = -128.f * sv[e];
          }
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const uint32_t xx = x[kk] ^ 0x80808080u;
            const uint32_t r0 = cvt_pk_bf16(__builtin_fmaf((float)(xx & 0xffu), sv[0], nb[0]),
                                            __builtin_fmaf((float)((xx >> 8) & 0xffu), sv[1], nb[1]));
            const uint32_t r1 = cvt_pk_bf16(__builtin_fmaf((float)((xx >> 16) & 0xffu), sv[2], nb[2]),
                                            __builtin_fmaf((float)(xx >> 24), sv[3], nb[3]));
            // dim 16 (dh0 + kk) + dlo: 16 dims * 32 bytes apart; token group m: 8 bytes
            *reinterpret_cast<u32x2*>(dst + v_dst + 512 * kk + 8 * m) = u32x2{r0, r1};
          }
        }
      }
    }
  };
  // Three tiles in flight from the start (clamped: a short context re-reads its last tile, so
  // every wave's count of outstanding pieces follows the same pattern); int8 pools: a fourth
  // goes into the first int8 stage once its codes are converted.
  if constexpr (I8) {
    fetch(jb, read_ids(jb), q8a, sca);
    fetch(min(jt0 + 1, jlast), read_ids(min(jt0 + 1, jlast)), q8b, scb);
    fetch(min(jt0 + 2, jlast), read_ids(min(jt0 + 2, jlast)), q8c, scc);
  } else {
    fetch(jb, read_ids(jb), lds0, sca);
    fetch(min(jt0 + 1, jlast), read_ids(min(jt0 + 1, jlast)), lds1, sca);
    fetch(min(jt0 + 2, jlast), read_ids(min(jt0 + 2, jlast)), lds2, sca);
  }

  // ---- per-row state (Q^T was loaded with the first block ids, above) ----------------------
  // msub: the running row max times c, in exp2 units (the same in both lanes of a row; -inf
  // until the row's first key); l_lane: this lane's share of the row sum; o: O^T, element e of
  // block mb = dim 32mb + 8(e/4) + 4h + e%4.
  float msub = -INFINITY, l_lane = 0.f;
  floatx16 o[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[mb][e] = 0.f;
  const float c = a.scale_log2;

  // Key order of the score product: MFMA row m of a 32-key block reads key swap23(m), so that
  // output element e of lane (col, h) is key 16(e/8) + 8h + e%8 of the block.
  const int kq = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);
  // K: chunk h (dims 8h .. +8 of k-step 0) of the key's token; k-step k adds 2k chunks.
  const uint32_t k_lane = (uint32_t)(((kq >> 4) * TE + (h * 16 + (kq & 15)) * 8) * 2);  // bytes
  // V^T: dim col of the 32-dim block, tokens 8h .. +8 of the k-step's pool tile.
  const uint32_t v_lane = (uint32_t)((col * 16 + 8 * h) * 2);  // bytes

  if constexpr (I8) {
    // Tiles 0-2 (and Q) have landed and are published; tiles 0 and 1 are converted by every
    // wave and published, then tile 3 streams into the first int8 stage (read by then).
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    barrier_no_fence();
    convert(jb, q8a, sca, lds0);
    convert(min(jt0 + 1, jlast), q8b, scb, lds1);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    barrier_no_fence();
    fetch(min(jt0 + 3, jlast), read_ids(min(jt0 + 3, jlast)), q8a, sca);
  } else {
    // Tiles 0 and 1 must have landed (at most this wave's pieces of tile 2 outstanding).
    wait_vmcnt(my_pieces);
    __syncthreads();
  }

  // V slots of keys at or past the context (only in the last 64-key tile) may hold anything,
  // NaN included, and p = 0 times NaN is NaN: once that tile has landed, the workgroup zeroes
  // them in LDS and meets at one more barrier before anyone reads it.
  auto zero_tail = [&](uint16_t (&stage)[8][TE], int jt) {
    if (jt != ntiles - 1 || 64 * ntiles <= L) return;  // workgroup-uniform
    for (int i = tid; i < 4 * D; i += blockDim.x) {
      const int t = i / D, d = i % D;  // V pool tile t of the stage, dim d: 16 tokens
      uint16_t* row = &stage[4 + t][d * 16];
      const int k0 = 64 * jt + 16 * t;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (k0 + u >= L) row[u] = 0;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this thread's LDS writes are done
    barrier_no_fence();
  };
  if constexpr (!I8) {  // (int8 pools: the conversion zeroes them)
    zero_tail(lds0, jt0);
    zero_tail(lds1, jt0 + 1);
  }

  // Attention of this wave's 32 rows against one 32-key block (pool tiles 2b, 2b+1 of the
  // stage).  `edge`: the block reaches past the wave's first row (causal diagonal) or past the
  // context, so its scores are masked.
  // The three phases of a 32-key block (pool tiles 2b, 2b+1 of the stage).
  auto qk = [&](const uint16_t (&stage)[8][TE], int b) -> floatx16 {
    const char* kt = reinterpret_cast<const char*>(stage[2 * b]) + k_lane;
    floatx16 sc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sc[e] = 0.f;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      // chunk 2k + h of the key's pool tile
      const bf16x8 ka = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kt + k * 2 * 16 * 16));
      sc = mfma32(ka, qb[k], sc);
    }
    return sc;
  };
  // The row's max over a block's scores, in three parts that can go into separate chunks: the
  // lane's scores 0-6, then 7-12, then 13-15 and the other half of the row (lanes l and l ^ 32
  // hold the same row).  IEEE maximum (no NaN quieting needed: a masked score is -inf).
  auto max_part = [&](const floatx16& sc, float& cm, int part) {
    auto mx3 = [](float x, float y, float z) {
      return __builtin_elementwise_maximum(__builtin_elementwise_maximum(x, y), z);
    };
    if (part == 0) {
      cm = mx3(sc[0], sc[1], sc[2]);
      cm = mx3(cm, sc[3], sc[4]);
      cm = mx3(cm, sc[5], sc[6]);
    } else if (part == 1) {
      cm = mx3(cm, sc[7], sc[8]);
      cm = mx3(cm, sc[9], sc[10]);
      cm = mx3(cm, sc[11], sc[12]);
    } else {
      cm = mx3(cm, sc[13], sc[14]);
      cm = __builtin_elementwise_maximum(cm, sc[15]);
      float x, y;
      swap32(cm, x, y);
      cm = __builtin_elementwise_maximum(x, y);
    }
  };
  // Masks the scores of an edge block (past the wave's first row on the causal diagonal, or past
  // the context), then raises the running max where a row's max grew by more than 2^8 in exp2
  // units (lazy: P stays <= 256 and the rescale is rare).  `cmax`: the row's max over the
  // unmasked scores when `have` (made beside the matrix work); an edge block makes it afresh.
  auto row_max = [&](floatx16& sc, int kb, bool edge, float cmax, bool have) {
    if (edge) {
      // keys of this lane: kb + 16 (e / 8) + 8 h' + e % 8 (h' recomputed from the lane id here
      // rather than held in a register through the loop)
      uint32_t ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      const int hh = (int)((ln >> 5) & 1);
      const int lim = min(prow, L - 1) - kb - 8 * hh;  // e is visible iff 16 (e / 8) + e % 8 <= lim
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (16 * (e >> 3) + (e & 7) > lim) sc[e] = -INFINITY;
      have = false;
    }
    if (!have) {
      max_part(sc, cmax, 0);
      max_part(sc, cmax, 1);
      max_part(sc, cmax, 2);
    }
    // true on a row's first key (msub = -inf); false for a row with no key yet (NaN)
    const float cm = cmax * c;
    const bool grow = cm - msub > 8.f;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? cm : msub;
      const float alpha = grow ? fast_exp2(msub - m_new) : 1.f;  // 0 on the first key
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) o[mb] *= alpha;
      l_lane *= alpha;
      msub = m_new;
    }
  };
  // Software pipeline over the wave's 32-key blocks: finishing block b (softmax, P.V) goes with
  // the score product of block b+1, so each wave always has matrix work in flight beside its
  // softmax and the waves of a SIMD need not take turns.  sc holds the scores of the block being
  // finished.  Edge blocks (past the wave's first row or the context) take the masked path.
  // Issue order of one finish, chunk by chunk (see PfSched).
  using Sched = PfSched<D>;
  // finish(blk, cur, nst, stride, sc, sn): block blk of stage `cur` (its scores in sc, already
  // masked, with the running max raised for them), with the score product of the wave's next
  // block blk + stride (1 for a whole-block wave, 2 for a half wave) from `nst` into sn; then
  // that next block's mask and row max, issued behind the last P.V MFMAs so that they overlap.
  auto finish = [&](int blk, const uint16_t (&cur)[8][TE], const uint16_t (&nst)[8][TE], int stride,
                    const floatx16& sc, floatx16& sn) {
    const int kb = 32 * blk;
    if (kb >= kew) return;  // wave-uniform
    // A row without a visible key yet (possible in a half wave: its first block may lie wholly
    // past the row's position) keeps msub = -inf; subtract 0 for it, so that its masked scores
    // give p = 0 rather than exp2(-inf + inf) = NaN.
    const float nms = msub > -INFINITY ? -msub : 0.f;
    // operands: K of the next block (in the same stage or the next one; past the wave's keys
    // its scores are never used), V^T of block blk
    const char* kt = reinterpret_cast<const char*>(nst[2 * ((blk + stride) & 1)]) + k_lane;
    const char* vt0 = reinterpret_cast<const char*>(cur[4 + 2 * (blk & 1)]) + v_lane;
    const char* vt1 = reinterpret_cast<const char*>(cur[5 + 2 * (blk & 1)]) + v_lane;
    auto load_op = [&](int u) -> u32x4 {
      if (u < KS) return *reinterpret_cast<const u32x4*>(kt + u * 2 * 16 * 16);  // chunk 2u + h
      const int j = (u - KS) / MB, mb = (u - KS) % MB;
      return *reinterpret_cast<const u32x4*>((j ? vt1 : vt0) + mb * 32 * 16 * 2);
    };
    u32x4 ops[Sched::N];
    ops[0] = load_op(Sched::op(0));
    ops[1] = load_op(Sched::op(1));
#pragma unroll
    for (int e = 0; e < 16; ++e) sn[e] = 0.f;
    uint32_t pk[8];
    float cmax_n = 0.f;  // the next block's row max (unmasked), made in the last chunks
    float e0 = 0.f, e1 = 0.f;  // exp2 results waiting for their pack stage
    __builtin_amdgcn_sched_barrier(0);
    // Chunks pinned in place: at most one MFMA, the operand load two MFMAs ahead, and at most one
    // exp2 pair of the softmax (the two scores' exp2, their bf16 pack and row sum), spread so
    // that the VALU work stays under the matrix core's.
#pragma unroll
    for (int ci = 0; ci < Sched::N; ++ci) {
      const int u = Sched::op(ci);
      if (u >= 0) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, ops[Sched::slot(ci)]);
        if (u < KS) {
          sn = mfma32(av, qb[u], sn);
        } else {
          const int j = (u - KS) / MB, mb = (u - KS) % MB;
          const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[4 * j], pk[4 * j + 1], pk[4 * j + 2], pk[4 * j + 3]});
          o[mb] = mfma32(av, pb, o[mb]);
        }
        const int nx = Sched::next_load(ci);
        if (nx >= 0) ops[Sched::slot_of_load(nx)] = load_op(Sched::op(nx));
      }
      const int mp = Sched::max_part(ci);
      if (mp >= 0) max_part(sn, cmax_n, mp);
      const int ep = Sched::exp_pair(ci), pp = Sched::pack_pair(ci);
      float p0 = 0.f, p1 = 0.f;
      if (ep >= 0) {
        p0 = fast_exp2(__builtin_fmaf(sc[2 * ep], c, nms));
        p1 = fast_exp2(__builtin_fmaf(sc[2 * ep + 1], c, nms));
      }
      if (pp >= 0) {
        // the pair's exp2 results: this chunk's, or the ones an earlier chunk left in e0, e1
        const float x0 = pp == ep ? p0 : e0, x1 = pp == ep ? p1 : e1;
        pk[pp] = cvt_pk_bf16(x0, x1);
        // row sum of the fp32 values (plain adds: the bf16 dot2 would take matrix-pipe slots)
        l_lane += x0 + x1;
      }
      if (ep >= 0 && pp != ep) {
        e0 = p0;
        e1 = p1;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const int kn = 32 * (blk + stride);
    if (kn < kew) row_max(sn, kn, kn + 31 > pw0 || kn + 32 > L, cmax_n, Sched::max_part(Sched::N - 1) >= 0);  // wave-uniform
  };
  // the wave's first block: the range's first, or its second for an odd half wave; whole-block
  // waves alternate their scores between sa and sb, half waves keep theirs in sa
  floatx16 sa, sb;
#pragma unroll
  for (int e = 0; e < 16; ++e) sa[e] = sb[e] = 0.f;
  if (kew > 64 * jt0 + 32 * par) {
    sa = qk(lds0, par);
    const int k0 = 64 * jt0 + 32 * par;
    row_max(sa, k0, k0 + 31 > pw0 || k0 + 32 > L, 0.f, false);
  }

  // One 64-key tile j (stage `cur`).  bf16: tile j+3 starts streaming into `fst` (the fourth
  // stage, free since its last reader, tile j-1, was done before the barrier that ended the
  // previous step); the blocks of tile j are finished, their successors' score products reading
  // `nxt1` (published a step ago); then tile j+2 (issued a step ago, in `nxt2`) is waited for
  // and published.  int8: tile j+4 starts streaming into `fst` (the int8 stage of tile j+1,
  // converted in the previous step); every wave converts its units of tile j+2 (its codes
  // published by the barrier that ended the previous step) from `cst` into `nxt2` (last read as
  // tile j-1); the blocks of tile j are finished as above; then the codes of tile j+3 (issued a
  // step ago) are waited for, and the barrier publishes them with the bf16 tile j+2.
  auto step = [&](int j, uint16_t (&cur)[8][TE], uint16_t (&nxt1)[8][TE], uint16_t (&nxt2)[8][TE],
                  auto&& fst, auto&& fsc, auto&& cst, auto&& csc) {
    // the ids of tile j+3; refill the id cache first when they lie past it (rare: only past
    // 16K keys; workgroup-uniform)
    const int jf = min(j + (I8 ? 4 : 3), jlast);
    if (4 * jf + 3 - ids0 >= IDS) {
      __syncthreads();
      ids0 = 4 * jf;
      load_ids(ids0);
      __syncthreads();
    }
    fetch(jf, read_ids(jf), fst, fsc);
    if constexpr (I8) convert(min(j + 2, jlast), cst, csc, nxt2);
    // whole-block waves: blocks 2j and 2j+1; half waves: block 2j + parity, then the same parity
    // in tile j+1 (wave-uniform)
    if (!half) {
      finish(2 * j, cur, cur, 1, sa, sb);
      sa = sb;
    }
    finish(2 * j + (half ? par : 1), cur, nxt1, half ? 2 : 1, sa, sb);
    sa = sb;
    if constexpr (I8) {
      // tile j+3's codes have landed once at most this wave's pieces of tile j+4 are
      // outstanding; the conversion's writes are done (lgkmcnt(0))
      wait_vmcnt(my_pieces);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      barrier_no_fence();
    } else {
      // tile j+2 has landed once at most this wave's pieces of tile j+3 are outstanding; every
      // wave's share of it is visible after the barrier
      wait_vmcnt(my_pieces);
      barrier_no_fence();
      zero_tail(nxt2, j + 2);
    }
  };
  if constexpr (I8) {
    // three bf16 and three int8 stages: the pattern repeats every 3 tiles
    for (int j = jt0; j < jt1; j += 3) {
      step(j, lds0, lds1, lds2, q8b, scb, q8c, scc);
      if (j + 1 < jt1) step(j + 1, lds1, lds2, lds0, q8c, scc, q8a, sca);
      if (j + 2 < jt1) step(j + 2, lds2, lds0, lds1, q8a, sca, q8b, scb);
    }
  } else {
    for (int j = jt0; j < jt1; j += 4) {
      step(j, lds0, lds1, lds2, lds3, sca, sca, sca);
      if (j + 1 < jt1) step(j + 1, lds1, lds2, lds3, lds0, sca, sca, sca);
      if (j + 2 < jt1) step(j + 2, lds2, lds3, lds0, lds1, sca, sca, sca);
      if (j + 3 < jt1) step(j + 3, lds3, lds0, lds1, lds2, sca, sca, sca);
    }
  }
  // The last steps re-read the last tile into free stages: drain those loads before the stages
  // are reused below or the workgroup's LDS is released.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // ---- half pairs: the odd wave hands its (max, sum, O^T) to the even one through LDS --------
  if (F < W) {  // workgroup-uniform
    // every wave is done with the stages (the last step ended on a barrier); pair p uses half
    // of stage array p / 2 for O^T (64 x 16 MB floats) and s_ids for (max, sum)
    constexpr int OF = 16 * MB;  // O^T floats per lane
    const int pair = half ? (wave - F) >> 1 : 0;
    uint16_t(*st)[TE] = (pair >> 1) == 0 ? lds0 : (pair >> 1) == 1 ? lds1 : lds2;
    float* ob = reinterpret_cast<float*>(&st[0][0]) + (pair & 1) * 64 * OF;
    float* ml = reinterpret_cast<float*>(s_ids) + pair * 128;
    if (half && par == 1) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) ob[(16 * mb + e) * 64 + lane] = o[mb][e];
      ml[lane] = msub;
      ml[64 + lane] = l_lane;
    }
    __syncthreads();
    if (half && par == 0) {
      const float m1 = ml[lane], l1 = ml[64 + lane];
      const float mm = __builtin_elementwise_maximum(msub, m1);
      // a wave with no key of the row (msub or m1 = -inf, its o and l 0) weighs 0; under key
      // ranges neither wave may have one (mm = -inf: the row's partial stays empty)
      const float a0 = msub == -INFINITY ? 0.f : fast_exp2(msub - mm);
      const float a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - mm);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[mb][e] = o[mb][e] * a0 + ob[(16 * mb + e) * 64 + lane] * a1;
      l_lane = l_lane * a0 + l1 * a1;
      msub = mm;
    }
  }

  // ---- normalise and store: lane (col, h) holds dims 32mb + 8q + 4h .. +4 of its row --------
  {
    float x, y;
    swap32(l_lane, x, y);
    const float lrow = x + y;
    if (NKR > 1) {
      // key range kj of a split row tile: the row's unnormalised partial, relative to its max
      // (exp2 units; -inf when the range holds none of the row's keys)
      if (valid && !(half && par == 1)) {
        const size_t slot = row_index() * NKR + kj;
        float* po = a.pf_part_o + slot * D + 4 * h;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<floatx4*>(po + 32 * mb + 8 * q) =
                floatx4{o[mb][4 * q], o[mb][4 * q + 1], o[mb][4 * q + 2], o[mb][4 * q + 3]};
        if (h == 0) *reinterpret_cast<float2*>(a.pf_part_ml + 2 * slot) = make_float2(msub, lrow);
      }
    } else if (valid && !(half && par == 1)) {  // a half pair's even wave stores the merged rows
      const float inv = 1.f / lrow;
      uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + row_index() * D + 4 * h;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w0 = f32_to_bf16_bits(o[mb][4 * q] * inv) | (f32_to_bf16_bits(o[mb][4 * q + 1] * inv) << 16);
          const uint32_t w1 = f32_to_bf16_bits(o[mb][4 * q + 2] * inv) | (f32_to_bf16_bits(o[mb][4 * q + 3] * inv) << 16);
          *reinterpret_cast<uint2*>(op + 32 * mb + 8 * q) = make_uint2(w0, w1);
        }
      }
    }
  }
}

long long prefill_wg_count(const int* rows, int n, int num_kv_heads, int rblk) {
  long long wgs = 0;
  for (int i = 0; i < n; ++i) {
    const long long nblk = ((long long)rows[i] + 31) / 32;
    wgs += (nblk + rblk - 1) / rblk * num_kv_heads;
  }
  return wgs;
}

namespace {

// Per 64-key tile cost of a workgroup of `w` waves over `r` row blocks, relative: waves w, w+4,
// w+8 share a SIMD, a whole-block wave counts 1 and a half wave 1/2, and the tile time is a
// fixed part plus the load of the busiest SIMD (measured on MI355X: about 1.0 + 0.45 x load
// microseconds per 64-key tile); a busiest SIMD with a single wave cannot hide its own
// latencies (measured 25-30% slower).
double prefill_tile_cost(int w, int r) {
  const int f = 2 * r - w;
  double load[4] = {0, 0, 0, 0};
  int nw[4] = {0, 0, 0, 0};
  for (int i = 0; i < w; ++i) {
    load[i & 3] += i < f ? 1.0 : 0.5;
    ++nw[i & 3];
  }
  int bs = 0;
  for (int k = 1; k < 4; ++k)
    if (load[k] > load[bs] || (load[k] == load[bs] && nw[k] < nw[bs])) bs = k;
  return (1.0 + 0.45 * load[bs]) * (nw[bs] <= 1 ? 1.3 : 1.0);
}

// Makespan of wgs workgroups cut into k key ranges each, over n 64-key tiles: one workgroup per
// CU at a time (LDS-bound), rounds(k) = ceil(k wgs / CUs) rounds of workgroups over n/k tiles
// plus their start and drain (about 8.5 tile times, measured), and the merge launch when k > 1
// (about 7).
double prefill_makespan(long long wgs, int k, double n, int num_cus, double tile) {
  const long long rounds = (wgs * k + num_cus - 1) / num_cus;
  return (double)rounds * (n / k + 8.5) * tile + (k > 1 ? 7.0 : 0.0);
}

int max_ksplit(int max_ctx) {
  const int n = (max_ctx + 63) / 64;
  return std::max(1, std::min(8, n / 4));  // ranges of at least 4 tiles
}

}  // namespace

void prefill_plan(const int* rows, int n, int num_kv_heads, int num_cus, bool whole_only,
                  int max_ctx, int* waves, int* rblk, int* ksplit) {
  // The (W, R, k) of least makespan, W/2 <= R <= W with at most 6 pairs (R = W and k = 1 when
  // whole_only), then the fewest workgroups, then the fewest waves.  The three are chosen
  // together: a shape that is slower per tile but holds more row blocks per workgroup can
  // still win once its row tiles are cut into key ranges that fill the CUs (a 512-token chunk
  // over a 32K prefix, 40/8 heads: W = 8, R = 4 in 3 ranges 441 us; W = 12, R = 10 in 4 ranges
  // 341 us).
  const double nt = (double)((max_ctx + 63) / 64);
  const int kmax = whole_only ? 1 : max_ksplit(max_ctx);
  int bw = 8, br = 8, bk = 1;
  double best_cost = 1e300;
  for (int w = 4; w <= 12; ++w) {
    for (int r = whole_only ? w : std::max((w + 1) / 2, w - 6); r <= w; ++r) {
      const double tile = prefill_tile_cost(w, r);
      const long long wgs = prefill_wg_count(rows, n, num_kv_heads, r);
      for (int k = 1; k <= kmax; ++k) {
        const double cost = prefill_makespan(wgs, k, nt, num_cus, tile) +
                            1e-4 * (double)(wgs * k) / num_cus + 1e-6 * w;
        if (cost < best_cost) {
          best_cost = cost;
          bw = w;
          br = r;
          bk = k;
        }
      }
    }
  }
  *waves = bw;
  *rblk = br;
  *ksplit = bk;
}

int prefill_ksplit(long long wgs, int num_cus, int max_ctx, int waves, int rblk,
                   bool deterministic) {
  if (deterministic || wgs <= 0 || num_cus <= 0) return 1;
  const double nt = (double)((max_ctx + 63) / 64);
  const double tile = prefill_tile_cost(waves, rblk);
  int best_k = 1;
  double best = prefill_makespan(wgs, 1, nt, num_cus, tile);
  for (int k = 2; k <= max_ksplit(max_ctx); ++k) {
    const double cost = prefill_makespan(wgs, k, nt, num_cus, tile);
    if (cost < best - 1e-9) {
      best = cost;
      best_k = k;
    }
  }
  return best_k;
}

hipError_t launch_attn_prefill_mfma(const AttnArgs& a, int head_dim, int waves, long long wgs,
                                    bool i8, hipStream_t st) {
  // at least 4 waves: the prologue's block-id loads cover the id cache with 256 threads, and
  // the DMA issue deals a stage's 8 pool tiles to at least 4 waves
  if (waves < 4 || waves > 12 || wgs < 0 || wgs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (i8 && (!a.k_scale_layer || !a.v_scale_layer)) return hipErrorInvalidConfiguration;
  // R row blocks with W/2 <= R <= W; at most 6 half pairs (their merge uses 3 stage arrays)
  if (2 * a.pf_rblk < waves || a.pf_rblk > waves || waves - a.pf_rblk > 6) return hipErrorInvalidConfiguration;
  if (wgs == 0) return hipSuccess;
  if (a.pf_ksplit < 1 || a.pf_ksplit > 8 || wgs * a.pf_ksplit > 0x7fffffffLL)
    return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(wgs * a.pf_ksplit));
  if (i8) {
    if (head_dim == 128)
      attn_prefill_mfma_kernel<128, true><<<grid, 64 * waves, 0, st>>>(a);
    else
      attn_prefill_mfma_kernel<64, true><<<grid, 64 * waves, 0, st>>>(a);
  } else {
    if (head_dim == 128)
      attn_prefill_mfma_kernel<128, false><<<grid, 64 * waves, 0, st>>>(a);
    else
      attn_prefill_mfma_kernel<64, false><<<grid, 64 * waves, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace kvp
