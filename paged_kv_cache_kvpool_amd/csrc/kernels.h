// Launchers of the gfx950 kernels, called by the C ABI layer (kvpool.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace kvp {

struct AppendArgs {
  void* k_layer;
  void* v_layer;
  const void* k_new;
  const void* v_new;
  const int32_t* block_tables;
  const int32_t* ctx_lens;
  const int32_t* q_lens;
  float* k_scale_layer;  // int8 pools: per-(block, KV head, token) fp32 scales of the layer
  float* v_scale_layer;
  int32_t num_seqs, total_q, num_kv_heads, head_dim, block_size, num_blocks;
  int32_t max_blocks_per_seq;
};

struct CopyArgs {
  void* k;
  void* v;
  void* k_scale;  // int8 pools: scale arrays, else null
  void* v_scale;
  const int32_t* src;
  const int32_t* dst;
  int32_t num_blocks;
  size_t block_bytes;        // one block of one layer: Hkv * block_size * head_dim * elt
  size_t block_scale_bytes;  // one block of one layer of scales: Hkv * block_size * 4
};

// Append of bf16/fp32 rows into a pool of the same dtype (elt_bytes 2 or 4), or of bf16 rows
// quantised into an int8 pool (elt_bytes 1).
hipError_t launch_append(const AppendArgs& a, int elt_bytes, int max_q_len, hipStream_t st);
hipError_t launch_copy_blocks(const CopyArgs& a, int n, int num_layers, hipStream_t st);

// Pool geometry for moving whole pages (one block across every layer: K, V and, for int8
// pools, the K and V scales) between the pool and a pinned host page store.
struct PageArgs {
  void* k;
  void* v;
  float* k_scale;       // int8 pools, else null
  float* v_scale;
  int32_t num_blocks;
  int32_t tensors;      // 2 (K, V) or 4 (K, V, K scales, V scales)
  int32_t segs;         // segments per page: num_layers * tensors
  size_t block_bytes;   // one block of one layer of K or V
  size_t scale_bytes;   // one block of one layer of K or V scales
  size_t page_stride;   // bytes between page slots in the host store
};
// Hash partials of pool blocks blocks[0..n): partial[2 (j * segs + seg) + {0, 1}].
hipError_t launch_page_hash(const PageArgs& a, const int32_t* blocks, int n, uint64_t* partial,
                            hipStream_t st);
// pairs: [n][2] = (pool block, store slot) for park, (store slot, pool block) for restore.
hipError_t launch_page_park(const PageArgs& a, const int32_t* pairs, int n, char* store,
                            hipStream_t st);
hipError_t launch_page_restore(const PageArgs& a, const int32_t* pairs, int n, const char* store,
                               hipStream_t st);
// Byte comparison of n page pairs: triples[3j] = pool block, triples[3j + 1] = 0 (the other page
// is store slot triples[3j + 2]) or 1 (pool block triples[3j + 2]); diff[j * segs + seg] = 1 when
// that segment differs, else 0.
hipError_t launch_page_compare(const PageArgs& a, const int32_t* triples, int n, const char* store,
                               uint32_t* diff, hipStream_t st);

// Split-K attention on the matrix cores (bf16) for the sequences with q_len <= split_q_max:
// items of (row tile of <= 32 rows, split, KV head, sequence) dealt round-robin to persistent
// waves (num_cus sizes the grid), or, for forced splits longer than 2048 keys, one 4-wave
// workgroup per item.  `splits`: most splits of any sequence (at most 65535 for the 4-wave
// variant).
// int8_kv: the pool holds int8 codes with per-token scales (a.k_scale_layer / v_scale_layer).
hipError_t launch_attn_split_mfma(const AttnArgs& a, int head_dim, int rows_per_tile,
                                  int splits, int num_cus, bool int8_kv, hipStream_t st);
// Vector-ALU attention (fp32 and bf16), one wave per (row tile of <= 8 rows, split, KV head,
// sequence); sequences past split_q_max make one pass in split slot 0.
hipError_t launch_attn_vec(const AttnArgs& a, int elt_bytes, int head_dim, int rows_per_tile,
                           int grid_x, hipStream_t st);
// Prefill attention on the matrix cores (bf16) for the sequences with q_len > split_q_max:
// `waves` (4..12) waves over a.pf_rblk 32-row blocks share LDS-staged K/V tiles; the workgroups, numbered sequence
// by sequence (KV heads x row tiles of each prefill-class sequence), are found on the device
// from q_lens.  `wgs`: grid size, at least the number of workgroups there are (extra ones exit).
// int8_kv: the pool holds int8 codes with per-token scales, converted to bf16 in LDS: the
// path for int8 pools when the workspace has no room for a bf16 copy.
hipError_t launch_attn_prefill_mfma(const AttnArgs& a, int head_dim, int waves, long long wgs,
                                    bool int8_kv, hipStream_t st);
// Workgroups of the prefill kernel for prefill-class sequences of rows[i] = q_len * G rows each,
// with rblk 32-row blocks per workgroup.
long long prefill_wg_count(const int* rows, int n, int num_kv_heads, int rblk);
// Key ranges per prefill row tile (1..8) for a given workgroup shape (waves, rblk): more when
// the row tiles alone, wgs of them, leave CUs idle; 1 in deterministic mode.  max_ctx: the
// longest context (ranges of whole 64-key tiles, at least 4 each).
int prefill_ksplit(long long wgs, int num_cus, int max_ctx, int waves, int rblk,
                   bool deterministic);
// Workgroup shape and key ranges for such a set of sequences, chosen together for the least
// modelled makespan: waves (4..12), row blocks per workgroup (waves/2 .. waves; the waves beyond
// 2*rblk - waves share a row block in pairs) and key ranges per row tile (1..8).
// whole_only: rblk = waves (no pairs) and one key range.
void prefill_plan(const int* rows, int n, int num_kv_heads, int num_cus, bool whole_only,
                  int max_ctx, int* waves, int* rblk, int* ksplit);
// Prefill over an int8 pool, when the workspace holds the copy: the prefill-class sequences'
// tiles dequantized to bf16 into a workspace pool (max_seqs sequences of blocks_per_seq 16-token
// blocks) and its block table [num_seqs][blocks_per_seq]; the grid covers max_seqs sequences
// of blocks_per_seq tiles.
struct DequantOut {
  uint16_t* k;
  uint16_t* v;
  int32_t* tables;
  int32_t blocks_per_seq;
  int32_t max_seqs;
};
hipError_t launch_dequant_prefill(const AttnArgs& a, const DequantOut& o, int head_dim,
                                  hipStream_t st);
// Cross-split merge of the split-K partials: one workgroup per (partial row, q-head).
hipError_t launch_attn_reduce(const AttnArgs& a, int elt_bytes, int head_dim, hipStream_t st);
// Merge of the prefill kernel's key-range partials (a.pf_ksplit > 1, at most 8): one workgroup
// per (query token, group of 256 (q-head, 4-dim) slices).  both: the cross-split merge of the
// split-K partials in the same launch (its workgroups first; the merges touch disjoint rows);
// with no key ranges it is then launch_attn_reduce alone.
hipError_t launch_attn_reduce_prefill(const AttnArgs& a, int elt_bytes, int head_dim, bool both,
                                      hipStream_t st);

}  // namespace kvp
