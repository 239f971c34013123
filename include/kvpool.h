/*
 * kvpool.h - C ABI of the paged-KV attention library for MI355X (gfx950).
 *
 * What the library computes: attention of new query tokens against keys and values held in
 * a block-paged KV pool that all sequences share.  The pool is sized once and each request
 * owns a list of fixed-size token blocks; blocks of a shared prefix are shared rather than
 * copied (sparkinfer server README, "Request isolation & continuous batching" and
 * "Automatic prefix cache"; NInfer serving doc, "Execution behavior").  One call covers
 *   - single-token decode for a batch of sequences (NInfer serving doc, "Execution behavior"),
 *   - verification of 1 + k draft tokens, causal among themselves (sparkinfer server README,
 *     "Serve Qwen3.8 with DSpark"; NInfer serving doc, "Server options", --spec/--draft-tokens),
 *   - prefix-reuse prefill, where only the uncached suffix is computed against the cached
 *     prefix (sparkinfer server README, "Automatic prefix cache").
 * For sequence s with L = ctx_lens[s] keys and T = q_lens[s] query tokens, query row i sits at
 * position L - T + i and attends to keys 0 .. L - T + i.  q-head h reads KV head
 * h / (num_q_heads / num_kv_heads) (GQA).  Softmax runs in fp32 with the caller's scale.
 *
 * Conventions shared by every entry point
 *   - Ownership: the caller owns every device buffer (pool storage, q, out, metadata,
 *     workspace).  No call allocates device memory and the library keeps no pointer beyond
 *     kvpool_create's storage pointers; its one piece of device memory is the static scratch of
 *     kvattn_forward_noalloc (KVATTN_NOALLOC_SCRATCH_BYTES on each GPU that loads the library,
 *     placed there by the runtime with the library's code).
 *   - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the null stream) with no
 *     host synchronisation, so calls can be captured in a HIP graph.  Faults inside kernels
 *     surface at the caller's next synchronisation.
 *   - Errors: a non-zero return enqueues no work; kvpool_last_error() then describes it.  The
 *     library never falls back silently to another method: unsupported shapes are rejected
 *     (compare the pages' rule that requested features are refused rather than silently
 *     degraded, sparkinfer server README, "Serve Qwen3.8 with DSpark").
 *   - Metadata checks: scalar arguments are always checked on the host.  Device metadata
 *     (block tables, lengths, block ids) is trusted unless the environment variable
 *     KVPOOL_VALIDATE=1 is set, in which case it is copied to the host (synchronising the
 *     stream) and every violation returns KV_ERANGE.  Without validation, kernels clamp ids and
 *     lengths into range so that bad metadata gives wrong values, never an out-of-bounds access.
 *   - Determinism: no float atomics, so every call is bitwise reproducible.  The split of a
 *     decode or verification sequence's keys depends only on that sequence's own lengths, so its
 *     output is bitwise independent of the rest of the batch and of where its blocks sit in the
 *     pool.  Prefill-class sequences are batch-invariant too with KVATTN_DETERMINISTIC=1 (see
 *     kvattn_forward); the pages' decode path has no float atomics and their deterministic mode
 *     is batch-invariant (sparkinfer server README, "Determinism").
 *
 * Pool storage layout (K and V are separate buffers of identical size).  Element type: fp32
 * or bf16; X = 16 bytes / element size (4 for fp32, 8 for bf16).  For layer l, block b,
 * KV head h, in-block token t (0 .. block_size-1) and dim d (0 .. head_dim-1):
 *   tile  = ((l * num_blocks + b) * num_kv_heads + h) * (block_size / 16) + t / 16
 *   K at element  tile * 16 * head_dim + ((d / X) * 16 + t % 16) * X + d % X
 *   V at element  tile * 16 * head_dim + d * 16 + t % 16
 * Every 16-token slice of a block is a contiguous tile of 16*head_dim elements: K as 16-byte
 * dim chunks (chunk-major, 16 tokens per chunk) and V transposed (dims-major).  One tile is
 * 4 KiB for bf16 at head_dim 128, so each tile is one coalesced read, and it can be copied
 * to LDS verbatim in the order the matrix cores consume it.
 *
 * int8 pools (KV_I8; the pages' int8 KV cache: NInfer serving doc, "Server options",
 * --kv-dtype bf16|int8; sparkinfer server README, "Env", SPARKINFER_KV_INT8).  Each (token,
 * KV head) row x of K or V is stored as codes q = rint(x / s) in [-127, 127] with one fp32
 * scale s = absmax(x) / 127 (fp32, correctly rounded, ties to even; s = 0 and q = 0 for a zero
 * row); it stands for q * s.  Tiles of 16 tokens, one byte per element:
 *   K at byte  tile * 16 * head_dim + ((d / 16) * 16 + t % 16) * 16 + d % 16
 *   V at byte  tile * 16 * head_dim + (((t % 16) / 4 * 16 + d % 16) * (head_dim / 16) + d / 16) * 4 + t % 4
 * (V puts the 4 keys of one dim of each 16-dim group side by side).  Scales: two fp32 arrays
 * (K, V) [num_layers][num_blocks][num_kv_heads][block_size], caller-owned like the storage.
 * Rows appended to an int8 pool, and q / out of attention on it, are bf16.
 */
#ifndef KVPOOL_H
#define KVPOOL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define KVPOOL_API __attribute__((visibility("default")))
#else
#define KVPOOL_API
#endif

typedef struct kvpool kvpool_t; /* opaque; immutable after creation, so thread-safe to share */

typedef enum {
  KV_OK = 0,
  KV_EINVAL = -1,        /* null handle/pointer, bad scalar argument, misaligned buffer   */
  KV_ERANGE = -2,        /* metadata out of range (only reported with KVPOOL_VALIDATE=1)   */
  KV_EUNSUPPORTED = -3,  /* head_dim, block_size, dtype or GQA ratio the kernels don't have */
  KV_EDEVICE = -4,       /* a HIP runtime call failed                                       */
  KV_ENOMEM = -5         /* workspace smaller than kvattn_workspace_size() asks for         */
} kv_status;

typedef enum { KV_F32 = 0, KV_BF16 = 1, KV_I8 = 2 } kv_dtype;

/* Bytes of ONE of the two storage buffers (K or V) for this geometry, written to *bytes.
 * Supported: block_size in {16, 64}, head_dim in {64, 128}, dtype KV_F32, KV_BF16 or KV_I8. */
KVPOOL_API int kvpool_storage_bytes(int32_t num_layers, int32_t num_blocks, int32_t block_size,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                    size_t *bytes);

/* Wraps caller-owned device storage as a pool (the block pool sized once for the whole
 * context, sparkinfer server README, "Serve Qwen3.8 with DSpark"; NInfer serving doc,
 * "Execution behavior").  k_storage and v_storage: device pointers, 16-byte aligned, each of
 * kvpool_storage_bytes() bytes, laid out as described above.  The handle records the current
 * HIP device.  *out receives the handle (host memory, freed by kvpool_destroy). */
KVPOOL_API int kvpool_create(kvpool_t **out, int32_t num_layers, int32_t num_blocks,
                             int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                             int32_t dtype, void *k_storage, void *v_storage);

/* Bytes of ONE of the two scale arrays (K or V) of an int8 pool of this geometry. */
KVPOOL_API int kvpool_scale_bytes(int32_t num_layers, int32_t num_blocks, int32_t block_size,
                                  int32_t num_kv_heads, size_t *bytes);

/* An int8 pool (the layout above) over caller-owned device storage: k_storage / v_storage of
 * kvpool_storage_bytes(..., KV_I8) bytes and k_scales / v_scales of kvpool_scale_bytes() bytes,
 * all 16-byte aligned.  kvpool_create refuses KV_I8 (it has no scale arrays). */
KVPOOL_API int kvpool_create_int8(kvpool_t **out, int32_t num_layers, int32_t num_blocks,
                                  int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                  void *k_storage, void *v_storage, void *k_scales,
                                  void *v_scales);

/* Frees the handle only, never the storage.  NULL is accepted. */
KVPOOL_API int kvpool_destroy(kvpool_t *pool);

/* Writes the K/V rows of each sequence's new tokens into its blocks: row i of sequence s
 * (rows packed in sequence order, q_lens[s] rows each) goes to position ctx_lens[s] - q_lens[s]
 * + i, i.e. block block_tables[s * max_blocks_per_seq + pos / block_size], slot
 * pos % block_size.  This is how only the uncached suffix enters the pool on a prefix hit
 * (sparkinfer server README, "Automatic prefix cache").  Bit copy; every other slot keeps its
 * bits.
 *   k_new, v_new   device, [total_q][num_kv_heads][head_dim] of the pool dtype (bf16 for an
 *                  int8 pool, quantised on the way in), row-major
 *   block_tables   device int32 [num_seqs][max_blocks_per_seq]
 *   ctx_lens       device int32 [num_seqs], length after the append (counts the new tokens)
 *   q_lens         device int32 [num_seqs], new tokens per sequence; sum == total_q
 *   max_q_len      host upper bound of q_lens (sizes the grid)
 * Blocks written here must not be shared with another live sequence (copy them first with
 * kvpool_copy_blocks). */
KVPOOL_API int kvpool_append(kvpool_t *pool, int32_t layer, const void *k_new,
                             const void *v_new, const int32_t *block_tables,
                             int32_t max_blocks_per_seq, const int32_t *ctx_lens,
                             const int32_t *q_lens, int32_t num_seqs, int32_t total_q,
                             int32_t max_q_len, void *stream);

/* pool[dst[i]] <- pool[src[i]] for i < n, every layer, K and V: the copy-on-write step for a
 * shared prefix block that a sequence is about to write (blocks are shared, not copied, until
 * they diverge: sparkinfer server README, "Automatic prefix cache"); an int8 pool's scales
 * move with their codes.  src, dst: device int32 [n].  dst ids must be distinct and disjoint from src ids (then the result does not depend on
 * order; KV_ERANGE under validation otherwise).  Bit copy. */
KVPOOL_API int kvpool_copy_blocks(kvpool_t *pool, const int32_t *src, const int32_t *dst,
                                  int32_t n, void *stream);

/* Workspace bytes kvattn_forward needs for these bounds (written to *bytes; may be 0).
 * q_lens_host: the optional host mirror of q_lens that kvattn_forward will get (NULL: sized for
 * any q_lens within the bounds).  On an int8 pool with prefill-class sequences this counts a
 * bf16 copy of those sequences' keys and values (2 x ceil(max_ctx_len / 16) x num_kv_heads x 16
 * x head_dim x 2 bytes per such sequence, plus its block table), which is the faster way; a
 * smaller workspace without room for the copy is accepted, and the prefill kernel then converts
 * the codes in LDS, with the same output bits. */
KVPOOL_API int kvattn_workspace_size(const kvpool_t *pool, int32_t num_q_heads,
                                     int32_t num_seqs, int32_t total_q, int32_t max_ctx_len,
                                     int32_t max_q_len, const int32_t *q_lens_host,
                                     size_t *bytes);

/* Attention of every sequence's q_lens[s] query rows against its ctx_lens[s] keys (the new
 * tokens' K/V must already be appended).  One call may batch every kind of sequence: decode
 * (q_len 1), verification of 1 + k drafts and prefill chunks over a cached prefix, as a serving
 * step packs every ready request into one batch (NInfer serving doc, "Execution behavior";
 * sparkinfer server README, "Request isolation & continuous batching").  A sequence with
 * q_len * (num_q_heads / num_kv_heads) <= 128 takes the split-K kernel (its keys cut into splits
 * of a size set by its own ctx_len and q_len, merged in a fixed order; when q_lens_host shows
 * sequences of at most 16 rows per KV head beside longer ones, the two kinds run in two
 * launches of 16- and 32-row tiles, with the same bits as one); a longer one takes the prefill
 * kernel.  Decode and verification sequences: the path and the arithmetic follow from the
 * sequence's own lengths, so their output bits never depend on the rest of the batch or on the
 * bounds passed here.  Prefill-class sequences: the workgroup plan follows the call (for speed,
 * a row block may be split between two waves whose partial results are merged, and when the
 * call's prefill row tiles leave CUs idle each row tile's keys are cut into ranges whose
 * partials a second launch merges in range order), so their bits may differ from batch to
 * batch, within the same tolerance; with the environment variable KVATTN_DETERMINISTIC=1
 * every row block is reduced by one wave in key order and their bits, too, depend on the
 * sequence alone (the pages' servers likewise offer bit-reproducible,
 * batch-invariant output as a mode that costs prefill time: sparkinfer server README,
 * "Determinism").
 *   q    device, [total_q][num_q_heads][head_dim], pool dtype (bf16 for an int8 pool), rows
 *        packed in sequence order
 *   out  device, same shape and dtype as q; each element is written exactly once, rounded to
 *        nearest-even from the fp32 result
 *   scale            softmax scale applied to q.k (e.g. 1/sqrt(head_dim))
 *   block_tables     device int32 [num_seqs][max_blocks_per_seq]
 *   ctx_lens, q_lens device int32 [num_seqs]; 0 <= q_lens[s] <= ctx_lens[s]
 *                    <= max_blocks_per_seq * block_size; q_lens[s] == 0 produces no rows
 *   max_ctx_len, max_q_len  host upper bounds of ctx_lens / q_lens (size the grid)
 *   q_lens_host      optional host copy of q_lens (read during the call, not kept; NULL
 *                    allowed).  With it, the grids and the workspace are exact and no kernel is
 *                    launched for a path no sequence takes; without it they are sized from the
 *                    bounds.  It must equal the device q_lens (checked under KVPOOL_VALIDATE=1).
 *   workspace        device scratch of at least kvattn_workspace_size() bytes (same bounds and
 *                    mirror; int8 pools: less without room for the bf16 copy, see there),
 *                    256-byte aligned; contents on entry don't matter.  Calls that may run at
 *                    the same time (other streams) need workspaces of their own.  KV_ENOMEM
 *                    names the bytes required when it is too small.
 * num_q_heads must be a multiple of the pool's num_kv_heads with at most 16 q-heads per KV
 * head. */
KVPOOL_API int kvattn_forward(kvpool_t *pool, int32_t layer, const void *q, void *out,
                              int32_t num_q_heads, float scale, const int32_t *block_tables,
                              int32_t max_blocks_per_seq, const int32_t *ctx_lens,
                              const int32_t *q_lens, int32_t num_seqs, int32_t total_q,
                              int32_t max_ctx_len, int32_t max_q_len,
                              const int32_t *q_lens_host, void *workspace,
                              size_t workspace_bytes, void *stream);

/* kvattn_forward for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  It takes no workspace: the library keeps
 * one static scratch buffer of KVATTN_NOALLOC_SCRATCH_BYTES per GPU, which each GPU that loads
 * the library holds until the process ends; its device address is taken once per device by
 * kvpool_create.  The call allocates nothing (no hipMalloc or hipFree, no events: with
 * kvpool_profile enabled its launches are not timed) and makes no host synchronisation unless
 * KVPOOL_VALIDATE=1.  Arguments, outputs and bits: those of kvattn_forward with the same
 * arguments.  Errors: those of kvattn_forward; KV_ENOMEM when the call needs more scratch than
 * the buffer holds (kvattn_workspace_size with the same bounds tells how much, less the bf16 copy
 * for an int8 pool, which this entry point leaves out when it does not fit; use kvattn_forward
 * then); KV_EDEVICE when the buffer's address could not be taken on the pool's
 * device.  Every call on one GPU shares that GPU's buffer, which keeps the last call's partial
 * results (no kernel needs it cleared on entry): calls ordered on one stream are safe, calls
 * that may overlap on one GPU (several streams or threads) race and must not be made. */
#define KVATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
KVPOOL_API int kvattn_forward_noalloc(kvpool_t *pool, int32_t layer, const void *q, void *out,
                                      int32_t num_q_heads, float scale,
                                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                                      const int32_t *ctx_lens, const int32_t *q_lens,
                                      int32_t num_seqs, int32_t total_q, int32_t max_ctx_len,
                                      int32_t max_q_len, const int32_t *q_lens_host,
                                      void *stream);

/* kvpool_append followed by kvattn_forward, in one call: the new tokens' K/V rows (k_new,
 * v_new, as for kvpool_append) are written into the pool, then every sequence attends as in
 * kvattn_forward (the pages' serving step appends a layer's new K/V and attends over the pool:
 * NInfer serving doc, "Execution behavior").  The result, pool and output, is bit for bit that
 * of the two calls.  On a bf16 pool, when every sequence takes the split-K kernel (decode and
 * verification rows only, judged from q_lens_host when given, else from max_q_len), that
 * kernel writes each new token itself, in the work item whose keys hold it, before reading it:
 * one launch fewer per step.  On an int8 pool the same holds when every sequence also has more
 * than 16 query rows per KV head (verification: 32-row tiles), the kernel quantising the new
 * rows as the append kernel does.  Otherwise (other int8 calls, fp32 pools, prefill chunks)
 * the append kernel runs first.  Arguments: those of both calls, with
 * max_q_len bounding q_lens for both; each call's argument errors and (KVPOOL_VALIDATE)
 * metadata checks apply, and a nonzero return enqueues no work.  The workspace is
 * kvattn_workspace_size's. */
KVPOOL_API int kvattn_append_forward(kvpool_t *pool, int32_t layer, const void *k_new,
                                     const void *v_new, const void *q, void *out,
                                     int32_t num_q_heads, float scale,
                                     const int32_t *block_tables, int32_t max_blocks_per_seq,
                                     const int32_t *ctx_lens, const int32_t *q_lens,
                                     int32_t num_seqs, int32_t total_q, int32_t max_ctx_len,
                                     int32_t max_q_len, const int32_t *q_lens_host,
                                     void *workspace, size_t workspace_bytes, void *stream);

/* kvattn_forward with sink + window sparsity: a query row at absolute position p (= ctx_len -
 * q_len + i) with p + 1 >= min_ctx_len reads only the keys j <= p with j < sink_tokens or
 * j >= p + 1 - window_tokens; rows below the threshold read all their keys.  The pages' decode
 * mode attends only to a sequence's first KV block and its last 4096 tokens once it holds 16384
 * (sparkinfer server README, "Env", SPARKINFER_SPARSE_GQA6): sink_tokens = the pool's
 * block_size, window_tokens = 4096, min_ctx_len = 16384.  The skipped keys are not read from
 * HBM.  Arguments, workspace (kvattn_workspace_size with the same bounds is enough) and the
 * batch-invariance guarantee are those of kvattn_forward.
 * Errors: KV_EINVAL for sink_tokens < 0, window_tokens < 1 or min_ctx_len < 0;
 * KV_EUNSUPPORTED for an fp32 pool, or when a sequence may be longer than the split-K path
 * takes (q_len * num_q_heads / num_kv_heads > 128; judged from q_lens_host when given, else
 * from max_q_len): sparse attention serves decode and verification rows only. */
KVPOOL_API int kvattn_forward_sparse(kvpool_t *pool, int32_t layer, const void *q, void *out,
                                     int32_t num_q_heads, float scale,
                                     const int32_t *block_tables, int32_t max_blocks_per_seq,
                                     const int32_t *ctx_lens, const int32_t *q_lens,
                                     int32_t num_seqs, int32_t total_q, int32_t max_ctx_len,
                                     int32_t max_q_len, int32_t sink_tokens,
                                     int32_t window_tokens, int32_t min_ctx_len,
                                     const int32_t *q_lens_host, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* kvpool_append followed by kvattn_forward_sparse, in one call (the sparse decode step of the
 * same serving loop as kvattn_append_forward).  The result, pool and output, is bit for bit that
 * of the two calls.  On a bf16 pool the split-K kernel writes each new token itself, in the work
 * item whose (sparse) key range holds it: new tokens are the last q_len positions, which every
 * row's window holds, so they always lie past the keys that sparsity skips.  On an int8 pool
 * likewise when every sequence runs in 32-row tiles (more than 16 rows per KV head), else the
 * append kernel runs first.  Arguments and errors: those of both calls (the sparse parameter
 * checks come first); a nonzero return enqueues no work. */
KVPOOL_API int kvattn_append_forward_sparse(kvpool_t *pool, int32_t layer, const void *k_new,
                                            const void *v_new, const void *q, void *out,
                                            int32_t num_q_heads, float scale,
                                            const int32_t *block_tables,
                                            int32_t max_blocks_per_seq, const int32_t *ctx_lens,
                                            const int32_t *q_lens, int32_t num_seqs,
                                            int32_t total_q, int32_t max_ctx_len,
                                            int32_t max_q_len, int32_t sink_tokens,
                                            int32_t window_tokens, int32_t min_ctx_len,
                                            const int32_t *q_lens_host, void *workspace,
                                            size_t workspace_bytes, void *stream);

/* ---- host page store: park / restore pool blocks over PCIe ----------------------------------
 * Evicted sequences can be parked in pinned host memory instead of being discarded, each taking
 * only its real size, and computed prefixes restored over PCIe instead of being recomputed,
 * with branches that share a prefix deduplicating against the same stored pages (NInfer serving
 * doc, "Server options", --host-kv-cache-mib and --kv-host-cache-mib).
 * A page is one pool block across every layer: for layer 0, 1, ...: the block's K bytes, its V
 * bytes and, for an int8 pool, its K and V scale bytes, each in storage order.  Pages with the
 * same content are stored once, with a reference count, so only pages the store lacks are
 * written over PCIe.  A 128-bit hash computed on the GPU nominates the candidates (each 64-bit
 * little-endian word w_i of the page, i = 0, 1, ..., contributes fmix64(w_i + 0x9E3779B97F4A7C15
 * (i + 1)) to the first half and fmix64(w_i ^ 0xD6E8FEB86659FD93 (i + 1)) to the second, sums
 * mod 2^64; fmix64 is the MurmurHash3 finalizer) and the bytes decide: before a block shares a
 * page, the GPU compares it with that page (a stored page is read back over PCIe, a page new in
 * the same call is read from the pool), so pages with equal hashes but different bytes, whether
 * by chance or crafted, are stored apart.
 * The kernels read and write the pinned store directly (no device memory is allocated).
 * A store serves pools of the geometry (layers, block size, KV heads, head dim, dtype) it was
 * created for.  Calls on one store are serialised by a lock; park, restore and page_hash are
 * enqueued on `stream` and wait for it to finish before returning.  Block and page lists are
 * host arrays. */
typedef struct kvhost kvhost_t;

/* Bytes of one page of `pool` (written to *bytes). */
KVPOOL_API int kvhost_page_bytes(const kvpool_t *pool, size_t *bytes);

/* A store holding up to budget_bytes / page slot (the page rounded up to 256 bytes) pages, in
 * one pinned host allocation made here.  KV_EINVAL if the budget holds no page; KV_ENOMEM if the
 * pinned allocation fails (the caller then runs without a store). */
KVPOOL_API int kvhost_create(kvhost_t **out, const kvpool_t *pool, size_t budget_bytes);
KVPOOL_API int kvhost_destroy(kvhost_t *store);   /* frees the pinned memory; NULL is a no-op */

/* Stores pool blocks blocks[0..n) and writes their page ids to page_ids[0..n): a block whose
 * content equals a stored page (or another block of the call) gets that page's id and adds a
 * reference.  All or nothing: KV_ENOMEM, with nothing stored, when the distinct new pages do not
 * fit.  KV_ERANGE for a block id outside the pool. */
KVPOOL_API int kvhost_park(kvhost_t *store, kvpool_t *pool, const int32_t *blocks, int32_t n,
                           int64_t *page_ids, void *stream);

/* Writes page page_ids[i] into pool block dst_blocks[i], bit for bit, for i < n.  Destination
 * blocks must be distinct; page ids must be live (KV_EINVAL otherwise, nothing written).  The
 * references are kept (release them when the pages are no longer needed). */
KVPOOL_API int kvhost_restore(kvhost_t *store, kvpool_t *pool, const int64_t *page_ids,
                              const int32_t *dst_blocks, int32_t n, void *stream);

/* Drops one reference per listed id; a page left with none is removed and its id goes stale
 * (a stale id is refused, never confused with a later page).  All or nothing: KV_EINVAL, with
 * nothing released, if an id is not live or is listed more often than it is referenced. */
KVPOOL_API int kvhost_release(kvhost_t *store, const int64_t *page_ids, int32_t n);

/* Pages stored, page capacity and live references. */
KVPOOL_API int kvhost_stats(const kvhost_t *store, int64_t *pages, int64_t *capacity,
                            int64_t *references);

/* The 128-bit content hashes of pool blocks blocks[0..n): hashes[2i], hashes[2i + 1] (host). */
KVPOOL_API int kvhost_page_hash(kvhost_t *store, kvpool_t *pool, const int32_t *blocks,
                                int32_t n, uint64_t *hashes, void *stream);

/* Opt-in per-kernel timing for measurement.  With enable != 0, every kernel launch made by this
 * library (any pool, any thread) is bracketed by a pair of HIP events recorded on the launch's
 * stream, and earlier records are dropped; with enable == 0 recording stops (records are kept).
 * It measures without changing what is computed, like the per-phase timings the pages' servers
 * log (NInfer serving doc, "Structured request log").  Costs a few microseconds per launch. */
KVPOOL_API int kvpool_profile(int32_t enable);

/* Totals for kernel `index` (0, 1, ... in a fixed order) since the last kvpool_profile(1): its
 * name (static string), the number of recorded launches and the summed event time in
 * milliseconds.  Waits for the recorded events to complete.  KV_ERANGE past the last kernel. */
KVPOOL_API int kvpool_profile_kernel(int32_t index, const char **name, int32_t *launches,
                                     double *total_ms);

/* Message for the last non-OK return on this thread ("" if none).  Valid until the next call
 * on the same thread. */
KVPOOL_API const char *kvpool_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVPOOL_H */
