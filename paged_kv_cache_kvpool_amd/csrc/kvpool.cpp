// C ABI of the paged-KV attention library: handle, argument checks, optional metadata
// validation, split planning and kernel dispatch.  Declared in include/kvpool.h.
#include "../../include/kvpool.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "host_dedup.h"
#include "kernels.h"

struct kvpool {
  int32_t num_layers, num_blocks, block_size, num_kv_heads, head_dim, dtype;
  void* k;
  void* v;
  float* k_scale;      // int8 pools: [layers][blocks][Hkv][block_size] fp32 scales, else null
  float* v_scale;
  size_t layer_elems;  // elements of one layer of K (or V)
  int device;
  int num_cus;         // compute units of that device
};

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return KV_OK;
}

int elt_bytes(int32_t dtype) { return dtype == KV_F32 ? 4 : dtype == KV_I8 ? 1 : 2; }

bool env_flag(const char* name) {
  const char* v = getenv(name);
  return v && *v && strcmp(v, "0") != 0;
}

bool env_is(const char* name, const char* value) {
  const char* v = getenv(name);
  return v && strcmp(v, value) == 0;
}

// Keys per split in split mode: 0 selects the per-sequence rule the kernels apply (about L/128
// rounded up to 32 keys, within [split_floor, 2048]), KVATTN_SPLIT_TOKENS fixes a count for
// tuning sweeps.  Neither
// depends on the rest of the batch, so each sequence's reduction order is a function of its own
// length and row count only.
int split_tokens() {
  const char* v = getenv("KVATTN_SPLIT_TOKENS");
  if (!v || !*v) return 0;
  int s = std::max(32, std::min(atoi(v), 1 << 20));
  return (s + 31) / 32 * 32;
}

// Upper bound of a sequence's split count over all lengths <= max_ctx.
int max_split_count(int split, int max_ctx) {
  if (split > 0) return std::max(1, (max_ctx + split - 1) / split);
  // The rule (ceil(L/128) rounded up to 32, within [256 or 512, 2048]) gives at most
  // min(128, ceil(L/256)) splits up to 262144 keys and ceil(L/2048) past that.
  return std::max(std::max(1, std::min(128, (max_ctx + 255) / 256)), (max_ctx + 2047) / 2048);
}

// The split-K path serves decode and verification (few query rows per KV head): a sequence's
// context is cut into splits so that even one sequence fills the GPU.  A sequence whose q_len
// times the group size exceeds this many rows (a prefill chunk) carries enough rows to fill it
// without splitting and takes the prefill kernel.  The class depends on the sequence alone.
constexpr int kSplitRowsMax = 128;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_geometry(int32_t num_layers, int32_t num_blocks, int32_t block_size,
                   int32_t num_kv_heads, int32_t head_dim, int32_t dtype) {
  if (num_layers <= 0 || num_blocks <= 0 || num_kv_heads <= 0)
    return fail(KV_EINVAL, "num_layers, num_blocks and num_kv_heads must be positive");
  if (block_size != 16 && block_size != 64)
    return fail(KV_EUNSUPPORTED, "block_size %d not supported (16 or 64)", block_size);
  if (head_dim != 64 && head_dim != 128)
    return fail(KV_EUNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (dtype != KV_F32 && dtype != KV_BF16 && dtype != KV_I8)
    return fail(KV_EUNSUPPORTED, "dtype %d not supported (KV_F32, KV_BF16 or KV_I8)", dtype);
  return KV_OK;
}

hipError_t current_device_matches(const kvpool* p) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  return dev == p->device ? hipSuccess : hipErrorInvalidDevice;
}

struct HostMeta {
  std::vector<int32_t> tables, ctx, ql;
};

int fetch_meta(const int32_t* tables, int32_t max_blocks, const int32_t* ctx, const int32_t* ql,
               int32_t num_seqs, hipStream_t st, HostMeta& m) {
  m.tables.resize((size_t)num_seqs * max_blocks);
  m.ctx.resize(num_seqs);
  m.ql.resize(num_seqs);
  hipError_t e = hipMemcpyAsync(m.tables.data(), tables, m.tables.size() * 4,
                                hipMemcpyDeviceToHost, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(m.ctx.data(), ctx, (size_t)num_seqs * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(m.ql.data(), ql, (size_t)num_seqs * 4, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(KV_EDEVICE, "metadata copy failed: %s", hipGetErrorString(e));
  return KV_OK;
}

int validate_meta(const kvpool* p, const HostMeta& m, int32_t max_blocks, int32_t num_seqs,
                  int32_t total_q, int32_t max_ctx_len, int32_t max_q_len) {
  long long sum_q = 0;
  for (int s = 0; s < num_seqs; ++s) {
    const int L = m.ctx[s], T = m.ql[s];
    if (T < 0 || L < T) return fail(KV_ERANGE, "seq %d: need 0 <= q_len (%d) <= ctx_len (%d)", s, T, L);
    if ((long long)L > (long long)max_blocks * p->block_size)
      return fail(KV_ERANGE, "seq %d: ctx_len %d exceeds max_blocks_per_seq*block_size", s, L);
    if (L > max_ctx_len) return fail(KV_ERANGE, "seq %d: ctx_len %d > max_ctx_len %d", s, L, max_ctx_len);
    if (T > max_q_len) return fail(KV_ERANGE, "seq %d: q_len %d > max_q_len %d", s, T, max_q_len);
    const int nb = (L + p->block_size - 1) / p->block_size;
    for (int b = 0; b < nb; ++b) {
      const int id = m.tables[(size_t)s * max_blocks + b];
      if (id < 0 || id >= p->num_blocks)
        return fail(KV_ERANGE, "seq %d: block table entry %d = %d outside [0, %d)", s, b, id, p->num_blocks);
    }
    sum_q += T;
  }
  if (sum_q != total_q) return fail(KV_ERANGE, "sum of q_lens (%lld) != total_q (%d)", sum_q, total_q);
  return KV_OK;
}

// Opt-in per-kernel timing: a HIP event pair around every launch, on the launch's stream.
enum KernelId {
  K_APPEND, K_COPY, K_SPLIT_MFMA, K_VEC, K_PREFILL_MFMA, K_REDUCE, K_DEQUANT,
  K_PAGE_HASH, K_PAGE_PARK, K_PAGE_RESTORE, K_REDUCE_PF, K_PAGE_COMPARE, K_COUNT
};
const char* const kKernelNames[K_COUNT] = {"kv_append", "kv_copy_blocks", "attn_split_mfma",
                                           "attn_vec", "attn_prefill_mfma", "attn_reduce",
                                           "kv_dequant_prefill", "page_hash", "page_park",
                                           "page_restore", "attn_reduce_prefill",
                                           "page_compare"};
struct ProfRec {
  int kernel;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_prof_free;

hipEvent_t prof_event() {
  if (!g_prof_free.empty()) {
    hipEvent_t e = g_prof_free.back();
    g_prof_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Set for the duration of an allocation-free call (kvattn_forward_noalloc): its launches are
// never bracketed by events, which the runtime may allocate.
thread_local bool g_no_events = false;

template <class F>
hipError_t timed(int kernel, hipStream_t st, F launch) {
  std::unique_lock<std::mutex> lk(g_prof_mu);
  if (!g_prof_on || g_no_events) {
    lk.unlock();
    return launch();
  }
  hipEvent_t a = prof_event(), b = prof_event();
  if (a) hipEventRecord(a, st);
  hipError_t e = launch();
  if (b) hipEventRecord(b, st);
  if (a && b) g_prof_recs.push_back({kernel, a, b});
  return e;
}

}  // namespace

extern "C" {

int kvpool_profile(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (enable) {
    for (auto& r : g_prof_recs) {
      g_prof_free.push_back(r.a);
      g_prof_free.push_back(r.b);
    }
    g_prof_recs.clear();
  }
  g_prof_on = enable != 0;
  return ok();
}

int kvpool_profile_kernel(int32_t index, const char** name, int32_t* launches, double* total_ms) {
  if (index < 0 || index >= K_COUNT) return fail(KV_ERANGE, "kernel index %d out of range", index);
  if (!name || !launches || !total_ms) return fail(KV_EINVAL, "NULL output pointer");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int n = 0;
  double ms = 0.0;
  for (auto& r : g_prof_recs) {
    if (r.kernel != index) continue;
    hipError_t e = hipEventSynchronize(r.b);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
    if (e != hipSuccess) return fail(KV_EDEVICE, "event timing: %s", hipGetErrorString(e));
    ms += t;
    ++n;
  }
  *name = kKernelNames[index];
  *launches = n;
  *total_ms = ms;
  return ok();
}

int kvpool_storage_bytes(int32_t num_layers, int32_t num_blocks, int32_t block_size,
                         int32_t num_kv_heads, int32_t head_dim, int32_t dtype, size_t* bytes) {
  if (!bytes) return fail(KV_EINVAL, "bytes is NULL");
  int rc = check_geometry(num_layers, num_blocks, block_size, num_kv_heads, head_dim, dtype);
  if (rc) return rc;
  *bytes = (size_t)num_layers * num_blocks * num_kv_heads * block_size * head_dim * elt_bytes(dtype);
  return ok();
}

}  // extern "C"

// ---- scratch of the allocation-free entry point ----------------------------------------------
// The workspace of kvattn_forward_noalloc.  Every GPU that loads this library's code holds its
// own copy, zero at load, until the process ends.  In host code this name stands for a host-side
// shadow, not for device memory: its device address on each GPU is taken once with
// hipGetSymbolAddress (scratch_setup) and only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[KVATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  bool done;
  hipError_t err;
  void* ptr;  // device address of `scratch` on this device
};
std::mutex g_scratch_mu;
ScratchSlot g_scratch[kMaxDevices];

// Takes the scratch array's device address on device `dev`, which must be current (called by
// kvpool_create, the library's set-up call).  Once per device; a failure is recorded and reported
// by kvattn_forward_noalloc, never by the pool's other entry points.
void scratch_setup(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  ScratchSlot& sl = g_scratch[dev];
  if (sl.done) return;
  void* p = nullptr;
  sl.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  sl.ptr = sl.err == hipSuccess ? p : nullptr;
  sl.done = true;
}

}  // namespace

namespace {

int create_pool(kvpool_t** out, int32_t num_layers, int32_t num_blocks, int32_t block_size,
                int32_t num_kv_heads, int32_t head_dim, int32_t dtype, void* k_storage,
                void* v_storage, void* k_scales, void* v_scales) {
  if (!out) return fail(KV_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = check_geometry(num_layers, num_blocks, block_size, num_kv_heads, head_dim, dtype);
  if (rc) return rc;
  if (dtype == KV_I8 && (!k_scales || !v_scales || !aligned16(k_scales) || !aligned16(v_scales)))
    return fail(KV_EINVAL, "int8 pools need 16-byte aligned K and V scale arrays");
  if (!k_storage || !v_storage) return fail(KV_EINVAL, "storage pointers must not be NULL");
  if (!aligned16(k_storage) || !aligned16(v_storage))
    return fail(KV_EINVAL, "storage pointers must be 16-byte aligned");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KV_EDEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  kvpool* p = new (std::nothrow) kvpool;
  if (!p) return fail(KV_EINVAL, "out of host memory");
  p->num_layers = num_layers;
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->num_kv_heads = num_kv_heads;
  p->head_dim = head_dim;
  p->dtype = dtype;
  p->k = k_storage;
  p->v = v_storage;
  p->k_scale = dtype == KV_I8 ? static_cast<float*>(k_scales) : nullptr;
  p->v_scale = dtype == KV_I8 ? static_cast<float*>(v_scales) : nullptr;
  p->layer_elems = (size_t)num_blocks * num_kv_heads * block_size * head_dim;
  p->device = dev;
  scratch_setup(dev);
  p->num_cus = 256;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
    p->num_cus = cus;
  *out = p;
  return ok();
}

}  // namespace

namespace {

// Checks (and, under KVPOOL_VALIDATE, validates) an append; *nothing = true when there is no
// row to write.  Shared by kvpool_append and kvattn_append_forward.
int append_check(kvpool_t* pool, int32_t layer, const void* k_new, const void* v_new,
                 const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* ctx_lens,
                 const int32_t* q_lens, int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                 hipStream_t st, bool* nothing) {
  *nothing = false;
  if (!pool) return fail(KV_EINVAL, "pool is NULL");
  if (layer < 0 || layer >= pool->num_layers) return fail(KV_EINVAL, "layer %d out of range", layer);
  if (num_seqs < 0 || total_q < 0 || max_q_len < 0 || max_blocks_per_seq < 0)
    return fail(KV_EINVAL, "negative size argument");
  if (num_seqs > 65535) return fail(KV_EUNSUPPORTED, "num_seqs %d > 65535", num_seqs);
  if (num_seqs == 0 || total_q == 0 || max_q_len == 0) {
    *nothing = true;
    return ok();
  }
  if (!k_new || !v_new || !block_tables || !ctx_lens || !q_lens)
    return fail(KV_EINVAL, "NULL device pointer");
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(KV_EINVAL, "k_new/v_new must be 16-byte aligned");
  if (current_device_matches(pool) != hipSuccess)
    return fail(KV_EINVAL, "current HIP device is not the pool's device %d", pool->device);
  if (env_flag("KVPOOL_VALIDATE")) {
    HostMeta m;
    int rc = fetch_meta(block_tables, max_blocks_per_seq, ctx_lens, q_lens, num_seqs, st, m);
    if (rc) return rc;
    rc = validate_meta(pool, m, max_blocks_per_seq, num_seqs, total_q, INT32_MAX, max_q_len);
    if (rc) return rc;
    // Blocks being written must belong to exactly one sequence of this call.
    std::vector<int> owner(pool->num_blocks, -1);
    for (int s = 0; s < num_seqs; ++s) {
      const int nb = (m.ctx[s] + pool->block_size - 1) / pool->block_size;
      for (int b = 0; b < nb; ++b) {
        const int id = m.tables[(size_t)s * max_blocks_per_seq + b];
        if (owner[id] >= 0 && owner[id] != s) {
          const int first_new = (m.ctx[s] - m.ql[s]) / pool->block_size;
          if (b >= first_new) return fail(KV_ERANGE, "seq %d writes block %d shared with seq %d", s, id, owner[id]);
        }
        owner[id] = s;
      }
    }
  }
  return ok();
}

// The append kernel's launch (arguments already checked).
int append_launch(kvpool_t* pool, int32_t layer, const void* k_new, const void* v_new,
                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* ctx_lens, const int32_t* q_lens, int32_t num_seqs,
                  int32_t total_q, int32_t max_q_len, hipStream_t st) {
  kvp::AppendArgs a;
  const size_t lo = (size_t)layer * pool->layer_elems * elt_bytes(pool->dtype);
  a.k_layer = static_cast<char*>(pool->k) + lo;
  a.v_layer = static_cast<char*>(pool->v) + lo;
  a.k_new = k_new;
  a.v_new = v_new;
  const size_t so = (size_t)layer * pool->num_blocks * pool->num_kv_heads * pool->block_size;
  a.k_scale_layer = pool->k_scale ? pool->k_scale + so : nullptr;
  a.v_scale_layer = pool->v_scale ? pool->v_scale + so : nullptr;
  a.block_tables = block_tables;
  a.ctx_lens = ctx_lens;
  a.q_lens = q_lens;
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.num_kv_heads = pool->num_kv_heads;
  a.head_dim = pool->head_dim;
  a.block_size = pool->block_size;
  a.num_blocks = pool->num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  hipError_t e = timed(K_APPEND, st, [&] { return kvp::launch_append(a, elt_bytes(pool->dtype), max_q_len, st); });
  if (e != hipSuccess) return fail(KV_EDEVICE, "append launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int kvpool_create(kvpool_t** out, int32_t num_layers, int32_t num_blocks, int32_t block_size,
                  int32_t num_kv_heads, int32_t head_dim, int32_t dtype, void* k_storage,
                  void* v_storage) {
  if (dtype == KV_I8) {
    if (out) *out = nullptr;
    return fail(KV_EINVAL, "int8 pools are created with kvpool_create_int8 (they need scale arrays)");
  }
  return create_pool(out, num_layers, num_blocks, block_size, num_kv_heads, head_dim, dtype,
                     k_storage, v_storage, nullptr, nullptr);
}

int kvpool_create_int8(kvpool_t** out, int32_t num_layers, int32_t num_blocks, int32_t block_size,
                       int32_t num_kv_heads, int32_t head_dim, void* k_storage, void* v_storage,
                       void* k_scales, void* v_scales) {
  return create_pool(out, num_layers, num_blocks, block_size, num_kv_heads, head_dim, KV_I8,
                     k_storage, v_storage, k_scales, v_scales);
}

int kvpool_scale_bytes(int32_t num_layers, int32_t num_blocks, int32_t block_size,
                       int32_t num_kv_heads, size_t* bytes) {
  if (!bytes) return fail(KV_EINVAL, "bytes is NULL");
  int rc = check_geometry(num_layers, num_blocks, block_size, num_kv_heads, 64, KV_I8);
  if (rc) return rc;
  *bytes = (size_t)num_layers * num_blocks * num_kv_heads * block_size * sizeof(float);
  return ok();
}

int kvpool_destroy(kvpool_t* pool) {
  delete pool;
  return ok();
}

int kvpool_append(kvpool_t* pool, int32_t layer, const void* k_new, const void* v_new,
                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* ctx_lens, const int32_t* q_lens, int32_t num_seqs,
                  int32_t total_q, int32_t max_q_len, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  bool nothing = false;
  if (int rc = append_check(pool, layer, k_new, v_new, block_tables, max_blocks_per_seq, ctx_lens,
                            q_lens, num_seqs, total_q, max_q_len, st, &nothing))
    return rc;
  if (nothing) return ok();
  return append_launch(pool, layer, k_new, v_new, block_tables, max_blocks_per_seq, ctx_lens,
                       q_lens, num_seqs, total_q, max_q_len, st);
}

int kvpool_copy_blocks(kvpool_t* pool, const int32_t* src, const int32_t* dst, int32_t n,
                       void* stream) {
  if (!pool) return fail(KV_EINVAL, "pool is NULL");
  if (n < 0) return fail(KV_EINVAL, "n must be >= 0");
  if (n == 0) return ok();
  if (!src || !dst) return fail(KV_EINVAL, "NULL device pointer");
  if (n > INT32_MAX / 2) return fail(KV_EINVAL, "n too large");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (current_device_matches(pool) != hipSuccess)
    return fail(KV_EINVAL, "current HIP device is not the pool's device %d", pool->device);
  if (env_flag("KVPOOL_VALIDATE")) {
    std::vector<int32_t> hs(n), hd(n);
    hipError_t e = hipMemcpyAsync(hs.data(), src, (size_t)n * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipMemcpyAsync(hd.data(), dst, (size_t)n * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(KV_EDEVICE, "metadata copy failed: %s", hipGetErrorString(e));
    std::vector<char> is_src(pool->num_blocks, 0), is_dst(pool->num_blocks, 0);
    for (int i = 0; i < n; ++i) {
      if (hs[i] < 0 || hs[i] >= pool->num_blocks || hd[i] < 0 || hd[i] >= pool->num_blocks)
        return fail(KV_ERANGE, "copy pair %d (%d -> %d) outside [0, %d)", i, hs[i], hd[i], pool->num_blocks);
      is_src[hs[i]] = 1;
    }
    for (int i = 0; i < n; ++i) {
      if (is_dst[hd[i]]) return fail(KV_ERANGE, "dst block %d appears twice", hd[i]);
      if (is_src[hd[i]]) return fail(KV_ERANGE, "dst block %d is also a src block", hd[i]);
      is_dst[hd[i]] = 1;
    }
  }
  kvp::CopyArgs a;
  a.k = pool->k;
  a.v = pool->v;
  a.k_scale = pool->k_scale;
  a.v_scale = pool->v_scale;
  a.block_scale_bytes = (size_t)pool->num_kv_heads * pool->block_size * sizeof(float);
  a.src = src;
  a.dst = dst;
  a.num_blocks = pool->num_blocks;
  a.block_bytes = (size_t)pool->num_kv_heads * pool->block_size * pool->head_dim * elt_bytes(pool->dtype);
  hipError_t e = timed(K_COPY, st, [&] { return kvp::launch_copy_blocks(a, n, pool->num_layers, st); });
  if (e != hipSuccess) return fail(KV_EDEVICE, "copy launch: %s", hipGetErrorString(e));
  return ok();
}

namespace {

struct Plan {
  int split_q_max;    // sequences with q_len <= split_q_max take the split-K path
  bool split_k;       // some sequence may take the split-K path with at least one row
  bool prefill;       // some sequence may take the prefill kernel
  int split_rows;     // rows per KV head of the longest split-K sequence (bound)
  int split_rows_min; // rows per KV head of the shortest split-K sequence with rows (0: unknown)
  int split;          // fixed keys per split, or 0 for the per-length rule
  int max_splits;     // split slots per partial row
  int part_rows;      // partial rows: the split-K path's query tokens (or a bound of them)
  int waves;          // prefill workgroup size
  int rblk;           // prefill 32-row blocks per workgroup
  long long pf_wgs;   // prefill grid: its workgroups (or a bound of them)
  int pf_ks;          // prefill key ranges per row tile (1: no partials)
  size_t pf_o_off, pf_ml_off;  // their partials in the workspace
  size_t o_bytes;     // partial outputs, rounded up to 256 bytes
  // int8 pools with prefill-class sequences: their tiles dequantized to a bf16 workspace pool
  // first (the faster way), when the workspace holds it; else the prefill kernel converts the
  // codes in LDS (bitwise the same results)
  int dq_seqs;        // prefill sequences it holds (exact or a bound)
  int dq_mpb;         // 16-token blocks per sequence (ceil(max_ctx_len / 16))
  size_t dq_off;      // byte offsets in the workspace: K pool, V pool, block table
  size_t dq_v_off, dq_tbl_off;
  size_t bytes_lean;  // the workspace without the bf16 copy (= bytes when there is none)
  size_t bytes;       // the workspace asked for
};

// The plan of one call.  With the host mirror of q_lens, the split-K rows, the prefill
// sequences and the grids are exact; without it, they are bounds from (num_seqs, total_q,
// max_q_len).  Either way the kernels decide each sequence's path from the device q_lens.
Plan make_plan(const kvpool* p, int32_t num_q_heads, int32_t num_seqs, int32_t total_q,
               int32_t max_ctx_len, int32_t max_q_len, const int32_t* q_lens_host) {
  Plan pl{};
  const int G = num_q_heads / p->num_kv_heads;
  const int sqm = kSplitRowsMax / G;
  pl.split_q_max = sqm;
  pl.split = split_tokens();
  pl.max_splits = max_split_count(pl.split, max_ctx_len);
  std::vector<int> pf_rows;
  int n_pf_exact = 0;
  if (q_lens_host) {
    long long split_tokens_sum = 0;
    int split_t = 0, split_t_min = 0;
    for (int s = 0; s < num_seqs; ++s) {
      const int T = std::max(0, std::min(q_lens_host[s], max_q_len));
      if (T <= sqm) {
        split_tokens_sum += T;
        split_t = std::max(split_t, T);
        if (T > 0) split_t_min = split_t_min ? std::min(split_t_min, T) : T;
      } else {
        pf_rows.push_back(T * G);
        ++n_pf_exact;
      }
    }
    pl.split_k = split_tokens_sum > 0;
    pl.split_rows = split_t * G;
    pl.split_rows_min = split_t_min * G;
    pl.part_rows = (int)std::min<long long>(split_tokens_sum, total_q);
    pl.prefill = !pf_rows.empty();
  } else {
    pl.split_k = true;
    pl.split_rows = std::min(max_q_len, sqm) * G;
    pl.split_rows_min = 0;
    pl.prefill = max_q_len > sqm;
    // When every sequence is split-K, all query tokens are; otherwise each split-K sequence
    // holds at most split_q_max of them.
    pl.part_rows = pl.prefill ? (int)std::min<long long>(total_q, (long long)num_seqs * sqm) : total_q;
    // For the workgroup size: as many sequences of max_q_len tokens as total_q allows.
    if (pl.prefill) {
      const int n = (int)std::min<long long>(num_seqs, (total_q + max_q_len - 1) / max_q_len);
      pf_rows.assign(std::max(n, 1), max_q_len * G);
    }
  }
  int pf_ks_plan = 1;
  if (pl.prefill) {
    // Deterministic mode (KVATTN_DETERMINISTIC=1): whole-block plans only.  A row block is then
    // always reduced by one wave over its keys in key order, whatever (W, R) the batch leads to,
    // so a prefill-class sequence's output bits no longer depend on the rest of the batch.  By
    // default a row block may also be split between a pair of half waves (even and odd key
    // blocks, merged at the end): faster when the batch is small, but the merge rounds
    // differently, so the bits follow the plan.
    // The key ranges (below) are chosen with the shape, as part of one makespan model.
    kvp::prefill_plan(pf_rows.data(), (int)pf_rows.size(), p->num_kv_heads, p->num_cus,
                      env_flag("KVATTN_DETERMINISTIC"), max_ctx_len, &pl.waves, &pl.rblk,
                      &pf_ks_plan);
    // sweeps and tests: KVATTN_PREFILL_WAVES fixes W in [4, 12] (then R = W unless
    // KVATTN_PREFILL_RBLK fixes R within [W/2, W], at most 6 pairs)
    if (const char* v = getenv("KVATTN_PREFILL_WAVES")) {
      pl.waves = std::max(4, std::min(12, atoi(v)));
      pl.rblk = pl.waves;
      if (const char* r = getenv("KVATTN_PREFILL_RBLK"))
        pl.rblk = std::max(std::max((pl.waves + 1) / 2, pl.waves - 6), std::min(pl.waves, atoi(r)));
      pf_ks_plan = 0;  // the ranges for the forced shape, below
    }
    if (q_lens_host) {
      pl.pf_wgs = kvp::prefill_wg_count(pf_rows.data(), (int)pf_rows.size(), p->num_kv_heads, pl.rblk);
    } else {
      // n prefill sequences (at most total_q / (split_q_max + 1)) of sum(T) <= total_q hold at
      // most (total_q * G + 31 n) / 32 row blocks, in at most (blocks + n (R - 1)) / R row
      // tiles per KV head.
      const long long n = std::min<long long>(num_seqs, total_q / (sqm + 1));
      const long long blocks = ((long long)total_q * G + 31 * n) / 32;
      pl.pf_wgs = (blocks + n * (pl.rblk - 1)) / pl.rblk * p->num_kv_heads;
    }
  }
  // [partial outputs, fp32][partial (max, sum) pairs, fp32]
  const size_t slots = (size_t)pl.part_rows * num_q_heads * pl.max_splits;
  pl.o_bytes = (slots * p->head_dim * 4 + 255) / 256 * 256;
  pl.bytes = slots ? pl.o_bytes + (slots * 2 * 4 + 255) / 256 * 256 : 0;
  // Prefill key ranges when the row tiles alone leave CUs idle (never in deterministic mode:
  // the ranges follow the batch); KVATTN_PREFILL_KSPLIT fixes their number (tests, sweeps).
  // Partials [total_q][Hq][ranges] of D floats and of (max, sum) pairs.
  pl.pf_ks = 1;
  if (pl.prefill && p->dtype != KV_F32) {  // (fp32 pools run every sequence in attn_vec)
    const bool det = env_flag("KVATTN_DETERMINISTIC");
    pl.pf_ks = pf_ks_plan > 0 ? pf_ks_plan
                              : kvp::prefill_ksplit(pl.pf_wgs, p->num_cus, max_ctx_len, pl.waves,
                                                    pl.rblk, det);
    if (const char* v = getenv("KVATTN_PREFILL_KSPLIT")) pl.pf_ks = std::max(1, std::min(8, atoi(v)));
    if (det) pl.pf_ks = 1;
  }
  if (pl.pf_ks > 1) {
    const size_t pslots = (size_t)total_q * num_q_heads * pl.pf_ks;
    pl.pf_o_off = pl.bytes;
    pl.pf_ml_off = pl.pf_o_off + (pslots * p->head_dim * 4 + 255) / 256 * 256;
    pl.bytes = pl.pf_ml_off + (pslots * 2 * 4 + 255) / 256 * 256;
  }
  pl.bytes_lean = pl.bytes;
  if (p->dtype == KV_I8 && pl.prefill) {
    // [dequantized K][dequantized V][block table], each 256-byte aligned
    pl.dq_seqs = q_lens_host ? n_pf_exact
                             : (int)std::min<long long>(num_seqs, total_q / (sqm + 1));
    pl.dq_mpb = (max_ctx_len + 15) / 16;
    const size_t pool_bytes = (size_t)pl.dq_seqs * pl.dq_mpb * p->num_kv_heads * 16 * p->head_dim * 2;
    pl.dq_off = pl.bytes;
    pl.dq_v_off = pl.dq_off + (pool_bytes + 255) / 256 * 256;
    pl.dq_tbl_off = pl.dq_v_off + (pool_bytes + 255) / 256 * 256;
    pl.bytes = pl.dq_tbl_off + ((size_t)num_seqs * pl.dq_mpb * 4 + 255) / 256 * 256;
  }
  return pl;
}

}  // namespace

int kvattn_workspace_size(const kvpool_t* pool, int32_t num_q_heads, int32_t num_seqs,
                          int32_t total_q, int32_t max_ctx_len, int32_t max_q_len,
                          const int32_t* q_lens_host, size_t* bytes) {
  if (!pool || !bytes) return fail(KV_EINVAL, "pool or bytes is NULL");
  if (num_q_heads <= 0 || num_q_heads % pool->num_kv_heads)
    return fail(KV_EINVAL, "num_q_heads must be a positive multiple of num_kv_heads");
  if (num_seqs < 0 || total_q < 0 || max_ctx_len < 0 || max_q_len < 0)
    return fail(KV_EINVAL, "negative size argument");
  *bytes = make_plan(pool, num_q_heads, num_seqs, total_q, max_ctx_len, max_q_len, q_lens_host).bytes;
  return ok();
}

}  // extern "C"

namespace {

// Sink + window sparsity of a call (window == 0: dense).
struct Sparse {
  int sink, window, min_len;
};

// k_new / v_new (kvattn_append_forward, arguments already checked by append_check): the new
// tokens' rows to append first; null for a plain forward.
int forward_impl(kvpool_t* pool, int32_t layer, const void* q, void* out, int32_t num_q_heads,
                 float scale, const int32_t* block_tables, int32_t max_blocks_per_seq,
                 const int32_t* ctx_lens, const int32_t* q_lens, int32_t num_seqs,
                 int32_t total_q, int32_t max_ctx_len, int32_t max_q_len, Sparse sp,
                 const int32_t* q_lens_host, void* workspace, size_t workspace_bytes,
                 void* stream, const void* k_new = nullptr, const void* v_new = nullptr) {
  if (!pool) return fail(KV_EINVAL, "pool is NULL");
  if (layer < 0 || layer >= pool->num_layers) return fail(KV_EINVAL, "layer %d out of range", layer);
  if (num_q_heads <= 0 || num_q_heads % pool->num_kv_heads)
    return fail(KV_EINVAL, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                num_q_heads, pool->num_kv_heads);
  const int G = num_q_heads / pool->num_kv_heads;
  if (G > 16) return fail(KV_EUNSUPPORTED, "%d q-heads per KV head (at most 16)", G);
  if (num_seqs < 0 || total_q < 0 || max_ctx_len < 0 || max_q_len < 0 || max_blocks_per_seq < 0)
    return fail(KV_EINVAL, "negative size argument");
  if (num_seqs > 65535) return fail(KV_EUNSUPPORTED, "num_seqs %d > 65535", num_seqs);
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY) return fail(KV_EINVAL, "scale must be finite");
  if (num_seqs == 0 || total_q == 0 || max_q_len == 0 || max_ctx_len == 0) return ok();
  if (max_q_len > max_ctx_len) return fail(KV_EINVAL, "max_q_len > max_ctx_len");
  // Every context length is capped at max_blocks_per_seq * block_size: no key, no row.
  if (max_blocks_per_seq == 0) return ok();
  if (!q || !out || !block_tables || !ctx_lens || !q_lens)
    return fail(KV_EINVAL, "NULL device pointer");
  if (!aligned16(q) || !aligned16(out)) return fail(KV_EINVAL, "q and out must be 16-byte aligned");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (current_device_matches(pool) != hipSuccess)
    return fail(KV_EINVAL, "current HIP device is not the pool's device %d", pool->device);
  const Plan pl = make_plan(pool, num_q_heads, num_seqs, total_q, max_ctx_len, max_q_len, q_lens_host);
  if (sp.window > 0) {
    // Sparse attention is a decode / verification mode: the split-K kernel serves it.
    if (pool->dtype == KV_F32)
      return fail(KV_EUNSUPPORTED, "sink + window sparse attention needs a bf16 or int8 pool");
    if (pl.prefill)
      return fail(KV_EUNSUPPORTED,
                  "sink + window sparse attention serves decode and verification rows only "
                  "(q_len <= %d here); %s", pl.split_q_max,
                  q_lens_host ? "a sequence has a longer q_len"
                              : "max_q_len allows longer ones (pass q_lens_host or a smaller max_q_len)");
  }
  if (pl.max_splits > 65535)
    return fail(KV_ERANGE, "%d splits per sequence exceed the launch grid (65535)", pl.max_splits);
  if ((long long)total_q * num_q_heads >= (1ll << 31))
    return fail(KV_ERANGE, "total_q * num_q_heads must stay below 2^31");
  if ((long long)num_seqs * pool->num_kv_heads * 8 * pl.max_splits >= (1ll << 30))
    return fail(KV_ERANGE, "too many work items (splits x KV heads x row tiles) in one call");
  // int8 prefill: the bf16 copy when the workspace holds it (and KVATTN_INT8_PREFILL is not
  // "lds"), else the conversion in LDS, which needs only bytes_lean
  const bool dq = pl.bytes > pl.bytes_lean && workspace && workspace_bytes >= pl.bytes &&
                  !env_is("KVATTN_INT8_PREFILL", "lds");
  const size_t need = dq ? pl.bytes : pl.bytes_lean;
  if (g_no_events && need > workspace_bytes)
    return fail(KV_ENOMEM,
                "this call needs %zu bytes of scratch; the static buffer of the allocation-free "
                "entry point holds %zu (call kvattn_forward with a workspace instead)",
                need, workspace_bytes);
  if (need) {
    if (!workspace) return fail(KV_ENOMEM, "workspace of %zu bytes required", pl.bytes);
    if (workspace_bytes < need)
      return fail(KV_ENOMEM, "workspace has %zu bytes, %zu required", workspace_bytes, need);
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
      return fail(KV_EINVAL, "workspace must be 256-byte aligned");
  }
  if (env_flag("KVPOOL_VALIDATE")) {
    HostMeta m;
    int rc = fetch_meta(block_tables, max_blocks_per_seq, ctx_lens, q_lens, num_seqs, st, m);
    if (rc) return rc;
    rc = validate_meta(pool, m, max_blocks_per_seq, num_seqs, total_q, max_ctx_len, max_q_len);
    if (rc) return rc;
    if (q_lens_host)
      for (int s = 0; s < num_seqs; ++s)
        if (q_lens_host[s] != m.ql[s])
          return fail(KV_ERANGE, "seq %d: q_lens_host %d != q_lens %d", s, q_lens_host[s], m.ql[s]);
  }

  kvp::AttnArgs a;
  a.split_rows_lo = 0;
  a.split_rows_hi = INT32_MAX;
  const size_t lo = (size_t)layer * pool->layer_elems * elt_bytes(pool->dtype);
  a.q = q;
  a.out = out;
  a.k_layer = static_cast<const char*>(pool->k) + lo;
  a.v_layer = static_cast<const char*>(pool->v) + lo;
  const size_t so = (size_t)layer * pool->num_blocks * pool->num_kv_heads * pool->block_size;
  a.k_scale_layer = pool->k_scale ? pool->k_scale + so : nullptr;
  a.v_scale_layer = pool->v_scale ? pool->v_scale + so : nullptr;
  a.block_tables = block_tables;
  a.ctx_lens = ctx_lens;
  a.q_lens = q_lens;
  char* ws = static_cast<char*>(workspace);
  a.part_o = pl.bytes ? reinterpret_cast<float*>(ws) : nullptr;
  a.part_ml = pl.bytes ? reinterpret_cast<float*>(ws + pl.o_bytes) : nullptr;
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.group = G;
  a.block_size = pool->block_size;
  a.block_shift = pool->block_size == 64 ? 6 : 4;
  a.num_blocks = pool->num_blocks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.split_tokens = pl.split;
  a.max_splits = pl.max_splits;
  a.split_q_max = pl.split_q_max;
  a.part_rows = pl.part_rows;
  a.pf_rblk = pl.rblk;
  a.pf_ksplit = pl.pf_ks;
  a.pf_part_o = pl.pf_ks > 1 ? reinterpret_cast<float*>(ws + pl.pf_o_off) : nullptr;
  a.pf_part_ml = pl.pf_ks > 1 ? reinterpret_cast<float*>(ws + pl.pf_ml_off) : nullptr;
  a.sparse_sink = sp.sink;
  a.sparse_window = sp.window;
  a.sparse_min = sp.min_len;
  a.scale_log2 = scale * kvp::LOG2E;
  a.k_new = nullptr;
  a.v_new = nullptr;

  // q / out element bytes (bf16 for int8 pools)
  const int eb = pool->dtype == KV_F32 ? 4 : 2;
  const bool i8 = pool->dtype == KV_I8;
  hipError_t e = hipSuccess;
  const bool vec = pool->dtype == KV_F32 || (pool->dtype == KV_BF16 && sp.window == 0 && !pl.prefill &&
                                              max_q_len == 1 && env_flag("KVATTN_DECODE_VEC"));
  // Split-K sequences of at most 16 rows per KV head beside longer ones (host q_lens): two
  // launches, 16- and 32-row tiles (see below).
  const bool two_launches = pl.split_rows > 16 && pl.split_rows_min > 0 && pl.split_rows_min <= 16;
  if (k_new) {
    // Append inside the split-K kernel when every sequence takes it on persistent waves: bf16
    // pools, and int8 pools whose sequences all run in 32-row tiles (one wave per SIMD, with
    // registers to spare for the quantisation; at two waves per SIMD the 16-row int8 kernel has
    // none).  Otherwise the append kernel runs first, as kvpool_append would.
    const bool fuse = (pool->dtype == KV_BF16 || (i8 && pl.split_rows > 16 && !two_launches)) &&
                      !vec && !pl.prefill && pl.split_k && (pl.split == 0 || pl.split <= 2048);
    if (fuse) {
      a.k_new = k_new;
      a.v_new = v_new;
    } else if (int rc = append_launch(pool, layer, k_new, v_new, block_tables, max_blocks_per_seq,
                                      ctx_lens, q_lens, num_seqs, total_q, max_q_len, st)) {
      return rc;
    }
  }
  if (vec) {
    // One launch for every sequence: split-K sequences in splits, longer ones in one pass.
    // Rows per wave: the template instance just large enough (1, 2, 4, 5 or 8).
    const int rows = max_q_len * G;
    const int r8 = std::min(rows, 8);
    const int rpt = r8 <= 1 ? 1 : r8 <= 2 ? 2 : r8 <= 4 ? 4 : r8 <= 5 ? 5 : 8;
    a.row_tiles = (rows + rpt - 1) / rpt;
    e = timed(K_VEC, st, [&] { return kvp::launch_attn_vec(a, eb, pool->head_dim, rpt, a.row_tiles * pl.max_splits, st); });
  } else {
    // Split-K sequences (decode, verification) on persistent waves, then the prefill kernel
    // for the longer query blocks of the same call.  Each kernel skips the other's sequences.
    if (pl.split_k) {
      // Sequences with rows per KV head in (lo, hi], in 16- or 32-row tiles.
      auto split_launch = [&](int rows, int lo_rows, int hi_rows) {
        const int rpt = rows <= 16 ? 16 : 32;
        kvp::AttnArgs as = a;
        as.row_tiles = (rows + rpt - 1) / rpt;
        as.split_rows_lo = lo_rows;
        as.split_rows_hi = hi_rows;
        return kvp::launch_attn_split_mfma(as, pool->head_dim, rpt, pl.max_splits, pool->num_cus,
                                           i8, st);
      };
      // When the host's q_lens show sequences of at most 16 rows per KV head (decode) beside
      // longer ones (verification), the short ones take the 16-row kernel, which runs twice the
      // waves, and the others the 32-row kernel, one launch after the other.  (One 32-row launch
      // for all would leave most of a decode item's tile empty.)  Timed as one stage.
      e = timed(K_SPLIT_MFMA, st, [&] {
        if (!two_launches) return split_launch(pl.split_rows, 0, INT32_MAX);
        hipError_t r = split_launch(16, 0, 16);
        return r == hipSuccess ? split_launch(pl.split_rows, 16, INT32_MAX) : r;
      });
    }
    if (e == hipSuccess && pl.prefill) {
      kvp::AttnArgs ap = a;
      if (i8 && dq) {
        // dequantize the prefill sequences' tiles into the workspace pool, then run the bf16
        // kernel on it (16-token blocks, its own block table)
        kvp::DequantOut o;
        o.k = reinterpret_cast<uint16_t*>(ws + pl.dq_off);
        o.v = reinterpret_cast<uint16_t*>(ws + pl.dq_v_off);
        o.tables = reinterpret_cast<int32_t*>(ws + pl.dq_tbl_off);
        o.blocks_per_seq = pl.dq_mpb;
        o.max_seqs = pl.dq_seqs;
        e = timed(K_DEQUANT, st, [&] { return kvp::launch_dequant_prefill(a, o, pool->head_dim, st); });
        ap.k_layer = o.k;
        ap.v_layer = o.v;
        ap.block_tables = o.tables;
        ap.max_blocks_per_seq = pl.dq_mpb;
        ap.block_size = 16;
        ap.block_shift = 4;
        ap.num_blocks = std::max(1, pl.dq_seqs * pl.dq_mpb);
      }
      // (int8 pools without the copy: the prefill kernel converts the codes in LDS)
      const bool conv = i8 && !dq;
      if (e == hipSuccess)
        e = timed(K_PREFILL_MFMA, st, [&] { return kvp::launch_attn_prefill_mfma(ap, pool->head_dim, pl.waves, pl.pf_wgs, conv, st); });
    }
  }
  if (e != hipSuccess) return fail(KV_EDEVICE, "attention launch: %s", hipGetErrorString(e));
  // Rows whose keys all fall in split 0 are finished by the attention kernels; when no sequence
  // can have a second split the reduce has nothing to do.  Every split holds at least the rule's
  // floor for the call's longest split-K rows per KV head (a sparse call may have a gap).
  const int min_split = pl.split > 0 ? pl.split
                                     : kvp::split_floor(pl.split_rows, sp.window > 0, i8);
  const bool need_reduce = pl.split_k && max_ctx_len > min_split;
  // The prefill key-range merge, with the split-K merge in the same launch when both are needed
  // (timed as the reduce then).  Both read only metadata and partials, so the original
  // arguments serve (the prefill partials are in them).
  const bool pf_merge = pl.prefill && pl.pf_ks > 1;
  if (pf_merge)
    e = timed(need_reduce ? K_REDUCE : K_REDUCE_PF, st, [&] {
      return kvp::launch_attn_reduce_prefill(a, eb, pool->head_dim, need_reduce, st);
    });
  else if (need_reduce)
    e = timed(K_REDUCE, st, [&] { return kvp::launch_attn_reduce(a, eb, pool->head_dim, st); });
  if (e != hipSuccess) return fail(KV_EDEVICE, "reduce launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int kvattn_forward(kvpool_t* pool, int32_t layer, const void* q, void* out, int32_t num_q_heads,
                   float scale, const int32_t* block_tables, int32_t max_blocks_per_seq,
                   const int32_t* ctx_lens, const int32_t* q_lens, int32_t num_seqs,
                   int32_t total_q, int32_t max_ctx_len, int32_t max_q_len,
                   const int32_t* q_lens_host, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return forward_impl(pool, layer, q, out, num_q_heads, scale, block_tables, max_blocks_per_seq,
                      ctx_lens, q_lens, num_seqs, total_q, max_ctx_len, max_q_len, Sparse{0, 0, 0},
                      q_lens_host, workspace, workspace_bytes, stream);
}

int kvattn_forward_noalloc(kvpool_t* pool, int32_t layer, const void* q, void* out,
                           int32_t num_q_heads, float scale, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* ctx_lens,
                           const int32_t* q_lens, int32_t num_seqs, int32_t total_q,
                           int32_t max_ctx_len, int32_t max_q_len, const int32_t* q_lens_host,
                           void* stream) {
  if (!pool) return fail(KV_EINVAL, "pool is NULL");
  ScratchSlot sl{false, hipSuccess, nullptr};
  if (pool->device >= 0 && pool->device < kMaxDevices) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    sl = g_scratch[pool->device];
  }
  if (!sl.done || sl.err != hipSuccess || !sl.ptr)
    return fail(KV_EDEVICE, "no static scratch on device %d: %s", pool->device,
                sl.done ? hipGetErrorString(sl.err) : "not set up (device id out of range)");
  g_no_events = true;
  const int rc = forward_impl(pool, layer, q, out, num_q_heads, scale, block_tables,
                              max_blocks_per_seq, ctx_lens, q_lens, num_seqs, total_q, max_ctx_len,
                              max_q_len, Sparse{0, 0, 0}, q_lens_host, sl.ptr,
                              KVATTN_NOALLOC_SCRATCH_BYTES, stream);
  g_no_events = false;
  return rc;
}

}  // extern "C"

namespace {
int append_forward_impl(kvpool_t* pool, int32_t layer, const void* k_new, const void* v_new,
                        const void* q, void* out, int32_t num_q_heads, float scale,
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* ctx_lens, const int32_t* q_lens, int32_t num_seqs,
                        int32_t total_q, int32_t max_ctx_len, int32_t max_q_len, Sparse sp,
                        const int32_t* q_lens_host, void* workspace, size_t workspace_bytes,
                        void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  bool nothing = false;
  if (int rc = append_check(pool, layer, k_new, v_new, block_tables, max_blocks_per_seq, ctx_lens,
                            q_lens, num_seqs, total_q, max_q_len, st, &nothing))
    return rc;
  if (nothing)
    return forward_impl(pool, layer, q, out, num_q_heads, scale, block_tables, max_blocks_per_seq,
                        ctx_lens, q_lens, num_seqs, total_q, max_ctx_len, max_q_len, sp,
                        q_lens_host, workspace, workspace_bytes, stream);
  // (forward_impl returns before its launches only when it has no row: then nothing may be
  // appended either, which these bounds guarantee)
  if (max_ctx_len < max_q_len) return fail(KV_EINVAL, "max_q_len > max_ctx_len");
  return forward_impl(pool, layer, q, out, num_q_heads, scale, block_tables, max_blocks_per_seq,
                      ctx_lens, q_lens, num_seqs, total_q, max_ctx_len, max_q_len, sp,
                      q_lens_host, workspace, workspace_bytes, stream, k_new, v_new);
}
}  // namespace

extern "C" {

int kvattn_append_forward(kvpool_t* pool, int32_t layer, const void* k_new, const void* v_new,
                          const void* q, void* out, int32_t num_q_heads, float scale,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* ctx_lens, const int32_t* q_lens, int32_t num_seqs,
                          int32_t total_q, int32_t max_ctx_len, int32_t max_q_len,
                          const int32_t* q_lens_host, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return append_forward_impl(pool, layer, k_new, v_new, q, out, num_q_heads, scale, block_tables,
                             max_blocks_per_seq, ctx_lens, q_lens, num_seqs, total_q, max_ctx_len,
                             max_q_len, Sparse{0, 0, 0}, q_lens_host, workspace, workspace_bytes,
                             stream);
}

int kvattn_append_forward_sparse(kvpool_t* pool, int32_t layer, const void* k_new,
                                 const void* v_new, const void* q, void* out,
                                 int32_t num_q_heads, float scale, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* ctx_lens,
                                 const int32_t* q_lens, int32_t num_seqs, int32_t total_q,
                                 int32_t max_ctx_len, int32_t max_q_len, int32_t sink_tokens,
                                 int32_t window_tokens, int32_t min_ctx_len,
                                 const int32_t* q_lens_host, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (sink_tokens < 0 || window_tokens < 1 || min_ctx_len < 0)
    return fail(KV_EINVAL, "sparse attention needs sink_tokens >= 0, window_tokens >= 1, "
                "min_ctx_len >= 0 (got %d, %d, %d)", sink_tokens, window_tokens, min_ctx_len);
  return append_forward_impl(pool, layer, k_new, v_new, q, out, num_q_heads, scale, block_tables,
                             max_blocks_per_seq, ctx_lens, q_lens, num_seqs, total_q, max_ctx_len,
                             max_q_len, Sparse{sink_tokens, window_tokens, min_ctx_len},
                             q_lens_host, workspace, workspace_bytes, stream);
}

int kvattn_forward_sparse(kvpool_t* pool, int32_t layer, const void* q, void* out,
                          int32_t num_q_heads, float scale, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* ctx_lens,
                          const int32_t* q_lens, int32_t num_seqs, int32_t total_q,
                          int32_t max_ctx_len, int32_t max_q_len, int32_t sink_tokens,
                          int32_t window_tokens, int32_t min_ctx_len,
                          const int32_t* q_lens_host, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (sink_tokens < 0 || window_tokens < 1 || min_ctx_len < 0)
    return fail(KV_EINVAL, "sparse attention needs sink_tokens >= 0, window_tokens >= 1, "
                "min_ctx_len >= 0 (got %d, %d, %d)", sink_tokens, window_tokens, min_ctx_len);
  return forward_impl(pool, layer, q, out, num_q_heads, scale, block_tables, max_blocks_per_seq,
                      ctx_lens, q_lens, num_seqs, total_q, max_ctx_len, max_q_len,
                      Sparse{sink_tokens, window_tokens, min_ctx_len}, q_lens_host, workspace,
                      workspace_bytes, stream);
}

const char* kvpool_last_error(void) { return g_err.c_str(); }

}  // extern "C"

// ---- host page store ----------------------------------------------------------------------
// Pinned host pages that pool blocks are parked in and restored from (park evicted sequences
// in host RAM, restore computed prefixes over PCIe, store pages shared by several sequences
// once: NInfer serving doc, "Server options", --host-kv-cache-mib and --kv-host-cache-mib).

namespace {

using kvp::PageHash;
using kvp::PageHashHasher;

// Pinned host allocation mapped into the GPU's address space: *host for the host, *dev (the
// address the device uses for it) for kernels.
bool alloc_pinned(size_t bytes, void** host, void** dev) {
  *host = *dev = nullptr;
  if (hipHostMalloc(host, bytes, hipHostMallocDefault) != hipSuccess || !*host) {
    *host = nullptr;
    return false;
  }
  if (hipHostGetDevicePointer(dev, *host, 0) != hipSuccess || !*dev) {
    hipHostFree(*host);
    *host = *dev = nullptr;
    return false;
  }
  return true;
}

// Grows a pinned host buffer to at least `bytes` (contents are not kept).
bool grow_pinned(void** p, void** dp, size_t* cap, size_t bytes) {
  if (*cap >= bytes) return true;
  if (*p) hipHostFree(*p);
  *p = *dp = nullptr;
  *cap = 0;
  const size_t want = std::max(bytes, (size_t)4096);
  if (!alloc_pinned(want, p, dp)) return false;
  *cap = want;
  return true;
}

}  // namespace

struct kvhost {
  // geometry of the pools it serves
  int32_t num_layers, num_blocks, block_size, num_kv_heads, head_dim, dtype;
  size_t block_bytes, scale_bytes, page_bytes, page_stride;
  int tensors, segs;
  char* arena = nullptr;  // pinned: capacity page slots of page_stride bytes
  char* arena_dev = nullptr;  // its device address
  int64_t capacity = 0;
  std::vector<int32_t> refs;    // per slot: references (0: free)
  std::vector<uint32_t> gen;    // per slot: generation of the page it holds
  std::vector<PageHash> hash_of;
  std::vector<int32_t> free_slots;
  kvp::PageIndex index;  // stored pages by content hash (several slots only after a collision)
  int64_t references = 0;
  // pinned scratch the kernels read or write
  void* partial = nullptr;  // hash partials
  void* partial_dev = nullptr;
  size_t partial_cap = 0;
  void* ints = nullptr;     // block lists, (block, slot) pairs and comparison triples
  void* ints_dev = nullptr;
  size_t ints_cap = 0;
  std::mutex mu;
};

namespace {

int host_matches(const kvhost* h, const kvpool* p) {
  if (!h || !p) return fail(KV_EINVAL, "store or pool is NULL");
  if (p->num_layers != h->num_layers || p->block_size != h->block_size ||
      p->num_kv_heads != h->num_kv_heads || p->head_dim != h->head_dim || p->dtype != h->dtype)
    return fail(KV_EINVAL, "pool geometry differs from the store's (layers, block size, KV heads, "
                "head dim and dtype must match)");
  if (current_device_matches(p) != hipSuccess)
    return fail(KV_EINVAL, "current HIP device is not the pool's device %d", p->device);
  return KV_OK;
}

kvp::PageArgs page_args(const kvhost* h, const kvpool* p) {
  kvp::PageArgs a;
  a.k = p->k;
  a.v = p->v;
  a.k_scale = p->k_scale;
  a.v_scale = p->v_scale;
  a.num_blocks = p->num_blocks;
  a.tensors = h->tensors;
  a.segs = h->segs;
  a.block_bytes = h->block_bytes;
  a.scale_bytes = h->scale_bytes;
  a.page_stride = h->page_stride;
  return a;
}

int64_t page_id(const kvhost* h, int32_t slot) { return ((int64_t)h->gen[slot] << 32) | slot; }

// Slot of a live page id, or -1.
int32_t slot_of(const kvhost* h, int64_t id) {
  if (id < 0) return -1;
  const int64_t slot = id & 0xffffffffll;
  if (slot >= h->capacity) return -1;
  if (h->refs[slot] <= 0 || (uint32_t)(id >> 32) != h->gen[slot]) return -1;
  return (int32_t)slot;
}

// Hashes of pool blocks blocks[0..n) (host array; validated) into out[n].
int hash_blocks(kvhost* h, kvpool* pool, const int32_t* blocks, int32_t n, hipStream_t st,
                std::vector<PageHash>& out) {
  out.assign(n, PageHash{0, 0});
  if (n == 0) return KV_OK;
  if (!grow_pinned(&h->partial, &h->partial_dev, &h->partial_cap,
                   (size_t)n * h->segs * 2 * sizeof(uint64_t)) ||
      !grow_pinned(&h->ints, &h->ints_dev, &h->ints_cap, (size_t)n * 2 * sizeof(int32_t)))
    return fail(KV_ENOMEM, "pinned host scratch for %d pages", n);
  std::memcpy(h->ints, blocks, (size_t)n * sizeof(int32_t));
  const kvp::PageArgs a = page_args(h, pool);
  const int32_t* ids_dev = static_cast<const int32_t*>(h->ints_dev);
  uint64_t* part_dev = static_cast<uint64_t*>(h->partial_dev);
  const uint64_t* part = static_cast<const uint64_t*>(h->partial);
  hipError_t e = timed(K_PAGE_HASH, st, [&] { return kvp::launch_page_hash(a, ids_dev, n, part_dev, st); });
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(KV_EDEVICE, "page hash: %s", hipGetErrorString(e));
  for (int32_t j = 0; j < n; ++j) {
    uint64_t x = 0, y = 0;  // sums mod 2^64 of the page's segment partials
    for (int g = 0; g < h->segs; ++g) {
      x += part[2 * ((size_t)j * h->segs + g)];
      y += part[2 * ((size_t)j * h->segs + g) + 1];
    }
    out[j] = PageHash{x, y};
  }
  // Test knob: KVHOST_HASH_BITS=k keeps only the low k bits of the hash (k = 0: every page has
  // the same hash), so that distinct pages collide and only the byte comparison tells them apart.
  if (const char* v = getenv("KVHOST_HASH_BITS")) {
    const int k = std::max(0, std::min(64, atoi(v)));
    const uint64_t mask = k >= 64 ? ~0ull : ((1ull << k) - 1);
    for (auto& hh : out) hh = PageHash{hh.a & mask, 0};
  }
  return KV_OK;
}

// Byte comparison of the pairs of one dedup round on the GPU: block pairs[k].block of the call
// (pool block blocks[...]) against a stored page (read from the pinned store over PCIe) or
// against another pool block (read from HBM).  equal[k] = 1 when every segment is the same.
int compare_pages(kvhost* h, kvpool* pool, const int32_t* blocks,
                  const std::vector<kvp::DedupPair>& pairs, std::vector<char>& equal,
                  hipStream_t st);

int check_blocks(const kvpool* pool, const int32_t* blocks, int32_t n, const char* what) {
  for (int32_t j = 0; j < n; ++j)
    if (blocks[j] < 0 || blocks[j] >= pool->num_blocks)
      return fail(KV_ERANGE, "%s[%d] = %d outside [0, %d)", what, j, blocks[j], pool->num_blocks);
  return KV_OK;
}

int compare_pages(kvhost* h, kvpool* pool, const int32_t* blocks,
                  const std::vector<kvp::DedupPair>& pairs, std::vector<char>& equal,
                  hipStream_t st) {
  const size_t m = pairs.size();
  if (!grow_pinned(&h->partial, &h->partial_dev, &h->partial_cap, m * h->segs * sizeof(uint32_t)) ||
      !grow_pinned(&h->ints, &h->ints_dev, &h->ints_cap, m * 3 * sizeof(int32_t)))
    return fail(KV_ENOMEM, "pinned host scratch for %zu page comparisons", m);
  int32_t* tri = static_cast<int32_t*>(h->ints);
  for (size_t k = 0; k < m; ++k) {
    tri[3 * k] = blocks[pairs[k].block];
    tri[3 * k + 1] = pairs[k].stored ? 0 : 1;
    tri[3 * k + 2] = pairs[k].stored ? pairs[k].id : blocks[pairs[k].id];
  }
  const kvp::PageArgs a = page_args(h, pool);
  hipError_t e = timed(K_PAGE_COMPARE, st, [&] {
    return kvp::launch_page_compare(a, static_cast<const int32_t*>(h->ints_dev), (int)m,
                                    h->arena_dev, static_cast<uint32_t*>(h->partial_dev), st);
  });
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(KV_EDEVICE, "page compare: %s", hipGetErrorString(e));
  const uint32_t* diff = static_cast<const uint32_t*>(h->partial);
  for (size_t k = 0; k < m; ++k) {
    uint32_t d = 0;
    for (int g = 0; g < h->segs; ++g) d |= diff[k * h->segs + g];
    equal[k] = d == 0;
  }
  return KV_OK;
}

}  // namespace

extern "C" {

int kvhost_page_bytes(const kvpool_t* pool, size_t* bytes) {
  if (!pool || !bytes) return fail(KV_EINVAL, "pool or bytes is NULL");
  const size_t bb = (size_t)pool->num_kv_heads * pool->block_size * pool->head_dim * elt_bytes(pool->dtype);
  const size_t sb = pool->dtype == KV_I8 ? (size_t)pool->num_kv_heads * pool->block_size * sizeof(float) : 0;
  *bytes = (size_t)pool->num_layers * (2 * bb + 2 * sb);
  return ok();
}

int kvhost_create(kvhost_t** out, const kvpool_t* pool, size_t budget_bytes) {
  if (!out) return fail(KV_EINVAL, "out is NULL");
  *out = nullptr;
  if (!pool) return fail(KV_EINVAL, "pool is NULL");
  size_t pb = 0;
  kvhost_page_bytes(pool, &pb);
  const size_t stride = (pb + 255) / 256 * 256;
  const int64_t cap = (int64_t)(budget_bytes / stride);
  if (cap < 1) return fail(KV_EINVAL, "budget of %zu bytes holds no page of %zu bytes", budget_bytes, stride);
  if (cap > 0x7fffffffll) return fail(KV_ERANGE, "budget holds more than 2^31 - 1 pages");
  kvhost* h = new (std::nothrow) kvhost();
  if (!h) return fail(KV_ENOMEM, "host allocation failed");
  h->num_layers = pool->num_layers;
  h->num_blocks = pool->num_blocks;
  h->block_size = pool->block_size;
  h->num_kv_heads = pool->num_kv_heads;
  h->head_dim = pool->head_dim;
  h->dtype = pool->dtype;
  h->block_bytes = (size_t)pool->num_kv_heads * pool->block_size * pool->head_dim * elt_bytes(pool->dtype);
  h->scale_bytes = pool->dtype == KV_I8 ? (size_t)pool->num_kv_heads * pool->block_size * sizeof(float) : 0;
  h->tensors = pool->dtype == KV_I8 ? 4 : 2;
  h->segs = pool->num_layers * h->tensors;
  h->page_bytes = pb;
  h->page_stride = stride;
  void *arena = nullptr, *arena_dev = nullptr;
  if (!alloc_pinned((size_t)cap * stride, &arena, &arena_dev)) {
    delete h;
    return fail(KV_ENOMEM, "pinned host allocation of %zu bytes failed", (size_t)cap * stride);
  }
  h->arena = static_cast<char*>(arena);
  h->arena_dev = static_cast<char*>(arena_dev);
  h->capacity = cap;
  h->refs.assign(cap, 0);
  h->gen.assign(cap, 0);
  h->hash_of.assign(cap, PageHash{0, 0});
  h->free_slots.reserve(cap);
  for (int64_t i = cap - 1; i >= 0; --i) h->free_slots.push_back((int32_t)i);
  *out = h;
  return ok();
}

int kvhost_destroy(kvhost_t* h) {
  if (!h) return ok();
  if (h->arena) hipHostFree(h->arena);
  if (h->partial) hipHostFree(h->partial);
  if (h->ints) hipHostFree(h->ints);
  delete h;
  return ok();
}

int kvhost_page_hash(kvhost_t* h, kvpool_t* pool, const int32_t* blocks, int32_t n,
                     uint64_t* hashes, void* stream) {
  int rc = host_matches(h, pool);
  if (rc) return rc;
  if (n < 0 || (n > 0 && (!blocks || !hashes))) return fail(KV_EINVAL, "bad block list or output");
  if ((rc = check_blocks(pool, blocks, n, "blocks"))) return rc;
  std::lock_guard<std::mutex> lk(h->mu);
  std::vector<PageHash> hv;
  if ((rc = hash_blocks(h, pool, blocks, n, reinterpret_cast<hipStream_t>(stream), hv))) return rc;
  for (int32_t j = 0; j < n; ++j) {
    hashes[2 * j] = hv[j].a;
    hashes[2 * j + 1] = hv[j].b;
  }
  return ok();
}

int kvhost_park(kvhost_t* h, kvpool_t* pool, const int32_t* blocks, int32_t n, int64_t* page_ids,
                void* stream) {
  int rc = host_matches(h, pool);
  if (rc) return rc;
  if (n < 0 || (n > 0 && (!blocks || !page_ids))) return fail(KV_EINVAL, "bad block list or output");
  if ((rc = check_blocks(pool, blocks, n, "blocks"))) return rc;
  if (n == 0) return ok();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lk(h->mu);
  std::vector<PageHash> hv;
  if ((rc = hash_blocks(h, pool, blocks, n, st, hv))) return rc;
  // Which stored page, or which new page of this call, each block holds: equal hashes only
  // nominate candidates, bytes decide (compared on the GPU).
  std::vector<kvp::DedupRef> ref;
  rc = kvp::dedup_resolve(hv, h->index, [&](const std::vector<kvp::DedupPair>& pairs,
                                            std::vector<char>& equal) {
    return compare_pages(h, pool, blocks, pairs, equal, st);
  }, ref);
  if (rc) return rc;
  // Distinct new pages of this call (the first block holding each), in block order.
  std::vector<int32_t> news;
  for (int32_t j = 0; j < n; ++j)
    if (!ref[j].stored && ref[j].id == j) news.push_back(j);
  if ((int64_t)news.size() > (int64_t)h->free_slots.size())
    return fail(KV_ENOMEM, "store has room for %zu more pages, %zu new ones needed (nothing parked)",
                h->free_slots.size(), news.size());
  if (!grow_pinned(&h->ints, &h->ints_dev, &h->ints_cap, news.size() * 2 * sizeof(int32_t)))
    return fail(KV_ENOMEM, "pinned host scratch for %zu pages", news.size());
  std::vector<int32_t> slots(news.size());
  std::vector<int32_t> slot_of_rep(n, -1);
  int32_t* pairs = static_cast<int32_t*>(h->ints);
  for (size_t k = 0; k < news.size(); ++k) {
    slots[k] = h->free_slots[h->free_slots.size() - 1 - k];
    slot_of_rep[news[k]] = slots[k];
    pairs[2 * k] = blocks[news[k]];
    pairs[2 * k + 1] = slots[k];
  }
  const kvp::PageArgs a = page_args(h, pool);
  hipError_t e = timed(K_PAGE_PARK, st, [&] {
    return kvp::launch_page_park(a, static_cast<const int32_t*>(h->ints_dev), (int)news.size(),
                                 h->arena_dev, st);
  });
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(KV_EDEVICE, "page park: %s", hipGetErrorString(e));
  // The copies are done: commit.
  h->free_slots.resize(h->free_slots.size() - news.size());
  for (size_t k = 0; k < news.size(); ++k) {
    const int32_t sl = slots[k];
    h->gen[sl] += 1;
    h->hash_of[sl] = hv[news[k]];
    h->index[hv[news[k]]].push_back(sl);
  }
  for (int32_t j = 0; j < n; ++j) {
    const int32_t sl = ref[j].stored ? ref[j].id : slot_of_rep[ref[j].id];
    h->refs[sl] += 1;
    page_ids[j] = page_id(h, sl);
  }
  h->references += n;
  return ok();
}

int kvhost_restore(kvhost_t* h, kvpool_t* pool, const int64_t* page_ids, const int32_t* dst_blocks,
                   int32_t n, void* stream) {
  int rc = host_matches(h, pool);
  if (rc) return rc;
  if (n < 0 || (n > 0 && (!page_ids || !dst_blocks))) return fail(KV_EINVAL, "bad page or block list");
  if ((rc = check_blocks(pool, dst_blocks, n, "dst_blocks"))) return rc;
  if (n == 0) return ok();
  std::vector<char> seen(pool->num_blocks, 0);
  for (int32_t j = 0; j < n; ++j) {
    if (seen[dst_blocks[j]]) return fail(KV_EINVAL, "dst_blocks[%d] = %d appears twice", j, dst_blocks[j]);
    seen[dst_blocks[j]] = 1;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lk(h->mu);
  if (!grow_pinned(&h->ints, &h->ints_dev, &h->ints_cap, (size_t)n * 2 * sizeof(int32_t)))
    return fail(KV_ENOMEM, "pinned host scratch for %d pages", n);
  int32_t* pairs = static_cast<int32_t*>(h->ints);
  for (int32_t j = 0; j < n; ++j) {
    const int32_t sl = slot_of(h, page_ids[j]);
    if (sl < 0) return fail(KV_EINVAL, "page_ids[%d] = %lld is not a live page", j, (long long)page_ids[j]);
    pairs[2 * j] = sl;
    pairs[2 * j + 1] = dst_blocks[j];
  }
  const kvp::PageArgs a = page_args(h, pool);
  hipError_t e = timed(K_PAGE_RESTORE, st, [&] {
    return kvp::launch_page_restore(a, static_cast<const int32_t*>(h->ints_dev), n, h->arena_dev,
                                    st);
  });
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return fail(KV_EDEVICE, "page restore: %s", hipGetErrorString(e));
  return ok();
}

int kvhost_release(kvhost_t* h, const int64_t* page_ids, int32_t n) {
  if (!h) return fail(KV_EINVAL, "store is NULL");
  if (n < 0 || (n > 0 && !page_ids)) return fail(KV_EINVAL, "bad page list");
  std::lock_guard<std::mutex> lk(h->mu);
  std::unordered_map<int32_t, int32_t> drop;  // slot -> references dropped by this call
  for (int32_t j = 0; j < n; ++j) {
    const int32_t sl = slot_of(h, page_ids[j]);
    if (sl < 0 || ++drop[sl] > h->refs[sl])
      return fail(KV_EINVAL, "page_ids[%d] = %lld is not a live reference (nothing released)", j,
                  (long long)page_ids[j]);
  }
  for (const auto& d : drop) {
    const int32_t sl = d.first;
    h->refs[sl] -= d.second;
    if (h->refs[sl] == 0) {
      auto it = h->index.find(h->hash_of[sl]);
      if (it != h->index.end()) {
        std::vector<int32_t>& v = it->second;
        v.erase(std::remove(v.begin(), v.end(), sl), v.end());
        if (v.empty()) h->index.erase(it);
      }
      h->free_slots.push_back(sl);
    }
  }
  h->references -= n;
  return ok();
}

int kvhost_stats(const kvhost_t* h, int64_t* pages, int64_t* capacity, int64_t* references) {
  if (!h || !pages || !capacity || !references) return fail(KV_EINVAL, "NULL argument");
  std::lock_guard<std::mutex> lk(const_cast<kvhost*>(h)->mu);
  *pages = h->capacity - (int64_t)h->free_slots.size();
  *capacity = h->capacity;
  *references = h->references;
  return ok();
}

}  // extern "C"
