// Pool blocks <-> pinned host pages: content hashing, park (device -> host) and restore
// (host -> device).
//
// Evicted sequences can be parked in pinned host memory instead of being discarded, and computed
// prefixes restored over PCIe instead of being recomputed, with pages shared by several
// sequences stored once (NInfer serving doc, "Server options": --host-kv-cache-mib and
// --kv-host-cache-mib).  A page is one pool block across every layer: for each layer its K
// bytes, its V bytes and, for an int8 pool, its K and V scale bytes.  The host keeps the store;
// these kernels move the data.  The host page store is mapped into the GPU's address space
// (pinned with hipHostMalloc), so the copies are plain kernel loads and stores over PCIe with
// no staging buffer in device memory.
//
// Work unit: one 256-thread workgroup per (pair, segment), a segment being one (layer, tensor)
// slice of a page.  Page hashes: word w_i (64-bit little-endian, i counted over the whole page)
// contributes fmix64(w_i + K1 (i + 1)) to h1 and fmix64(w_i ^ K2 (i + 1)) to h2, summed mod
// 2^64 (fmix64: the MurmurHash3 finalizer); each workgroup writes its segment's two partial
// sums, and the host adds a page's segments.  Integer sums do not depend on their order, so the
// hash is exact whatever the thread layout.
#include "common.h"
#include "kernels.h"

namespace kvp {

namespace {

__device__ __forceinline__ uint64_t fmix64(uint64_t k) {
  k ^= k >> 33;
  k *= 0xFF51AFD7ED558CCDull;
  k ^= k >> 33;
  k *= 0xC4CEB9FE1A85EC53ull;
  k ^= k >> 33;
  return k;
}
constexpr uint64_t KEY1 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t KEY2 = 0xD6E8FEB86659FD93ull;

// Segment `seg` of a page: its device address for pool block b, its byte offset within the
// page and its length.
__device__ __forceinline__ void segment(const PageArgs& a, int b, int seg, const char*& dev,
                                        size_t& page_off, size_t& bytes) {
  const int layer = seg / a.tensors, t = seg - layer * a.tensors;
  const size_t per_layer = 2 * a.block_bytes + (a.tensors > 2 ? 2 * a.scale_bytes : 0);
  const size_t lb = (size_t)layer * a.num_blocks + b;
  if (t < 2) {
    dev = static_cast<const char*>(t == 0 ? a.k : a.v) + lb * a.block_bytes;
    page_off = (size_t)layer * per_layer + t * a.block_bytes;
    bytes = a.block_bytes;
  } else {
    dev = reinterpret_cast<const char*>(t == 2 ? a.k_scale : a.v_scale) + lb * a.scale_bytes;
    page_off = (size_t)layer * per_layer + 2 * a.block_bytes + (t - 2) * a.scale_bytes;
    bytes = a.scale_bytes;
  }
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__global__ __launch_bounds__(256) void page_hash_kernel(PageArgs a, const int32_t* blocks,
                                                        uint64_t* partial) {
  const int j = blockIdx.x / a.segs, seg = blockIdx.x - j * a.segs;
  const int b = blocks[j];
  const char* src;
  size_t off, bytes;
  segment(a, b, seg, src, off, bytes);
  const u32x4* p = reinterpret_cast<const u32x4*>(src);
  const size_t n16 = bytes / 16;
  const uint64_t w0 = off / 8;  // page word index of the segment's first word
  uint64_t h1 = 0, h2 = 0;
  for (size_t u = threadIdx.x; u < n16; u += 256) {
    const u32x4 x = p[u];
    const uint64_t wa = (uint64_t)x[0] | ((uint64_t)x[1] << 32);
    const uint64_t wb = (uint64_t)x[2] | ((uint64_t)x[3] << 32);
    const uint64_t ia = w0 + 2 * u + 1, ib = ia + 1;  // positions counted from 1
    h1 += fmix64(wa + KEY1 * ia) + fmix64(wb + KEY1 * ib);
    h2 += fmix64(wa ^ (KEY2 * ia)) + fmix64(wb ^ (KEY2 * ib));
  }
  h1 = wave_sum_u64(h1);
  h2 = wave_sum_u64(h2);
  __shared__ uint64_t s[2][4];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s[0][wave] = h1;
    s[1][wave] = h2;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t* o = partial + 2 * (size_t)blockIdx.x;
    o[0] = s[0][0] + s[0][1] + s[0][2] + s[0][3];
    o[1] = s[1][0] + s[1][1] + s[1][2] + s[1][3];
  }
}

// pairs[2j] = pool block, pairs[2j + 1] = page slot in the host store.
__global__ __launch_bounds__(256) void page_park_kernel(PageArgs a, const int32_t* pairs,
                                                        char* store) {
  const int j = blockIdx.x / a.segs, seg = blockIdx.x - j * a.segs;
  const int b = pairs[2 * j], slot = pairs[2 * j + 1];
  const char* src;
  size_t off, bytes;
  segment(a, b, seg, src, off, bytes);
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  u32x4* d = reinterpret_cast<u32x4*>(store + (size_t)slot * a.page_stride + off);
  const int n16 = (int)(bytes / 16);
  for (int u = threadIdx.x; u < n16; u += 256) __builtin_nontemporal_store(s[u], d + u);
}

// pairs[2j] = page slot in the host store, pairs[2j + 1] = destination pool block.  Each thread
// issues its host reads four at a time (they cross PCIe), then writes them.
__global__ __launch_bounds__(256) void page_restore_kernel(PageArgs a, const int32_t* pairs,
                                                           const char* store) {
  const int j = blockIdx.x / a.segs, seg = blockIdx.x - j * a.segs;
  const int slot = pairs[2 * j], b = pairs[2 * j + 1];
  const char* dst;
  size_t off, bytes;
  segment(a, b, seg, dst, off, bytes);
  const u32x4* s = reinterpret_cast<const u32x4*>(store + (size_t)slot * a.page_stride + off);
  u32x4* d = reinterpret_cast<u32x4*>(const_cast<char*>(dst));
  const int n16 = (int)(bytes / 16);
  int u = threadIdx.x;
  for (; u + 3 * 256 < n16; u += 4 * 256) {
    const u32x4 x0 = s[u], x1 = s[u + 256], x2 = s[u + 512], x3 = s[u + 768];
    d[u] = x0;
    d[u + 256] = x1;
    d[u + 512] = x2;
    d[u + 768] = x3;
  }
  for (; u < n16; u += 256) d[u] = s[u];
}

// triples[3j] = pool block; triples[3j + 1] = 0: compare with store slot triples[3j + 2] (read
// over PCIe), 1: with pool block triples[3j + 2].  diff[(j, seg)] = 1 when the segment differs.
// Dedup merges two pages only when every segment compares equal (a hash only nominates them).
__global__ __launch_bounds__(256) void page_compare_kernel(PageArgs a, const int32_t* triples,
                                                           const char* store, uint32_t* diff) {
  const int j = blockIdx.x / a.segs, seg = blockIdx.x - j * a.segs;
  const int b = triples[3 * j], kind = triples[3 * j + 1], other = triples[3 * j + 2];
  const char* src;
  size_t off, bytes;
  segment(a, b, seg, src, off, bytes);
  const u32x4* x = reinterpret_cast<const u32x4*>(src);
  const u32x4* y;
  if (kind == 0) {
    y = reinterpret_cast<const u32x4*>(store + (size_t)other * a.page_stride + off);
  } else {
    const char* src2;
    size_t off2, bytes2;
    segment(a, other, seg, src2, off2, bytes2);
    y = reinterpret_cast<const u32x4*>(src2);
  }
  const int n16 = (int)(bytes / 16);
  uint32_t d = 0;
  for (int u = threadIdx.x; u < n16; u += 256) {
    const u32x4 p = x[u], q = y[u];
    d |= (p[0] ^ q[0]) | (p[1] ^ q[1]) | (p[2] ^ q[2]) | (p[3] ^ q[3]);
  }
  const int any = __syncthreads_or(d != 0u);
  if (threadIdx.x == 0) diff[blockIdx.x] = any ? 1u : 0u;
}

}  // namespace

hipError_t launch_page_compare(const PageArgs& a, const int32_t* triples, int n, const char* store,
                               uint32_t* diff, hipStream_t st) {
  const long long wgs = (long long)n * a.segs;
  if (wgs <= 0) return hipSuccess;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  page_compare_kernel<<<(unsigned)wgs, 256, 0, st>>>(a, triples, store, diff);
  return hipGetLastError();
}

hipError_t launch_page_hash(const PageArgs& a, const int32_t* blocks, int n, uint64_t* partial,
                            hipStream_t st) {
  const long long wgs = (long long)n * a.segs;
  if (wgs <= 0) return hipSuccess;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  page_hash_kernel<<<(unsigned)wgs, 256, 0, st>>>(a, blocks, partial);
  return hipGetLastError();
}

hipError_t launch_page_park(const PageArgs& a, const int32_t* pairs, int n, char* store,
                            hipStream_t st) {
  const long long wgs = (long long)n * a.segs;
  if (wgs <= 0) return hipSuccess;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  page_park_kernel<<<(unsigned)wgs, 256, 0, st>>>(a, pairs, store);
  return hipGetLastError();
}

hipError_t launch_page_restore(const PageArgs& a, const int32_t* pairs, int n, const char* store,
                               hipStream_t st) {
  const long long wgs = (long long)n * a.segs;
  if (wgs <= 0) return hipSuccess;
  if (wgs > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  page_restore_kernel<<<(unsigned)wgs, 256, 0, st>>>(a, pairs, store);
  return hipGetLastError();
}

}  // namespace kvp
