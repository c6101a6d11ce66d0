// block_ops.hip -- whole-block operations on the paged KV pools for gfx950: copy-on-write
// block copies inside the pools and block swap between the device pools and pinned host
// pools, behind the C ABI declared in include/pagedkv.h ("vllm-project-vllm -- L2", section 9
// "Memory Management": COW sharing and forks, swapping blocks to CPU memory).  Both are plain
// HBM (or host-link) streams: one workgroup per (block pair, pool), 16-byte accesses, four in
// flight per thread.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "host_util.h"
#include "pagedkv.h"

namespace {

using namespace pkv_host;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Copy-on-write copies inside a pool pair: workgroup (i, pool) copies block src[i] to dst[i]
// of the K (pool 0) or V (pool 1) cache, 16 bytes per thread per step.  A pair with an id
// outside [0, num_blocks) is skipped.
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* kc, char* vc, const int32_t* src,
                                                         const int32_t* dst, int num_blocks,
                                                         long long chunks) {
  const int i = blockIdx.x;
  const int sb = src[i], db = dst[i];
  if (sb < 0 || sb >= num_blocks || db < 0 || db >= num_blocks) return;
  char* pool = blockIdx.y ? vc : kc;
  const u32x4* from = (const u32x4*)(pool + (size_t)sb * (size_t)chunks * 16);
  u32x4* to = (u32x4*)(pool + (size_t)db * (size_t)chunks * 16);
  long long j = threadIdx.x;
  for (; j + 768 < chunks; j += 1024) {
    const u32x4 a = from[j], b = from[j + 256], c = from[j + 512], d = from[j + 768];
    to[j] = a;
    to[j + 256] = b;
    to[j + 512] = c;
    to[j + 768] = d;
  }
  for (; j < chunks; j += 256) to[j] = from[j];
}

// Block swap between a device pool and a pinned host pool of the same block shape: workgroup
// (i, pool) moves device block dev[i] to host block host[i] (to_host) or back.  The host
// pools are addressed through their device-visible mapping; the transfer crosses the host
// link.  A pair with an id outside its pool is skipped.
__global__ __launch_bounds__(256) void swap_blocks_kernel(char* kc, char* vc, char* hk, char* hv,
                                                         const int32_t* dev, const int32_t* host,
                                                         int num_blocks, int num_host_blocks,
                                                         long long chunks, int to_host) {
  const int i = blockIdx.x;
  const int db = dev[i], hb = host[i];
  if (db < 0 || db >= num_blocks || hb < 0 || hb >= num_host_blocks) return;
  char* dpool = blockIdx.y ? vc : kc;
  char* hpool = blockIdx.y ? hv : hk;
  u32x4* d = (u32x4*)(dpool + (size_t)db * (size_t)chunks * 16);
  u32x4* h = (u32x4*)(hpool + (size_t)hb * (size_t)chunks * 16);
  const u32x4* from = to_host ? d : h;
  u32x4* to = to_host ? h : d;
  long long j = threadIdx.x;
  for (; j + 768 < chunks; j += 1024) {
    const u32x4 a = from[j], b = from[j + 256], c = from[j + 512], e = from[j + 768];
    to[j] = a;
    to[j + 256] = b;
    to[j + 512] = c;
    to[j + 768] = e;
  }
  for (; j < chunks; j += 256) to[j] = from[j];
}

// Bytes of one block of a pool, or -1 for an unsupported shape.
long long block_bytes_of(int block_size, int num_kv_heads, int head_dim, int cache_dtype) {
  if (block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0) return -1;
  if (cache_dtype != PKV_F16 && cache_dtype != PKV_BF16 && cache_dtype != PKV_FP8_E4M3) return -1;
  const long long e = cache_dtype == PKV_FP8_E4M3 ? 1 : 2;
  const long long bytes = (long long)block_size * num_kv_heads * head_dim * e;
  return bytes % 16 == 0 ? bytes : -1;
}

// Device-visible address of pinned host memory covering [p, p + bytes), or nullptr.  A failed
// query leaves an error in the runtime's last-error slot; it is cleared here so that it is not
// reported by a later call's launch check.
char* mapped_host(void* p, size_t bytes) {
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, p, 0) != hipSuccess || !d) {
    (void)hipGetLastError();
    return nullptr;
  }
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)d) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  const uintptr_t lo = (uintptr_t)base, at = (uintptr_t)d;
  if (at < lo || at - lo + bytes > size) return nullptr;
  return (char*)d;
}

// Checked mode: every id in range, targets b distinct, and (same_pool) no target is also a
// source (a copy would then read another copy's result).
bool check_pairs(const int32_t* a, const int32_t* b, int n, int na, int nb, bool same_pool,
                 hipStream_t st) {
  std::vector<int32_t> ha, hb;
  if (!copy_to_host(ha, a, (size_t)n, st) || !copy_to_host(hb, b, (size_t)n, st)) return false;
  std::vector<char> seen_b((size_t)nb, 0), is_a((size_t)na, 0);
  for (int i = 0; i < n; ++i) {
    if (ha[i] < 0 || ha[i] >= na || hb[i] < 0 || hb[i] >= nb) return false;
    is_a[(size_t)ha[i]] = 1;
  }
  for (int i = 0; i < n; ++i) {
    if (seen_b[(size_t)hb[i]]) return false;
    seen_b[(size_t)hb[i]] = 1;
    if (same_pool && is_a[(size_t)hb[i]]) return false;
  }
  return true;
}

}  // namespace

extern "C" {

int paged_kv_copy_blocks(void* key_cache, void* value_cache, const int32_t* src_blocks,
                         const int32_t* dst_blocks, int num_pairs, int num_blocks, int block_size,
                         int num_kv_heads, int head_dim, int cache_dtype, void* stream) {
  if (num_pairs < 0 || num_blocks < 0) return PKV_ERR_SHAPE;
  if (cache_dtype != PKV_F16 && cache_dtype != PKV_BF16 && cache_dtype != PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  const long long bb = block_bytes_of(block_size, num_kv_heads, head_dim, cache_dtype);
  if (bb < 0) return PKV_ERR_SHAPE;
  if (num_pairs == 0) return PKV_OK;
  if (!key_cache || !value_cache || !src_blocks || !dst_blocks) return PKV_ERR_NULL;
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16) || !aligned(src_blocks, 4) ||
      !aligned(dst_blocks, 4))
    return PKV_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  if (check_mode() && !check_pairs(src_blocks, dst_blocks, num_pairs, num_blocks, num_blocks, true, st))
    return PKV_ERR_CHECK;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, 2), dim3(256), 0, st, (char*)key_cache,
                     (char*)value_cache, src_blocks, dst_blocks, num_blocks, bb / 16);
  return launch_status();
}

int paged_kv_swap_blocks(void* key_cache, void* value_cache, void* host_key, void* host_value,
                         const int32_t* dev_blocks, const int32_t* host_blocks, int num_pairs,
                         int num_blocks, int num_host_blocks, int block_size, int num_kv_heads,
                         int head_dim, int cache_dtype, int to_host, void* stream) {
  if (num_pairs < 0 || num_blocks < 0 || num_host_blocks < 0) return PKV_ERR_SHAPE;
  if (cache_dtype != PKV_F16 && cache_dtype != PKV_BF16 && cache_dtype != PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  const long long bb = block_bytes_of(block_size, num_kv_heads, head_dim, cache_dtype);
  if (bb < 0 || (to_host != 0 && to_host != 1)) return PKV_ERR_SHAPE;
  if (num_pairs == 0) return PKV_OK;
  if (!key_cache || !value_cache || !host_key || !host_value || !dev_blocks || !host_blocks)
    return PKV_ERR_NULL;
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16) || !aligned(host_key, 16) ||
      !aligned(host_value, 16) || !aligned(dev_blocks, 4) || !aligned(host_blocks, 4))
    return PKV_ERR_ALIGN;
  const size_t host_bytes = (size_t)num_host_blocks * (size_t)bb;
  char* hk = mapped_host(host_key, host_bytes);
  char* hv = mapped_host(host_value, host_bytes);
  if (!hk || !hv) return PKV_ERR_HOST;
  hipStream_t st = (hipStream_t)stream;
  if (check_mode()) {
    // targets must be distinct; sources may repeat
    const bool ok = to_host ? check_pairs(dev_blocks, host_blocks, num_pairs, num_blocks, num_host_blocks, false, st)
                            : check_pairs(host_blocks, dev_blocks, num_pairs, num_host_blocks, num_blocks, false, st);
    if (!ok) return PKV_ERR_CHECK;
  }
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(num_pairs, 2), dim3(256), 0, st, (char*)key_cache,
                     (char*)value_cache, hk, hv, dev_blocks, host_blocks, num_blocks, num_host_blocks,
                     bb / 16, to_host);
  return launch_status();
}

}  // extern "C"
