// kv_append and block_copy for the paged KV cache (gfx950).
//
// kv_append writes each new token's K and V into the slot its slot mapping names
// (the ml-canon page's block-table sketch writes the token into the sequence's last
// block; "Stop Wasting GPU Memory" page, Technical Details, "Single Sequence
// Generation": new tokens fill the remaining slots of the current block).
// block_copy is the device half of copy-on-write: only the diverging block is
// duplicated (same page, "Copy-on-Write for Parallel Sampling").
//
// Both are pure byte movement: bit-exact, no arithmetic on the values.
#include <cstdlib>
#include <cstring>
#include <unordered_set>
#include <vector>

#include "pa_device.h"
#include "pa_status.h"

namespace pa {

// One thread per (token, kv head, 16-byte chunk of head_dim).  K goes to the 16-byte
// chunk [blk][h][chunk][off][0..X) as one vector store; V goes to [blk][h][d][off]
// element by element (V is stored with tokens fastest).
template <int EB>
__device__ __forceinline__ void kv_append_one(const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
                                              const int32_t* __restrict__ slots, int64_t gid, int64_t total,
                                              uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                                              int64_t num_slots, int H, int D, int B) {
  constexpr int X = 16 / EB;
  if (gid >= total) return;
  const int chunks = D / X;
  const int c = static_cast<int>(gid % chunks);
  const int64_t th = gid / chunks;
  const int h = static_cast<int>(th % H);
  const int64_t t = th / H;
  const int32_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / B;
  const int off = slot % B;
  const int64_t src = ((t * H + h) * D + static_cast<int64_t>(c) * X) * EB;
  const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(k_new + src);
  const u32x4_t vv = *reinterpret_cast<const u32x4_t*>(v_new + src);
  const int64_t kdst = ((((blk * H + h) * chunks + c) * B + off) * X) * EB;
  *reinterpret_cast<u32x4_t*>(k_cache + kdst) = kv;
  const int64_t vrow = (blk * H + h) * D + static_cast<int64_t>(c) * X;  // element index of (blk, h, d=c*X)
  if constexpr (EB == 4) {
    float* vc = reinterpret_cast<float*>(v_cache);
#pragma unroll
    for (int e = 0; e < 4; ++e) vc[(vrow + e) * B + off] = __uint_as_float(vv[e]);
  } else {
    uint16_t* vc = reinterpret_cast<uint16_t*>(v_cache);
#pragma unroll
    for (int e = 0; e < 8; ++e) vc[(vrow + e) * B + off] = static_cast<uint16_t>(vv[e / 2] >> (16 * (e % 2)));
  }
}

template <int EB>
__global__ __launch_bounds__(256) void kv_append_kernel(const uint8_t* __restrict__ k_new,
                                                        const uint8_t* __restrict__ v_new,
                                                        const int32_t* __restrict__ slots, int64_t total,
                                                        uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                                                        int64_t num_slots, int H, int D, int B) {
  kv_append_one<EB>(k_new, v_new, slots, static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x, total, k_cache,
                    v_cache, num_slots, H, D, B);
}

// Grid x = pair * chunks_per_block + chunk (4 KiB per workgroup), y = 0 for K, 1 for V.
__global__ __launch_bounds__(256) void block_copy_kernel(uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                                                         const int32_t* __restrict__ pairs, int64_t num_blocks,
                                                         int64_t block_bytes, int64_t chunks_per_block) {
  const int64_t pair = blockIdx.x / chunks_per_block;
  const int64_t chunk = blockIdx.x % chunks_per_block;
  const int32_t src = pairs[2 * pair];
  const int32_t dst = pairs[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint8_t* base = blockIdx.y == 0 ? k_cache : v_cache;
  const int64_t off = chunk * 4096 + static_cast<int64_t>(threadIdx.x) * 16;
  if (off >= block_bytes) return;
  const u32x4_t x = *reinterpret_cast<const u32x4_t*>(base + src * block_bytes + off);
  *reinterpret_cast<u32x4_t*>(base + dst * block_bytes + off) = x;
}


// Copy bytes (a multiple of 4) from pinned host memory the device can address into device
// memory, 16 bytes per thread and a tail of 4-byte words: one kernel on the caller's stream.
__device__ __forceinline__ void stage_copy_one(uint32_t* __restrict__ dst, const uint32_t* __restrict__ src,
                                               int64_t words, int64_t i) {
  const int64_t v = i * 4;
  if (v + 3 < words) {
    *reinterpret_cast<u32x4_t*>(dst + v) = *reinterpret_cast<const u32x4_t*>(src + v);
  } else {
    for (int64_t w = v; w < words; ++w) dst[w] = src[w];
  }
}

__global__ __launch_bounds__(256) void stage_copy_kernel(uint32_t* __restrict__ dst, const uint32_t* __restrict__ src,
                                                         int64_t words) {
  stage_copy_one(dst, src, words, static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x);
}

// Both at once: workgroups [0, copy_wgs) copy, the rest append.  The two parts share no memory.
template <int EB>
__global__ __launch_bounds__(256) void stage_append_kernel(uint32_t* __restrict__ dst, const uint32_t* __restrict__ src,
                                                           int64_t words, int64_t copy_wgs,
                                                           const uint8_t* __restrict__ k_new,
                                                           const uint8_t* __restrict__ v_new,
                                                           const int32_t* __restrict__ slots, int64_t total,
                                                           uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                                                           int64_t num_slots, int H, int D, int B) {
  const int64_t wg = blockIdx.x;
  if (wg < copy_wgs) {
    stage_copy_one(dst, src, words, wg * blockDim.x + threadIdx.x);
  } else {
    kv_append_one<EB>(k_new, v_new, slots, (wg - copy_wgs) * blockDim.x + threadIdx.x, total, k_cache, v_cache,
                      num_slots, H, D, B);
  }
}

static bool cache_desc_ok(const pa_cache_desc* c) {
  if (!c || c->num_blocks <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0 || c->block_size <= 0) return false;
  if (!valid_dtype(c->dtype)) return false;
  const int x = 16 / elem_bytes(c->dtype);
  return c->head_dim % x == 0;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The address a kernel uses for p: pinned host memory goes through the device pointer HIP
// reports for it; device memory is used as is.  nullptr if p is neither.
static const void* device_view(const void* p, bool host_only) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (attr.type == hipMemoryTypeHost) return attr.devicePointer;
  if (host_only) return nullptr;
  return (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) ? p : nullptr;
}

// Debug checks (environment PA_DEBUG_CHECKS set and not "0"): the call reads its device index
// arrays back to the host (a synchronous copy) and rejects what the kernels leave undefined, before
// launching anything.
static bool debug_checks() {
  const char* e = std::getenv("PA_DEBUG_CHECKS");
  return e && *e && std::strcmp(e, "0") != 0;
}

static int32_t read_back(std::vector<int32_t>* out, const int32_t* dev, size_t n, void* stream, const char* what) {
  out->resize(n);
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = hipMemcpy(out->data(), dev, n * sizeof(int32_t), hipMemcpyDefault);
  return PA_HIP_STATUS(what, e);
}

// Copy pairs whose blocks are in range must have src != dst, distinct destinations, and no destination
// that is also a source of the same call (the copies run in parallel).
static bool pairs_ok(const std::vector<int32_t>& v, int64_t num_blocks) {
  std::unordered_set<int32_t> srcs, dsts;
  const size_t n = v.size() / 2;
  for (size_t i = 0; i < n; ++i) {
    const int32_t s = v[2 * i], d = v[2 * i + 1];
    if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) continue;  // skipped by the kernel
    if (s == d || !dsts.insert(d).second) return false;
    srcs.insert(s);
  }
  for (int32_t d : dsts)
    if (srcs.count(d)) return false;
  return true;
}

// Slots in range must be distinct (two tokens written to one slot race).
static bool slots_ok(const std::vector<int32_t>& v, int64_t num_slots) {
  std::unordered_set<int32_t> seen;
  for (int32_t s : v)
    if (s >= 0 && s < num_slots && !seen.insert(s).second) return false;
  return true;
}

}  // namespace pa

using namespace pa;

extern "C" int32_t kv_append(const void* k_new, const void* v_new, const int32_t* slot_mapping, int32_t num_tokens,
                             void* k_cache, void* v_cache, const pa_cache_desc* cache, void* stream) {
  if (!cache_desc_ok(cache) || num_tokens < 0) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return PA_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_INVALID_ARG;
  const int eb = elem_bytes(cache->dtype);
  const int64_t total = static_cast<int64_t>(num_tokens) * cache->num_kv_heads * (cache->head_dim / (16 / eb));
  const int64_t num_slots = cache->num_blocks * cache->block_size;
  const dim3 grid(static_cast<uint32_t>((total + 255) / 256));
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // drop an error some earlier, unrelated HIP call left behind
  if (debug_checks()) {
    std::vector<int32_t> v;
    const int32_t rc = read_back(&v, slot_mapping, static_cast<size_t>(num_tokens), stream, "kv_append: debug check");
    if (rc != PA_OK) return rc;
    if (!slots_ok(v, num_slots)) return PA_ERR_INVALID_ARG;
  }
  if (eb == 4) {
    hipLaunchKernelGGL(kv_append_kernel<4>, grid, dim3(256), 0, s, static_cast<const uint8_t*>(k_new),
                       static_cast<const uint8_t*>(v_new), slot_mapping, total, static_cast<uint8_t*>(k_cache),
                       static_cast<uint8_t*>(v_cache), num_slots, cache->num_kv_heads, cache->head_dim,
                       cache->block_size);
  } else {
    hipLaunchKernelGGL(kv_append_kernel<2>, grid, dim3(256), 0, s, static_cast<const uint8_t*>(k_new),
                       static_cast<const uint8_t*>(v_new), slot_mapping, total, static_cast<uint8_t*>(k_cache),
                       static_cast<uint8_t*>(v_cache), num_slots, cache->num_kv_heads, cache->head_dim,
                       cache->block_size);
  }
  return PA_HIP_STATUS("kv_append", hipGetLastError());
}

extern "C" int32_t block_copy(void* k_cache, void* v_cache, const int32_t* pairs, int32_t num_pairs,
                              const pa_cache_desc* cache, void* stream) {
  if (!cache_desc_ok(cache) || num_pairs < 0) return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !pairs) return PA_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_INVALID_ARG;
  const int64_t block_bytes = static_cast<int64_t>(cache->num_kv_heads) * cache->head_dim * cache->block_size *
                              elem_bytes(cache->dtype);
  const int64_t chunks = (block_bytes + 4095) / 4096;
  const int64_t nwg = chunks * num_pairs;
  if (nwg > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
  (void)hipGetLastError();  // drop an error some earlier, unrelated HIP call left behind
  if (debug_checks()) {
    std::vector<int32_t> v;
    const int32_t rc = read_back(&v, pairs, 2 * static_cast<size_t>(num_pairs), stream, "block_copy: debug check");
    if (rc != PA_OK) return rc;
    if (!pairs_ok(v, cache->num_blocks)) return PA_ERR_INVALID_ARG;
  }
  hipLaunchKernelGGL(block_copy_kernel, dim3(static_cast<uint32_t>(nwg), 2), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                     pairs, cache->num_blocks, block_bytes, chunks);
  return PA_HIP_STATUS("block_copy", hipGetLastError());
}

extern "C" int32_t pa_device_address(const void* p, const void** out) {
  if (!p || !out) return PA_ERR_INVALID_ARG;
  const void* d = device_view(p, false);
  if (!d) return PA_ERR_INVALID_ARG;
  *out = d;
  return PA_OK;
}

extern "C" int32_t pa_stage_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (bytes == 0) return PA_OK;
  if (!dst || !src || bytes % 4 != 0) return PA_ERR_INVALID_ARG;
  if (!aligned16(dst) || !aligned16(src)) return PA_ERR_INVALID_ARG;
  const int64_t words = static_cast<int64_t>(bytes / 4);
  const int64_t threads = (words + 3) / 4;
  if ((threads + 255) / 256 > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
  (void)hipGetLastError();  // drop an error some earlier, unrelated HIP call left behind
  // src must be pinned host memory the device can address; use the address HIP reports for it.
  const uint32_t* dsrc = static_cast<const uint32_t*>(device_view(src, true));
  if (!dsrc || !aligned16(dsrc)) return PA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(stage_copy_kernel, dim3(static_cast<uint32_t>((threads + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint32_t*>(dst), dsrc, words);
  return PA_HIP_STATUS("pa_stage_copy", hipGetLastError());
}

extern "C" int32_t pa_stage_append(void* dst, const void* src, size_t bytes, const void* k_new, const void* v_new,
                                   const int32_t* slot_mapping, int32_t num_tokens, void* k_cache, void* v_cache,
                                   const pa_cache_desc* cache, void* stream) {
  if (!cache_desc_ok(cache) || num_tokens < 0) return PA_ERR_INVALID_ARG;
  if (bytes % 4 != 0 || (bytes > 0 && (!dst || !src || !aligned16(dst) || !aligned16(src)))) return PA_ERR_INVALID_ARG;
  if (num_tokens > 0 && (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache)) return PA_ERR_INVALID_ARG;
  if (num_tokens > 0 && (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache)))
    return PA_ERR_INVALID_ARG;
  if (bytes == 0 && num_tokens == 0) return PA_OK;
  (void)hipGetLastError();  // drop an error some earlier, unrelated HIP call left behind
  const uint32_t* dsrc = nullptr;
  if (bytes > 0) {
    dsrc = static_cast<const uint32_t*>(device_view(src, true));
    if (!dsrc || !aligned16(dsrc)) return PA_ERR_INVALID_ARG;
  }
  const int32_t* dslots = nullptr;
  if (num_tokens > 0) {
    dslots = static_cast<const int32_t*>(device_view(slot_mapping, false));
    if (!dslots) return PA_ERR_INVALID_ARG;
  }
  const int64_t words = static_cast<int64_t>(bytes / 4);
  const int64_t copy_wgs = ((words + 3) / 4 + 255) / 256;
  const int eb = elem_bytes(cache->dtype);
  const int64_t total = static_cast<int64_t>(num_tokens) * cache->num_kv_heads * (cache->head_dim / (16 / eb));
  const int64_t append_wgs = (total + 255) / 256;
  if (copy_wgs + append_wgs > 0x7fffffffLL) return PA_ERR_UNSUPPORTED;
  const int64_t num_slots = cache->num_blocks * cache->block_size;
  const dim3 grid(static_cast<uint32_t>(copy_wgs + append_wgs));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (eb == 4) {
    hipLaunchKernelGGL(stage_append_kernel<4>, grid, dim3(256), 0, st, static_cast<uint32_t*>(dst), dsrc, words,
                       copy_wgs, static_cast<const uint8_t*>(k_new), static_cast<const uint8_t*>(v_new), dslots, total,
                       static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), num_slots, cache->num_kv_heads,
                       cache->head_dim, cache->block_size);
  } else {
    hipLaunchKernelGGL(stage_append_kernel<2>, grid, dim3(256), 0, st, static_cast<uint32_t*>(dst), dsrc, words,
                       copy_wgs, static_cast<const uint8_t*>(k_new), static_cast<const uint8_t*>(v_new), dslots, total,
                       static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache), num_slots, cache->num_kv_heads,
                       cache->head_dim, cache->block_size);
  }
  return PA_HIP_STATUS("pa_stage_append", hipGetLastError());
}
