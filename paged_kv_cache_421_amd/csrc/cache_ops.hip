// pa_write_kv, pa_copy_blocks and pa_swap_blocks for gfx950.
//
// write: each decode iteration stores the new token's K and V in its
// sequence's current block (ybb.press, "vLLM PagedAttention 大模型推理架构深度实战",
// §6); the destination of each row is a flat slot = block * 16 + offset.
// copy: copy-on-write duplicates a shared block before it is modified
// (same page, §2.3); a pair copies the whole block of both caches.
// swap: the same whole-block copies between the device cache and a pinned
// host pool, when sequences are swapped out under memory pressure and back
// in (same page, §3.2, §6, §9 item 5).
//
// All kernels are pure data movement: one lane moves 16 source bytes, so a
// wave moves 1 KiB per instruction with fully coalesced accesses.
#include <hip/hip_runtime.h>

#include <cmath>

#include "debug_checks.h"
#include "device_common.h"
#include "status.h"

namespace pagedkv {

// One lane per 16-byte chunk of a source row [Hkv][D]; grid.y selects K or V.
// A token's row of one head is contiguous in the cache, so every chunk is
// one store.
template <typename SrcChunk, int kElems, int kFmt>
__global__ void __launch_bounds__(256)
write_kv_kernel(char* __restrict__ k_cache, char* __restrict__ v_cache,
                const char* __restrict__ k, const char* __restrict__ v,
                const int64_t* __restrict__ slot_mapping, int64_t num_chunks,
                int chunks_per_row, int chunks_per_head, int hkv, int d, int bs,
                float k_inv, float v_inv) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= num_chunks) return;
  const bool is_v = blockIdx.y != 0;
  const int64_t tok = idx / chunks_per_row;
  const int rem = static_cast<int>(idx - tok * chunks_per_row);
  const int64_t slot = slot_mapping[tok];
  if (slot < 0) return;
  const int g = rem / chunks_per_head;
  const int c = rem - g * chunks_per_head;
  const int64_t blk = slot / bs;
  const int off = static_cast<int>(slot % bs);
  const int64_t dst_elem = ((blk * hkv + g) * bs + off) * d + c * kElems;
  const SrcChunk src = reinterpret_cast<const SrcChunk*>(is_v ? v : k)[idx];
  char* cache = is_v ? v_cache : k_cache;
  if constexpr (kFmt == PA_FP8_E4M3) {
    const float inv = is_v ? v_inv : k_inv;
    uint32_t codes[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      codes[2 * i] = e4m3_encode(bf16_lo(src[i]) * inv);
      codes[2 * i + 1] = e4m3_encode(bf16_hi(src[i]) * inv);
    }
    u32x2_t out;
    out[0] = codes[0] | (codes[1] << 8) | (codes[2] << 16) | (codes[3] << 24);
    out[1] = codes[4] | (codes[5] << 8) | (codes[6] << 16) | (codes[7] << 24);
    *reinterpret_cast<u32x2_t*>(cache + dst_elem) = out;
  } else {
    constexpr int kBytes = sizeof(SrcChunk) / kElems;
    *reinterpret_cast<SrcChunk*>(cache + dst_elem * kBytes) = src;
  }
}

// Whole-block copies from one pool to another (the same pool for
// copy-on-write; device cache and pinned host pool for swapping).  One lane
// per 16-byte chunk of a block; grid.y = pair, grid.z = K or V.
__global__ void __launch_bounds__(256)
copy_blocks_kernel(const char* __restrict__ src_k, const char* __restrict__ src_v,
                   char* __restrict__ dst_k, char* __restrict__ dst_v,
                   const int32_t* __restrict__ pairs, int64_t block_bytes) {
  const int64_t chunk = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (chunk * 16 >= block_bytes) return;
  const int64_t src = pairs[2 * blockIdx.y];
  const int64_t dst = pairs[2 * blockIdx.y + 1];
  const char* from = blockIdx.z ? src_v : src_k;
  char* to = blockIdx.z ? dst_v : dst_k;
  const u32x4_t x = *reinterpret_cast<const u32x4_t*>(from + src * block_bytes + chunk * 16);
  *reinterpret_cast<u32x4_t*>(to + dst * block_bytes + chunk * 16) = x;
}

int dtype_bytes(int dt) {
  switch (dt) {
    case PA_F32: return 4;
    case PA_BF16: return 2;
    case PA_FP8_E4M3: return 1;
    default: return 0;
  }
}

pa_status check_desc(const pa_cache_desc* c, const char* fn) {
  if (!c) return fail(PA_ERR_INVALID_ARG, "%s: null cache descriptor", fn);
  if (c->block_size != 8 && c->block_size != 16 && c->block_size != 32 && c->block_size != 64)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (8, 16, 32 or 64)", fn, c->block_size);
  if (c->num_blocks < 0 || c->num_kv_heads <= 0)
    return fail(PA_ERR_INVALID_ARG, "%s: num_blocks %d, num_kv_heads %d", fn,
                c->num_blocks, c->num_kv_heads);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128)", fn, c->head_dim);
  if (dtype_bytes(c->cache_dtype) == 0)
    return fail(PA_ERR_INVALID_ARG, "%s: cache_dtype %d", fn, c->cache_dtype);
  if (c->cache_dtype == PA_FP8_E4M3 &&
      !(std::isfinite(c->k_scale) && c->k_scale > 0.f && std::isfinite(c->v_scale) &&
        c->v_scale > 0.f))
    return fail(PA_ERR_INVALID_ARG, "%s: fp8 scales must be finite and > 0", fn);
  return PA_OK;
}

pa_status launch_status(const char* fn) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return PA_OK;
}

}  // namespace pagedkv

using namespace pagedkv;

extern "C" size_t pa_cache_bytes(const pa_cache_desc* c) {
  if (check_desc(c, "pa_cache_bytes") != PA_OK) return 0;
  return static_cast<size_t>(c->num_blocks) * c->num_kv_heads * c->block_size * c->head_dim *
         dtype_bytes(c->cache_dtype);
}

extern "C" pa_status pa_write_kv(const pa_cache_desc* c, void* k_cache, void* v_cache,
                                 const void* k, const void* v, int32_t src_dtype,
                                 const int64_t* slot_mapping, int32_t num_tokens,
                                 void* stream) {
  pa_status st = check_desc(c, "pa_write_kv");
  if (st != PA_OK) return st;
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "pa_write_kv: num_tokens < 0");
  const bool ok_combo = (src_dtype == PA_F32 && c->cache_dtype == PA_F32) ||
                        (src_dtype == PA_BF16 && c->cache_dtype == PA_BF16) ||
                        (src_dtype == PA_BF16 && c->cache_dtype == PA_FP8_E4M3);
  if (!ok_combo)
    return fail(PA_ERR_UNSUPPORTED, "pa_write_kv: source dtype %d into cache dtype %d",
                src_dtype, c->cache_dtype);
  if (num_tokens == 0) return PA_OK;
  if (!k_cache || !v_cache || !k || !v || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "pa_write_kv: null pointer");
  PA_DEBUG_CHECK(debug::check_slots(c, slot_mapping, num_tokens, stream, "pa_write_kv"));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int hkv = c->num_kv_heads, d = c->head_dim;
  const int elems = (src_dtype == PA_F32) ? 4 : 8;
  const int chunks_per_head = d / elems;
  const int chunks_per_row = hkv * chunks_per_head;
  const int64_t num_chunks = static_cast<int64_t>(num_tokens) * chunks_per_row;
  const int64_t grid_x = (num_chunks + 255) / 256;
  if (grid_x > INT32_MAX) return fail(PA_ERR_INVALID_ARG, "pa_write_kv: too many tokens");
  dim3 grid(static_cast<unsigned>(grid_x), 2);
  const float k_inv = (c->cache_dtype == PA_FP8_E4M3) ? 1.0f / c->k_scale : 1.f;
  const float v_inv = (c->cache_dtype == PA_FP8_E4M3) ? 1.0f / c->v_scale : 1.f;
  char* kc = static_cast<char*>(k_cache);
  char* vc = static_cast<char*>(v_cache);
  const char* kk = static_cast<const char*>(k);
  const char* vv = static_cast<const char*>(v);
  if (c->cache_dtype == PA_FP8_E4M3) {
    write_kv_kernel<u32x4_t, 8, PA_FP8_E4M3><<<grid, 256, 0, s>>>(
        kc, vc, kk, vv, slot_mapping, num_chunks, chunks_per_row, chunks_per_head, hkv, d,
        c->block_size, k_inv, v_inv);
  } else if (src_dtype == PA_BF16) {
    write_kv_kernel<u32x4_t, 8, PA_BF16><<<grid, 256, 0, s>>>(
        kc, vc, kk, vv, slot_mapping, num_chunks, chunks_per_row, chunks_per_head, hkv, d,
        c->block_size, k_inv, v_inv);
  } else {
    write_kv_kernel<u32x4_t, 4, PA_F32><<<grid, 256, 0, s>>>(
        kc, vc, kk, vv, slot_mapping, num_chunks, chunks_per_row, chunks_per_head, hkv, d,
        c->block_size, k_inv, v_inv);
  }
  return launch_status("pa_write_kv");
}

extern "C" pa_status pa_copy_blocks(const pa_cache_desc* c, void* k_cache, void* v_cache,
                                    const int32_t* pairs, int32_t num_pairs, void* stream) {
  pa_status st = check_desc(c, "pa_copy_blocks");
  if (st != PA_OK) return st;
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: num_pairs < 0");
  if (num_pairs == 0) return PA_OK;
  if (num_pairs > 65535)
    return fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: %d pairs (at most 65535 per call)",
                num_pairs);
  if (!k_cache || !v_cache || !pairs) return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: null pointer");
  PA_DEBUG_CHECK(debug::check_pairs(pairs, num_pairs, c->num_blocks, true, stream, "pa_copy_blocks"));
  const int64_t block_bytes = static_cast<int64_t>(c->num_kv_heads) * c->block_size *
                              c->head_dim * dtype_bytes(c->cache_dtype);
  const int64_t chunks = block_bytes / 16;
  dim3 grid(static_cast<unsigned>((chunks + 255) / 256), num_pairs, 2);
  copy_blocks_kernel<<<grid, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const char*>(k_cache), static_cast<const char*>(v_cache),
      static_cast<char*>(k_cache), static_cast<char*>(v_cache), pairs, block_bytes);
  return launch_status("pa_copy_blocks");
}

namespace {

// True if the GPU can address `p`: device memory, or host memory allocated
// pinned (hipHostMalloc) or managed.  Pageable host memory is not.
bool gpu_addressable(const void* p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();     // the query leaves its error behind
    return false;
  }
  switch (attr.type) {
    case hipMemoryTypeDevice:
    case hipMemoryTypeManaged:
    case hipMemoryTypeUnified:
      return true;
    case hipMemoryTypeHost:
      return attr.devicePointer != nullptr;
    default:
      return false;
  }
}

}  // namespace

extern "C" pa_status pa_swap_blocks(const pa_cache_desc* c, const void* src_k,
                                    const void* src_v, void* dst_k, void* dst_v,
                                    const int32_t* pairs, int32_t num_pairs, void* stream) {
  pa_status st = check_desc(c, "pa_swap_blocks");
  if (st != PA_OK) return st;
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: num_pairs < 0");
  if (num_pairs == 0) return PA_OK;
  if (num_pairs > 65535)
    return fail(PA_ERR_UNSUPPORTED, "pa_swap_blocks: %d pairs (at most 65535 per call)",
                num_pairs);
  if (!src_k || !src_v || !dst_k || !dst_v || !pairs)
    return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: null pointer");
  const void* ptrs[5] = {src_k, src_v, dst_k, dst_v, pairs};
  const char* names[5] = {"src_k", "src_v", "dst_k", "dst_v", "pairs"};
  for (int i = 0; i < 5; ++i)
    if (!gpu_addressable(ptrs[i]))
      return fail(PA_ERR_INVALID_ARG,
                  "pa_swap_blocks: %s is not device or pinned host memory", names[i]);
  // the pools' sizes are not passed, so only signs and distinct destinations
  PA_DEBUG_CHECK(debug::check_pairs(pairs, num_pairs, -1, false, stream, "pa_swap_blocks"));
  const int64_t block_bytes = static_cast<int64_t>(c->num_kv_heads) * c->block_size *
                              c->head_dim * dtype_bytes(c->cache_dtype);
  const int64_t chunks = block_bytes / 16;
  dim3 grid(static_cast<unsigned>((chunks + 255) / 256), num_pairs, 2);
  copy_blocks_kernel<<<grid, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const char*>(src_k), static_cast<const char*>(src_v),
      static_cast<char*>(dst_k), static_cast<char*>(dst_v), pairs, block_bytes);
  return launch_status("pa_swap_blocks");
}
