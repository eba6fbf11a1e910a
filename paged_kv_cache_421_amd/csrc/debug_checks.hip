// Host-side validation of device arrays for PA_DEBUG builds (see
// debug_checks.h).  Out-of-range block ids, slots, lengths or copy pairs are
// undefined behaviour in a release build; a debug build reports them as
// PA_ERR_INVALID_ARG before launching anything.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <unordered_set>
#include <vector>

#include "debug_checks.h"
#include "status.h"

namespace pagedkv {
namespace debug {
namespace {

// Copies `count` elements of `src` (device or pinned host memory) to the
// host once the work queued on `stream` before this call has finished.
template <typename T>
pa_status fetch(const T* src, int64_t count, void* stream, std::vector<T>* out, const char* fn) {
  out->resize(static_cast<size_t>(std::max<int64_t>(count, 0)));
  if (count <= 0) return PA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(out->data(), src, static_cast<size_t>(count) * sizeof(T),
                                hipMemcpyDefault, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess)
    return fail(PA_ERR_HIP, "%s (PA_DEBUG): reading a device array back failed: %s", fn,
                hipGetErrorString(e));
  return PA_OK;
}

}  // namespace

pa_status check_slots(const pa_cache_desc* c, const int64_t* slots, int32_t n, void* stream,
                      const char* fn) {
  std::vector<int64_t> h;
  pa_status st = fetch(slots, n, stream, &h, fn);
  if (st != PA_OK) return st;
  const int64_t cap = static_cast<int64_t>(c->num_blocks) * c->block_size;
  std::vector<int64_t> used;
  for (int32_t i = 0; i < n; ++i) {
    if (h[i] < 0) continue;
    if (h[i] >= cap)
      return fail(PA_ERR_INVALID_ARG, "%s (PA_DEBUG): slot_mapping[%d] = %lld, the cache holds %lld slots",
                  fn, i, static_cast<long long>(h[i]), static_cast<long long>(cap));
    used.push_back(h[i]);
  }
  std::sort(used.begin(), used.end());
  for (size_t i = 1; i < used.size(); ++i)
    if (used[i] == used[i - 1])
      return fail(PA_ERR_INVALID_ARG, "%s (PA_DEBUG): slot %lld appears twice in slot_mapping",
                  fn, static_cast<long long>(used[i]));
  return PA_OK;
}

pa_status check_pairs(const int32_t* pairs, int32_t n, int32_t num_blocks, bool same_pool,
                      void* stream, const char* fn) {
  std::vector<int32_t> h;
  pa_status st = fetch(pairs, 2 * static_cast<int64_t>(n), stream, &h, fn);
  if (st != PA_OK) return st;
  std::unordered_set<int32_t> src, dst;
  for (int32_t i = 0; i < n; ++i) {
    for (int k = 0; k < 2; ++k) {
      const int32_t b = h[2 * i + k];
      if (b < 0 || (num_blocks >= 0 && b >= num_blocks))
        return fail(PA_ERR_INVALID_ARG, "%s (PA_DEBUG): pairs[%d][%d] = %d out of range (%d blocks)",
                    fn, i, k, b, num_blocks);
    }
    src.insert(h[2 * i]);
    if (!dst.insert(h[2 * i + 1]).second)
      return fail(PA_ERR_INVALID_ARG, "%s (PA_DEBUG): destination block %d appears twice", fn,
                  h[2 * i + 1]);
  }
  // within one pool a block must not be both read and written by one call;
  // between two pools (a swap) the ids name different blocks
  for (int32_t d : dst)
    if (same_pool && src.count(d))
      return fail(PA_ERR_INVALID_ARG, "%s (PA_DEBUG): block %d is both a source and a destination",
                  fn, d);
  return PA_OK;
}

pa_status check_tables(const pa_cache_desc* c, const int32_t* block_tables, int32_t max_blocks,
                       const int32_t* context_lens, int32_t max_len, int32_t B, void* stream,
                       const char* fn) {
  std::vector<int32_t> L, bt;
  pa_status st = fetch(context_lens, B, stream, &L, fn);
  if (st != PA_OK) return st;
  st = fetch(block_tables, static_cast<int64_t>(B) * max_blocks, stream, &bt, fn);
  if (st != PA_OK) return st;
  for (int32_t s = 0; s < B; ++s) {
    if (L[s] < 0 || L[s] > max_len)
      return fail(PA_ERR_INVALID_ARG, "%s (PA_DEBUG): context_lens[%d] = %d outside [0, %d]", fn,
                  s, L[s], max_len);
    const int64_t nb = (static_cast<int64_t>(L[s]) + c->block_size - 1) / c->block_size;
    for (int64_t j = 0; j < nb; ++j) {
      const int32_t b = bt[static_cast<size_t>(s) * max_blocks + j];
      if (b < 0 || b >= c->num_blocks)
        return fail(PA_ERR_INVALID_ARG,
                    "%s (PA_DEBUG): block_tables[%d][%lld] = %d is not a block id (%d blocks)",
                    fn, s, static_cast<long long>(j), b, c->num_blocks);
    }
  }
  return PA_OK;
}

pa_status check_groups(const int32_t* block_tables, int32_t max_blocks, int32_t B,
                       const int32_t* groups, int32_t num_groups, void* stream, const char* fn) {
  std::vector<int32_t> bt;
  pa_status st = fetch(block_tables, static_cast<int64_t>(B) * max_blocks, stream, &bt, fn);
  if (st != PA_OK) return st;
  for (int32_t k = 0; k < num_groups; ++k) {
    const int32_t f = groups[3 * k], n = groups[3 * k + 1], m = groups[3 * k + 2];
    for (int32_t i = 1; i < n; ++i)
      for (int32_t j = 0; j < m; ++j)
        if (bt[static_cast<size_t>(f + i) * max_blocks + j] != bt[static_cast<size_t>(f) * max_blocks + j])
          return fail(PA_ERR_INVALID_ARG,
                      "%s (PA_DEBUG): group %d: sequence %d's table entry %d differs from "
                      "sequence %d's inside the shared run",
                      fn, k, f + i, j, f);
  }
  return PA_OK;
}

pa_status check_order(const int32_t* order, int64_t n, void* stream, const char* fn) {
  std::vector<int32_t> h;
  pa_status st = fetch(order, n, stream, &h, fn);
  if (st != PA_OK) return st;
  for (int64_t i = 0; i < n; ++i)
    if (h[i] < 0 || h[i] >= n)
      return fail(PA_ERR_INVALID_ARG, "%s (PA_DEBUG): chunk_order[%lld] = %d outside [0, %lld)",
                  fn, static_cast<long long>(i), h[i], static_cast<long long>(n));
  return PA_OK;
}

}  // namespace debug
}  // namespace pagedkv
