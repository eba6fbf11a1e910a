// Internal: host-side validation of the values inside device arrays, built
// only with PA_DEBUG.  Each check copies the array to the host (after the
// work already queued on `stream`, which it waits for) and returns
// PA_ERR_INVALID_ARG, with a message naming the offending entry, before any
// kernel could read an out-of-range value.  A debug build therefore
// synchronises inside its calls and cannot be captured in a graph.
#pragma once

#include "pagedkv.h"

namespace pagedkv {
namespace debug {

// slot_mapping[n]: each slot negative (skipped) or below num_blocks * bs, and
// the non-negative ones distinct.
pa_status check_slots(const pa_cache_desc* c, const int64_t* slots, int32_t n, void* stream,
                      const char* fn);

// pairs[n][2] of (src, dst) blocks: destinations distinct, and with
// same_pool (a copy inside one pool) none of them a source; with
// num_blocks >= 0 every id is below it (else only >= 0).
pa_status check_pairs(const int32_t* pairs, int32_t n, int32_t num_blocks, bool same_pool,
                      void* stream, const char* fn);

// context_lens[B] within [0, max_len]; the first ceil(L / bs) entries of each
// row of block_tables[B][max_blocks] are valid block ids.
pa_status check_tables(const pa_cache_desc* c, const int32_t* block_tables, int32_t max_blocks,
                       const int32_t* context_lens, int32_t max_len, int32_t B, void* stream,
                       const char* fn);

// groups[k] = (first, count, shared): every member's first `shared` table
// entries equal the first member's.
pa_status check_groups(const int32_t* block_tables, int32_t max_blocks, int32_t B,
                       const int32_t* groups, int32_t num_groups, void* stream, const char* fn);

// chunk_order[n]: every entry within [0, n).
pa_status check_order(const int32_t* order, int64_t n, void* stream, const char* fn);

}  // namespace debug
}  // namespace pagedkv

#ifdef PA_DEBUG
#define PA_DEBUG_CHECK(expr)            \
  do {                                  \
    const pa_status pa_dbg_st_ = (expr); \
    if (pa_dbg_st_ != PA_OK) return pa_dbg_st_; \
  } while (0)
#else
#define PA_DEBUG_CHECK(expr) \
  do {                       \
  } while (0)
#endif
