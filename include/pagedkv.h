/*
 * pagedkv.h -- C ABI of libpagedkv: paged KV cache and single-query decode
 * attention for AMD Instinct MI355X (gfx950).
 *
 * What the library does (sources are web pages on vLLM / PagedAttention):
 *   - The KV cache is split into fixed-size blocks (16 tokens by default;
 *     8, 32 or 64 may be chosen to suit request lengths, unionyoga.cn,
 *     section "在真实架构中扮演什么角色？") that need not be
 *     contiguous; each sequence owns a block table from logical to physical
 *     block (explore.n1n.ai, "vLLM 深度解析：PagedAttention 如何让大模型推理更快、
 *     更省钱", 映射机制详解; ybb.press, "vLLM PagedAttention 大模型推理架构深度
 *     实战", §2.2).
 *   - The attention kernel walks ceil(len / block_size) table entries of a sequence
 *     and reads the blocks they name (unionyoga.cn, "vLLM：重塑大模型推理性能的
 *     关键引擎", PagedAttention section, kernel sketch).
 *   - Each decode iteration writes the new token's K/V into its block and
 *     then checks whether the sequence needs a new block (ybb.press, §6).
 *   - Shared blocks carry reference counts; a sequence about to modify a
 *     block shared with others copies it first (ybb.press, §2.3).
 *
 * Conventions for every call:
 *   - Return value: PA_OK (0) or a negative pa_status.  On error nothing was
 *     launched and no state changed; pa_last_error() returns a message
 *     (thread-local, valid until the next failing call on that thread).
 *   - Device pointers are caller-owned device memory (for example torch
 *     tensors); the library never allocates, frees or synchronises device
 *     memory.  Device calls are asynchronous on `stream` (a hipStream_t passed
 *     as void*; NULL = the null stream).
 *   - Arguments are validated on the host before any launch.  Values inside
 *     device arrays (block ids, slots, context lengths) cannot be checked on
 *     the host; out-of-range values there are undefined behaviour.
 *
 * Cache layout (one K and one V tensor, same shape and dtype; bs = block_size):
 *   cache[num_blocks][num_kv_heads][bs][head_dim], row-major, so element
 *   (block b, kv head g, slot t, dim d) is at ((b*Hkv + g)*bs + t)*D + d and
 *   one (block, head) tile is bs*D contiguous elements; a token's row of one
 *   head is D contiguous elements, so appending a token writes whole rows.
 *   Below, "16" in slot and table formulas stands for the block size.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,        /* null pointer, bad size, bad enum value */
  PA_ERR_UNSUPPORTED = -2,        /* valid but not implemented combination */
  PA_ERR_NO_BLOCKS = -3,          /* block manager: free pool too small */
  PA_ERR_UNKNOWN_SEQ = -4,        /* block manager: no such sequence id */
  PA_ERR_SEQ_EXISTS = -5,         /* block manager: id already in use */
  PA_ERR_WORKSPACE_TOO_SMALL = -6,
  PA_ERR_HIP = -7,                /* a HIP runtime call or launch failed */
  PA_ERR_SWAPPED = -8             /* block manager: sequence is in the other pool */
} pa_status;

typedef enum {
  PA_F32 = 0,       /* IEEE binary32 */
  PA_BF16 = 1,      /* bfloat16 */
  PA_FP8_E4M3 = 2   /* OCP E4M3 ("e4m3fn"): bias 7, max 448, no inf, NaN 0x7F/0xFF */
} pa_dtype;

#define PA_BLOCK_SIZE 16
/* Context positions per partition of the general (fp32) decode path. */
#define PA_PARTITION_TOKENS 512
/* Largest chunk of new tokens per sequence pa_decode_chunk takes. */
#define PA_MAX_CHUNK 16
/* Most shared-prefix groups one pa_decode_shared_prefix call takes. */
#define PA_MAX_PREFIX_GROUPS 128

typedef struct {
  int32_t num_blocks;    /* physical blocks in each of the K and V caches */
  int32_t block_size;    /* tokens per block: 8, 16 (PA_BLOCK_SIZE), 32 or 64;
                            decode streams tiles of 16 tokens: 2 or 4 per block
                            of 32 or 64, and a tile of two 8-token blocks (one
                            buffer descriptor over a cache under 2 GiB - 128
                            KiB, 64-bit per-lane addresses beyond) */
  int32_t num_kv_heads;  /* Hkv >= 1 */
  int32_t head_dim;      /* D: 64 or 128 */
  int32_t cache_dtype;   /* pa_dtype of both caches */
  float k_scale;         /* PA_FP8_E4M3 only: stored K value = code value * k_scale */
  float v_scale;         /* PA_FP8_E4M3 only: same for V; both finite and > 0 */
} pa_cache_desc;

/* Version string of the library build. */
const char* pa_version(void);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* pa_last_error(void);

/* Bytes of one (K or V) cache tensor described by `c`; 0 if `c` is invalid. */
size_t pa_cache_bytes(const pa_cache_desc* c);

/*
 * pa_write_kv -- store new K/V rows into their cache slots (the "write KV
 * into its block" step of each decode iteration, ybb.press §6).
 *   k, v          : [num_tokens][num_kv_heads][head_dim] contiguous, dtype
 *                   src_dtype (device).
 *   slot_mapping  : int64 [num_tokens] (device); slot = block * bs + offset;
 *                   a negative slot skips that row.  Non-negative slots must
 *                   be distinct and < num_blocks * bs.
 *   Supported (src_dtype -> cache_dtype): F32 -> F32, BF16 -> BF16 (bit
 *   copies) and BF16 -> FP8_E4M3 (code = round-to-nearest-even of
 *   min(|x * fp32(1/scale)|, 448) with x's sign; NaN -> 0x7F).
 *   Bytes of slots that are not written are left untouched.
 */
pa_status pa_write_kv(const pa_cache_desc* c, void* k_cache, void* v_cache,
                      const void* k, const void* v, int32_t src_dtype,
                      const int64_t* slot_mapping, int32_t num_tokens,
                      void* stream);

/*
 * pa_copy_blocks -- copy-on-write block duplication (ybb.press §2.3).
 *   pairs : int32 [num_pairs][2] (device), each (src, dst): the whole block
 *           -- every KV head, all bs slots -- of both caches is copied byte
 *           for byte from src to dst.  Destinations must be distinct and none
 *           may also be a source (the block manager never emits otherwise).
 */
pa_status pa_copy_blocks(const pa_cache_desc* c, void* k_cache, void* v_cache,
                         const int32_t* pairs, int32_t num_pairs, void* stream);

/*
 * Workspace bytes pa_decode needs for this cache and batch shape; 0 if the
 * arguments are invalid or no workspace is needed.  The size depends on the
 * decode path the shape takes (and, for the bf16 / fp8 path, on the number
 * of compute units of the current device), not on the context lengths.
 */
size_t pa_decode_workspace_bytes(const pa_cache_desc* c, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t max_context_len);

/* The same for pa_decode_chunk with chunk_len new tokens per sequence. */
size_t pa_decode_chunk_workspace_bytes(const pa_cache_desc* c, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t chunk_len,
                                       int32_t max_context_len);

/*
 * pa_decode_workspace_init -- zero-fill `workspace_bytes` bytes of a decode
 * workspace on `stream` (a plain fill kernel, so it may be captured in a
 * graph).  A workspace must be zero-filled once before its first pa_decode
 * (this call, or any other zero fill such as torch.zeros); every pa_decode
 * or pa_decode_chunk that completes leaves it zero-filled again.  workspace must be 4-byte
 * aligned.
 */
pa_status pa_decode_workspace_init(void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * pa_decode -- single-query decode attention through block tables.
 *   For every sequence s < num_seqs and query head h < num_q_heads:
 *     g = h / (num_q_heads / num_kv_heads)         (contiguous head groups)
 *     L = context_lens[s]; token t < L lives in block block_tables[s][t/16],
 *     slot t % 16;
 *     out[s][h] = sum_t softmax_t(scale * q[s][h] . K[t]) * V[t]
 *   which is exact attention, computed blockwise with online-softmax
 *   renormalisation (ybb.press §5.1).  L == 0 gives a zero row.  Only the first
 *   ceil(L/16) table entries and the first L slots are read.
 *   q, out       : [num_seqs][num_q_heads][head_dim] contiguous (device),
 *                  16-byte aligned.  q dtype: F32 with an F32 cache, BF16
 *                  with a BF16 or FP8 cache; out has q's dtype.
 *                  Accumulation is fp32.
 *   block_tables : int32 [num_seqs][max_blocks_per_seq] (device).
 *   context_lens : int32 [num_seqs] (device), each in [0, max_context_len].
 *   max_context_len: host-side upper bound on context_lens, sizes the grid.
 *   workspace    : device scratch of at least
 *                  pa_decode_workspace_bytes(c, num_seqs, num_q_heads,
 *                  max_context_len) bytes, 16-byte aligned, zero-filled
 *                  before its first use (pa_decode_workspace_init); may be
 *                  NULL when that size is 0.  It holds partial results and
 *                  arrival counters of one call at a time: calls that may
 *                  overlap (different streams) need separate workspaces.
 *   A context is processed in pieces whose partial (max, sum, output) are
 *   merged by the log-sum-exp rule: with a bf16 or fp8 cache and head_dim
 *   64 or 128, pieces are equal shares of the whole batch's KV tiles (a KV
 *   head with G > 16 query heads is streamed as the fewest equal blocks of
 *   at most 16 of them, each reading the head's tiles; at most 511 such
 *   blocks over all KV heads); otherwise (fp32 caches) pieces are
 *   PA_PARTITION_TOKENS-token partitions.  Pieces are merged in a fixed order, so repeated calls give
 *   bit-identical results.
 */
pa_status pa_decode(const pa_cache_desc* c, const void* k_cache,
                    const void* v_cache, const void* q, int32_t q_dtype,
                    void* out, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens,
                    int32_t max_context_len, int32_t num_seqs,
                    int32_t num_q_heads, float scale, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * pa_decode_noalloc -- pa_decode without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, serving
 * loops and harnesses that forbid allocation.  Same arguments (minus the
 * workspace), results (bit for bit: same kernels, same work split) and
 * errors as pa_decode.
 *   Scratch: a static device array inside the library, one per GPU, held
 *   until the process ends: 256 KiB of arrival counters (at most 65536
 *   sequences x KV heads per call) and 24 MiB of partial results.  A batch
 *   that needs more returns PA_ERR_WORKSPACE_TOO_SMALL and launches nothing
 *   (the bf16 / fp8 path needs about 2 * 4 * CUs * min(G, 16) * (head_dim +
 *   2) * 4 bytes: 17 MiB at G = 16, head_dim 128 on 256 CUs, and one counter
 *   per sequence and block of at most 16 query heads; the fp32 path needs
 *   num_seqs * num_q_heads * ceil(max_context_len / 512) * (head_dim + 2) * 4
 *   bytes once a context spans more than one partition).
 *   The first call on a device looks the array up and clears its counters
 *   with a fill kernel on `stream`; every completed call leaves them zero.
 *   The call itself allocates nothing and uses no memset.  All calls on one
 *   GPU share the array: calls that may overlap on one GPU (different
 *   streams, or graphs replayed concurrently) race and must be serialised by
 *   the caller.  Like pa_decode it consumes a pa_time_next_call request.
 */
pa_status pa_decode_noalloc(const pa_cache_desc* c, const void* k_cache,
                            const void* v_cache, const void* q, int32_t q_dtype,
                            void* out, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t max_context_len, int32_t num_seqs,
                            int32_t num_q_heads, float scale, void* stream);

/*
 * pa_decode_chunk -- attention of a chunk of chunk_len = T new tokens per
 * sequence (1 <= T <= PA_MAX_CHUNK), as in chunked prefill (ybb.press §7.1,
 * §7.2) and draft-token verification in speculative decoding (ybb.press §9
 * item 2).  The chunk's K/V rows are already in the cache (pa_write_kv) and
 * context_lens[s] = L counts them.  Chunk token i sits at position L - T + i
 * and attends positions 0 .. L - T + i only (causal order inside the chunk):
 *     out[s][i][h] = sum_{t <= L-T+i} softmax_t(scale * q[s][i][h] . K[t]) V[t]
 *   with the head map, scales and dtypes of pa_decode.  A token with no
 *   position to see (L - T + i < 0) gets a zero row.
 *   q, out    : [num_seqs][chunk_len][num_q_heads][head_dim] contiguous.
 *   workspace : at least pa_decode_chunk_workspace_bytes(c, num_seqs,
 *               num_q_heads, chunk_len, max_context_len) bytes, same rules
 *               as pa_decode's.
 *   With a bf16 or fp8 cache the KV tiles are streamed once per pass of
 *   floor(16 / G) chunk tokens (each pass's G * tokens query rows share the
 *   tile loads; G > 16 is split into blocks of at most 16 query heads as for
 *   pa_decode, one token per pass); other caches take the partition path.
 *   pa_decode is pa_decode_chunk with chunk_len = 1.
 */
pa_status pa_decode_chunk(const pa_cache_desc* c, const void* k_cache,
                          const void* v_cache, const void* q, int32_t q_dtype,
                          void* out, int32_t chunk_len,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t max_context_len,
                          int32_t num_seqs, int32_t num_q_heads, float scale,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_window -- pa_decode_chunk with a sliding window (ybb.press §7.2:
 * sliding-window attention for long contexts): with window = W > 0 a token
 * at position p attends only positions max(0, p - W + 1) .. p (its own and
 * the W - 1 before it), so a chunk token i of a length-L context sees
 * max(0, L - T + i + 1 - W) .. L - T + i.  window = 0 is no window.  Blocks
 * wholly before every chunk token's window are not read.  Same arguments,
 * workspace (pa_decode_chunk_workspace_bytes) and errors as pa_decode_chunk;
 * window < 0 is PA_ERR_INVALID_ARG.
 */
pa_status pa_decode_window(const pa_cache_desc* c, const void* k_cache,
                           const void* v_cache, const void* q, int32_t q_dtype,
                           void* out, int32_t chunk_len, int32_t window,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t max_context_len,
                           int32_t num_seqs, int32_t num_q_heads, float scale,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Host block manager (plain host memory, no GPU calls).  One owner; not
 * thread-safe.  Policy: the free pool is a FIFO queue initialised from
 * `free_order` (a permutation of 0..num_blocks-1; NULL = 0,1,2,...);
 * allocation pops the front and a block whose reference count drops to zero
 * is pushed to the back, a freed sequence releasing its blocks in logical
 * order.  Appending token p to a sequence: if p % 16 == 0 a fresh block is
 * appended to its table; otherwise, if its last block is shared (count > 1),
 * that block is replaced by a fresh one and the pair (old, new) is reported
 * for pa_copy_blocks.  Every mutating call is all-or-nothing.
 * ------------------------------------------------------------------------- */
typedef struct pa_bm pa_bm;

/* A pool of num_blocks device blocks of block_size tokens, all free: the
 * block pool that logical blocks are mapped onto (explore.n1n.ai,
 * "vLLM 深度解析", 映射机制详解; ybb.press §2.2, block division and
 * allocation on demand).  NULL on invalid arguments (see pa_last_error). */
pa_bm* pa_bm_create(int32_t num_blocks, int32_t block_size,
                    const int32_t* free_order);
/* The same with a pool of num_host_blocks host blocks for swapping
 * (host_free_order: a permutation of 0..num_host_blocks-1, NULL = 0,1,...). */
pa_bm* pa_bm_create_ex(int32_t num_blocks, int32_t block_size,
                       const int32_t* free_order, int32_t num_host_blocks,
                       const int32_t* host_free_order);
void pa_bm_destroy(pa_bm* bm);

/* A new sequence with an empty block table (ybb.press §6: the block manager
 * allocates a new prompt's blocks; they are taken as tokens are appended). */
pa_status pa_bm_add_seq(pa_bm* bm, int64_t seq_id);
/* child shares all of parent's blocks (each gains one reference): samples of
 * one prompt start from the same block table, with reference counts on the
 * shared blocks (ybb.press §2.3, copy-on-write and parallel sampling). */
pa_status pa_bm_fork(pa_bm* bm, int64_t parent_id, int64_t child_id);
/* Append one token: *slot receives its cache slot; *cow_src / *cow_dst
 * receive the copy pair, or -1 / -1 when no copy is needed.  Each decode
 * iteration writes the new token's KV into its block, then checks whether a
 * new block is needed (ybb.press §6); a block is taken only when the
 * sequence needs it (§2.2, allocation on demand); a shared block is copied
 * before it is modified (§2.3). */
pa_status pa_bm_append_slot(pa_bm* bm, int64_t seq_id, int64_t* slot,
                            int32_t* cow_src, int32_t* cow_dst);
/* Append n >= 0 tokens (a prompt, or several decode steps; ybb.press §6):
 * slots[n]; at most one copy pair (the first token, ybb.press §2.3). */
pa_status pa_bm_append_tokens(pa_bm* bm, int64_t seq_id, int32_t n,
                              int64_t* slots, int32_t* cow_src,
                              int32_t* cow_dst);
/* One decode step for a batch (ybb.press §6, the decode loop of the running
 * batch): append one token to each of seq_ids[0..n-1], in order.  slots[n] receive the slots; cow_pairs[2*k], cow_pairs[2*k+1]
 * the k-th copy pair (room for n pairs); *num_pairs their count.  All or
 * nothing across the whole batch. */
pa_status pa_bm_append_batch(pa_bm* bm, const int64_t* seq_ids, int32_t n,
                             int64_t* slots, int32_t* cow_pairs,
                             int32_t* num_pairs);
/* A finished sequence gives back its references; blocks whose count reaches
 * zero return to the pool at once (ybb.press §2.2, blocks are reclaimed as
 * soon as a sequence ends). */
pa_status pa_bm_free_seq(pa_bm* bm, int64_t seq_id);

/* Blocks an allocation can take (free, plus evictable with prefix caching). */
int32_t pa_bm_num_free(const pa_bm* bm);
/* Reference count of `block`, or -1 if out of range (the counts copy-on-write
 * tests, ybb.press §2.3). */
int32_t pa_bm_refcount(const pa_bm* bm, int32_t block);
/* Context length of a sequence in *len. */
pa_status pa_bm_length(const pa_bm* bm, int64_t seq_id, int32_t* len);
/* Pack tables of seq_ids[0..n-1]: block_tables[n][cap] padded with -1,
 * context_lens[n].  Host memory.  These are the per-sequence block tables
 * (logical block -> physical block, explore.n1n.ai, "vLLM 深度解析",
 * 映射机制详解) and lengths that pa_decode reads. */
pa_status pa_bm_pack(const pa_bm* bm, const int64_t* seq_ids, int32_t n,
                     int32_t* block_tables, int32_t cap, int32_t* context_lens);

/* ---------------------------------------------------------------------------
 * Swapping (ybb.press §3.2: when device memory runs short the KV cache of
 * low-priority sequences moves to CPU memory and is resumed later; §6: the
 * scheduler swaps sequences out and in; §9 item 5: it stays in host memory).
 *
 * pa_bm_swap_out moves the sequences seq_ids[0..n-1] to the host pool: every
 * distinct device block they reference, in walk order (sequences as listed,
 * each table in logical order), gets one host block popped from the host
 * pool, and pairs[k] = (device block, host block) is the k-th copy to make
 * (pa_swap_blocks, device cache -> host pool).  Each table entry then names
 * the host copy; each device block loses the set's references and returns
 * to the device pool, in walk order, when its count reaches zero -- a block
 * also used by sequences outside the set stays on the device for them.
 * pa_bm_swap_in is the mirror (pairs = (host block, device block)).
 * pairs: int32 [pairs_cap][2] host array; *num_pairs receives the count.
 * All or nothing: PA_ERR_NO_BLOCKS when the destination pool is short,
 * PA_ERR_SWAPPED when a sequence is already in the destination pool,
 * PA_ERR_INVALID_ARG for a repeated id or a pairs buffer that is too small.
 * A swapped-out sequence cannot append, fork or be packed (PA_ERR_SWAPPED);
 * pa_bm_free_seq releases its host blocks.
 * ------------------------------------------------------------------------- */
pa_status pa_bm_swap_out(pa_bm* bm, const int64_t* seq_ids, int32_t n,
                         int32_t* pairs, int32_t pairs_cap, int32_t* num_pairs);
pa_status pa_bm_swap_in(pa_bm* bm, const int64_t* seq_ids, int32_t n,
                        int32_t* pairs, int32_t pairs_cap, int32_t* num_pairs);
int32_t pa_bm_num_free_host(const pa_bm* bm);
/* Reference count of a host block, -1 if out of range. */
int32_t pa_bm_host_refcount(const pa_bm* bm, int32_t block);
/* *swapped = 1 if the sequence is in the host pool, else 0. */
pa_status pa_bm_is_swapped(const pa_bm* bm, int64_t seq_id, int32_t* swapped);

/* ---------------------------------------------------------------------------
 * Prefix caching (explore.n1n.ai, "vLLM 深度解析", section "vLLM 生态的核心功能
 * 亮点": requests sharing a system prompt or documents reuse its cached KV;
 * ybb.press §7.3: automatic prefix caching shares the KV blocks of
 * identical prefixes across requests; gheillcoat.github.io, "概念-vLLM",
 * section 3).  Off until pa_bm_enable_prefix_caching.
 *
 * A full block written with token ids (pa_bm_add_seq_prompt,
 * pa_bm_append_token_ids) is registered under a key: FNV-1a 64 over its
 * parent block's key (8 bytes little-endian, 0 for a first block) then its
 * 16 token ids (4 bytes little-endian each), so the key covers the whole
 * prefix.  pa_bm_add_seq_prompt creates a sequence with tokens[0..n-1]: the
 * longest run of leading full blocks whose key, parent key and ids all match
 * a registered block is reused (each gains a reference); *num_cached
 * receives that many tokens -- their KV is already in the cache, the caller
 * writes only tokens num_cached..n-1 -- and the rest are appended.  slots[n]
 * receives every token's slot.  A registered block whose count drops to
 * zero is kept as evictable rather than freed; allocation takes free blocks
 * first, then evicts the least recently released evictable block, and a hit
 * revives one.  pa_bm_num_free counts free plus evictable blocks.
 * pa_bm_append_tokens / pa_bm_append_batch (ids unknown) stop registering a
 * sequence's later blocks.  All calls are all-or-nothing as above.
 * ------------------------------------------------------------------------- */
pa_status pa_bm_enable_prefix_caching(pa_bm* bm);
pa_status pa_bm_add_seq_prompt(pa_bm* bm, int64_t seq_id, const int32_t* tokens,
                               int32_t n, int64_t* slots, int32_t* num_cached);
pa_status pa_bm_append_token_ids(pa_bm* bm, int64_t seq_id, const int32_t* tokens,
                                 int32_t n, int64_t* slots, int32_t* cow_src,
                                 int32_t* cow_dst);
/* Prompt full blocks looked up, blocks reused, registered and evictable blocks. */
pa_status pa_bm_cache_stats(const pa_bm* bm, int64_t* queried_blocks, int64_t* hit_blocks,
                            int32_t* registered_blocks, int32_t* evictable_blocks);

/* ---------------------------------------------------------------------------
 * Shared prefixes: attention over a prompt prefix that several sequences
 * share is computed once for all of them (prefix caching makes such
 * sharing common: explore.n1n.ai, "vLLM 深度解析", section "vLLM 生态的核心功能
 * 亮点"; ybb.press §7.3).
 *
 * pa_bm_shared_prefix_groups -- runs of adjacent sequences of seq_ids (in
 * that order) whose tables start with the same block, as groups[k] =
 * (index in seq_ids of the first member, member count, shared blocks):
 * shared = the longest common run of leading table entries that leaves
 * every member at least one more token (shared * block_size < length).
 * Runs of one sequence or with nothing shared are left out.  groups: host
 * int32 [cap][3]; *num_groups receives the count (PA_ERR_INVALID_ARG if it
 * would exceed cap).
 *
 * pa_decode_shared_prefix -- pa_decode for a batch in which groups[k] =
 * (first, count, shared) says sequences first .. first+count-1 hold the
 * same valid block ids in their first `shared` table entries (host array,
 * at most PA_MAX_PREFIX_GROUPS disjoint groups; a member no longer than shared * block_size
 * sees only its own length of them).  The result is pa_decode's (up to
 * rounding order); the prefix is attended once per
 * (group, KV head) on MFMA with all members' query rows and folded into each
 * row by the log-sum-exp rule.  With at most 256 sequences this is one
 * launch of pa_decode's tile stream in which each (group, KV head) is one
 * segment: the prefix tiles, seen by every member's rows up to its own
 * length, then each member's own tiles, seen by that member's rows only.  A
 * group whose rows of a KV head (members x G) exceed 16 is cut into row
 * groups of 16 / G members, each such a segment over the same prefix, and
 * the tile stream then runs KV head by KV head so that the row groups of a
 * head read its prefix tiles from one L2.  With more sequences, groups
 * whose rows of a KV head fit 16 run the prefix through the same tile
 * stream with the members as query rows and the suffixes are decoded
 * afterwards (a group with a member no longer than shared * block_size is
 * then decoded whole by the suffix pass; same result); larger groups use a
 * kernel that shares each prefix tile among up to 128 rows in LDS, then the
 * suffix pass.
 * Needs the bf16 / fp8 fast path (head_dim 64 or 128, G <= 16, block size a
 * multiple of 16), single-token decode, a positive scale (with groups).  workspace: zero-filled before first
 * use, 256-byte aligned, pa_decode_shared_prefix_workspace_bytes(...) bytes;
 * it holds suffix tables and lengths and per-row prefix records besides
 * pa_decode's scratch.  num_groups = 0 is pa_decode.
 * ------------------------------------------------------------------------- */
pa_status pa_bm_shared_prefix_groups(const pa_bm* bm, const int64_t* seq_ids, int32_t n,
                                     int32_t* groups, int32_t cap, int32_t* num_groups);
size_t pa_decode_shared_prefix_workspace_bytes(const pa_cache_desc* c, int32_t num_seqs,
                                               int32_t num_q_heads,
                                               int32_t max_blocks_per_seq,
                                               int32_t max_context_len);
pa_status pa_decode_shared_prefix(const pa_cache_desc* c, const void* k_cache,
                                  const void* v_cache, const void* q, int32_t q_dtype,
                                  void* out, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t max_context_len, int32_t num_seqs,
                                  int32_t num_q_heads, float scale, const int32_t* groups,
                                  int32_t num_groups, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * pa_swap_blocks -- whole-block copies between two pools with the layout of
 * `c`: for each pairs[i] = (s, d), block d of dst_k / dst_v receives block s
 * of src_k / src_v, byte for byte (every KV head, all 16 slots).  Each pool
 * pointer is device memory or pinned host memory (hipHostMalloc); the call
 * checks that the GPU can address all four (PA_ERR_INVALID_ARG otherwise,
 * e.g. for pageable host memory).  pairs: int32 [num_pairs][2] in device or
 * pinned host memory.  Destinations must be distinct; the two pools must not
 * overlap.  The copy is a kernel on `stream` (it reads or writes host memory
 * over the host link directly).  num_pairs <= 65535 per call.
 */
pa_status pa_swap_blocks(const pa_cache_desc* c, const void* src_k, const void* src_v,
                         void* dst_k, void* dst_v, const int32_t* pairs,
                         int32_t num_pairs, void* stream);

/* ---------------------------------------------------------------------------
 * Diagnostics (not part of the attention path).
 *
 * pa_read_probe -- reads floor(bytes / 4096) chunks of 4 KiB of the device
 * buffer `buf` with the decode kernel's load form (16-byte non-temporal
 * buffer loads), 8 waves per compute unit: in address order, or, with
 * chunk_order (int32 [chunks], device memory, each < chunks), chunk c taken
 * from offset chunk_order[c] * 4096 -- the scattered pattern of paged
 * blocks.  Timing a call gives the streaming-read rate decode's bandwidth is
 * compared with.  sink: device scratch of pa_read_probe_sink_bytes(num_cus)
 * bytes (its contents are meaningless).
 * ------------------------------------------------------------------------- */
size_t pa_read_probe_sink_bytes(int32_t num_cus);

/*
 * pa_time_next_call -- the next pa_decode, pa_decode_noalloc, pa_decode_chunk
 * or pa_decode_window made on the calling thread launches its kernels through hipExtLaunchKernel
 * with these events (hipEvent_t, created by the caller; either may be null):
 * start_event is recorded as its first kernel starts, stop_event as its last
 * kernel ends, by the dispatches themselves, so no marker packet sits in the
 * stream between the previous work and the kernel.  The request is consumed
 * by that call whatever its outcome (a call that launches nothing records
 * nothing); other entry points leave it pending.  Always PA_OK.
 */
pa_status pa_time_next_call(void* start_event, void* stop_event);
pa_status pa_read_probe(const void* buf, size_t bytes, const int32_t* chunk_order,
                        void* sink, int32_t num_cus, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
