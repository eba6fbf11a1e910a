// pa_decode for gfx950: single-query attention over a paged KV cache.
//
// The method (vLLM PagedAttention, as described on the pages): the cache
// is split into 16-token blocks scattered through a pool, and the kernel
// reaches a sequence's blocks through its block table, walking ceil(L/16)
// entries (unionyoga.cn, "vLLM：重塑大模型推理性能的关键引擎", PagedAttention
// section; ybb.press, "vLLM PagedAttention 大模型推理架构深度实战", §2.2).
// Partial softmax results of separate pieces of the context are combined
// with online-softmax renormalisation (ybb.press §5.1).  Query heads that
// share a KV head (GQA, ybb.press §9 item 3) are processed together so each
// KV tile is read once.
//
// Decode reads every KV byte once and does 2*G flops per KV element, so it
// is bound by HBM bandwidth (ybb.press §9, 九、前沿进展与未来展望, item 4: decode
// is the memory-bound phase).
//
// Fast path (bf16 or fp8 cache, bf16 q, head_dim 64/128; a KV head with G > 16
// query heads runs as blocks of at most 16 of them, each a head of its own):
//  * Work unit: a tile = one 16-token block of one KV head (16 x D elements
//    of K and of V, contiguous in the cache).  The tiles of all sequences
//    form one ordered list, (sequence, KV head, block) with the block index
//    fastest; a "segment" is the run of tiles of one (sequence, KV head).
//  * Persistent waves, one per work-group: the list is cut into equal
//    contiguous ranges, one per wave, so every wave streams the same number
//    of bytes whatever the length mix.  A wave keeps kNT tiles in flight
//    across segment boundaries; the next block ids, the next sequence's
//    length and the next segment's q are fetched while earlier tiles are
//    being used, so the load pipeline never drains inside a range.
//  * Tiles are read with buffer loads whose range is the tile's valid rows:
//    slots past the context length read as zero and move no data, and a
//    slot of the ring with nothing to load has range 0.
//  * Both products of a tile are MFMAs with the cache tile as the A operand.
//    Logits are formed transposed, S^T = K q^T (16x16x32 bf16, one per 32
//    dims, q zero-padded to 16 heads), with K read from HBM straight into
//    operand layout; this leaves lane (head h, quad) holding
//    S[h][4*quad..+3] -- exactly the B operand layout of the 16x16x16 bf16
//    MFMA that forms O^T = V^T P^T, so P never moves between lanes.  That
//    MFMA wants 4 tokens of one dim per lane, the transpose of how the
//    token-major V tile is stored: V rows are loaded whole, staged in a
//    per-wave LDS tile, and read back down its columns.  The running max is moved only when a logit exceeds it by more
//    than 2^8 (any reference max gives the same softmax): the common path
//    has no cross-lane step at all.  P is rounded to bf16 once and the sum
//    takes the rounded values, so the weights applied are exactly
//    normalised.
//  * A segment that lies inside one wave's range writes its output row
//    directly.  A segment cut between waves leaves each piece's (max, sum,
//    unnormalised output) in the workspace; an arrival counter per segment
//    tells the last piece to finish, which merges all pieces by the
//    log-sum-exp rule and resets the counter to zero.
//
// General path (fp32 cache, or shapes the fast path does not cover): one
// wave per (512-token partition, query head, sequence), one token at a time,
// plus a separate log-sum-exp reduce kernel.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "debug_checks.h"
#include "device_common.h"
#include "status.h"

namespace pagedkv {

int dtype_bytes(int dt);
pa_status check_desc(const pa_cache_desc* c, const char* fn);
pa_status launch_status(const char* fn);

namespace {

constexpr float kRescaleSlack = 8.0f;   // log2 units: exponentials stay <= 2^8
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kAuxNonTemporal = 2;      // buffer load cache policy: nt
constexpr int kWavesPerCU = 4;          // fast path: persistent waves per CU (one per SIMD)
constexpr int kWavesPerGroup = 1;       // fast path: waves per work-group
constexpr int kPadLds = 0;              // fast path: extra LDS per work-group (occupancy cap)
constexpr int kMinTilesPerWave = 8;     // fast path: at least this many tiles per wave
constexpr int kNT = 3;                  // fast path: tiles in flight per wave
constexpr int kCap = 512;               // fast path: tile descriptors per round (LDS)
constexpr int kGather = 4;              // fast path: block-id loads in flight per lane
constexpr int kAuxCoherent = 16;        // buffer cache policy sc1: device-coherent access
constexpr int kMaxRows = 16;            // fast path: query rows per pass (MFMA columns)
constexpr float kNoMax = -1e30f;        // running max of a row that has seen no position yet
constexpr int kOutOfRange = 0x7FFFFF00; // buffer offset past any range: the load reads 0
constexpr int kTile = 16;               // fast path: tokens per MFMA tile (a block holds 1, 2 or 4)
constexpr int kSeqBits = 26;            // descriptor word 2: sequence | window start << 26
constexpr uint32_t kSeqMask = (1u << kSeqBits) - 1;

// DPP controls (GFX9 encoding).
constexpr int kDppQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int kCtrl>
__device__ __forceinline__ float dpp_c(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, false));
}

// Max / sum over the 16 lanes of a DPP row, result in every lane of the row.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_c<kDppQuadSwap1>(x));
  x = fmaxf(x, dpp_c<kDppQuadSwap2>(x));
  x = fmaxf(x, dpp_c<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp_c<kDppRowMirror>(x));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_c<kDppQuadSwap1>(x);
  x += dpp_c<kDppQuadSwap2>(x);
  x += dpp_c<kDppRowHalfMirror>(x);
  x += dpp_c<kDppRowMirror>(x);
  return x;
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}
__device__ __forceinline__ int readlane_i(int x, int lane) {
  return __builtin_amdgcn_readlane(x, lane);
}
// floor(x / d) for 0 <= x < 2^12 and 1 <= d <= 32, given rcp = 1/d to within
// 2 ulp: (x + 1/2) / d is at least 1/(2d) >= 2^-6 away from an integer,
// while the float error of the product is below 2^12 * 2^-22 = 2^-10.  A
// handful of instructions instead of the ~25 of an integer division by a
// runtime value.
__device__ __forceinline__ int div_small(int x, float rcp) {
  return static_cast<int>((static_cast<float>(x) + 0.5f) * rcp);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, kRsrcWord3);
}
// The same for a base and size that are wave-uniform but that the compiler
// may not prove so (values merged across branches): taken through
// readfirstlane, the descriptor stays in scalar registers instead of a
// loop over lanes around every load that uses it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_uniform(const char* base, int64_t off,
                                                                     int bytes) {
  const uint64_t o = static_cast<uint64_t>(off);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(o & 0xFFFFFFFFu)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(o >> 32)));
  const int n = __builtin_amdgcn_readfirstlane(bytes);
  return make_rsrc(base + static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo), n);
}

// Inclusive prefix sum over the 64 lanes of a wave, by DPP operand moves
// (register-to-register, no LDS round trips): shifts right by 1, 2, 4 and 8
// lanes inside each 16-lane row (lanes shifted in from outside the row add
// 0), then lane 15's total is added to rows 1 and 3 and lane 31's to rows 2
// and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 1, 0xf, 0xf, true);
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 2, 0xf, 0xf, true);
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 4, 0xf, 0xf, true);
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 8, 0xf, 0xf, true);
  x += __builtin_amdgcn_update_dpp(0, x, kRowBcast15, 0xa, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, kRowBcast31, 0xc, 0xf, false);
  return x;
}
// Sum over the 64 lanes of a wave, as a wave-uniform value.
__device__ __forceinline__ int wave_sum(int x) {
  return __builtin_amdgcn_readlane(wave_incl_scan(x), 63);
}
// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, then for the other waves; global loads stay in flight (a
// full __syncthreads also waits for every outstanding global access).  The
// memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Transposing LDS read of 16-bit data (gfx950): each lane addresses 8
// bytes; within every 16 lanes, lane i receives in element k element i mod 4
// of the bytes lane 4k + i/4 addressed.  p must point into LDS.
__device__ __forceinline__ u32x2_t lds_read_tr16(const char* p) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p)));
}

// Maximum over the 64 lanes of a wave, as a wave-uniform value.
__device__ __forceinline__ int wave_max_int(int x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x = max(x, __shfl_xor(x, d));
  return __builtin_amdgcn_readfirstlane(x);
}

// Result of one (partition, query head or KV head, sequence) of the general
// path: either the final output rows, or partial results for the reduce.
struct PartOut {
  void* out;            // [B][Hq][D], q dtype
  float* ws_o;          // [B][Hq][P][D]
  float* ws_ml;         // [B][Hq][P][2]  (max in log2 units, sum)
  int num_parts;        // P (workspace stride)
};

template <bool kOutF32>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v) {
  if constexpr (kOutF32) {
    static_cast<float*>(out)[idx] = v;
  } else {
    static_cast<uint16_t*>(out)[idx] = static_cast<uint16_t>(f32_to_bf16_bits(v));
  }
}

// ---------------------------------------------------------------------------
// Fast path.
// A pass covers `rows` = G * (chunk tokens of the pass) <= 16 query rows per
// KV head: row n is chunk token t_first + n / G of query head g*G + n % G.
// Single-token decode is chunk = 1, one pass with rows = G.
// A KV head with more than 16 query heads is decoded as kv_split row blocks
// of G = (query heads per KV head) / kv_split heads each: the kernel's
// "heads" (hkv of them, hkv = cache heads * kv_split) are those blocks, and
// block g reads cache head g / kv_split.  Query head gG + h of the kernel's
// numbering is the same query head as in the caller's, so q, out and the
// arrival counters need no other change.
struct StreamArgs {
  const char* k_cache;
  const char* v_cache;
  const uint16_t* q;          // [B][chunk][Hq][D] bf16
  uint16_t* out;              // [B][chunk][Hq][D] bf16
  const int32_t* block_tables;
  const int32_t* context_lens;
  uint32_t* counters;         // [B * Hkv], zero between calls
  float* partials;            // [num_waves][2][rows][kD + 2]
  int num_seqs;
  int hkv;                    // kernel heads: cache KV heads * kv_split
  int kv_split;               // row blocks per cache KV head (1 unless G > 16)
  int max_blocks;
  int num_waves;
  int group;                  // G: query heads per kernel head
  int chunk;                  // T: new tokens per sequence
  int window;                 // W > 0: attend only the last W positions; 0: all
  int sub_shift;              // log2(block size / 16): tiles per block = 1 << sub_shift
  int pair_nrec;              // 8-token blocks: bytes of one cache (< 2^31 - 2^16), or 0
                              // for a larger cache (a descriptor per block)
  // shared prefixes (null when unused): a sequence with prefix_len[s] > 0
  // has the attention over its first prefix_len[s] positions in
  // prefix_rec[(s*Hq + h)*(kD + 4)]: unnormalised o[kD], max m (log2 units),
  // sum l, 2 floats of padding (16-byte rows); the tables and lengths this
  // kernel reads are the suffixes'.
  const int32_t* prefix_len;
  const float* prefix_rec;
  int t_first;                // first chunk token of this pass
  int rows;                   // query rows of this pass (<= kMaxRows)
  float logit_scale;          // scale * k_scale * log2(e)
  float v_scale;
  // q rows (of Hq heads each) from one sequence's to the next (the chunk
  // length T; 1 in a group pass) and in all of q: loads past them read 0
  int q_seq_rows;
  int q_total_rows;
  int causal;                 // 1: chunk token t sees positions < L - T + 1 + t; 0: all < L
  // group pass (null otherwise): "sequence" s leads a group of rec_count[s]
  // consecutive sequences whose rows are the chunk tokens (T = the most
  // members of any group); its length and table are the group's shared
  // prefix.  Each member row's attention over it is written as a record
  // rec_out[((s + t)*Hq + h)*(kD + 4)]: unnormalised o[kD], max m (log2
  // units), sum l -- the prefix records a later pass folds in.
  float* rec_out;
  const int32_t* rec_count;
  // group mode only (kGrp), 1: the tile list is ordered by KV head first,
  // then by segment-starting sequence, and wave w of the grid works on the
  // range of index (w mod 8) * (waves / 8) + w / 8 (waves a multiple of 8):
  // the dispatcher deals work-groups to the 8 XCDs in turn, so the waves of
  // one XCD take one eighth of the list, i.e. the segments of 1/8 of the KV
  // heads, and a prefix read by many row groups of a head stays in that
  // XCD's L2.  0: (sequence, KV head) order, wave w takes range w.
  int head_major;
};

// Groups of a shared-prefix batch decoded in one launch (kGrp), one word per
// sequence (at most 256): bit 0 -- the sequence is a member of a group
// whose first `shared` table entries name the same blocks; bit 1 -- it is
// the group's first member (its leader); bits 2..10 -- the group's member
// count, in the leader's word only; bits 11..31 -- shared.  Sequences
// outside groups (and past the batch) have word 0.
struct GroupTable {
  uint32_t info[256];
};
constexpr uint32_t kGrpMember = 1u, kGrpLeader = 2u;
__host__ __device__ constexpr uint32_t grp_count(uint32_t w) { return (w >> 2) & 511u; }
__host__ __device__ constexpr uint32_t grp_shared(uint32_t w) { return w >> 11; }
constexpr uint32_t kGrpMaxShared = (1u << 21) - 1;
struct NoGroupTable {
  int num;
};

// kD: head_dim; kFp8: E4M3 cache (else bf16); kAux: cache policy bits of the
// KV loads; kPair: 8-token blocks; kGrp: shared-prefix groups in one launch.
//
// kGrp (at most 256 sequences, single-token decode, block size a multiple
// of 16): a group is one segment per KV head -- the tiles of the shared
// prefix, then each member's own tiles past it -- with the members' query
// rows (member t, head h: row t * G + h, q rows one sequence apart) as the
// pass's rows.  Every member row sees the prefix tiles (up to its own
// length), a member's own tiles are seen by its rows only, so each row's
// result is its sequence's attention over its whole context; the segment is
// split between waves and merged like any other.  Sequences outside groups
// are segments of their own, written for one sequence's rows.
template <int kD, bool kFp8, int kAux, bool kPair, bool kGrp = false>
__global__ void __launch_bounds__(64 * kWavesPerGroup)
decode_stream_kernel(StreamArgs a,
                     typename std::conditional<kGrp, GroupTable, NoGroupTable>::type gt) {
  constexpr int kE = kFp8 ? 1 : 2;                 // bytes per cache element
  constexpr int kRowBytes = kD * kE;
  constexpr int kTileBytes = kTile * kRowBytes;
  constexpr int kKK = kD / 32;                     // QK MFMA steps over head_dim
  constexpr int kVC = kD / 16;                     // P.V MFMAs (16 dims each)
  constexpr int kLanesPerRow = kD / 8;             // V: lanes covering one token row
  constexpr int kRowsPerLoad = 64 / kLanesPerRow;  // V: token rows per load
  constexpr int kVLoads = kTile / kRowsPerLoad;   // V: loads per lane
  // LDS row pitch of the V staging tile, which holds bf16 rows (an fp8
  // cache's V is widened on its way in, exactly): rows are read 8 bytes per
  // lane, 4 rows by each 16 lanes (pitch = 32 mod 256 puts them on
  // distinct banks)
  constexpr int kVStride = kD * 2 + 32;
  constexpr int kRowOutBytes = kD * 2;             // one bf16 output row
  using Chunk = typename std::conditional<kFp8, u32x2_t, u32x4_t>::type;

  // waves of a work-group are independent (no barriers): a work-group only
  // places kWavesPerGroup waves on one CU together
  const int wig = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w_grid = blockIdx.x * kWavesPerGroup + wig;
  const bool hmaj = kGrp && a.head_major != 0;
  // the wave's range index (head-major group mode: XCD-major, see StreamArgs)
  const int w = hmaj ? (w_grid & 7) * (a.num_waves >> 3) + (w_grid >> 3) : w_grid;
  const int lane = threadIdx.x & 63;
  const int B = a.num_seqs;
  const int hkv = a.hkv;
  const int G = a.group;
  const int nchunk = a.chunk;
  const int R = a.rows;
  const int hq = hkv * G;
  const int slot_floats = (R * (kD + 2) + 3) & ~3; // floats per partial slot (16-byte multiple)
  const float rcp_R = __builtin_amdgcn_rcpf(static_cast<float>(R));   // for div_small (R, G <= 16)
  const float rcp_G = __builtin_amdgcn_rcpf(static_cast<float>(G));
  // With a window, a (sequence, KV head) segment covers the blocks from the
  // one holding the first chunk token's window start to the last.
  const int win = a.window;
  auto first_blk = [&](int L) -> int { return win > 0 ? max(0, L - nchunk + 1 - win) / kTile : 0; };
  auto tiles_of = [&](int L) -> int { return (L + kTile - 1) / kTile - first_blk(L); };
  const __amdgpu_buffer_rsrc_t lens_rsrc = make_rsrc(a.context_lens, B * 4);

  // ---- 1. total tile count; zero rows of empty sequences s = w (mod waves).
  // The lengths of the first 256 sequences stay in registers (Lr[r] holds
  // sequence 64*r + lane): batches up to 256 need a single length load.
  int Lr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
    Lr[r] = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(lens_rsrc, (64 * r + lane) * 4, 0, 0));

  // kGrp: each sequence's group word (Inf: lane l of register r holds
  // sequence 64r + l), read from the kernel arguments beside the lengths,
  // and the tiles per KV head of the segment the sequence starts (Ur: a
  // group's leader counts the prefix and every member's own tiles, the
  // other members 0, a sequence outside groups its own tiles)
  uint32_t Inf[4] = {0u, 0u, 0u, 0u};
  int Ur[4] = {0, 0, 0, 0};
  const int tile_shift = a.sub_shift;                      // block tiles = 1 << tile_shift
  if constexpr (kGrp) {
#pragma unroll
    for (int r = 0; r < 4; ++r) Inf[r] = gt.info[64 * r + lane];
    int suf[4], S[4], carry = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int P = static_cast<int>(grp_shared(Inf[r]) << tile_shift) * kTile;
      suf[r] = (Inf[r] & kGrpMember) ? (max(Lr[r] - P, 0) + kTile - 1) / kTile : 0;
      S[r] = wave_incl_scan(suf[r]) + carry;
      carry = readlane_i(S[r], 63);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int sq = 64 * r + lane;
      const bool lead = (Inf[r] & kGrpLeader) != 0;
      const int end = lead ? sq + static_cast<int>(grp_count(Inf[r])) - 1 : sq;   // the group's last member
      const int e_same = __shfl(S[r], end & 63);
      const int e_next = __shfl(S[r < 3 ? r + 1 : 3], end & 63);
      const int s_end = (end >> 6) == r ? e_same : e_next;
      Ur[r] = !(Inf[r] & kGrpMember) ? (sq < B ? (Lr[r] + kTile - 1) / kTile : 0)
              : lead ? static_cast<int>(grp_shared(Inf[r]) << tile_shift) + s_end - S[r] + suf[r] : 0;
    }
  }
  (void)gt;
  // the first sequence that starts a segment (head-major walk: where each
  // head's block of the list begins)
  int s_first = B;
  if constexpr (kGrp) {
#pragma unroll
    for (int r = 3; r >= 0; --r) {
      const uint64_t m = __builtin_amdgcn_ballot_w64(Ur[r] > 0);
      if (m != 0) s_first = 64 * r + __builtin_ctzll(m);
    }
  }
  // group word of sequence sq (< 256), wave-uniform
  auto info_of = [&](int sq) -> uint32_t {
    const int r = sq >> 6;
    const uint32_t v = (r == 0) ? Inf[0] : (r == 1) ? Inf[1] : (r == 2) ? Inf[2] : Inf[3];
    return static_cast<uint32_t>(readlane_i(static_cast<int>(v), sq & 63));
  };
  auto ut_of = [&](int sq) -> int {
    const int r = sq >> 6;
    const int v = (r == 0) ? Ur[0] : (r == 1) ? Ur[1] : (r == 2) ? Ur[2] : Ur[3];
    return readlane_i(v, sq & 63);
  };
  // sequences whose rows a segment started by sq writes: its group's
  // members for a group leader, else sq alone
  auto seg_count = [&](int sq) -> int {
    if constexpr (kGrp) {
      const uint32_t inf = info_of(sq);
      return (inf & kGrpLeader) ? static_cast<int>(grp_count(inf)) : 1;
    } else {
      return R / G;
    }
  };
  auto round_blocks = [&](int s0, const int (&L)[4]) -> int {   // blocks of s0..s0+255
    int c = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = s0 + 64 * r + lane;
      c += kGrp ? Ur[r] : tiles_of(L[r]);
      const uint64_t empty = __builtin_amdgcn_ballot_w64(s < B && L[r] == 0 && s % a.num_waves == w &&
                                                         a.rec_out == nullptr && !(Inf[r] & kGrpMember));
      for (uint64_t m = empty; m != 0; m &= m - 1) {
        const int se = s0 + 64 * r + __builtin_ctzll(m);
        uint16_t* orow = a.out + (static_cast<int64_t>(se) * nchunk + a.t_first) * hq * kD;
        if (a.prefix_len != nullptr && a.prefix_len[se] > 0) {
          // all of it is shared prefix (single-token decode): its record alone
          for (int i = lane; i < hq * kD / 8; i += 64) {
            const int h = i / (kD / 8), d0 = 8 * i - h * kD;
            const float* rec = a.prefix_rec + (static_cast<int64_t>(se) * hq + h) * (kD + 4);
            const float lp = rec[kD + 1];
            const float inv = lp > 0.f ? a.v_scale * __builtin_amdgcn_rcpf(lp) : 0.f;
            const f32x4_t x0 = *reinterpret_cast<const f32x4_t*>(rec + d0);
            const f32x4_t x1 = *reinterpret_cast<const f32x4_t*>(rec + d0 + 4);
            const bf16x8_t v = {static_cast<__bf16>(x0[0] * inv), static_cast<__bf16>(x0[1] * inv),
                                static_cast<__bf16>(x0[2] * inv), static_cast<__bf16>(x0[3] * inv),
                                static_cast<__bf16>(x1[0] * inv), static_cast<__bf16>(x1[1] * inv),
                                static_cast<__bf16>(x1[2] * inv), static_cast<__bf16>(x1[3] * inv)};
            reinterpret_cast<u32x4_t*>(orow)[i] = __builtin_bit_cast(u32x4_t, v);
          }
        } else {
          for (int i = lane; i < (kGrp ? 1 : R / G) * hq * kD / 8; i += 64)
            reinterpret_cast<u32x4_t*>(orow)[i] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
    return wave_sum(c);
  };
  int T = round_blocks(0, Lr);
  for (int s0 = 256; s0 < B; s0 += 256) {
    int L[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      L[r] = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(lens_rsrc, (s0 + 64 * r + lane) * 4, 0, 0));
    T += round_blocks(s0, L);
  }
  const int Tg = T;                                       // tiles of one KV head
  T *= hkv;
  const int per = (T + a.num_waves - 1) / a.num_waves;
  const int t_begin = w * per;
  if (per == 0 || t_begin >= T) return;

  // ---- 2. the segment and block of tile t_begin: the first sequence whose
  // inclusive tile prefix passes t_begin
  // (head-major: the head of tile t_begin, then the segment inside its
  // block of Tg tiles)
  int s_cur = -1, off = 0, L_cur = 0, U_cur = 0, seg0 = 0;
  const int g_hm = hmaj ? t_begin / Tg : 0;
  const int tgt = t_begin - g_hm * Tg;
  {
    int base = 0;
    auto scan64 = [&](int s0, int L, int U) {
      const int c = hmaj ? U : hkv * (kGrp ? U : tiles_of(L));
      const int incl = wave_incl_scan(c);
      const uint64_t m = __builtin_amdgcn_ballot_w64(base + incl > tgt);
      if (m != 0) {
        const int l0 = __builtin_ctzll(m);
        s_cur = s0 + l0;
        const int excl = base + readlane_i(incl, l0) - readlane_i(c, l0);
        off = tgt - excl;
        L_cur = readlane_i(L, l0);
        U_cur = readlane_i(U, l0);
        seg0 = excl;
      }
      base += readlane_i(incl, 63);
    };
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (s_cur < 0) scan64(64 * r, Lr[r], Ur[r]);
    for (int s0 = 256; s0 < B && s_cur < 0; s0 += 64)
      scan64(s0, static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(lens_rsrc, (s0 + lane) * 4, 0, 0)),
             0);
  }
  // lengths changed under us: nothing safe to do
  if (s_cur < 0 || (kGrp ? U_cur <= 0 : L_cur <= 0)) return;
  // tile t_begin is block j0 of KV head g0 of sequence s_cur (kGrp: tile j0
  // of the segment s_cur starts)
  const int nb0 = kGrp ? U_cur : tiles_of(L_cur);
  const int g0 = hmaj ? g_hm : off / nb0;
  const int j0 = first_blk(L_cur) + (off - (hmaj ? 0 : g0) * nb0);
  const int n_total = min(per, T - t_begin);

  // q of a segment travels with each ring slot, loaded straight into the
  // MFMA B-operand layout of S^T = K q^T: lane (row, quad) holds dims
  // 32*kk + 8*quad .. +7 of query row `row`; rows past R read as zero.
  // Row `row` is chunk token t_row, query head g*G + h_row; it may see the
  // context up to L - mshift positions (causal order inside the chunk).
  const int row = lane & 15;
  const int quad = lane >> 4;
  const bool row_ok = row < R;
  const int t_row = a.t_first + (row_ok ? row / G : 0);
  const int h_row = row_ok ? row - (row / G) * G : 0;
  const int mshift = a.causal ? nchunk - 1 - t_row : 0;
  // the largest shift of the pass (its first chunk token): a tile with at
  // least 16 + mshift_max rows to the context's end masks nothing
  const int mshift_max = a.causal ? nchunk - 1 - a.t_first : 0;
  // one segment's q rows (kGrp: up to R / G member sequences, one apart)
  const int q_bytes = (((kGrp ? R / G : nchunk) - 1) * hq + G) * kD * 2;
  const int64_t q_all_bytes = static_cast<int64_t>(a.q_total_rows) * hq * kD * 2;
  // q in the B-operand layout, dims matching K's: bf16 step kk, quad q
  // holds dims 32kk + 8q .. +7; fp8 K is loaded 16 dims per lane (one
  // 16-byte load for two steps: half the cache-line requests of 8-byte
  // loads), so there step kk, quad q holds dims 64 (kk/2) + 16q + 8 (kk%2)
  // .. +7 -- a permutation of the contraction's dims, applied to both sides
  const int q_lane_off = row_ok ? ((t_row * hq + h_row) * kD + (kFp8 ? 16 : 8) * quad) * 2 : kOutOfRange;
  auto q_step_off = [](int kk) -> int { return kFp8 ? 128 * (kk >> 1) + 16 * (kk & 1) : 64 * kk; };

  // ---- 3. tile descriptors, built in LDS in rounds of up to kCap tiles
  // word 0: tile index block * Hkv + g (the block's position in the table
  //         while building); word 1: rows to the context's end, min(31, L - 16j)
  //         (the tile's valid rows are min(16, that)) | first << 5 | last << 6 |
  //         g << 7 | tiles of the segment << 16; word 2: sequence | window code
  // << 26 (0 without a window, else 17 + the first chunk token's window
  // start relative to the segment's first block, clamped at -16); word 3:
  // list index of the
  // segment's first tile.  "first"/"last" mark the ends of a piece: a
  // segment's ends or the ends of this wave's range.
  __shared__ u32x4_t s_desc_all[kWavesPerGroup][kCap];
  u32x4_t* s_desc = s_desc_all[wig];
  // 8-token blocks: a tile is two blocks; word 0 holds the first block's
  // 8-row tile index (block * Hkv + head), this the second's
  __shared__ uint32_t s_pair_all[kWavesPerGroup][kPair ? kCap : 1];
  uint32_t* s_pair = s_pair_all[wig];
  // V tile staging (token-major rows, padded pitch): it turns the V tile's
  // rows into the P.V MFMA's operand, 4 tokens of one dim per lane
  __shared__ __align__(16) char s_v_all[kWavesPerGroup][kTile * kVStride];
  char* s_v = s_v_all[wig];
  // output staging: the rows of a finished segment are gathered here so
  // that each row goes to memory as whole 16-byte pieces, 256 contiguous
  // bytes per row (partial-line stores are slow on this memory path)
  constexpr int kOPitch = kRowOutBytes + 16;
  __shared__ __align__(16) char s_o_all[kWavesPerGroup][kMaxRows * kOPitch];
  char* s_o = s_o_all[wig];
  // this wave's (at most two) partial pieces, parked here while the ring
  // runs and published to the workspace once it has drained
  constexpr int kSlotBytesMax = kMaxRows * (kD + 2) * 4;
  __shared__ __align__(16) char s_p_all[kWavesPerGroup][2 * kSlotBytesMax];
  char* s_p = s_p_all[wig];
  int w_s = s_cur, w_g = g0, w_j = j0, w_L = L_cur, w_nb = kGrp ? U_cur : (L_cur + kTile - 1) / kTile;
  int w_jf = first_blk(L_cur), w_seg = hmaj ? g_hm * Tg + seg0 : seg0 + g0 * nb0;
  // The first chunk token's window starts at L - T + 1 - W; a row of chunk
  // token t starts t later.  Code = that start relative to the segment's
  // first block, clamped at -16 (rows then cut nothing), plus 17: 1..32.
  auto lo_code = [&](int L, int jf) -> uint32_t {
    return win > 0 ? static_cast<uint32_t>(max(L - nchunk + 1 - win - kTile * jf, -kTile) + kTile + 1)
                   : 0u;
  };
  // lengths for the walk: from Lr for the first 256 sequences, past them
  // from a window of 64 (lane i -> sequence lwin_base + i) loaded on demand
  int lwin_base = -1, lwin = 0;
  auto len_of = [&](int sq) -> int {
    if (sq < 256) {
      const int r = sq >> 6;
      const int v = (r == 0) ? Lr[0] : (r == 1) ? Lr[1] : (r == 2) ? Lr[2] : Lr[3];
      return readlane_i(v, sq & 63);
    }
    if (lwin_base < 0 || sq - lwin_base >= 64) {
      lwin_base = sq;
      lwin = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(lens_rsrc, (lwin_base + lane) * 4, 0, 0));
    }
    return readlane_i(lwin, sq - lwin_base);
  };
  const int tbl_bytes = B * a.max_blocks * 4;
  const __amdgpu_buffer_rsrc_t tbl_rsrc = make_rsrc(a.block_tables, tbl_bytes);
  // the cache head a kernel head reads (row blocks of one KV head share its tiles)
  const int kv_split = a.kv_split;
  const uint32_t hkv_cache = static_cast<uint32_t>(hkv / kv_split);
  auto cache_head = [&](uint32_t g) -> uint32_t {
    return kv_split == 1 ? g : g / static_cast<uint32_t>(kv_split);
  };

  // Lane offsets inside a (block, KV head) tile [16][D], in bytes.
  //  K: MFMA A operand of S^T = K q^T, lane (row, quad) holds token `row`,
  //    dims 32*kk + 8*quad .. +7.
  //  V: plain rows, lane l holds token l / kLanesPerRow (+ kRowsPerLoad per
  //    load), dims 8 * (l % kLanesPerRow) .. +7; they pass through LDS.
  const int k_off = kFp8 ? row * kRowBytes + 16 * quad           // fp8: + 64*j, j < kKK/2
                         : (row * kD + 8 * quad) * kE;            // bf16: + 32*kk*kE
  const int v_c = lane % kLanesPerRow;
  const int v_r = lane / kLanesPerRow;
  const int v_off = (v_r * kD + 8 * v_c) * kE;                // + i*kRowsPerLoad*kRowBytes

  // ---- 4. consumer state: online softmax of the current segment piece.
  // Logits are computed transposed (S^T = K q^T), so lane (row, quad) holds
  // S[query row][tokens 4*quad + r], r = 0..3 -- which is exactly the layout
  // of the B operand of the 16x16x16 MFMA that forms P.V.  m_ref is the
  // reference max of the row, the same in its four lanes (kNoMax while the
  // row has seen no position: masked logits then still weigh exactly 0);
  // lacc holds the row's exponent sum (every element: it is formed by an
  // MFMA of the rounded weights with an all-ones operand); oacc[c][r] =
  // O[query row][16*c + 4*quad + r].
  bf16x8_t qa[kKK];
  float m_ref = kNoMax;
  // kGrp: this lane's row may see the prefix below g_plim (its member's
  // length, capped at the prefix); g_short: some row of the segment stops
  // inside the prefix
  int g_plim = 1 << 30;
  bool g_short = false;
  f32x4_t lacc = {0.f, 0.f, 0.f, 0.f};
  f32x4_t oacc[kVC];
  // A operand of the exponent-sum MFMA: bf16 1.0 in every element, so
  // D[i][row] = sum over the tile's tokens of the row's rounded weights
  const s16x4_t ones = {0x3F80, 0x3F80, 0x3F80, 0x3F80};
  int pend_s[2] = {-1, -1}, pend_g[2] = {0, 0}, pend_seg[2] = {0, 0}, pend_nb[2] = {0, 0};

  auto slot_ptr = [&](int wave, int seg) -> int64_t {       // byte offset of a partial slot
    const int which = (seg <= wave * per) ? 0 : 1;
    return static_cast<int64_t>(wave * 2 + which) * slot_floats * 4;
  };
  const __amdgpu_buffer_rsrc_t part_rsrc = make_rsrc(a.partials, 0x7FFFFFFF);

  // Writes the R staged rows of (sequence s, KV head g) to `out`: lane l
  // moves 16 bytes of row r0 + l / (kD/8) per pass.
  auto store_rows = [&](int s, int g) {
    constexpr int kLPR = kRowOutBytes / 16;                // lanes per row
    constexpr int kRPP = 64 / kLPR;                        // rows per pass
    const int rr = lane / kLPR;
    const int ch = lane - rr * kLPR;
    const int nrows = kGrp ? seg_count(s) * G : R;         // kGrp: the segment's members only
    // the segment's first output row (wave-uniform); row n is chunk token (or
    // member) n / G, one token or sequence = hq rows further
    uint16_t* const obase = a.out + ((static_cast<int64_t>(s) * nchunk + a.t_first) * hq + g * G) * kD;
    for (int r0 = 0; r0 < nrows; r0 += kRPP) {
      const int n = r0 + rr;
      if (n < nrows) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(s_o + n * kOPitch + ch * 16);
        const int nt = div_small(n, rcp_G);
        *reinterpret_cast<u32x4_t*>(obase + (nt * hq + (n - nt * G)) * kD + ch * 8) = v;
      }
    }
  };

  auto finalize = [&](int s, int g, int seg, int nb) {
    float l_tot = lacc[0];
    // the whole segment lies in this wave's range [t_begin, t_begin + per)
    const bool whole = seg >= t_begin && seg + nb <= t_begin + per;
    if (whole && a.rec_out != nullptr) {   // group pass: the member rows' records
      const int cnt = a.rec_count[s];
      if (row_ok && t_row < cnt) {
        float* rec = a.rec_out + ((static_cast<int64_t>(s) + t_row) * hq + g * G + h_row) * (kD + 4);
#pragma unroll
        for (int c = 0; c < kVC; ++c) *reinterpret_cast<f32x4_t*>(rec + 16 * c + 4 * quad) = oacc[c];
        if (quad == 0) *reinterpret_cast<f32x2_t*>(rec + kD) = f32x2_t{m_ref, l_tot};
      }
      return;
    }
    if (whole) {   // the whole segment was in this wave: write the output
      if (row_ok) {
        if (a.prefix_len != nullptr) {                       // fold in the shared prefix
          // the record is read together with the prefix length (one round
          // trip in the middle of the ring, not two); a sequence without a
          // prefix ignores what it read and keeps its values exactly
          const float* rec = a.prefix_rec + (static_cast<int64_t>(s) * hq + g * G + h_row) * (kD + 4);
          const int plen = a.prefix_len[s];
          const f32x2_t ml = *reinterpret_cast<const f32x2_t*>(rec + kD);
          f32x4_t po[kVC];
#pragma unroll
          for (int c = 0; c < kVC; ++c) po[c] = *reinterpret_cast<const f32x4_t*>(rec + 16 * c + 4 * quad);
          const bool has = plen > 0;
          const float mp = has ? ml[0] : kNoMax, lp = has ? ml[1] : 0.f;
          const float mn = fmaxf(m_ref, mp);
          const float fa = __builtin_amdgcn_exp2f(m_ref - mn);
          const float fb = has ? __builtin_amdgcn_exp2f(mp - mn) : 0.f;
          l_tot = l_tot * fa + lp * fb;
#pragma unroll
          for (int c = 0; c < kVC; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) oacc[c][r] = oacc[c][r] * fa + (has ? po[c][r] : 0.f) * fb;
        }
        // a row that saw no position has l = 0 and o = 0: a zero row
        const float inv = (l_tot > 0.f) ? a.v_scale * __builtin_amdgcn_rcpf(l_tot) : 0.f;
        char* srow = s_o + row * kOPitch + 8 * quad;
#pragma unroll
        for (int c = 0; c < kVC; ++c) {
          const bf16x4_t pk = {static_cast<__bf16>(oacc[c][0] * inv), static_cast<__bf16>(oacc[c][1] * inv),
                               static_cast<__bf16>(oacc[c][2] * inv), static_cast<__bf16>(oacc[c][3] * inv)};
          *reinterpret_cast<bf16x4_t*>(srow + 32 * c) = pk;
        }
      }
      store_rows(s, g);
      return;
    }
    // A piece of a segment shared with other waves: only the first and the
    // last segment of a range can be shared, so a wave has at most two
    // pieces, in slots 0 and 1, kept in LDS until the ring has drained (a
    // device-coherent store in the middle of the ring would hold up the
    // loads issued after it).  Slot layout (floats): o as [kD/16][4][R][4]
    // -- lane (row, quad)'s 4 values of dims 16c + 4quad .. +3 at
    // ((c*4 + quad)*R + row)*4, so every store instruction writes one
    // contiguous range -- then (m, l) pairs [R][2]
    // (floats).  Pieces are published with device-coherent stores (sc1:
    // written through to the point of coherence of all XCDs); the arrival
    // count follows once they have completed, after the ring has drained.
    // No L2 write-back or invalidation is needed: nothing else is shared.
    const int which = (seg <= w * per) ? 0 : 1;
    char* lslot = s_p + which * kSlotBytesMax;
    if (row_ok) {
#pragma unroll
      for (int c = 0; c < kVC; ++c)
        *reinterpret_cast<f32x4_t*>(lslot + (((c * 4 + quad) * R + row) * 4) * 4) = oacc[c];
      if (quad == 0)
        *reinterpret_cast<f32x2_t*>(lslot + (R * kD + 2 * row) * 4) = f32x2_t{m_ref, l_tot};
    }
    pend_s[which] = s;
    pend_g[which] = g;
    pend_seg[which] = seg;
    pend_nb[which] = nb;
  };

  // The last piece of a segment merges all of them:
  // out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p, computed online.
  // Lane l handles the 4-float groups l + 64*i of the slot layout above
  // (group q: row q % R, dims 16*(q / (4R)) + 4*((q / R) % 4) .. +3).  A
  // piece in which a row saw no position holds m = kNoMax, l = 0, o = 0 and
  // adds nothing; a row that saw none in any piece gets a zero row.
  auto merge = [&](int s, int g, int seg, int nb, int own) {
    const int wf = seg / per;
    const int wl = (seg + nb - 1) / per;
    uint32_t* ctr = a.counters + static_cast<int64_t>(s) * hkv + g;
    constexpr int kE4 = (kMaxRows * kD / 4 + 63) / 64;    // 4-float groups per lane, at most
    const int n_el = R * kD;
    const int n_grp = n_el / 4;
    float M[kE4], den[kE4];
    f32x4_t num[kE4];
#pragma unroll
    for (int i = 0; i < kE4; ++i) {
      M[i] = kNoMax;
      den[i] = 0.f;
      num[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // The rounding is spelled out (a product, then one fused multiply-add;
    // no contraction left to the compiler): the function is inlined at
    // several places, and which place takes a given piece depends on which
    // wave merges, so every place must round alike for the result not to
    // depend on arrival order.
    auto combine = [&](const f32x4_t (&op)[kE4], const float (&mp)[kE4], const float (&lp)[kE4]) {
#pragma clang fp contract(off)
#pragma unroll
      for (int i = 0; i < kE4; ++i) {
        if (64 * i >= n_grp) break;                        // wave-uniform
        const float mn = fmaxf(M[i], mp[i]);
        const float f_old = __builtin_amdgcn_exp2f(M[i] - mn);
        const float f_new = __builtin_amdgcn_exp2f(mp[i] - mn);
        den[i] = __builtin_fmaf(lp[i], f_new, den[i] * f_old);
#pragma unroll
        for (int e = 0; e < 4; ++e) num[i][e] = __builtin_fmaf(op[i][e], f_new, num[i][e] * f_old);
        M[i] = mn;
      }
    };
    // Pieces are combined in wave order whoever merges, so the result does
    // not depend on which piece arrived last.  The other waves' pieces are
    // loaded two at a time (a segment of up to three pieces takes one round
    // trip); this wave's own piece comes from its LDS slot and is combined
    // at its place in the order.
    const char* own_slot = s_p + own * kSlotBytesMax;
    auto from_lds = [&](f32x4_t (&op)[kE4], float (&mp)[kE4], float (&lp)[kE4]) {
#pragma unroll
      for (int i = 0; i < kE4; ++i) {
        if (64 * i >= n_grp) break;
        const int q = min(lane + 64 * i, n_grp - 1);
        op[i] = *reinterpret_cast<const f32x4_t*>(own_slot + q * 16);
        const f32x2_t ml = *reinterpret_cast<const f32x2_t*>(own_slot + (n_el + 2 * (q - div_small(q, rcp_R) * R)) * 4);
        mp[i] = ml[0];
        lp[i] = ml[1];
      }
    };
    auto own_piece = [&]() {
      f32x4_t oo[kE4];
      float mo_[kE4], lo_[kE4];
      from_lds(oo, mo_, lo_);
      combine(oo, mo_, lo_);
    };
    bool own_done = false;
    int pa = (wf == w) ? wf + 1 : wf;                      // first remote piece
    while (pa <= wl) {
      int pb = pa + 1;                                     // the next remote piece, if any
      if (pb == w) ++pb;
      const bool has_b = pb <= wl;
      f32x4_t oa[kE4], ob[kE4];
      float ma[kE4], la[kE4], mb[kE4], lb[kE4];
      const char* base = reinterpret_cast<const char*>(a.partials);
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(base + slot_ptr(pa, seg), slot_floats * 4);
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(base + (has_b ? slot_ptr(pb, seg) : 0),
                                                  has_b ? slot_floats * 4 : 0);
#pragma unroll
      for (int i = 0; i < kE4; ++i) {
        if (64 * i >= n_grp) break;
        const int q = min(lane + 64 * i, n_grp - 1);
        const int mo = (n_el + 2 * (q - div_small(q, rcp_R) * R)) * 4;
        oa[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, q * 16, 0, kAuxCoherent));
        ob[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rb, q * 16, 0, kAuxCoherent));
        const u32x2_t mla = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(ra, mo, 0, kAuxCoherent));
        const u32x2_t mlb = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rb, mo, 0, kAuxCoherent));
        ma[i] = __uint_as_float(mla[0]);
        la[i] = __uint_as_float(mla[1]);
        mb[i] = __uint_as_float(mlb[0]);
        lb[i] = __uint_as_float(mlb[1]);
      }
      if (!own_done && w < pa) {
        own_piece();
        own_done = true;
      }
      combine(oa, ma, la);
      if (has_b) {
        if (!own_done && w < pb) {
          own_piece();
          own_done = true;
        }
        combine(ob, mb, lb);
      }
      pa = pb + 1;
      if (pa == w) ++pa;
    }
    if (!own_done) own_piece();
    if (a.prefix_len != nullptr && a.prefix_len[s] > 0) {     // fold in the shared prefix
#pragma unroll
      for (int i = 0; i < kE4; ++i) {
        const int q = lane + 64 * i;
        if (q < n_grp) {
          const int cq = div_small(q, rcp_R);
          const int r = q - cq * R;
          const int nt = div_small(r, rcp_G);
          const float* rec = a.prefix_rec + ((static_cast<int64_t>(s) * nchunk + a.t_first + nt) * hq +
                                             g * G + (r - nt * G)) * (kD + 4);
          const float mp = rec[kD], lp = rec[kD + 1];
          const f32x4_t po = *reinterpret_cast<const f32x4_t*>(rec + 4 * cq);
          const float mn = fmaxf(M[i], mp);
          const float fa = __builtin_amdgcn_exp2f(M[i] - mn), fb = __builtin_amdgcn_exp2f(mp - mn);
          den[i] = den[i] * fa + lp * fb;
#pragma unroll
          for (int e = 0; e < 4; ++e) num[i][e] = num[i][e] * fa + po[e] * fb;
          M[i] = mn;
        }
      }
    }
    if (a.rec_out != nullptr) {                           // group pass: member records
      const int cnt = a.rec_count[s];
#pragma unroll
      for (int i = 0; i < kE4; ++i) {
        const int q = lane + 64 * i;
        const int cq = div_small(q, rcp_R);
        const int r = q - cq * R;
        const int rt = div_small(r, rcp_G);
        const int t = a.t_first + rt;
        if (q < n_grp && t < cnt) {
          float* rec = a.rec_out + ((static_cast<int64_t>(s) + t) * hq + g * G + (r - rt * G)) * (kD + 4);
          *reinterpret_cast<f32x4_t*>(rec + 4 * cq) = num[i];
          if (q < R) *reinterpret_cast<f32x2_t*>(rec + kD) = f32x2_t{M[i], den[i]};
        }
      }
      if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
#pragma unroll
    for (int i = 0; i < kE4; ++i) {
      const int q = lane + 64 * i;
      if (q < n_grp) {
        const int cq = div_small(q, rcp_R);                // c * 4 + quad
        const int r = q - cq * R;
        const float inv = (den[i] > 0.f) ? a.v_scale * __builtin_amdgcn_rcpf(den[i]) : 0.f;
        const bf16x4_t pk = {static_cast<__bf16>(num[i][0] * inv), static_cast<__bf16>(num[i][1] * inv),
                             static_cast<__bf16>(num[i][2] * inv), static_cast<__bf16>(num[i][3] * inv)};
        *reinterpret_cast<bf16x4_t*>(s_o + r * kOPitch + 8 * cq) = pk;
      }
    }
    store_rows(s, g);
    if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  // ring slots: tile data and the segment's q
  constexpr int kKLoads = kFp8 ? kKK / 2 : kKK;    // 16-byte K loads per lane
  u32x4_t kt[kNT][kKLoads];
  Chunk vt[kNT][kVLoads];
  u32x4_t qs[kNT][kKK];

  for (int done = 0; done < n_total;) {
    const int n = min(kCap, n_total - done);
    // pass 1: walk the pieces of this round, one lane per tile
    if constexpr (kGrp) {
      // a group's segment: the prefix tiles (table of the leader, rows to
      // the prefix end), then each member's own tiles (its table from the
      // prefix on, rows to its end), the member in word 2's top bits (1 +
      // its index; 0 for the prefix and for segments outside groups)
      for (int pos = 0; pos < n;) {
        const uint32_t inf = info_of(w_s);                    // a leader, or a lone sequence
        int sub_start = 0, sub_end = w_nb, tbase = 0, sublen = w_L, tseq = w_s, code = 0;
        if (inf & kGrpLeader) {
          const int Pt = static_cast<int>(grp_shared(inf) << tile_shift), P = Pt * kTile;
          if (w_j < Pt) {
            sub_end = Pt;
            sublen = P;
          } else {
            int cum = Pt;
            const int cnt = static_cast<int>(grp_count(inf));
            for (int m = 0; m < cnt; ++m) {
              const int Lm = len_of(w_s + m);
              const int sm = (max(Lm - P, 0) + kTile - 1) / kTile;
              if (w_j < cum + sm) {
                sub_start = cum;
                sub_end = cum + sm;
                tbase = Pt;
                sublen = Lm - P;
                tseq = w_s + m;
                code = m + 1;
                break;
              }
              cum += sm;
            }
          }
        }
        const int span = min(sub_end - w_j, n - pos);
        const uint32_t word2 = static_cast<uint32_t>(tseq) | (static_cast<uint32_t>(code) << kSeqBits);
        for (int c = lane; c < span; c += 64) {
          const int j = w_j + c;
          const int gpos = done + pos + c;                   // position in the range
          const uint32_t valid = static_cast<uint32_t>(min(31, sublen - kTile * (j - sub_start)));
          const uint32_t first = (j == 0 || gpos == 0) ? 1u : 0u;
          const uint32_t last = (j == w_nb - 1 || gpos == n_total - 1) ? 1u : 0u;
          s_desc[pos + c] = u32x4_t{static_cast<uint32_t>(tbase + j - sub_start),
                                    valid | (first << 5) | (last << 6) |
                                        (static_cast<uint32_t>(w_g) << 7) |
                                        (static_cast<uint32_t>(w_nb) << 16),
                                    word2, static_cast<uint32_t>(w_seg)};
        }
        pos += span;
        w_j += span;
        if (w_j == w_nb) {                                   // next segment
          w_seg += w_nb;
          if (hmaj) {                                        // the head's next sequence, then the next head
            do {
              w_s += seg_count(w_s);
              w_nb = (w_s < B) ? ut_of(w_s) : 0;
            } while (w_nb == 0 && w_s < B);
            if (w_s >= B && ++w_g < hkv) {
              w_s = s_first;
              w_nb = ut_of(s_first);
            }
            w_L = (w_s < B) ? len_of(w_s) : 0;
          } else if (++w_g == hkv) {                         // next segment-starting sequence
            w_g = 0;
            do {
              w_s += seg_count(w_s);
              w_nb = (w_s < B) ? ut_of(w_s) : 0;
            } while (w_nb == 0 && w_s < B);
            w_L = (w_s < B) ? len_of(w_s) : 0;
          }
          w_j = 0;
        }
      }
    } else
    for (int pos = 0; pos < n;) {
      const int span = min(w_nb - w_j, n - pos);
      const uint32_t word2 = static_cast<uint32_t>(w_s) | (lo_code(w_L, w_jf) << kSeqBits);
      for (int c = lane; c < span; c += 64) {
        const int j = w_j + c;
        const int gpos = done + pos + c;                     // position in the range
        const uint32_t valid = static_cast<uint32_t>(min(31, w_L - kTile * j));
        const uint32_t first = (j == w_jf || gpos == 0) ? 1u : 0u;
        const uint32_t last = (j == w_nb - 1 || gpos == n_total - 1) ? 1u : 0u;
        s_desc[pos + c] = u32x4_t{static_cast<uint32_t>(j),
                                  valid | (first << 5) | (last << 6) |
                                      (static_cast<uint32_t>(w_g) << 7) |
                                      (static_cast<uint32_t>(w_nb - w_jf) << 16),
                                  word2, static_cast<uint32_t>(w_seg)};
      }
      pos += span;
      w_j += span;
      if (w_j == w_nb) {                                     // next segment
        w_seg += w_nb - w_jf;
        if (++w_g == hkv) {                                  // next non-empty sequence
          w_g = 0;
          do {
            ++w_s;
            w_L = (w_s < B) ? len_of(w_s) : 0;
          } while (w_L == 0 && w_s + 1 < B);
          w_nb = (w_L + kTile - 1) / kTile;
          w_jf = first_blk(w_L);
        }
        w_j = w_jf;
      }
    }
    // pass 2: block ids from the tables, independent loads per lane
    if constexpr (kPair) {
      // tile j is blocks 2j (rows 0-7) and 2j+1 (rows 8-15); the second is
      // read only when the context reaches past the first
      for (int e0 = 0; e0 < n; e0 += 64 * kGather) {
        int ida[kGather], idb[kGather];
#pragma unroll
        for (int r = 0; r < kGather; ++r) {
          const int e = e0 + 64 * r + lane;
          ida[r] = idb[r] = 0;
          if (e < n) {
            const u32x4_t d = s_desc[e];
            const int base = static_cast<int>(d[2] & kSeqMask) * a.max_blocks + 2 * static_cast<int>(d[0]);
            ida[r] = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(tbl_rsrc, base * 4, 0, 0));
            idb[r] = (d[1] & 31u) > 8u
                         ? static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(tbl_rsrc, (base + 1) * 4, 0, 0))
                         : 0;
          }
        }
#pragma unroll
        for (int r = 0; r < kGather; ++r) {
          const int e = e0 + 64 * r + lane;
          if (e < n) {
            const uint32_t g = (s_desc[e][1] >> 7) & 511u;
            const uint32_t ua = static_cast<uint32_t>(ida[r]) * hkv_cache + cache_head(g);
            const bool two = (s_desc[e][1] & 31u) > 8u;
            s_desc[e][0] = ua;
            s_pair[e] = two ? static_cast<uint32_t>(idb[r]) * hkv_cache + cache_head(g) : ua;
          }
        }
      }
    } else
    for (int e0 = 0; e0 < n; e0 += 64 * kGather) {
      int ids[kGather];
#pragma unroll
      for (int r = 0; r < kGather; ++r) {
        const int e = e0 + 64 * r + lane;
        ids[r] = 0;
        if (e < n) {
          const u32x4_t d = s_desc[e];
          ids[r] = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(
              tbl_rsrc, (static_cast<int>(d[2] & kSeqMask) * a.max_blocks +
                         static_cast<int>(d[0] >> a.sub_shift)) * 4, 0, 0));
        }
      }
#pragma unroll
      for (int r = 0; r < kGather; ++r) {
        const int e = e0 + 64 * r + lane;
        if (e < n) {
          // tile j of the sequence is sub-tile j % (tiles per block) of its block
          const uint32_t g = (s_desc[e][1] >> 7) & 511u;
          const uint32_t u = s_desc[e][0] & ((1u << a.sub_shift) - 1u);
          s_desc[e][0] = ((static_cast<uint32_t>(ids[r]) * hkv_cache + cache_head(g)) << a.sub_shift) + u;
        }
      }
    }

    // ---- 5. the ring: kNT tiles in flight.  Every step issues the same
    // K and V loads (empty ranges move nothing), so the wait counts the
    // consumer needs never depend on the path taken.  The q rows are read
    // the same way, except in the KV-head-major group launches (the group
    // launches with the default cache policy, kAux = 0): there the row
    // groups' segments run over hundreds of tiles, nearly every tile starts
    // no piece, and the q loads are issued only where one starts (3% on a
    // batch of 256 requests sharing a 2048-token prompt).  Elsewhere the
    // branch costs more than the loads it skips (1% on the parallel-sampling
    // batch in group mode, 0.5% on the plain decode).
    auto issue = [&](int slot, int t) {
      int k_nrec = 0, v_nrec = 0, q_nrec = 0;
      int64_t tile_off = 0, q_off = 0;
      if (t < n) {
        const u32x4_t d = s_desc[t];
        const uint32_t tile = __builtin_amdgcn_readfirstlane(d[0]);
        const uint32_t info = __builtin_amdgcn_readfirstlane(d[1]);
        int s = __builtin_amdgcn_readfirstlane(static_cast<int>(d[2] & kSeqMask));
        if constexpr (kGrp) {                              // a member's tile: the group's leader
          const int code = __builtin_amdgcn_readfirstlane(static_cast<int>(d[2])) >> kSeqBits;
          s -= code > 0 ? code - 1 : 0;
        }
        k_nrec = min(static_cast<int>(info & 31u), kTile) * kRowBytes;   // rows past the context read 0
        v_nrec = k_nrec;
        tile_off = static_cast<int64_t>(tile) * kTileBytes;
        if (info & 32u) {
          q_off = (static_cast<int64_t>(s) * a.q_seq_rows * hq + static_cast<int>((info >> 7) & 511u) * G) * kD * 2;
          q_nrec = static_cast<int>(min(static_cast<int64_t>(q_bytes), q_all_bytes - q_off));
        }
      }
      const __amdgpu_buffer_rsrc_t rq = make_rsrc_uniform(reinterpret_cast<const char*>(a.q), q_off, q_nrec);
      constexpr bool kQAtStartsOnly = kGrp && kAux == 0;
      if (!kQAtStartsOnly || q_nrec > 0) {                 // (q_nrec is wave-uniform)
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk) qs[slot][kk] = __builtin_amdgcn_raw_buffer_load_b128(rq, q_lane_off + q_step_off(kk), 0, 0);
      } else {
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk) qs[slot][kk] = u32x4_t{0u, 0u, 0u, 0u};
      }
      if constexpr (kPair) {
        // one descriptor over the whole cache, per-lane offsets: rows 0-7
        // of the tile in the first block, rows 8-15 in the second; rows
        // past the context (and an empty slot) get an offset past the
        // cache, which reads 0
        uint32_t ha = 0, hb = 0;
        if (t < n) {
          ha = __builtin_amdgcn_readfirstlane(s_desc[t][0]);
          hb = __builtin_amdgcn_readfirstlane(s_pair[t]);
        }
        const int rows = k_nrec / kRowBytes;
        if (a.pair_nrec == 0) {
          // a cache of 2 GiB or more, beyond one descriptor's 32-bit offsets.
          // Each K load spans all 16 rows, so K is read with global loads
          // from per-lane 64-bit addresses (rows 0-7 in the first block,
          // 8-15 in the second), switched off for rows past the context,
          // whose registers are zeroed first; a V load covers rows of one
          // block only and keeps a buffer descriptor per block.
          const int64_t blk_a = static_cast<int64_t>(ha) * (8 * kRowBytes);
          const int64_t blk_b = static_cast<int64_t>(hb) * (8 * kRowBytes);
          const char* kp = a.k_cache + (row < 8 ? blk_a : blk_b) + (row & 7) * kRowBytes +
                           (kFp8 ? 16 : 8 * kE) * quad;
#pragma unroll
          for (int j = 0; j < kKLoads; ++j) kt[slot][j] = u32x4_t{0u, 0u, 0u, 0u};
          if (row < rows) {
#pragma unroll
            for (int j = 0; j < kKLoads; ++j)
              kt[slot][j] = __builtin_nontemporal_load(
                  reinterpret_cast<const u32x4_t*>(kp + (kFp8 ? 64 : 32 * kE) * j));
          }
          const __amdgpu_buffer_rsrc_t rva = make_rsrc(a.v_cache + blk_a, min(rows, 8) * kRowBytes);
          const __amdgpu_buffer_rsrc_t rvb = make_rsrc(a.v_cache + blk_b, max(rows - 8, 0) * kRowBytes);
          static_assert(8 % kRowsPerLoad == 0, "a V load stays inside one 8-row block");
#pragma unroll
          for (int i = 0; i < kVLoads; ++i) {
            const bool second = i * kRowsPerLoad >= 8;       // the block of this load's rows
            const int vo = ((v_r + i * kRowsPerLoad) & 7) * kRowBytes + 8 * v_c * kE;
            if constexpr (kFp8)
              vt[slot][i] = __builtin_bit_cast(Chunk, __builtin_amdgcn_raw_buffer_load_b64(second ? rvb : rva, vo, 0, kAux));
            else
              vt[slot][i] = __builtin_amdgcn_raw_buffer_load_b128(second ? rvb : rva, vo, 0, kAux);
          }
          (void)tile_off;
          (void)v_nrec;
          return;
        }
        auto row_at = [&](int r) -> int {                  // byte offset of tile row r
          return r < rows ? static_cast<int>((r < 8 ? ha : hb) * static_cast<uint32_t>(8 * kRowBytes)) +
                                (r & 7) * kRowBytes
                          : kOutOfRange;
        };
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k_cache, a.pair_nrec);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v_cache, a.pair_nrec);
        const int ko = row_at(row) + (kFp8 ? 16 : 8 * kE) * quad;
#pragma unroll
        for (int j = 0; j < kKLoads; ++j)
          kt[slot][j] = __builtin_amdgcn_raw_buffer_load_b128(rk, ko + (kFp8 ? 64 : 32 * kE) * j, 0, kAux);
#pragma unroll
        for (int i = 0; i < kVLoads; ++i) {
          const int vo = row_at(v_r + i * kRowsPerLoad) + 8 * v_c * kE;
          if constexpr (kFp8)
            vt[slot][i] = __builtin_bit_cast(Chunk, __builtin_amdgcn_raw_buffer_load_b64(rv, vo, 0, kAux));
          else
            vt[slot][i] = __builtin_amdgcn_raw_buffer_load_b128(rv, vo, 0, kAux);
        }
        (void)tile_off;
        (void)v_nrec;
        return;
      }
      const __amdgpu_buffer_rsrc_t rk = make_rsrc_uniform(a.k_cache, tile_off, k_nrec);
      const __amdgpu_buffer_rsrc_t rv = make_rsrc_uniform(a.v_cache, tile_off, v_nrec);
#pragma unroll
      for (int j = 0; j < kKLoads; ++j)
        kt[slot][j] = __builtin_amdgcn_raw_buffer_load_b128(rk, k_off + (kFp8 ? 64 : 32 * kE) * j, 0, kAux);
#pragma unroll
      for (int i = 0; i < kVLoads; ++i) {
        if constexpr (kFp8)
          vt[slot][i] = __builtin_bit_cast(Chunk, __builtin_amdgcn_raw_buffer_load_b64(rv, v_off + i * kRowsPerLoad * kRowBytes, 0, kAux));
        else
          vt[slot][i] = __builtin_amdgcn_raw_buffer_load_b128(rv, v_off + i * kRowsPerLoad * kRowBytes, 0, kAux);
      }
    };

    auto consume = [&](int slot, int t) {
      if (t >= n) return;
      const u32x4_t d = s_desc[t];
      const uint32_t info = __builtin_amdgcn_readfirstlane(d[1]);
      const int rows_left = static_cast<int>(info & 31u);   // min(31, L - 16j)
      // kGrp: the member code of the tile and the segment's first sequence
      int code = 0, lead = 0;
      if constexpr (kGrp) {
        code = __builtin_amdgcn_readfirstlane(static_cast<int>(d[2])) >> kSeqBits;
        lead = __builtin_amdgcn_readfirstlane(static_cast<int>(d[2] & kSeqMask)) - (code > 0 ? code - 1 : 0);
      }
      if (info & 32u) {                                      // a piece starts here
        if constexpr (kGrp) {
          // a group's rows see the prefix up to their own member's length
          const uint32_t inf = info_of(lead);
          if (inf & kGrpLeader) {
            const int P = static_cast<int>(grp_shared(inf) << tile_shift) * kTile;
            const int cnt = static_cast<int>(grp_count(inf));
            const int sq = lead + min(t_row, cnt - 1);        // < 256
            const int li = sq & 63, rb = sq >> 6;
            const int l0 = __shfl(Lr[0], li), l1 = __shfl(Lr[1], li);
            const int l2 = __shfl(Lr[2], li), l3 = __shfl(Lr[3], li);
            const int Lt = rb == 0 ? l0 : rb == 1 ? l1 : rb == 2 ? l2 : l3;
            g_plim = t_row < cnt ? min(Lt, P) : P;
            g_short = __builtin_amdgcn_ballot_w64(g_plim < P) != 0;
          } else {
            g_plim = 1 << 30;
            g_short = false;
          }
        }
        m_ref = kNoMax;
        lacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kVC; ++c) oacc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk) qa[kk] = __builtin_bit_cast(bf16x8_t, qs[slot][kk]);
      }

      // ---- logits, transposed: acc[r] = S[head row][token 4*quad + r]
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk) {
        bf16x8_t kb;
        if constexpr (kFp8) {
          const u32x4_t wv = kt[slot][kk >> 1];
          const int w0 = static_cast<int>(wv[2 * (kk & 1)]), w1 = static_cast<int>(wv[2 * (kk & 1) + 1]);
          const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
          const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
          const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
          const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
          kb = bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        } else {
          kb = __builtin_bit_cast(bf16x8_t, kt[slot][kk]);
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qa[kk], acc, 0, 0, 0);
      }
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = acc[r] * a.logit_scale;
      // Masks.  Only a tile that reaches the context's end (less the causal
      // shift), or one a window start cuts, has rows a query row may not
      // see; a wave-uniform test skips the masking for every other tile.
      if constexpr (kGrp) {
        // one masking step for every case (a member's tile: its rows only; a
        // prefix tile: each row up to its member's length; a tile at a
        // context's end), skipped by one wave-uniform test otherwise
        if (code != 0 || g_short || rows_left < kTile) {
          int lim = rows_left;
          if (code != 0) {
            lim = (t_row == code - 1) ? rows_left : 0;
          } else if (g_short) {
            const int jl = t_begin + done + t - __builtin_amdgcn_readfirstlane(static_cast<int>(d[3]));
            lim = min(rows_left, g_plim - kTile * jl);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (4 * quad + r >= lim) x[r] = -INFINITY;
        }
      }
      const uint32_t wcode =
          kGrp ? 0u : static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(d[2]))) >> kSeqBits;
      if (!kGrp && (wcode != 0u || rows_left - mshift_max < kTile)) {
        const int lim = rows_left - mshift;                  // tile rows this query row may see
        // window start: tile rows below `lo` are cut (never, without a window)
        int lo = -kTile;
        if (wcode != 0u) {
          const int j_local = t_begin + done + t - __builtin_amdgcn_readfirstlane(static_cast<int>(d[3]));
          lo = static_cast<int>(wcode) - (kTile + 1) + t_row - kTile * j_local;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * quad + r >= lim || 4 * quad + r < lo) x[r] = -INFINITY;
      }

      // ---- lazy running max: moved only when a logit exceeds it by more
      // than 2^kRescaleSlack (rare; a wave-uniform branch)
      const float xm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      if (__builtin_amdgcn_ballot_w64(xm > m_ref + kRescaleSlack) != 0) {
        float mt = xm;
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));                   // max over the head's 16 tokens
        const float mn = (mt > m_ref + kRescaleSlack) ? mt : m_ref;
        const float alpha = __builtin_amdgcn_exp2f(m_ref - mn);
        lacc[0] *= alpha;
#pragma unroll
        for (int c = 0; c < kVC; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) oacc[c][r] *= alpha;
        m_ref = mn;
      }

      // ---- P in bf16, two weights per conversion; the exponent sum takes the
      // rounded values (one MFMA against the all-ones operand), so the
      // weights the P.V MFMA applies are exactly normalised
      const bf16x2_t p01 = __builtin_convertvector(
          (f32x2_t{__builtin_amdgcn_exp2f(x[0] - m_ref), __builtin_amdgcn_exp2f(x[1] - m_ref)}),
          bf16x2_t);
      const bf16x2_t p23 = __builtin_convertvector(
          (f32x2_t{__builtin_amdgcn_exp2f(x[2] - m_ref), __builtin_amdgcn_exp2f(x[3] - m_ref)}),
          bf16x2_t);
      const bf16x4_t pb = {p01[0], p01[1], p23[0], p23[1]};
      lacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones, __builtin_bit_cast(s16x4_t, pb), lacc, 0, 0, 0);
      // V rows through LDS: rows past the context were read as zeros
#pragma unroll
      for (int i = 0; i < kVLoads; ++i) {
        char* dst = s_v + (v_r + i * kRowsPerLoad) * kVStride + 16 * v_c;   // 8 dims, bf16
        if constexpr (kFp8) {
          // 8 E4M3 codes (dims 8 v_c .. +7) to bf16, exactly: 2 per instruction
          const int w0 = static_cast<int>(vt[slot][i][0]), w1 = static_cast<int>(vt[slot][i][1]);
          const u32x4_t wide = {
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false)),
              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true))};
          *reinterpret_cast<u32x4_t*>(dst) = wide;
        } else {
          *reinterpret_cast<u32x4_t*>(dst) = vt[slot][i];
        }
      }
      // one transposing read per MFMA; lane (row, quad) addresses token
      // 4 quad + row/4, dims 16c + 4 (row mod 4) .. +3
      const char* vtr = s_v + (4 * quad + (row >> 2)) * kVStride + 8 * (row & 3);
#pragma unroll
      for (int c = 0; c < kVC; ++c) {
        const u32x2_t vw = lds_read_tr16(vtr + 32 * c);           // tokens 4*quad..+3 of dim 16c+row
        oacc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, vw),
                                                           __builtin_bit_cast(s16x4_t, pb),
                                                           oacc[c], 0, 0, 0);
      }

      if (info & 64u)                                        // a piece ends here
        finalize(kGrp ? lead : __builtin_amdgcn_readfirstlane(static_cast<int>(d[2] & kSeqMask)),
                 static_cast<int>((info >> 7) & 511u),
                 __builtin_amdgcn_readfirstlane(static_cast<int>(d[3])),
                 static_cast<int>(info >> 16));
    };

#pragma unroll
    for (int k = 0; k < kNT; ++k) issue(k, k);
    for (int t0 = 0; t0 < n; t0 += kNT) {
#pragma unroll
      for (int k = 0; k < kNT; ++k) {
        consume(k, t0 + k);
        issue(k, t0 + k + kNT);
      }
    }
    done += n;
  }

  // ---- 6. count the arrivals of the stored pieces (once every store of
  // this wave has completed; both counters at once), then merge the
  // segments of which this wave holds the last piece
  if (pend_s[0] >= 0 || pend_s[1] >= 0) {
    // publish the parked pieces: whole 16-byte chunks, device-coherent
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (pend_s[i] < 0) continue;
      const int64_t mine = slot_ptr(w, pend_seg[i]);
      const char* lslot = s_p + i * kSlotBytesMax;
      for (int off = 16 * lane; off < slot_floats * 4; off += 1024)
        __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4_t*>(lslot + off),
                                               part_rsrc, static_cast<int>(mine + off), 0,
                                               kAuxCoherent);
    }
    wait_memory_done();
    uint32_t prev[2] = {0u, 0u};
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        if (pend_s[i] >= 0)
          prev[i] = __hip_atomic_fetch_add(a.counters + static_cast<int64_t>(pend_s[i]) * hkv + pend_g[i],
                                           1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    compiler_fence();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (pend_s[i] < 0) continue;
      const int wf = pend_seg[i] / per;
      const int wl = (pend_seg[i] + pend_nb[i] - 1) / per;
      if (static_cast<uint32_t>(readlane_i(static_cast<int>(prev[i]), 0)) ==
          static_cast<uint32_t>(wl - wf))                      // the last piece
        merge(pend_s[i], pend_g[i], pend_seg[i], pend_nb[i], i);
    }
  }
}

// Zero-fill of a decode workspace.
__global__ void __launch_bounds__(256)
zero_fill_kernel(uint32_t* p, int64_t n_words) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n_words; i += stride)
    p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Shared prefixes.  Sequences first .. first+count-1 of a group share the
// physical blocks of their first `shared` table entries (a prompt reused
// through prefix caching).  Attention over those positions is one dense
// contraction per KV head -- every member's query rows against the same K
// and V -- so it is computed once per group, on MFMA, with many query rows
// per tile, and folded into each row's result by the log-sum-exp rule.
//
// What bounds it is moving the shared tiles from L2 into the CUs: a
// workgroup reads each tile of its position range once, so the bytes moved
// are the prefix's bytes times (rows / rows per workgroup).  A workgroup
// therefore takes 128 rows (8 waves of 16) that all read each tile from
// LDS, and the prefix's positions are split over several workgroups to
// fill the chip; the last split of a row block to finish merges the
// splits' records.
constexpr int kMaxGroups = PA_MAX_PREFIX_GROUPS;   // groups travel in the kernel arguments
constexpr int kPrefixWaves = 8;            // 16-row blocks per workgroup, one per wave
constexpr int kPrefixRows = 16 * kPrefixWaves;
constexpr int kPrefixTilesPerStep = 2;     // tiles loaded and run between barriers
static_assert(kPrefixTilesPerStep % 2 == 0, "P.V takes the tiles of a step in pairs");
constexpr int kMaxSplits = 8;

struct PrefixGroups {
  int num;
  int first[kMaxGroups];
  int count[kMaxGroups];
  int shared[kMaxGroups];          // blocks
  int wg_begin[kMaxGroups + 1];    // prefix sum of row workgroups: ceil(count * G / 128)
};


struct PrefixArgs {
  const char* k_cache;
  const char* v_cache;
  const uint16_t* q;            // [B][Hq][D] bf16
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t* suf_tables;          // [B][max_blocks]: tables without the shared blocks
  int32_t* suf_lens;            // [B]: lengths without them
  int32_t* prefix_len;          // [B]: positions of the prefix each sequence sees
  float* rec;                   // [splits][B*Hq][D+4]: o, m, l, padding; split 0 ends merged
  uint32_t* counters;           // [workgroups * Hkv]: split arrivals, zero between calls
  int64_t split_stride;         // floats between two splits' records
  int num_seqs;
  int hkv;
  int group;                    // G
  int max_blocks;
  int bs;
  int sub_shift;
  int splits;
  float logit_scale;
  // group pass (null otherwise): each group leader's prefix length and
  // member count, 0 for every other sequence (written by prefix_prep_kernel)
  int32_t* grp_lens;
  int32_t* grp_count;
  PrefixGroups gr;
};

// Side job of a shared-prefix call: every sequence's suffix table (its
// table without the group's shared blocks) and suffix length, the prefix
// length it sees, and for a group pass each leader's prefix length and
// member count.  s_grp: LDS for the group table; threads nthreads per
// workgroup, grid-strided over (sequence, table entry).
__device__ __forceinline__ void prefix_side_job(const PrefixArgs& a, int (*s_grp)[kMaxGroups],
                                                int tid, int nthreads) {
  // the groups' (first, count, shared) in LDS: looked up per lane at varying
  // indices, they would otherwise be read from the argument block one
  // scalar-cache line at a time
  for (int i = tid; i < a.gr.num; i += nthreads) {
    s_grp[0][i] = a.gr.first[i];
    s_grp[1][i] = a.gr.count[i];
    s_grp[2][i] = a.gr.shared[i];
  }
  __syncthreads();

  const int64_t entries = static_cast<int64_t>(a.num_seqs) * a.max_blocks;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * nthreads + tid; idx < entries;
       idx += static_cast<int64_t>(gridDim.x) * nthreads) {
    const int s = static_cast<int>(idx / a.max_blocks);
    const int j = static_cast<int>(idx - static_cast<int64_t>(s) * a.max_blocks);
    int gi = -1;
    for (int i = 0; i < a.gr.num; ++i)
      if (s >= s_grp[0][i] && s < s_grp[0][i] + s_grp[1][i]) gi = i;
    int m = gi >= 0 ? s_grp[2][gi] : 0;
    const int64_t row = static_cast<int64_t>(s) * a.max_blocks;
    const int L = a.context_lens[s];
    const int e_shift = (j + m < a.max_blocks) ? a.block_tables[row + j + m] : -1;
    if (a.grp_lens != nullptr && m > 0) {
      // the group pass gives every member all m blocks: a group with a
      // member no longer than them is left whole to the suffix pass (its
      // members' lengths and both table entries are read at once)
      const int f = s_grp[0][gi], n = s_grp[1][gi];
      const int e_own = a.block_tables[row + j];
      int Lm[kMaxRows];
#pragma unroll
      for (int i = 0; i < kMaxRows; ++i) Lm[i] = (i < n) ? a.context_lens[f + i] : 0x7FFFFFFF;
      bool short_member = false;
#pragma unroll
      for (int i = 0; i < kMaxRows; ++i) short_member |= Lm[i] <= m * a.bs;
      if (short_member) m = 0;
      a.suf_tables[row + j] = short_member ? e_own : e_shift;
    } else {
      a.suf_tables[row + j] = e_shift;
    }
    if (j == 0) {
      const int p = min(m * a.bs, max(L, 0));          // a member no longer than the prefix is all prefix
      a.suf_lens[s] = L - p;
      a.prefix_len[s] = p;
      if (a.grp_lens != nullptr) {
        const bool lead = m > 0 && s == s_grp[0][gi];
        a.grp_lens[s] = lead ? m * a.bs : 0;
        a.grp_count[s] = lead ? s_grp[1][gi] : 0;
      }
    }
  }
}

// The side job alone, for a group pass (the prefix itself runs through
// the decode kernel): a light grid without the prefix kernel's registers
// and LDS.
__global__ void __launch_bounds__(256) prefix_prep_kernel(PrefixArgs a) {
  __shared__ int s_grp[3][kMaxGroups];
  prefix_side_job(a, s_grp, threadIdx.x, 256);
}

// One workgroup of 8 waves per (KV head g, 128 query rows of a group, split
// of the prefix's positions): rows are (member, head) pairs, member-major,
// 16 per wave.  A step loads 2 tiles' K and V once, 16 bytes per thread,
// into LDS (two stages; eight steps in flight in registers); each wave then
// runs both tiles against its 16 rows on MFMA.  Workgroups are dispatched
// round-robin over the chip's 8 XCDs, so with g = block index mod Hkv all
// workgroups of a head run on the same XCD(s) and share its tiles in L2;
// workgroups of one group start their walk at different steps, so that the
// first reads of a tile, which miss L2, are spread over the prefix.  As a
// side job the grid writes every sequence's suffix table and length, and
// the positions of the prefix it sees, for the decode kernel that follows.
template <int kD, bool kFp8>
__global__ void __launch_bounds__(64 * kPrefixWaves)
shared_prefix_kernel(PrefixArgs a) {
  constexpr int kE = kFp8 ? 1 : 2;
  constexpr int kRowBytes = kD * kE;
  constexpr int kTileBytes = kTile * kRowBytes;
  constexpr int kKK = kD / 32;
  constexpr int kVC = kD / 16;
  // LDS row pitches: K rows are read 16 bytes per lane, 16 rows at once
  // (pitch = 16 mod 256 bytes puts them on distinct banks); V rows are
  // read 8 bytes per lane, 4 rows by each 16 lanes (pitch = 32 mod 256)
  constexpr int kPitch = kRowBytes + 16;
  constexpr int kVPitch = kRowBytes + 32;
  constexpr int kTileLds = kTile * (kPitch + kVPitch);   // one tile's K rows, then V rows
  constexpr int kStage = kPrefixTilesPerStep * kTileLds;
  constexpr int kThreads = 64 * kPrefixWaves;
  constexpr int kKPieces = kTileBytes / 16;              // 16-byte pieces of a K (or V) tile
  constexpr int kStepPieces = kPrefixTilesPerStep * 2 * kKPieces;
  constexpr int kPer = (kStepPieces + kThreads - 1) / kThreads;
  constexpr int kRing = 8;                               // steps in flight
  constexpr int kIdCap = 1024;                           // tile ids per round (LDS)
  constexpr int kRec = kD + 4;                           // record floats
  static_assert(kKPieces % 64 == 0 && kIdCap % (kPrefixTilesPerStep * kRing) == 0,
                "wave-uniform pieces, whole rings");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6) & (kPrefixWaves - 1);
  const int hkv = a.hkv, G = a.group, hq = hkv * G;

  // side job: suffix tables and lengths, prefix lengths
  __shared__ int s_grp[3][kMaxGroups];
  prefix_side_job(a, s_grp, tid, kThreads);

  const int g = static_cast<int>(blockIdx.x) % hkv;
  const int rest = static_cast<int>(blockIdx.x) / hkv;
  const int sp = rest % a.splits;
  const int wg = rest / a.splits;
  int gi = 0;
  while (gi + 1 < a.gr.num && wg >= a.gr.wg_begin[gi + 1]) ++gi;
  // the group's values, made wave-uniform explicitly: read from the
  // argument block at a computed index they would otherwise live in vector
  // registers, and every buffer descriptor built from them would need a
  // loop over lanes
  const int first = __builtin_amdgcn_readfirstlane(a.gr.first[gi]);
  const int count = __builtin_amdgcn_readfirstlane(a.gr.count[gi]);
  const int shared_blocks = __builtin_amdgcn_readfirstlane(a.gr.shared[gi]);
  const int wg_b = __builtin_amdgcn_readfirstlane(a.gr.wg_begin[gi]);
  const int wg_e = __builtin_amdgcn_readfirstlane(a.gr.wg_begin[gi + 1]);
  const int share = shared_blocks * a.bs;                // shared positions
  const int ntiles = shared_blocks << a.sub_shift;
  const int per_split = (ntiles + a.splits - 1) / a.splits;
  const int tb = min(ntiles, sp * per_split), te = min(ntiles, tb + per_split);
  const int wg_local = wg - wg_b;
  const int wg_count = wg_e - wg_b;
  const int row = lane & 15, quad = lane >> 4;
  const int ri = (wg_local * kPrefixWaves + wv) * 16 + row;   // row in the group
  const int member = ri / G;
  const bool row_ok = member < count;
  const int h = ri - member * G;
  const int s = first + (row_ok ? member : 0);
  const int32_t* trow = a.block_tables + static_cast<int64_t>(first) * a.max_blocks;
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.context_lens, a.num_seqs * 4);

  // loads that need nothing else, issued together: q rows in the B-operand
  // layout of S^T = K q^T (rows past the group read 0), this row's length,
  // the members' lengths
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.q), 0, a.num_seqs * hq * kD * 2, kRsrcWord3);
  const int q_off = row_ok ? ((s * hq + g * G + h) * kD + 8 * quad) * 2 : kOutOfRange;
  bf16x8_t qa[kKK];
#pragma unroll
  for (int kk = 0; kk < kKK; ++kk)
    qa[kk] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rq, q_off + 64 * kk, 0, 0));
  const int my_len = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(rl, row_ok ? s * 4 : kOutOfRange, 0, 0));
  // positions up to the longest member's share; rows past a shorter
  // member's length are masked, slots past the longest read as zero
  int span = 0;
  for (int i0 = 0; i0 < count; i0 += 256) {
    int v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + 64 * r + lane;
      v[r] = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(rl, i < count ? (first + i) * 4 : kOutOfRange, 0, 0));
    }
    span = max(span, max(max(v[0], v[1]), max(v[2], v[3])));
  }
  span = min(wave_max_int(span), share);
  const int lim = min(max(my_len, 0), share);            // positions this row sees

  __shared__ uint32_t s_tile[kIdCap];
  __shared__ __align__(16) char s_lds[2 * kStage];

  float m_ref = kNoMax;
  f32x4_t lacc = {0.f, 0.f, 0.f, 0.f};                   // the exponent sum, in every element
  const bf16x8_t ones8 = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  f32x4_t oacc[kVC];
#pragma unroll
  for (int c = 0; c < kVC; ++c) oacc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t buf[kRing][kPer];

  for (int c0 = tb; c0 < te; c0 += kIdCap) {
    const int n = min(kIdCap, te - c0);
    const int nsteps = (n + kPrefixTilesPerStep - 1) / kPrefixTilesPerStep;
    const int rot = static_cast<int>(static_cast<int64_t>(wg_local) * nsteps / wg_count);
    // walk position i is step (i + rot) mod nsteps: tiles c0 + 2*step + 0, 1
    auto step_at = [&](int i) -> int { return i + rot < nsteps ? i + rot : i + rot - nsteps; };
    __syncthreads();                                   // the previous round's ids are read
    for (int e = tid; e < n; e += kThreads) {
      const int j = c0 + e;
      const uint32_t id = static_cast<uint32_t>(trow[j >> a.sub_shift]);
      s_tile[e] = ((id * static_cast<uint32_t>(hkv) + static_cast<uint32_t>(g)) << a.sub_shift) +
                  (static_cast<uint32_t>(j) & ((1u << a.sub_shift) - 1u));
    }
    __syncthreads();
    // Load j of a thread is piece p = 64*wave + 512j + lane of the step:
    // tile p / (2 kKPieces), K or V by (p / kKPieces) & 1, bytes
    // 16 (p mod kKPieces); pieces past the step are none.  All of this is
    // the same for a whole wave, so every thread issues the same loads,
    // unconditionally (past the walk or the tile's rows the load reads 0),
    // and the waits before the LDS writes count.
    auto issue = [&](int slot, int i) {
      const int stp = i < nsteps ? step_at(i) : 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int pw = 64 * wv + kThreads * j;                     // the wave's first piece
        const int tx = pw / (2 * kKPieces);
        const bool is_k = ((pw / kKPieces) & 1) == 0;
        const int e = kPrefixTilesPerStep * stp + tx;              // tile in the round
        const bool live = pw < kStepPieces && i < nsteps && e < n;
        const uint32_t tile = __builtin_amdgcn_readfirstlane(live ? s_tile[e] : 0u);
        // (clamped in a vector register: readfirstlane keeps the descriptor scalar)
        const int nrec = __builtin_amdgcn_readfirstlane(
            live ? max(0, min(kTile, span - kTile * (c0 + e))) * kRowBytes : 0);
        const int64_t off = static_cast<int64_t>(tile) * kTileBytes;
        const __amdgpu_buffer_rsrc_t r = make_rsrc((is_k ? a.k_cache : a.v_cache) + off, nrec);
        buf[slot][j] = __builtin_amdgcn_raw_buffer_load_b128(r, 16 * (pw % kKPieces + lane), 0, 0);
      }
    };
    auto stage = [&](int slot, char* dst) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int pw = 64 * wv + kThreads * j;
        if (pw < kStepPieces) {
          const int tx = pw / (2 * kKPieces);
          const int kv = (pw / kKPieces) & 1;
          const int b = 16 * (pw % kKPieces + lane);               // byte in the tile
          const int r = b / kRowBytes;
          *reinterpret_cast<u32x4_t*>(dst + tx * kTileLds + (kv ? kTile * kPitch + r * kVPitch : r * kPitch) +
                                      (b - r * kRowBytes)) = buf[slot][j];
        }
      }
    };
    // One step's tiles against the wave's 16 rows.  The logits of every
    // tile are independent MFMA chains; the running max is checked once per
    // step; then O^T += V^T P^T takes a pair of tiles (32 positions) per
    // MFMA, K index 8 quad + e standing for position 4 quad + e of the
    // pair's first tile (e < 4) or 4 quad + e - 4 of its second, which is
    // how the logits' accumulator already holds them (lane (row, quad):
    // positions 4 quad .. +3 of row `row`).  The exponent sum runs on the
    // same pipe, against an all-ones operand, over the rounded weights.
    // live: tiles of the step inside the walk (the rest are masked).
    auto compute_step = [&](const char* stg, int e0, int live) {
      constexpr int kT = kPrefixTilesPerStep;
      f32x4_t acc[kT];
#pragma unroll
      for (int tx = 0; tx < kT; ++tx) acc[tx] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk) {
#pragma unroll
        for (int tx = 0; tx < kT; ++tx) {
          const char* sk = stg + tx * kTileLds + row * kPitch + 8 * quad * kE;
          bf16x8_t kb;
          if constexpr (kFp8) {
            const u32x2_t wv2 = *reinterpret_cast<const u32x2_t*>(sk + 32 * kk);
            const int w0 = static_cast<int>(wv2[0]), w1 = static_cast<int>(wv2[1]);
            const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
            const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
            const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
            const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
            kb = bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
          } else {
            kb = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(sk + 64 * kk));
          }
          acc[tx] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qa[kk], acc[tx], 0, 0, 0);
        }
      }
      // positions at or past a row's end are masked, where any lane has one
#pragma unroll
      for (int tx = 0; tx < kT; ++tx) {
        const int hi = tx < live ? lim : 0;                       // positions below hi count
        const int p0 = kTile * (c0 + e0 + tx) + 4 * quad;         // position of acc[tx][0]
        if (__builtin_amdgcn_ballot_w64(p0 + 3 >= hi) != 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[tx][r] = p0 + r < hi ? acc[tx][r] : -INFINITY;
        }
      }
      // the scale is positive: the largest logit is the scale times the
      // largest product, and each weight is exp2(fma(product, scale, -max))
      float xm = -INFINITY;
#pragma unroll
      for (int tx = 0; tx < kT; ++tx)
        xm = fmaxf(xm, fmaxf(fmaxf(acc[tx][0], acc[tx][1]), fmaxf(acc[tx][2], acc[tx][3])));
      xm *= a.logit_scale;
      if (__builtin_amdgcn_ballot_w64(xm > m_ref + kRescaleSlack) != 0) {
        float mt = xm;
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = (mt > m_ref + kRescaleSlack) ? mt : m_ref;
        const float alpha = __builtin_amdgcn_exp2f(m_ref - mn);
#pragma unroll
        for (int r = 0; r < 4; ++r) lacc[r] *= alpha;
#pragma unroll
        for (int c = 0; c < kVC; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) oacc[c][r] *= alpha;
        m_ref = mn;
      }
      bf16x4_t pb[kT];
#pragma unroll
      for (int tx = 0; tx < kT; ++tx)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          pb[tx][r] = static_cast<__bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(acc[tx][r], a.logit_scale, -m_ref)));
#pragma unroll
      for (int pr = 0; pr < kT / 2; ++pr) {
        const bf16x8_t pp = {pb[2 * pr][0], pb[2 * pr][1], pb[2 * pr][2], pb[2 * pr][3],
                             pb[2 * pr + 1][0], pb[2 * pr + 1][1], pb[2 * pr + 1][2], pb[2 * pr + 1][3]};
        lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pp, lacc, 0, 0, 0);
        // V rows of both tiles.  bf16: one transposing LDS read per tile and
        // dim block; within each 16 lanes it hands lane i, element k,
        // element i mod 4 of the 8 bytes that lane 4k + i/4 addressed; lane
        // (row, quad) addresses position 4 quad + row/4, dims 16c +
        // 4 (row mod 4) .. +3, so it receives positions 4 quad .. +3 of dim
        // 16c + row.  fp8: the same positions gathered a byte at a time.
        const char* tv0 = stg + (2 * pr) * kTileLds + kTile * kPitch;
        const char* tv1 = tv0 + kTileLds;
#pragma unroll
        for (int c = 0; c < kVC; ++c) {
          u32x2_t v0, v1;
          if constexpr (kFp8) {
            auto gather = [&](const char* tv) -> u32x2_t {
              const char* p = tv + 4 * quad * kVPitch + row + 16 * c;
              const uint32_t b0 = static_cast<uint8_t>(p[0]), b1 = static_cast<uint8_t>(p[kVPitch]);
              const uint32_t b2 = static_cast<uint8_t>(p[2 * kVPitch]), b3 = static_cast<uint8_t>(p[3 * kVPitch]);
              const int w4 = static_cast<int>(b0 | (b1 << 8) | (b2 << 16) | (b3 << 24));
              return u32x2_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w4, 1.0f, false)),
                             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w4, 1.0f, true))};
            };
            v0 = gather(tv0);
            v1 = gather(tv1);
          } else {
            const int tr = (4 * quad + (row >> 2)) * kVPitch + 8 * (row & 3) + 32 * c;
            v0 = lds_read_tr16(tv0 + tr);
            v1 = lds_read_tr16(tv1 + tr);
          }
          const u32x4_t vv = {v0[0], v0[1], v1[0], v1[1]};
          oacc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vv), pp, oacc[c], 0, 0, 0);
        }
      }
    };
    // step i: registers (slot i mod kRing) -> LDS stage i mod 2 -> MFMA.
    // One barrier per step: a thread writing stage i mod 2 has passed step
    // i-1's barrier, so every wave is done with step i-2 that used it.  The
    // barrier waits for the LDS writes only (lgkmcnt), not for the loads in
    // flight.  Rounds run whole rings: steps past the walk read zeros and
    // are masked.
    // (issued in slot order, which the loop's waits count on)
#pragma unroll
    for (int k = 0; k < kRing; ++k) {
      issue(k, k);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int i0 = 0; i0 < nsteps; i0 += kRing) {
#pragma unroll
      for (int k = 0; k < kRing; ++k) {
        const int i = i0 + k;
        char* stg = s_lds + (i & 1) * kStage;
        stage(k, stg);
        issue(k, i + kRing);
        lds_barrier();
        const int e0 = kPrefixTilesPerStep * (i < nsteps ? step_at(i) : 0);
        compute_step(stg, e0, i < nsteps ? min(kPrefixTilesPerStep, n - e0) : 0);
      }
    }
  }

  const float l_tot = lacc[0];
  const int64_t row_off = (static_cast<int64_t>(s) * hq + g * G + h) * kRec;
  if (a.splits == 1) {
    if (row_ok) {
      float* rec = a.rec + row_off;
#pragma unroll
      for (int c = 0; c < kVC; ++c) *reinterpret_cast<f32x4_t*>(rec + 16 * c + 4 * quad) = oacc[c];
      if (quad == 0) *reinterpret_cast<f32x2_t*>(rec + kD) = f32x2_t{m_ref, l_tot};
    }
    return;
  }
  // several splits: publish this split's records (device-coherent), count
  // the arrival; the last split of the row block merges them all into
  // split 0's records, in split order whichever split arrives last (the
  // result does not depend on timing), 4 splits' records in flight at once
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.rec, 0x7FFFFFFF);
  if (row_ok) {
    const int mine = static_cast<int>((sp * a.split_stride + row_off) * 4);
#pragma unroll
    for (int c = 0; c < kVC; ++c)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, oacc[c]), rr,
                                             mine + (16 * c + 4 * quad) * 4, 0, kAuxCoherent);
    if (quad == 0)
      __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{__float_as_uint(m_ref), __float_as_uint(l_tot)},
                                            rr, mine + kD * 4, 0, kAuxCoherent);
  }
  wait_memory_done();
  __shared__ uint32_t s_prev;
  __syncthreads();
  uint32_t* ctr = a.counters + static_cast<int64_t>(wg) * hkv + g;
  if (tid == 0)
    s_prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  compiler_fence();
  if (s_prev != static_cast<uint32_t>(a.splits - 1)) return;
  if (tid == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!row_ok) return;
  float M = kNoMax, Ls = 0.f;
#pragma unroll
  for (int c = 0; c < kVC; ++c) oacc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(a.rec, 0);          // reads 0
  for (int k0 = 0; k0 < a.splits; k0 += 4) {
    f32x4_t o[4][kVC];
    u32x2_t ml[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + u;
      const bool use = k < a.splits;
      const __amdgpu_buffer_rsrc_t ru = use ? rr : rz;
      const int off = use ? static_cast<int>((k * a.split_stride + row_off) * 4) : 0;
      ml[u] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(ru, off + kD * 4, 0, kAuxCoherent));
#pragma unroll
      for (int c = 0; c < kVC; ++c)
        o[u][c] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                  ru, off + (16 * c + 4 * quad) * 4, 0, kAuxCoherent));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + u;
      if (k >= a.splits) continue;
      const float mk = __uint_as_float(ml[u][0]), lk = __uint_as_float(ml[u][1]);
      const float mn = fmaxf(M, mk);
      const float fa = __builtin_amdgcn_exp2f(M - mn), fb = __builtin_amdgcn_exp2f(mk - mn);
#pragma unroll
      for (int c = 0; c < kVC; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[c][r] = oacc[c][r] * fa + o[u][c][r] * fb;
      Ls = Ls * fa + lk * fb;
      M = mn;
    }
  }
  float* rec = a.rec + row_off;
#pragma unroll
  for (int c = 0; c < kVC; ++c) *reinterpret_cast<f32x4_t*>(rec + 16 * c + 4 * quad) = oacc[c];
  if (quad == 0) *reinterpret_cast<f32x2_t*>(rec + kD) = f32x2_t{M, Ls};
}


// ---------------------------------------------------------------------------
// General path: any G, fp32 / bf16 / fp8 cache.  One wave per (partition,
// query row, sequence); one token at a time, dot product by a wave
// reduction, exact online softmax.  Used for fp32 caches and shapes the fast
// path does not cover.  Query row y = i * hq + h is chunk token i of query
// head h; it sees positions below n = L - chunk + 1 + i, from max(0, n - W)
// with a window of W > 0.  A partition with nothing to see records l = 0.
template <int kD, int kFmt, bool kOutF32>
__global__ void __launch_bounds__(64)
decode_simple_kernel(const char* __restrict__ k_cache, const char* __restrict__ v_cache,
                     const void* __restrict__ q, const int32_t* __restrict__ block_tables,
                     const int32_t* __restrict__ context_lens, int max_blocks, int hkv,
                     int bs, int group, int hq, int chunk, int window, float logit_scale,
                     float v_scale, PartOut po) {
  constexpr int kPer = kD / 64;
  const int part = blockIdx.x;
  const int y = blockIdx.y;
  const int s = blockIdx.z;
  const int h = y % hq;
  const int g = h / group;
  const int L = max(0, context_lens[s] - chunk + 1 + y / hq);
  const int nparts = (L + kPartTokens - 1) / kPartTokens;
  const int lane = threadIdx.x;
  if (part >= (nparts > 0 ? nparts : 1)) return;
  const int64_t orow = (static_cast<int64_t>(s) * gridDim.y + y) * kD;
  if (L == 0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) store_out<kOutF32>(po.out, orow + lane + 64 * i, 0.f);
    return;
  }
  auto elem = [&](const char* base, int64_t idx) -> float {
    if constexpr (kFmt == PA_F32) {
      return reinterpret_cast<const float*>(base)[idx];
    } else if constexpr (kFmt == PA_BF16) {
      return __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(base)[idx])
                             << 16);
    } else {
      const uint32_t code = reinterpret_cast<const uint8_t*>(base)[idx];
      return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(code, 1.0f, false)[0];
    }
  };
  float qv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if constexpr (kOutF32)
      qv[i] = static_cast<const float*>(q)[orow + lane + 64 * i];
    else
      qv[i] = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(q)[orow + lane + 64 * i]) << 16);
  }
  const int t0 = max(part * kPartTokens, window > 0 ? L - window : 0);
  const int t1 = min(L, part * kPartTokens + kPartTokens);
  float m = -INFINITY, l = 0.f, o[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) o[i] = 0.f;
  for (int t = t0; t < t1; ++t) {
    const int64_t id = block_tables[static_cast<int64_t>(s) * max_blocks + t / bs];
    const int64_t base = ((id * hkv + g) * bs + t % bs) * kD;
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) dot = fmaf(qv[i], elem(k_cache, base + lane + 64 * i), dot);
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) dot += __shfl_xor(dot, sh);
    const float x = dot * logit_scale;
    const float mn = fmaxf(m, x);
    const float a = __builtin_amdgcn_exp2f(m - mn);
    const float p = __builtin_amdgcn_exp2f(x - mn);
    l = l * a + p;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      o[i] = fmaf(p, elem(v_cache, base + lane + 64 * i), o[i] * a);
    m = mn;
  }
  const float inv = (l > 0.f) ? v_scale / l : 0.f;
  if (nparts == 1) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) store_out<kOutF32>(po.out, orow + lane + 64 * i, o[i] * inv);
  } else {
    const int64_t r = (static_cast<int64_t>(s) * gridDim.y + y) * po.num_parts + part;
#pragma unroll
    for (int i = 0; i < kPer; ++i) po.ws_o[r * kD + lane + 64 * i] = o[i] * inv;
    if (lane == 0) {
      po.ws_ml[2 * r] = m;
      po.ws_ml[2 * r + 1] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the partitions of one (sequence, query row):
//   out = sum_i 2^(m_i - M) l_i o_i / sum_i 2^(m_i - M) l_i,  M = max_i m_i.
template <int kD, bool kOutF32>
__global__ void __launch_bounds__(kD)
reduce_kernel(const int32_t* __restrict__ context_lens, int hq, int chunk, PartOut po) {
  const int y = blockIdx.x;
  const int s = blockIdx.y;
  const int L = max(0, context_lens[s] - chunk + 1 + y / hq);
  const int nparts = (L + kPartTokens - 1) / kPartTokens;
  if (nparts <= 1) return;     // written directly by the partition pass
  const int d = threadIdx.x;
  const int64_t r0 = (static_cast<int64_t>(s) * gridDim.x + y) * po.num_parts;
  float M = -INFINITY;
  for (int i = 0; i < nparts; ++i) M = fmaxf(M, po.ws_ml[2 * (r0 + i)]);
  float den = 0.f, num = 0.f;
  for (int i = 0; i < nparts; ++i) {
    const float li = po.ws_ml[2 * (r0 + i) + 1];
    const float a = (li > 0.f) ? __builtin_amdgcn_exp2f(po.ws_ml[2 * (r0 + i)] - M) * li : 0.f;
    den += a;
    num = fmaf(a, po.ws_o[(r0 + i) * kD + d], num);
  }
  store_out<kOutF32>(po.out, (static_cast<int64_t>(s) * gridDim.x + y) * kD + d, num / den);
}

// Events a caller asked the next decode call on this thread to record
// (pa_time_next_call): the first kernel's start and the last kernel's end.
struct CallTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
thread_local CallTiming t_next_call;

CallTiming take_call_timing() {
  const CallTiming t = t_next_call;
  t_next_call = CallTiming{};
  return t;
}

// Launches `kernel`; with events, through hipExtLaunchKernelGGL, which has
// the dispatch itself record them as the kernel starts and ends (no marker
// packets in the stream).
template <typename... KArgs, typename... Args>
void launch_k(void (*kernel)(KArgs...), dim3 grid, dim3 block, unsigned shmem, hipStream_t st,
              hipEvent_t e0, hipEvent_t e1, Args... args) {
  if (e0 != nullptr || e1 != nullptr)
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, e0, e1, 0, args...);
  else
    kernel<<<grid, block, shmem, st>>>(args...);
}

template <int kD>
void launch_simple(int fmt, dim3 grid, hipStream_t st, hipEvent_t e0, hipEvent_t e1,
                   const char* kc, const char* vc, const void* q, const int32_t* bt,
                   const int32_t* cl, int maxb, int hkv, int bs, int G, int hq, int T, int W,
                   float ls, float vs, PartOut po) {
  if (fmt == PA_F32)
    launch_k(decode_simple_kernel<kD, PA_F32, true>, grid, dim3(64), 0, st, e0, e1, kc, vc, q, bt, cl, maxb, hkv, bs, G, hq, T, W, ls, vs, po);
  else if (fmt == PA_BF16)
    launch_k(decode_simple_kernel<kD, PA_BF16, false>, grid, dim3(64), 0, st, e0, e1, kc, vc, q, bt, cl, maxb, hkv, bs, G, hq, T, W, ls, vs, po);
  else
    launch_k(decode_simple_kernel<kD, PA_FP8_E4M3, false>, grid, dim3(64), 0, st, e0, e1, kc, vc, q, bt, cl, maxb, hkv, bs, G, hq, T, W, ls, vs, po);
}


template <int kD>
void launch_stream(bool fp8, bool pair, int nw, hipStream_t st, const StreamArgs& a,
                   hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr) {
  const dim3 grid(nw / kWavesPerGroup), block(64 * kWavesPerGroup);
  const NoGroupTable ng{0};
  if (pair) {
    if (fp8)
      launch_k(decode_stream_kernel<kD, true, kAuxNonTemporal, true>, grid, block, kPadLds, st, e0, e1, a, ng);
    else
      launch_k(decode_stream_kernel<kD, false, kAuxNonTemporal, true>, grid, block, kPadLds, st, e0, e1, a, ng);
  } else if (fp8) {
    launch_k(decode_stream_kernel<kD, true, kAuxNonTemporal, false>, grid, block, kPadLds, st, e0, e1, a, ng);
  } else {
    launch_k(decode_stream_kernel<kD, false, kAuxNonTemporal, false>, grid, block, kPadLds, st, e0, e1, a, ng);
  }
}

// The same with shared-prefix groups decoded in the one launch.  In the
// head-major order the KV heads of one group run on neighbouring waves of
// one XCD, so its prefix tiles are read with the default policy and stay
// in that XCD's L2 for the next head; otherwise the loads are streamed.
template <int kD>
void launch_stream_groups(bool fp8, int nw, hipStream_t st, const StreamArgs& a,
                          const GroupTable& gt, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr) {
  const dim3 grid(nw / kWavesPerGroup), block(64 * kWavesPerGroup);
  if (a.head_major) {
    if (fp8)
      launch_k(decode_stream_kernel<kD, true, 0, false, true>, grid, block, kPadLds, st, e0, e1, a, gt);
    else
      launch_k(decode_stream_kernel<kD, false, 0, false, true>, grid, block, kPadLds, st, e0, e1, a, gt);
  } else if (fp8) {
    launch_k(decode_stream_kernel<kD, true, kAuxNonTemporal, false, true>, grid, block, kPadLds, st, e0, e1, a, gt);
  } else {
    launch_k(decode_stream_kernel<kD, false, kAuxNonTemporal, false, true>, grid, block, kPadLds, st, e0, e1, a, gt);
  }
}

}  // namespace

}  // namespace pagedkv

using namespace pagedkv;

namespace {

int num_partitions(int32_t max_context_len) {
  return (max_context_len + kPartTokens - 1) / kPartTokens;
}

// Largest cache (bytes of K, or of V) the 8-token-block mode addresses
// with one buffer descriptor (32-bit offsets, and room past it for the
// out-of-range offset of masked rows); larger caches take a descriptor per
// block, with K loaded once per block of the tile.
constexpr int64_t kPairCacheMax = int64_t{0x7FFF0000} - (int64_t{1} << 16);

bool fast_path(int fmt, int q_dtype, int G, int D, int bs) {
  return (fmt == PA_BF16 || fmt == PA_FP8_E4M3) && q_dtype == PA_BF16 && G >= 1 &&
         (D == 64 || D == 128) && (bs % kTile == 0 || bs == 8);
}

// Row blocks per KV head on the fast path: a KV head with more than 16
// query heads is decoded as the fewest equal blocks of at most 16 (the
// smallest divisor of G that brings G / split to 16 or below).
int head_split(int G) {
  if (G <= kMaxRows) return 1;
  for (int d = 2; d < G; ++d)
    if (G % d == 0 && G / d <= kMaxRows) return d;
  return G;
}

int64_t cache_bytes(const pa_cache_desc* c) {
  const int e = c->cache_dtype == PA_F32 ? 4 : c->cache_dtype == PA_BF16 ? 2 : 1;
  return static_cast<int64_t>(c->num_blocks) * c->num_kv_heads * c->block_size * c->head_dim * e;
}

// The fast path for this cache and head map.
bool fast_path(const pa_cache_desc* c, int q_dtype, int G) {
  return fast_path(c->cache_dtype, q_dtype, G, c->head_dim, c->block_size) &&
         static_cast<int64_t>(c->num_kv_heads) * head_split(G) <= 511;   // 9-bit head field
}

// Chunk tokens per fast-path pass: as many as fit G rows each in 16 columns.
int tokens_per_pass(int G, int T) { return std::min(T, std::max(1, kMaxRows / G)); }

// Compute units of the current device (256 on MI355X when it cannot be read).
int device_cus() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Fast path scratch: two partial slots per wave of `rows` query rows each.
size_t stream_partials_bytes(int rows, int D) {
  const size_t waves = static_cast<size_t>(device_cus()) * kWavesPerCU;
  const size_t slot_floats = (static_cast<size_t>(rows) * (D + 2) + 3) & ~static_cast<size_t>(3);
  return waves * 2 * slot_floats * sizeof(float);
}

// Fast path workspace: arrival counters, then the partial slots.
size_t stream_workspace_bytes(int num_seqs, int hkv, int rows, int D) {
  return align256(static_cast<size_t>(num_seqs) * hkv * sizeof(uint32_t)) +
         stream_partials_bytes(rows, D);
}

size_t general_workspace_bytes(int num_seqs, int num_q_heads, int T, int D, int max_context_len) {
  const int P = num_partitions(max_context_len);
  if (P <= 1) return 0;
  return static_cast<size_t>(num_seqs) * T * num_q_heads * P * (D + 2) * sizeof(float);
}

size_t workspace_bytes_for(const pa_cache_desc* c, int32_t num_seqs, int32_t num_q_heads,
                           int32_t T, int32_t max_context_len, const char* fn) {
  if (check_desc(c, fn) != PA_OK) return 0;
  if (num_seqs <= 0 || num_q_heads <= 0 || max_context_len <= 0 || T <= 0 ||
      num_q_heads % c->num_kv_heads != 0)
    return 0;
  const int G = num_q_heads / c->num_kv_heads;
  const int q_dtype = (c->cache_dtype == PA_F32) ? PA_F32 : PA_BF16;
  if (fast_path(c, q_dtype, G)) {
    const int split = head_split(G), Gk = G / split;
    return stream_workspace_bytes(num_seqs, c->num_kv_heads * split, Gk * tokens_per_pass(Gk, T),
                                  c->head_dim);
  }
  return general_workspace_bytes(num_seqs, num_q_heads, T, c->head_dim, max_context_len);
}

// pa_decode (T = 1, no window), pa_decode_chunk and pa_decode_window: one
// implementation.
pa_status attend(const char* fn, const pa_cache_desc* c, const void* k_cache,
                 const void* v_cache, const void* q, int32_t q_dtype, void* out, int32_t T,
                 int32_t W,
                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                 const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs,
                 int32_t num_q_heads, float scale, void* workspace, size_t workspace_bytes,
                 void* stream, const int32_t* prefix_len = nullptr,
                 const float* prefix_rec = nullptr, CallTiming tm = CallTiming{},
                 uint32_t* fixed_counters = nullptr) {
  // fixed_counters: the fast path's arrival counters live there (zero
  // between calls) and `workspace` holds only the partial results
  pa_status st = check_desc(c, fn);
  if (st != PA_OK) return st;
  const int hkv = c->num_kv_heads, D = c->head_dim, fmt = c->cache_dtype;
  if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0 || max_blocks_per_seq < 0)
    return fail(PA_ERR_INVALID_ARG, "%s: negative size", fn);
  if (T < 1 || T > PA_MAX_CHUNK)
    return fail(PA_ERR_INVALID_ARG, "%s: chunk_len %d (1..%d)", fn, T, PA_MAX_CHUNK);
  if (W < 0) return fail(PA_ERR_INVALID_ARG, "%s: window %d < 0", fn, W);
  if (num_q_heads % hkv != 0)
    return fail(PA_ERR_INVALID_ARG, "%s: %d query heads not a multiple of %d KV heads", fn,
                num_q_heads, hkv);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "%s: scale not finite", fn);
  const bool combo_ok = (fmt == PA_F32 && q_dtype == PA_F32) ||
                        (fmt == PA_BF16 && q_dtype == PA_BF16) ||
                        (fmt == PA_FP8_E4M3 && q_dtype == PA_BF16);
  if (!combo_ok)
    return fail(PA_ERR_UNSUPPORTED, "%s: q dtype %d with cache dtype %d", fn, q_dtype, fmt);
  const int bs = c->block_size;
  if (static_cast<int64_t>(max_blocks_per_seq) * bs < max_context_len)
    return fail(PA_ERR_INVALID_ARG, "%s: max_blocks_per_seq %d cannot hold max_context_len %d",
                fn, max_blocks_per_seq, max_context_len);
  if (num_seqs == 0) return PA_OK;
  if (!k_cache || !v_cache || !q || !out || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "%s: null pointer", fn);
  const int G = num_q_heads / hkv;
  const bool fast = fast_path(c, q_dtype, G);
  // the kernel's heads: row blocks of Gk query heads, split per KV head
  const int split = fast ? head_split(G) : 1, Gk = G / split, hk = hkv * split;
  const int tpp = tokens_per_pass(Gk, T);
  const int64_t max_tiles = static_cast<int64_t>(hk) * num_seqs *
                            ((static_cast<int64_t>(max_context_len) + kTile - 1) / kTile);
  if (fast && (max_tiles >= (int64_t{1} << 30) || num_seqs > static_cast<int32_t>(kSeqMask) ||
               static_cast<int64_t>(c->num_blocks) * hkv * std::max(1, bs / kTile) >= (int64_t{1} << 32) ||
               static_cast<int64_t>(max_blocks_per_seq) * 4 >= (int64_t{1} << 31) ||
               (static_cast<int64_t>(T - 1) * num_q_heads + Gk) * D * 2 >= (int64_t{1} << 30)))
    return fail(PA_ERR_UNSUPPORTED, "%s: %lld tiles in one call (limit 2^30)", fn,
                static_cast<long long>(max_tiles));
  if (!fast && (num_seqs > 65535 || static_cast<int64_t>(T) * num_q_heads > 65535))
    return fail(PA_ERR_UNSUPPORTED, "%s: num_seqs / chunk_len * num_q_heads above 65535", fn);
  if (fast && (reinterpret_cast<uintptr_t>(out) % 16 != 0 || reinterpret_cast<uintptr_t>(q) % 16 != 0))
    return fail(PA_ERR_INVALID_ARG, "%s: q and out must be 16-byte aligned", fn);
  const size_t need = !fast ? general_workspace_bytes(num_seqs, num_q_heads, T, D, max_context_len)
                     : fixed_counters ? stream_partials_bytes(Gk * tpp, D)
                                      : stream_workspace_bytes(num_seqs, hk, Gk * tpp, D);
  if (workspace_bytes < need || (need > 0 && !workspace))
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes, need %zu", fn,
                workspace_bytes, need);
  if (need > 0 && reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(PA_ERR_INVALID_ARG, "%s: workspace not 16-byte aligned", fn);
  PA_DEBUG_CHECK(debug::check_tables(c, block_tables, max_blocks_per_seq, context_lens,
                                     max_context_len, num_seqs, stream, fn));

  const float kscale = (fmt == PA_FP8_E4M3) ? c->k_scale : 1.f;
  const float vscale = (fmt == PA_FP8_E4M3) ? c->v_scale : 1.f;
  const float logit_scale =
      static_cast<float>(static_cast<double>(scale) * kscale * 1.4426950408889634);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* kc = static_cast<const char*>(k_cache);
  const char* vc = static_cast<const char*>(v_cache);

  if (fast) {
    if (max_context_len == 0) max_context_len = 1;
    const int64_t waves_max = static_cast<int64_t>(device_cus()) * kWavesPerCU;
    const int64_t by_size = (max_tiles + kMinTilesPerWave - 1) / kMinTilesPerWave;
    const int64_t nw = (std::max<int64_t>(std::min(waves_max, by_size), 1) + kWavesPerGroup - 1) /
                       kWavesPerGroup * kWavesPerGroup;
    StreamArgs a;
    a.k_cache = kc;
    a.v_cache = vc;
    a.q = static_cast<const uint16_t*>(q);
    a.out = static_cast<uint16_t*>(out);
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.counters = fixed_counters ? fixed_counters : static_cast<uint32_t*>(workspace);
    a.partials = fixed_counters ? static_cast<float*>(workspace)
                                : reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                           align256(static_cast<size_t>(num_seqs) * hk * 4));
    a.num_seqs = num_seqs;
    a.hkv = hk;
    a.kv_split = split;
    a.max_blocks = max_blocks_per_seq;
    a.num_waves = static_cast<int>(nw);
    a.group = Gk;
    a.chunk = T;
    a.window = W;
    a.sub_shift = bs == 64 ? 2 : bs == 32 ? 1 : 0;
    // 8-token blocks: one descriptor over a cache below 2 GiB - 128 KiB, else one per block
    a.pair_nrec = (bs == 8 && cache_bytes(c) <= kPairCacheMax) ? static_cast<int>(cache_bytes(c)) : 0;
    a.prefix_len = prefix_len;
    a.prefix_rec = prefix_rec;
    a.logit_scale = logit_scale;
    a.v_scale = vscale;
    a.q_seq_rows = T;
    a.q_total_rows = num_seqs * T;
    a.causal = 1;
    a.rec_out = nullptr;
    a.rec_count = nullptr;
    a.head_major = 0;
    // one pass per tpp chunk tokens; each pass leaves the counters zeroed
    for (int t0 = 0; t0 < T; t0 += tpp) {
      a.t_first = t0;
      a.rows = Gk * std::min(tpp, T - t0);
      hipEvent_t e0 = t0 == 0 ? tm.start : nullptr;
      hipEvent_t e1 = t0 + tpp >= T ? tm.stop : nullptr;
      if (D == 128) launch_stream<128>(fmt == PA_FP8_E4M3, bs == 8, a.num_waves, s, a, e0, e1);
      else launch_stream<64>(fmt == PA_FP8_E4M3, bs == 8, a.num_waves, s, a, e0, e1);
      st = launch_status(fn);
      if (st != PA_OK) return st;
    }
    return PA_OK;
  }

  const int P = max_context_len > 0 ? num_partitions(max_context_len) : 1;
  PartOut po;
  po.out = out;
  po.num_parts = P;
  po.ws_o = static_cast<float*>(workspace);
  po.ws_ml = need ? po.ws_o + static_cast<size_t>(num_seqs) * T * num_q_heads * P * D : nullptr;
  const int rows = T * num_q_heads;
  {
    dim3 grid(P, rows, num_seqs);
    hipEvent_t e1 = P > 1 ? nullptr : tm.stop;
    if (D == 128)
      launch_simple<128>(fmt, grid, s, tm.start, e1, kc, vc, q, block_tables, context_lens,
                         max_blocks_per_seq, hkv, bs, G, num_q_heads, T, W, logit_scale, vscale, po);
    else
      launch_simple<64>(fmt, grid, s, tm.start, e1, kc, vc, q, block_tables, context_lens,
                        max_blocks_per_seq, hkv, bs, G, num_q_heads, T, W, logit_scale, vscale, po);
  }
  st = launch_status(fn);
  if (st != PA_OK) return st;
  if (P > 1) {
    dim3 grid(rows, num_seqs);
    const bool of32 = (q_dtype == PA_F32);
    hipEvent_t e1 = tm.stop;
    if (D == 128) {
      if (of32) launch_k(reduce_kernel<128, true>, grid, dim3(128), 0, s, nullptr, e1, context_lens, num_q_heads, T, po);
      else launch_k(reduce_kernel<128, false>, grid, dim3(128), 0, s, nullptr, e1, context_lens, num_q_heads, T, po);
    } else {
      if (of32) launch_k(reduce_kernel<64, true>, grid, dim3(64), 0, s, nullptr, e1, context_lens, num_q_heads, T, po);
      else launch_k(reduce_kernel<64, false>, grid, dim3(64), 0, s, nullptr, e1, context_lens, num_q_heads, T, po);
    }
    st = launch_status(fn);
  }
  return st;
}

}  // namespace

extern "C" size_t pa_decode_workspace_bytes(const pa_cache_desc* c, int32_t num_seqs,
                                            int32_t num_q_heads, int32_t max_context_len) {
  return workspace_bytes_for(c, num_seqs, num_q_heads, 1, max_context_len,
                             "pa_decode_workspace_bytes");
}

extern "C" size_t pa_decode_chunk_workspace_bytes(const pa_cache_desc* c, int32_t num_seqs,
                                                  int32_t num_q_heads, int32_t chunk_len,
                                                  int32_t max_context_len) {
  if (chunk_len < 1 || chunk_len > PA_MAX_CHUNK) return 0;
  return workspace_bytes_for(c, num_seqs, num_q_heads, chunk_len, max_context_len,
                             "pa_decode_chunk_workspace_bytes");
}

extern "C" pa_status pa_decode_workspace_init(void* workspace, size_t workspace_bytes,
                                              void* stream) {
  if (workspace_bytes == 0) return PA_OK;
  if (!workspace) return fail(PA_ERR_INVALID_ARG, "pa_decode_workspace_init: null workspace");
  if (reinterpret_cast<uintptr_t>(workspace) % 4 != 0)
    return fail(PA_ERR_INVALID_ARG, "pa_decode_workspace_init: workspace not 4-byte aligned");
  const int64_t words = static_cast<int64_t>(workspace_bytes / 4);
  if (words > 0) {
    const int64_t grid = std::min<int64_t>((words + 255) / 256, 4096);
    zero_fill_kernel<<<static_cast<unsigned>(grid), 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<uint32_t*>(workspace), words);
  }
  return launch_status("pa_decode_workspace_init");
}

extern "C" pa_status pa_decode(const pa_cache_desc* c, const void* k_cache, const void* v_cache,
                               const void* q, int32_t q_dtype, void* out,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t max_context_len,
                               int32_t num_seqs, int32_t num_q_heads, float scale,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return attend("pa_decode", c, k_cache, v_cache, q, q_dtype, out, 1, 0, block_tables,
                max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads, scale,
                workspace, workspace_bytes, stream, nullptr, nullptr, take_call_timing());
}

extern "C" pa_status pa_decode_chunk(const pa_cache_desc* c, const void* k_cache,
                                     const void* v_cache, const void* q, int32_t q_dtype,
                                     void* out, int32_t chunk_len, const int32_t* block_tables,
                                     int32_t max_blocks_per_seq, const int32_t* context_lens,
                                     int32_t max_context_len, int32_t num_seqs,
                                     int32_t num_q_heads, float scale, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return attend("pa_decode_chunk", c, k_cache, v_cache, q, q_dtype, out, chunk_len, 0,
                block_tables, max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                num_q_heads, scale, workspace, workspace_bytes, stream, nullptr, nullptr,
                take_call_timing());
}

extern "C" pa_status pa_decode_window(const pa_cache_desc* c, const void* k_cache,
                                      const void* v_cache, const void* q, int32_t q_dtype,
                                      void* out, int32_t chunk_len, int32_t window,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t max_context_len,
                                      int32_t num_seqs, int32_t num_q_heads, float scale,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return attend("pa_decode_window", c, k_cache, v_cache, q, q_dtype, out, chunk_len, window,
                block_tables, max_blocks_per_seq, context_lens, max_context_len, num_seqs,
                num_q_heads, scale, workspace, workspace_bytes, stream, nullptr, nullptr,
                take_call_timing());
}

// ---------------------------------------------------------------------------
// pa_decode_noalloc: pa_decode with its scratch in a static device array
// instead of a caller workspace.  Layout: arrival counters of up to
// kStaticCounters (sequence, KV head) segments, which every completed call
// leaves at zero, then the partial results (written before they are read).
namespace {
constexpr size_t kStaticCounters = size_t{1} << 16;
constexpr size_t kStaticCounterBytes = kStaticCounters * sizeof(uint32_t);
constexpr size_t kStaticPartialBytes = size_t{24} << 20;
}  // namespace

static __device__ __align__(256) char scratch[kStaticCounterBytes + kStaticPartialBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch[kMaxDevices] = {};    // device address of `scratch`, per device

// The current device's address of `scratch`; on the first call for a device
// it is looked up and its counters are cleared on `st` (a fill kernel, so it
// precedes the caller's decode on that stream).
pa_status device_scratch(hipStream_t st, char** base, const char* fn) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess)
    return fail(PA_ERR_HIP, "%s: hipGetDevice failed", fn);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PA_ERR_UNSUPPORTED, "%s: device %d (at most %d devices)", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(PA_ERR_HIP, "%s: hipGetSymbolAddress of the static scratch: %s", fn,
                  hipGetErrorString(e));
    const int64_t words = static_cast<int64_t>(kStaticCounterBytes / 4);
    zero_fill_kernel<<<static_cast<unsigned>((words + 255) / 256), 256, 0, st>>>(
        static_cast<uint32_t*>(p), words);
    const pa_status ls = launch_status(fn);
    if (ls != PA_OK) return ls;
    g_scratch[dev] = static_cast<char*>(p);
  }
  *base = g_scratch[dev];
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_decode_noalloc(const pa_cache_desc* c, const void* k_cache,
                                       const void* v_cache, const void* q, int32_t q_dtype,
                                       void* out, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                                       int32_t max_context_len, int32_t num_seqs,
                                       int32_t num_q_heads, float scale, void* stream) {
  const char* fn = "pa_decode_noalloc";
  pa_status st = check_desc(c, fn);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0)
    return fail(PA_ERR_INVALID_ARG, "%s: negative size", fn);
  if (num_q_heads % c->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "%s: %d query heads not a multiple of %d KV heads", fn,
                num_q_heads, c->num_kv_heads);
  if (num_seqs == 0) return PA_OK;
  const int G = num_q_heads / c->num_kv_heads;
  const bool fast = fast_path(c, q_dtype, G);
  const int split = fast ? head_split(G) : 1;
  if (fast && static_cast<size_t>(num_seqs) * c->num_kv_heads * split > kStaticCounters)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL,
                "%s: %d sequences x %d KV heads x %d row blocks exceed the static scratch's %zu "
                "counters", fn, num_seqs, c->num_kv_heads, split, kStaticCounters);
  const size_t need = fast ? stream_partials_bytes(G / split, c->head_dim)
                           : general_workspace_bytes(num_seqs, num_q_heads, 1, c->head_dim,
                                                     max_context_len);
  if (need > kStaticPartialBytes)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL,
                "%s: this batch needs %zu bytes of scratch, the static scratch holds %zu", fn,
                need, kStaticPartialBytes);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* base = nullptr;
  st = device_scratch(hs, &base, fn);
  if (st != PA_OK) return st;
  return attend(fn, c, k_cache, v_cache, q, q_dtype, out, 1, 0, block_tables, max_blocks_per_seq,
                context_lens, max_context_len, num_seqs, num_q_heads, scale,
                base + kStaticCounterBytes, kStaticPartialBytes, stream, nullptr, nullptr,
                take_call_timing(), reinterpret_cast<uint32_t*>(base));
}

namespace {

// Row workgroups of a launch: each group rounds its count * G rows up to
// whole workgroups, at most one partial one per group.
int64_t max_prefix_wgs(int32_t B, int G) {
  return (static_cast<int64_t>(B) * G + kPrefixRows - 1) / kPrefixRows + kMaxGroups;
}

struct SharedPrefixLayout {
  size_t stream, tables, lens, plen, counters, grp_lens, grp_count, recs, total;
  int64_t split_stride;         // floats
};

SharedPrefixLayout shared_prefix_layout(const pa_cache_desc* c, int32_t B, int32_t Hq,
                                        int32_t max_blocks) {
  SharedPrefixLayout L{};
  const int G = Hq / c->num_kv_heads;
  // decode scratch for up to 16 query rows: the group pass's chunk rows
  L.stream = align256(stream_workspace_bytes(B, c->num_kv_heads, std::max(G, kMaxRows), c->head_dim));
  L.tables = L.stream;
  L.lens = L.tables + align256(static_cast<size_t>(B) * max_blocks * 4);
  L.plen = L.lens + align256(static_cast<size_t>(B) * 4);
  L.counters = L.plen + align256(static_cast<size_t>(B) * 4);
  L.grp_lens = L.counters + align256(static_cast<size_t>(c->num_kv_heads) * max_prefix_wgs(B, G) * 4);
  L.grp_count = L.grp_lens + align256(static_cast<size_t>(B) * 4);
  L.recs = L.grp_count + align256(static_cast<size_t>(B) * 4);
  L.split_stride = static_cast<int64_t>(B) * Hq * (c->head_dim + 4);
  L.total = L.recs + static_cast<size_t>(L.split_stride) * kMaxSplits * 4;
  return L;
}

}  // namespace

extern "C" size_t pa_decode_shared_prefix_workspace_bytes(const pa_cache_desc* c, int32_t num_seqs,
                                                          int32_t num_q_heads,
                                                          int32_t max_blocks_per_seq,
                                                          int32_t max_context_len) {
  if (check_desc(c, "pa_decode_shared_prefix_workspace_bytes") != PA_OK) return 0;
  if (num_seqs <= 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0 || max_context_len <= 0 ||
      num_q_heads % c->num_kv_heads != 0)
    return 0;
  const int G = num_q_heads / c->num_kv_heads;
  const int q_dtype = (c->cache_dtype == PA_F32) ? PA_F32 : PA_BF16;
  if (!fast_path(c, q_dtype, G) || G > kMaxRows || c->block_size % kTile != 0) return 0;
  return shared_prefix_layout(c, num_seqs, num_q_heads, max_blocks_per_seq).total;
}

extern "C" pa_status pa_decode_shared_prefix(
    const pa_cache_desc* c, const void* k_cache, const void* v_cache, const void* q,
    int32_t q_dtype, void* out, const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t max_context_len, int32_t num_seqs, int32_t num_q_heads,
    float scale, const int32_t* groups, int32_t num_groups, void* workspace,
    size_t workspace_bytes, void* stream) {
  const char* fn = "pa_decode_shared_prefix";
  if (num_groups < 0 || num_groups > kMaxGroups)
    return fail(PA_ERR_INVALID_ARG, "%s: num_groups %d (0..%d)", fn, num_groups, kMaxGroups);
  if (num_groups == 0)
    return attend(fn, c, k_cache, v_cache, q, q_dtype, out, 1, 0, block_tables,
                  max_blocks_per_seq, context_lens, max_context_len, num_seqs, num_q_heads,
                  scale, workspace, workspace_bytes, stream);
  pa_status st = check_desc(c, fn);
  if (st != PA_OK) return st;
  if (!groups) return fail(PA_ERR_INVALID_ARG, "%s: null groups", fn);
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(PA_ERR_INVALID_ARG, "%s: scale must be positive and finite", fn);
  if (num_seqs <= 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0 ||
      num_q_heads % c->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "%s: bad batch shape", fn);
  const int hkv = c->num_kv_heads, D = c->head_dim, G = num_q_heads / hkv, bs = c->block_size;
  if (!fast_path(c, q_dtype, G) || G > kMaxRows || bs % kTile != 0)
    return fail(PA_ERR_UNSUPPORTED, "%s: needs a bf16 or fp8 cache with bf16 q, head_dim 64 or "
                "128, G <= 16 and a block size that is a multiple of 16", fn);
  if (static_cast<int64_t>(num_seqs) * num_q_heads * D * 2 >= (int64_t{1} << 31) ||
      static_cast<int64_t>(num_seqs) * num_q_heads * (D + 4) * 4 * kMaxSplits >= (int64_t{1} << 31))
    return fail(PA_ERR_UNSUPPORTED, "%s: q or the prefix records larger than 2 GiB", fn);
  PrefixGroups gr{};
  gr.num = num_groups;
  std::vector<std::pair<int, int>> spans;
  int wgs = 0, max_tiles = 0, max_count = 0, max_shared = 0;
  for (int i = 0; i < num_groups; ++i) {
    const int f = groups[3 * i], n = groups[3 * i + 1], m = groups[3 * i + 2];
    max_count = std::max(max_count, n);
    max_shared = std::max(max_shared, m);
    if (f < 0 || n < 1 || m < 1 || static_cast<int64_t>(f) + n > num_seqs || m > max_blocks_per_seq)
      return fail(PA_ERR_INVALID_ARG, "%s: group %d = (%d, %d, %d) out of range", fn, i, f, n, m);
    gr.first[i] = f;
    gr.count[i] = n;
    gr.shared[i] = m;
    gr.wg_begin[i] = wgs;
    wgs += (n * G + kPrefixRows - 1) / kPrefixRows;
    max_tiles = std::max(max_tiles, m * (bs / kTile));
    spans.emplace_back(f, f + n);
  }
  gr.wg_begin[num_groups] = wgs;
  std::sort(spans.begin(), spans.end());
  for (size_t i = 1; i < spans.size(); ++i)
    if (spans[i].first < spans[i - 1].second)
      return fail(PA_ERR_INVALID_ARG, "%s: groups overlap", fn);
  const SharedPrefixLayout L = shared_prefix_layout(c, num_seqs, num_q_heads, max_blocks_per_seq);
  if (!workspace || workspace_bytes < L.total)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes, need %zu", fn,
                workspace_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(PA_ERR_INVALID_ARG, "%s: workspace not 256-byte aligned", fn);
  if (!k_cache || !v_cache || !q || !out || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "%s: null pointer", fn);
  PA_DEBUG_CHECK(debug::check_tables(c, block_tables, max_blocks_per_seq, context_lens,
                                     max_context_len, num_seqs, stream, fn));
  PA_DEBUG_CHECK(debug::check_groups(block_tables, max_blocks_per_seq, num_seqs, groups,
                                     num_groups, stream, fn));
  char* ws = static_cast<char*>(workspace);
  int32_t* suf_tables = reinterpret_cast<int32_t*>(ws + L.tables);
  int32_t* suf_lens = reinterpret_cast<int32_t*>(ws + L.lens);
  int32_t* plen = reinterpret_cast<int32_t*>(ws + L.plen);
  float* recs = reinterpret_cast<float*>(ws + L.recs);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const float kscale = (c->cache_dtype == PA_FP8_E4M3) ? c->k_scale : 1.f;
  PrefixArgs pa;
  pa.k_cache = static_cast<const char*>(k_cache);
  pa.v_cache = static_cast<const char*>(v_cache);
  pa.q = static_cast<const uint16_t*>(q);
  pa.block_tables = block_tables;
  pa.context_lens = context_lens;
  pa.suf_tables = suf_tables;
  pa.suf_lens = suf_lens;
  pa.prefix_len = plen;
  pa.rec = recs;
  pa.counters = reinterpret_cast<uint32_t*>(ws + L.counters);
  pa.split_stride = L.split_stride;
  // splits of the prefix: about one workgroup per CU, each split at least
  // 16 tiles
  const int64_t row_wgs = static_cast<int64_t>(wgs) * hkv;
  int splits = static_cast<int>(std::min<int64_t>(kMaxSplits, (device_cus() + row_wgs - 1) / row_wgs));
  splits = std::max(1, std::min(splits, max_tiles / 16));
  pa.splits = splits;
  pa.num_seqs = num_seqs;
  pa.hkv = hkv;
  pa.group = G;
  pa.max_blocks = max_blocks_per_seq;
  pa.bs = bs;
  pa.sub_shift = bs == 64 ? 2 : bs == 32 ? 1 : 0;
  pa.logit_scale = static_cast<float>(static_cast<double>(scale) * kscale * 1.4426950408889634);
  pa.gr = gr;
  pa.grp_lens = nullptr;
  pa.grp_count = nullptr;
  const bool fp8 = c->cache_dtype == PA_FP8_E4M3;
  // rows of a group of a KV head that fit one 16-row MFMA block
  const int msub = std::max(1, kMaxRows / G);
  const bool split_groups = max_count > msub;
  if (num_seqs <= 256 && static_cast<uint32_t>(max_shared) <= kGrpMaxShared) {
    // At most 256 sequences: one launch of the decode kernel in which each
    // (group, KV head) is one segment -- the prefix tiles, then every
    // member's own tiles -- with all members' rows (kGrp).  A group with
    // more rows than 16 is split into row groups of msub members, each a
    // segment over the shared prefix; the tile list is then ordered by KV
    // head first so that the row groups of one head, which read the same
    // prefix tiles, run on one XCD and find them in its L2.
    GroupTable gtab{};
    int64_t tiles = 0;
    int rows_max = 0;
    for (int i = 0; i < num_groups; ++i) {
      const int f = groups[3 * i], n = groups[3 * i + 1];
      const uint32_t sh = static_cast<uint32_t>(groups[3 * i + 2]) << 11;
      for (int b0 = 0; b0 < n; b0 += msub) {
        const int nn = std::min(msub, n - b0);
        rows_max = std::max(rows_max, nn * G);
        for (int m = 0; m < nn; ++m)
          gtab.info[f + b0 + m] =
              kGrpMember | sh | (m == 0 ? kGrpLeader | (static_cast<uint32_t>(nn) << 2) : 0u);
      }
    }
    tiles = static_cast<int64_t>(hkv) * num_seqs * ((static_cast<int64_t>(max_context_len) + kTile - 1) / kTile);
    const int64_t waves_max = static_cast<int64_t>(device_cus()) * kWavesPerCU;
    int64_t nw = std::max<int64_t>(1, std::min(waves_max, (tiles + kMinTilesPerWave - 1) / kMinTilesPerWave));
    const bool head_major = split_groups && nw >= 8;
    if (head_major) nw = nw / 8 * 8;                       // XCD-major wave order needs whole rounds
    StreamArgs a;
    a.k_cache = pa.k_cache;
    a.v_cache = pa.v_cache;
    a.q = pa.q;
    a.out = static_cast<uint16_t*>(out);
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.counters = reinterpret_cast<uint32_t*>(ws);        // decode scratch comes first
    a.partials = reinterpret_cast<float*>(ws + align256(static_cast<size_t>(num_seqs) * hkv * 4));
    a.num_seqs = num_seqs;
    a.hkv = hkv;
    a.kv_split = 1;
    a.max_blocks = max_blocks_per_seq;
    a.num_waves = static_cast<int>(nw);
    a.group = G;
    a.chunk = 1;
    a.window = 0;
    a.sub_shift = pa.sub_shift;
    a.pair_nrec = 0;
    a.prefix_len = nullptr;
    a.prefix_rec = nullptr;
    a.t_first = 0;
    a.rows = rows_max;
    a.logit_scale = pa.logit_scale;
    a.v_scale = (c->cache_dtype == PA_FP8_E4M3) ? c->v_scale : 1.f;
    a.q_seq_rows = 1;
    a.q_total_rows = num_seqs;
    a.causal = 0;
    a.rec_out = nullptr;
    a.rec_count = nullptr;
    a.head_major = head_major ? 1 : 0;
    if (D == 128) launch_stream_groups<128>(fp8, a.num_waves, hs, a, gtab);
    else launch_stream_groups<64>(fp8, a.num_waves, hs, a, gtab);
    return launch_status(fn);
  }
  if (max_count * G <= kMaxRows) {
    // Small groups (all members' rows of a KV head fit one 16-row MFMA
    // block): the prefix goes through the decode kernel's tile stream, each
    // group leader standing for its group, with the members' rows as chunk
    // tokens that all see the whole prefix.  The prefix kernel's grid only
    // prepares the tables, lengths and group lengths.
    pa.grp_lens = reinterpret_cast<int32_t*>(ws + L.grp_lens);
    pa.grp_count = reinterpret_cast<int32_t*>(ws + L.grp_count);
    const int64_t entries = static_cast<int64_t>(num_seqs) * max_blocks_per_seq;
    const unsigned side_grid = static_cast<unsigned>(
        std::max<int64_t>(1, std::min<int64_t>(8 * device_cus(), (entries + 255) / 256)));
    prefix_prep_kernel<<<side_grid, 256, 0, hs>>>(pa);
    st = launch_status(fn);
    if (st != PA_OK) return st;
    const int64_t prefix_tiles = static_cast<int64_t>(hkv) * num_groups * max_tiles;
    const int64_t waves_max = static_cast<int64_t>(device_cus()) * kWavesPerCU;
    const int64_t nw = std::max<int64_t>(
        1, std::min(waves_max, (prefix_tiles + kMinTilesPerWave - 1) / kMinTilesPerWave));
    StreamArgs a;
    a.k_cache = pa.k_cache;
    a.v_cache = pa.v_cache;
    a.q = pa.q;
    a.out = static_cast<uint16_t*>(out);                 // not written by a group pass
    a.block_tables = block_tables;
    a.context_lens = pa.grp_lens;
    a.counters = reinterpret_cast<uint32_t*>(ws);        // decode scratch comes first
    a.partials = reinterpret_cast<float*>(ws + align256(static_cast<size_t>(num_seqs) * hkv * 4));
    a.num_seqs = num_seqs;
    a.hkv = hkv;
    a.kv_split = 1;
    a.max_blocks = max_blocks_per_seq;
    a.num_waves = static_cast<int>(nw);
    a.group = G;
    a.chunk = max_count;
    a.window = 0;
    a.sub_shift = pa.sub_shift;
    a.pair_nrec = 0;
    a.prefix_len = nullptr;
    a.prefix_rec = nullptr;
    a.t_first = 0;
    a.rows = G * max_count;
    a.logit_scale = pa.logit_scale;
    a.v_scale = (c->cache_dtype == PA_FP8_E4M3) ? c->v_scale : 1.f;
    a.q_seq_rows = 1;
    a.q_total_rows = num_seqs;
    a.causal = 0;
    a.rec_out = recs;
    a.rec_count = pa.grp_count;
    a.head_major = 0;
    if (D == 128) launch_stream<128>(fp8, false, a.num_waves, hs, a);
    else launch_stream<64>(fp8, false, a.num_waves, hs, a);
    st = launch_status(fn);
    if (st != PA_OK) return st;
    return attend(fn, c, k_cache, v_cache, q, q_dtype, out, 1, 0, pa.suf_tables, max_blocks_per_seq,
                  pa.suf_lens, max_context_len, num_seqs, num_q_heads, scale, workspace, L.stream,
                  stream, pa.prefix_len, recs);
  }
  const unsigned grid = static_cast<unsigned>(row_wgs * splits);
  if (D == 128) {
    if (fp8) shared_prefix_kernel<128, true><<<grid, 64 * kPrefixWaves, 0, hs>>>(pa);
    else shared_prefix_kernel<128, false><<<grid, 64 * kPrefixWaves, 0, hs>>>(pa);
  } else {
    if (fp8) shared_prefix_kernel<64, true><<<grid, 64 * kPrefixWaves, 0, hs>>>(pa);
    else shared_prefix_kernel<64, false><<<grid, 64 * kPrefixWaves, 0, hs>>>(pa);
  }
  st = launch_status(fn);
  if (st != PA_OK) return st;
  return attend(fn, c, k_cache, v_cache, q, q_dtype, out, 1, 0, suf_tables, max_blocks_per_seq,
                suf_lens, max_context_len, num_seqs, num_q_heads, scale, workspace, L.stream,
                stream, plen, recs);
}

extern "C" pa_status pa_time_next_call(void* start_event, void* stop_event) {
  t_next_call.start = static_cast<hipEvent_t>(start_event);
  t_next_call.stop = static_cast<hipEvent_t>(stop_event);
  return PA_OK;
}
