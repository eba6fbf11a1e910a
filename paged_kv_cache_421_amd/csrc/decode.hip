// pa_decode for gfx950: single-query attention over a paged KV cache.
//
// The method (vLLM PagedAttention, as described on the pages): the cache
// is split into 16-token blocks scattered through a pool, and the kernel
// reaches a sequence's blocks through its block table, walking ceil(L/16)
// entries (unionyoga.cn, "vLLM：重塑大模型推理性能的关键引擎", PagedAttention
// section; ybb.press, "vLLM PagedAttention 大模型推理架构深度实战", §2.2).
// Partial softmax results of separate pieces of the context are combined
// with online-softmax renormalisation (ybb.press §5.1), here both inside a
// work-group and across partitions.  Query heads that share a KV head (GQA,
// ybb.press §9 item 3) are processed together so each KV tile is read once.
//
// Work decomposition: one work-group per (partition of 512 tokens, KV head,
// sequence).  Decode reads every KV byte once and does 2*G flops per KV
// element, so it is HBM-bound: the design goal is to keep HBM streaming.
//
// Fast path (bf16 or fp8 cache, bf16 q, head_dim 64/128, G <= 8), 4 waves:
//  * wave w takes the partition's blocks w, w+4, w+8, ... and keeps its own
//    online-softmax state; the next block's K and V are loaded before the
//    current one is used (two tiles in flight per wave);
//  * logits S[h][t] = q[h] . K[t] for the G heads and 16 tokens of a block
//    come from one 16x16x32 bf16 MFMA per 32 dims: q (heads, zero-padded to
//    16 rows) is the A operand, the K tile straight from HBM is the B
//    operand -- each lane loads 16 contiguous bytes of one token row, which
//    is exactly the operand layout, so K never passes through LDS;
//  * the row max over 16 tokens is four DPP steps inside a 16-lane row;
//    the running max is only moved when a block's max exceeds it by more
//    than 2^8 (exact: any reference max gives the same softmax, and the
//    exponentials stay <= 256), so the accumulator rescale is rare;
//  * P moves to the V layout through 512 bytes of LDS per wave; V is
//    accumulated with fp32 VALU FMAs (reduction over tokens would need a
//    transposed V for MFMA), each lane owning 8 dims of a quarter of the
//    tokens;
//  * waves merge (m, l, o) through LDS at the end; a single-partition
//    sequence writes its output row, otherwise the partition's normalised
//    output and (max, sum) go to the workspace for the reduce kernel.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "device_common.h"
#include "status.h"

namespace pagedkv {

int dtype_bytes(int dt);
pa_status check_desc(const pa_cache_desc* c, const char* fn);
pa_status launch_status(const char* fn);

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kRescaleSlack = 8.0f;   // log2 units: exponentials stay <= 2^8

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

// Result of one (partition, KV head, sequence) work-group: either the final
// output rows, or partial results for the reduce kernel.
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
// Fast path.  kFp8: cache holds E4M3 codes (else bf16).  kD: head_dim.
// kG: query heads per KV head (1..8).
template <int kD, int kG, bool kFp8>
__global__ void __launch_bounds__(kThreads)
decode_mfma_kernel(const char* __restrict__ k_cache, const char* __restrict__ v_cache,
                   const uint16_t* __restrict__ q, const int32_t* __restrict__ block_tables,
                   const int32_t* __restrict__ context_lens, int max_blocks, int hkv,
                   float logit_scale /* scale*k_scale*log2(e) */, float v_scale,
                   PartOut po) {
  constexpr int kE = kFp8 ? 1 : 2;                 // bytes per cache element
  constexpr int kKK = kD / 32;                     // MFMA steps over head_dim
  constexpr int kLanesPerRow = kD / 8;             // V: lanes covering one token row
  constexpr int kRowsPerLoad = 64 / kLanesPerRow;  // V: token rows per load
  constexpr int kVLoads = kBlock / kRowsPerLoad;   // V: loads (tokens) per lane
  constexpr int kGP = (kG + 3) / 4 * 4;            // heads padded to 4
  constexpr int kHG = kGP / 4;                     // 16-lane row groups with heads
  constexpr int64_t kTileBytes = kBlock * kD * kE;

  const int part = blockIdx.x;
  const int g = blockIdx.y;
  const int s = blockIdx.z;
  const int L = context_lens[s];
  const int nparts = (L + kPartTokens - 1) / kPartTokens;
  const int hq = hkv * kG;
  if (part >= (nparts > 0 ? nparts : 1)) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  __shared__ __align__(16) float s_p[kWaves][kBlock][kGP];
  __shared__ __align__(16) float s_o[kWaves][kG][kD];
  __shared__ float s_m[kWaves][kG];
  __shared__ float s_l[kWaves][kG];

  if (L == 0) {   // empty context: zero output rows
    for (int i = threadIdx.x; i < kG * kD; i += kThreads) {
      const int h = g * kG + i / kD;
      store_out<false>(po.out, (static_cast<int64_t>(s) * hq + h) * kD + i % kD, 0.f);
    }
    return;
  }

  const int blk0 = part * kPartBlocks;
  const int nblk = min(kPartBlocks, (L + kBlock - 1) / kBlock - blk0);

  // Physical block ids of this partition, one per lane (lanes < nblk).
  int my_id = 0;
  if (lane < nblk) my_id = block_tables[static_cast<int64_t>(s) * max_blocks + blk0 + lane];

  // q as the MFMA A operand: row i = head (zero rows past kG), lane l holds
  // dims 32*kk + 8*(l/16) .. +7 of head l%16.
  const int row = lane & 15;
  const int quad = lane >> 4;
  bf16x8_t qa[kKK];
  {
    const int h = g * kG + row;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (row < kG)
        w = *reinterpret_cast<const u32x4_t*>(q + (static_cast<int64_t>(s) * hq + h) * kD +
                                              32 * kk + 8 * quad);
      qa[kk] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  // Lane offsets inside a (block, head) tile, in bytes.
  const int k_off = (row * kD + 8 * quad) * kE;               // + 32*kk*kE
  const int v_c = lane % kLanesPerRow;                        // 8-dim chunk
  const int v_r = lane / kLanesPerRow;                        // first token row
  const int v_off = (v_r * kD + 8 * v_c) * kE;                // + i*kRowsPerLoad*kD*kE

  // Online-softmax state.  Logit rows of head group `quad` (heads 4*quad+r)
  // live in lanes of row group `quad`; m_ref is uniform within the row,
  // l_part is per lane (token l%16) and summed at the end.
  float m_ref[4], l_part[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m_ref[r] = -INFINITY;
    l_part[r] = 0.f;
  }
  float o[kG][8];
#pragma unroll
  for (int h = 0; h < kG; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) o[h][j] = 0.f;

  using KChunk = typename std::conditional<kFp8, u32x2_t, u32x4_t>::type;
  using VChunk = KChunk;
  const int64_t head_off = static_cast<int64_t>(g) * kTileBytes;
  const int64_t blk_stride = static_cast<int64_t>(hkv) * kTileBytes;

  auto load_tile = [&](int k, KChunk (&kt)[kKK], VChunk (&vt)[kVLoads]) {
    const int id = __builtin_amdgcn_readlane(my_id, wave + kWaves * k);
    const int64_t base = static_cast<int64_t>(id) * blk_stride + head_off;
    const char* kb = k_cache + base + k_off;
    const char* vb = v_cache + base + v_off;
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk)
      kt[kk] = *reinterpret_cast<const KChunk*>(kb + 32 * kk * kE);
#pragma unroll
    for (int i = 0; i < kVLoads; ++i)
      vt[i] = *reinterpret_cast<const VChunk*>(vb + i * kRowsPerLoad * kD * kE);
  };

  const int nk = (nblk - wave + kWaves - 1) / kWaves;   // blocks of this wave

  auto process = [&](int k, const KChunk (&kt)[kKK], const VChunk (&vt)[kVLoads]) {
    const int valid = L - (blk0 + wave + kWaves * k) * kBlock;   // >= 1

    // ---- logits: S[4*quad + r][row] in acc[r]
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kKK; ++kk) {
      bf16x8_t kb;
      if constexpr (kFp8) {
        const u32x2_t w = kt[kk];
        const int w0 = static_cast<int>(w[0]), w1 = static_cast<int>(w[1]);
        const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
        const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
        const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
        const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
        kb = bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
      } else {
        kb = __builtin_bit_cast(bf16x8_t, kt[kk]);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], kb, acc, 0, 0, 0);
    }

    float x[4], rmax[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = acc[r] * logit_scale;
      if (valid < kBlock && row >= valid) x[r] = -INFINITY;
      rmax[r] = row16_max(x[r]);
    }

    // ---- lazy running-max update (wave-uniform branch)
    bool need = false;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      need |= (quad * 4 + r < kG) && (rmax[r] > m_ref[r] + kRescaleSlack);
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      float alpha[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float mn = (rmax[r] > m_ref[r] + kRescaleSlack) ? rmax[r] : m_ref[r];
        alpha[r] = __builtin_amdgcn_exp2f(m_ref[r] - mn);
        l_part[r] *= alpha[r];
        m_ref[r] = mn;
      }
#pragma unroll
      for (int h = 0; h < kG; ++h) {
        const float a = readlane_f(alpha[h & 3], 16 * (h >> 2));
#pragma unroll
        for (int j = 0; j < 8; ++j) o[h][j] *= a;
      }
    }

    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = __builtin_amdgcn_exp2f(x[r] - m_ref[r]);
      l_part[r] += p[r];
    }
    // P to LDS: s_p[wave][token][head]
    if (quad < kHG)
      *reinterpret_cast<f32x4_t*>(&s_p[wave][row][4 * quad]) = f32x4_t{p[0], p[1], p[2], p[3]};

    // ---- o += P V over this lane's tokens v_r + i*kRowsPerLoad, dims 8*v_c..+7
#pragma unroll
    for (int i = 0; i < kVLoads; ++i) {
      const int t = v_r + i * kRowsPerLoad;
      float vf[8];
      if constexpr (kFp8) {
        const u32x2_t w = vt[i];
        const int w0 = static_cast<int>(w[0]), w1 = static_cast<int>(w[1]);
        const f32x2_t a0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w0, 1.0f, false);
        const f32x2_t a1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w0, 1.0f, true);
        const f32x2_t a2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w1, 1.0f, false);
        const f32x2_t a3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w1, 1.0f, true);
        vf[0] = a0[0]; vf[1] = a0[1]; vf[2] = a1[0]; vf[3] = a1[1];
        vf[4] = a2[0]; vf[5] = a2[1]; vf[6] = a3[0]; vf[7] = a3[1];
      } else {
        const u32x4_t w = vt[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vf[2 * j] = bf16_lo(w[j]);
          vf[2 * j + 1] = bf16_hi(w[j]);
        }
      }
      if (valid < kBlock && t >= valid) {   // unused slots may hold NaN
#pragma unroll
        for (int j = 0; j < 8; ++j) vf[j] = 0.f;
      }
      float pt[kGP];
#pragma unroll
      for (int h4 = 0; h4 < kHG; ++h4) {
        const f32x4_t pv = *reinterpret_cast<const f32x4_t*>(&s_p[wave][t][4 * h4]);
        pt[4 * h4 + 0] = pv[0];
        pt[4 * h4 + 1] = pv[1];
        pt[4 * h4 + 2] = pv[2];
        pt[4 * h4 + 3] = pv[3];
      }
#pragma unroll
      for (int h = 0; h < kG; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) o[h][j] = fmaf(pt[h], vf[j], o[h][j]);
    }
  };

  // Two tiles in flight: while block k is used, block k+1 is loading.
  KChunk kt0[kKK], kt1[kKK];
  VChunk vt0[kVLoads], vt1[kVLoads];
  if (nk > 0) load_tile(0, kt0, vt0);
  for (int k = 0; k < nk; k += 2) {
    if (k + 1 < nk) load_tile(k + 1, kt1, vt1);
    process(k, kt0, vt0);
    if (k + 1 < nk) {
      if (k + 2 < nk) load_tile(k + 2, kt0, vt0);
      process(k + 1, kt1, vt1);
    }
  }

  // ---- wave totals: l over the 16 token lanes, o over the lanes sharing v_c
  float l_sum[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) l_sum[r] = row16_sum(l_part[r]);
#pragma unroll
  for (int h = 0; h < kG; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v = o[h][j];
#pragma unroll
      for (int sh = kLanesPerRow; sh < 64; sh <<= 1) v += __shfl_xor(v, sh);
      o[h][j] = v;
    }
  if (lane < kLanesPerRow) {
#pragma unroll
    for (int h = 0; h < kG; ++h) {
      *reinterpret_cast<f32x4_t*>(&s_o[wave][h][8 * v_c]) =
          f32x4_t{o[h][0], o[h][1], o[h][2], o[h][3]};
      *reinterpret_cast<f32x4_t*>(&s_o[wave][h][8 * v_c + 4]) =
          f32x4_t{o[h][4], o[h][5], o[h][6], o[h][7]};
    }
  }
  if (row == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * quad + r;
      if (h < kG) {
        s_m[wave][h] = m_ref[r];
        s_l[wave][h] = (nk > 0) ? l_sum[r] : 0.f;
      }
    }
  }
  __syncthreads();

  // ---- merge the waves: thread -> (head, dim)
  for (int i = threadIdx.x; i < kG * kD; i += kThreads) {
    const int hh = i / kD;
    const int d = i % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (s_l[w][hh] > 0.f) M = fmaxf(M, s_m[w][hh]);
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (s_l[w][hh] > 0.f) {
        const float a = __builtin_amdgcn_exp2f(s_m[w][hh] - M);
        lsum = fmaf(a, s_l[w][hh], lsum);
        osum = fmaf(a, s_o[w][hh][d], osum);
      }
    }
    const int h = g * kG + hh;
    const float ohat = osum / lsum;
    if (nparts == 1) {
      store_out<false>(po.out, (static_cast<int64_t>(s) * hq + h) * kD + d, ohat * v_scale);
    } else {
      const int64_t r = (static_cast<int64_t>(s) * hq + h) * po.num_parts + part;
      po.ws_o[r * kD + d] = ohat * v_scale;
      if (d == 0) {
        po.ws_ml[2 * r] = M;
        po.ws_ml[2 * r + 1] = lsum;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// General path: any G, fp32 / bf16 / fp8 cache.  One wave per (partition,
// query head, sequence); one token at a time, dot product by a wave
// reduction, exact online softmax.  Used for fp32 caches and shapes the fast
// path does not cover.
template <int kD, int kFmt, bool kOutF32>
__global__ void __launch_bounds__(64)
decode_simple_kernel(const char* __restrict__ k_cache, const char* __restrict__ v_cache,
                     const void* __restrict__ q, const int32_t* __restrict__ block_tables,
                     const int32_t* __restrict__ context_lens, int max_blocks, int hkv,
                     int group, float logit_scale, float v_scale, PartOut po) {
  constexpr int kPer = kD / 64;
  const int part = blockIdx.x;
  const int h = blockIdx.y;
  const int s = blockIdx.z;
  const int hq = gridDim.y;
  const int g = h / group;
  const int L = context_lens[s];
  const int nparts = (L + kPartTokens - 1) / kPartTokens;
  const int lane = threadIdx.x;
  if (part >= (nparts > 0 ? nparts : 1)) return;
  const int64_t orow = (static_cast<int64_t>(s) * hq + h) * kD;
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
  const int t0 = part * kPartTokens;
  const int t1 = min(L, t0 + kPartTokens);
  float m = -INFINITY, l = 0.f, o[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) o[i] = 0.f;
  for (int t = t0; t < t1; ++t) {
    const int64_t id = block_tables[static_cast<int64_t>(s) * max_blocks + t / kBlock];
    const int64_t base = ((id * hkv + g) * kBlock + t % kBlock) * kD;
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
    for (int i = 0; i < kPer; ++i) o[i] = fmaf(p, elem(v_cache, base + lane + 64 * i), o[i] * a);
    m = mn;
  }
  if (nparts == 1) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) store_out<kOutF32>(po.out, orow + lane + 64 * i, o[i] / l * v_scale);
  } else {
    const int64_t r = (static_cast<int64_t>(s) * hq + h) * po.num_parts + part;
#pragma unroll
    for (int i = 0; i < kPer; ++i) po.ws_o[r * kD + lane + 64 * i] = o[i] / l * v_scale;
    if (lane == 0) {
      po.ws_ml[2 * r] = m;
      po.ws_ml[2 * r + 1] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the partitions of one (sequence, query head):
//   out = sum_i 2^(m_i - M) l_i o_i / sum_i 2^(m_i - M) l_i,  M = max_i m_i.
template <int kD, bool kOutF32>
__global__ void __launch_bounds__(kD)
reduce_kernel(const int32_t* __restrict__ context_lens, PartOut po) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int hq = gridDim.x;
  const int L = context_lens[s];
  const int nparts = (L + kPartTokens - 1) / kPartTokens;
  if (nparts <= 1) return;     // written directly by the partition pass
  const int d = threadIdx.x;
  const int64_t r0 = (static_cast<int64_t>(s) * hq + h) * po.num_parts;
  float M = -INFINITY;
  for (int i = 0; i < nparts; ++i) M = fmaxf(M, po.ws_ml[2 * (r0 + i)]);
  float den = 0.f, num = 0.f;
  for (int i = 0; i < nparts; ++i) {
    const float a = __builtin_amdgcn_exp2f(po.ws_ml[2 * (r0 + i)] - M) * po.ws_ml[2 * (r0 + i) + 1];
    den += a;
    num = fmaf(a, po.ws_o[(r0 + i) * kD + d], num);
  }
  store_out<kOutF32>(po.out, (static_cast<int64_t>(s) * hq + h) * kD + d, num / den);
}

template <int kD>
void launch_fast(int G, bool fp8, dim3 grid, hipStream_t st, const char* kc, const char* vc,
                 const uint16_t* q, const int32_t* bt, const int32_t* cl, int maxb, int hkv,
                 float ls, float vs, PartOut po) {
#define PA_FAST(GG)                                                                     \
  case GG:                                                                              \
    if (fp8)                                                                            \
      decode_mfma_kernel<kD, GG, true><<<grid, kThreads, 0, st>>>(kc, vc, q, bt, cl,    \
                                                                  maxb, hkv, ls, vs, po); \
    else                                                                                \
      decode_mfma_kernel<kD, GG, false><<<grid, kThreads, 0, st>>>(kc, vc, q, bt, cl,   \
                                                                   maxb, hkv, ls, vs, po); \
    break;
  switch (G) {
    PA_FAST(1) PA_FAST(2) PA_FAST(3) PA_FAST(4) PA_FAST(5) PA_FAST(6) PA_FAST(7) PA_FAST(8)
    default: break;
  }
#undef PA_FAST
}

template <int kD>
void launch_simple(int fmt, bool out_f32, dim3 grid, hipStream_t st, const char* kc,
                   const char* vc, const void* q, const int32_t* bt, const int32_t* cl,
                   int maxb, int hkv, int G, float ls, float vs, PartOut po) {
  if (fmt == PA_F32)
    decode_simple_kernel<kD, PA_F32, true><<<grid, 64, 0, st>>>(kc, vc, q, bt, cl, maxb, hkv, G, ls, vs, po);
  else if (fmt == PA_BF16)
    decode_simple_kernel<kD, PA_BF16, false><<<grid, 64, 0, st>>>(kc, vc, q, bt, cl, maxb, hkv, G, ls, vs, po);
  else
    decode_simple_kernel<kD, PA_FP8_E4M3, false><<<grid, 64, 0, st>>>(kc, vc, q, bt, cl, maxb, hkv, G, ls, vs, po);
  (void)out_f32;
}

}  // namespace

}  // namespace pagedkv

using namespace pagedkv;

static int num_partitions(int32_t max_context_len) {
  return (max_context_len + kPartTokens - 1) / kPartTokens;
}

extern "C" size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                            int32_t head_dim, int32_t max_context_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  const int P = num_partitions(max_context_len);
  if (P <= 1) return 0;
  return static_cast<size_t>(num_seqs) * num_q_heads * P * (head_dim + 2) * sizeof(float);
}

extern "C" pa_status pa_decode(const pa_cache_desc* c, const void* k_cache, const void* v_cache,
                               const void* q, int32_t q_dtype, void* out,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t max_context_len,
                               int32_t num_seqs, int32_t num_q_heads, float scale,
                               void* workspace, size_t workspace_bytes, void* stream) {
  pa_status st = check_desc(c, "pa_decode");
  if (st != PA_OK) return st;
  const int hkv = c->num_kv_heads, D = c->head_dim, fmt = c->cache_dtype;
  if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0 || max_blocks_per_seq < 0)
    return fail(PA_ERR_INVALID_ARG, "pa_decode: negative size");
  if (num_q_heads % hkv != 0)
    return fail(PA_ERR_INVALID_ARG, "pa_decode: %d query heads not a multiple of %d KV heads",
                num_q_heads, hkv);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "pa_decode: scale not finite");
  const bool combo_ok = (fmt == PA_F32 && q_dtype == PA_F32) ||
                        (fmt == PA_BF16 && q_dtype == PA_BF16) ||
                        (fmt == PA_FP8_E4M3 && q_dtype == PA_BF16);
  if (!combo_ok)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: q dtype %d with cache dtype %d", q_dtype, fmt);
  if (static_cast<int64_t>(max_blocks_per_seq) * kBlock < max_context_len)
    return fail(PA_ERR_INVALID_ARG,
                "pa_decode: max_blocks_per_seq %d cannot hold max_context_len %d",
                max_blocks_per_seq, max_context_len);
  if (num_seqs == 0) return PA_OK;
  if (!k_cache || !v_cache || !q || !out || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "pa_decode: null pointer");
  if (num_seqs > 65535 || num_q_heads > 65535)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: num_seqs / num_q_heads above 65535");
  const size_t need = pa_decode_workspace_bytes(num_seqs, num_q_heads, D, max_context_len);
  if (workspace_bytes < need || (need > 0 && !workspace))
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "pa_decode: workspace %zu bytes, need %zu",
                workspace_bytes, need);

  const int G = num_q_heads / hkv;
  const int P = max_context_len > 0 ? num_partitions(max_context_len) : 1;
  PartOut po;
  po.out = out;
  po.num_parts = P;
  po.ws_o = static_cast<float*>(workspace);
  po.ws_ml = need ? po.ws_o + static_cast<size_t>(num_seqs) * num_q_heads * P * D : nullptr;
  const float kscale = (fmt == PA_FP8_E4M3) ? c->k_scale : 1.f;
  const float vscale = (fmt == PA_FP8_E4M3) ? c->v_scale : 1.f;
  const float logit_scale =
      static_cast<float>(static_cast<double>(scale) * kscale * 1.4426950408889634);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* kc = static_cast<const char*>(k_cache);
  const char* vc = static_cast<const char*>(v_cache);

  const bool fast = (fmt == PA_BF16 || fmt == PA_FP8_E4M3) && G <= 8;
  if (fast) {
    dim3 grid(P, hkv, num_seqs);
    const auto* qb = static_cast<const uint16_t*>(q);
    if (D == 128)
      launch_fast<128>(G, fmt == PA_FP8_E4M3, grid, s, kc, vc, qb, block_tables, context_lens,
                       max_blocks_per_seq, hkv, logit_scale, vscale, po);
    else
      launch_fast<64>(G, fmt == PA_FP8_E4M3, grid, s, kc, vc, qb, block_tables, context_lens,
                      max_blocks_per_seq, hkv, logit_scale, vscale, po);
  } else {
    dim3 grid(P, num_q_heads, num_seqs);
    if (D == 128)
      launch_simple<128>(fmt, fmt == PA_F32, grid, s, kc, vc, q, block_tables, context_lens,
                         max_blocks_per_seq, hkv, G, logit_scale, vscale, po);
    else
      launch_simple<64>(fmt, fmt == PA_F32, grid, s, kc, vc, q, block_tables, context_lens,
                        max_blocks_per_seq, hkv, G, logit_scale, vscale, po);
  }
  st = launch_status("pa_decode (partition pass)");
  if (st != PA_OK) return st;
  if (P > 1) {
    dim3 grid(num_q_heads, num_seqs);
    const bool of32 = (q_dtype == PA_F32);
    if (D == 128) {
      if (of32) reduce_kernel<128, true><<<grid, 128, 0, s>>>(context_lens, po);
      else reduce_kernel<128, false><<<grid, 128, 0, s>>>(context_lens, po);
    } else {
      if (of32) reduce_kernel<64, true><<<grid, 64, 0, s>>>(context_lens, po);
      else reduce_kernel<64, false><<<grid, 64, 0, s>>>(context_lens, po);
    }
    st = launch_status("pa_decode (reduce)");
  }
  return st;
}
