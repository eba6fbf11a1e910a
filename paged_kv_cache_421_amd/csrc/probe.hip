// pa_read_probe: the device's streaming-read rate, measured the way the
// decode kernel reads the cache (16-byte non-temporal buffer loads), so that
// decode's bandwidth can be put beside what the memory system delivers on
// this box.  A diagnostic, not part of the attention path.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "debug_checks.h"
#include "status.h"

namespace pagedkv {

pa_status launch_status(const char* fn);

namespace {

constexpr int kProbeChunk = 4096;        // bytes: one 16-token bf16 tile of head_dim 128
constexpr int kProbeUnroll = 4;          // chunks in flight per wave
constexpr int kAuxNT = 2;                // buffer load policy: non-temporal

// Each wave reads whole 4 KiB chunks (64 lanes x 4 x 16 B), chunks
// w, w + W, w + 2W, ... (W = waves in the grid), kProbeUnroll at a time.
// With `order`, chunk c is read from offset order[c] * 4 KiB instead of c.
// The XOR of everything read goes to sink[wave] so nothing is optimised away.
__global__ void __launch_bounds__(256)
read_probe_kernel(const char* __restrict__ buf, int64_t num_chunks,
                  const int32_t* __restrict__ order, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  // wave-uniform, taken through readfirstlane so that the chunk descriptors
  // stay in scalar registers (no loop over lanes around each load)
  const int64_t wave = __builtin_amdgcn_readfirstlane(
      static_cast<int>((static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6));
  const int64_t waves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (int64_t c0 = wave; c0 < num_chunks; c0 += waves * kProbeUnroll) {
    u32x4_t v[kProbeUnroll][4];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const int64_t c = c0 + u * waves;
      const int64_t cc = c < num_chunks ? (order ? order[c] : c) : 0;
      const int nrec = c < num_chunks ? kProbeChunk : 0;     // past the end: reads 0
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(buf) + cc * kProbeChunk, 0, nrec, 0x00020000);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[u][i] = __builtin_amdgcn_raw_buffer_load_b128(r, (i * 64 + lane) * 16, 0, kAuxNT);
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc ^= v[u][i];
  }
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  sink[wave * 64 + lane] = x;
}

}  // namespace

}  // namespace pagedkv

using namespace pagedkv;

extern "C" size_t pa_read_probe_sink_bytes(int32_t num_cus) {
  return num_cus > 0 ? static_cast<size_t>(num_cus) * 8 * 64 * sizeof(uint32_t) : 0;
}

extern "C" pa_status pa_read_probe(const void* buf, size_t bytes, const int32_t* chunk_order,
                                   void* sink, int32_t num_cus, void* stream) {
  if (!buf || !sink || num_cus <= 0)
    return fail(PA_ERR_INVALID_ARG, "pa_read_probe: null buffer or sink, or num_cus <= 0");
  const int64_t chunks = static_cast<int64_t>(bytes / kProbeChunk);
  if (chunks == 0) return PA_OK;
  if (chunks >= (int64_t{1} << 31))
    return fail(PA_ERR_UNSUPPORTED, "pa_read_probe: buffer too large");
  if (chunk_order) PA_DEBUG_CHECK(debug::check_order(chunk_order, chunks, stream, "pa_read_probe"));
  // 8 waves per compute unit: two 4-wave blocks per CU
  const unsigned blocks = static_cast<unsigned>(num_cus) * 2;
  read_probe_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const char*>(buf), chunks, chunk_order, static_cast<uint32_t*>(sink));
  return launch_status("pa_read_probe");
}
