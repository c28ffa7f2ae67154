// Streaming probes for the benchmark's measured HBM ceilings (not part of
// the decode path or of include/tka.h; built into libtka_probe.so).
//
// Reads `bytes` (a multiple of 16) once with 16-byte non-temporal loads, the
// way the decode step's scan streams K: a persistent grid of `wg_per_cu`
// workgroups of 256 threads per compute unit, each workgroup one contiguous
// range, UNR loads in flight per lane. Every lane folds what it read into one
// word and writes it to sink[global thread id] (so the loads cannot be
// dropped): sink must hold grid * 256 words. Bytes moved per launch: `bytes`
// read + grid * 1 KiB written.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tka_probe {

constexpr int UNR = 8;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per, hi = min(lo + per, n16);
  uint32_t acc = 0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += 256 * UNR) {
    u32x4_t v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int64_t j = min(i + (int64_t)u * 256, hi - 1);  // past the end: re-read the last chunk, ignored below
      v[u] = __builtin_nontemporal_load(src + j);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      if (i + (int64_t)u * 256 < hi) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// Read with writes mixed in: each wave reads 8 KiB tiles (tile t = wave id, + number of waves,
// ...) with 16-byte non-temporal loads, 8 in flight per lane, and writes 1 KiB per tile (one
// 16-byte non-temporal store per lane, contiguous) at dst + 1 KiB t: the byte ratio of a scan that
// writes one fp32 score per 8 bytes of bf16 key row read (a row of d = 128 scored for 8 heads:
// 32 B written per 256 B read). src: ntiles 8 KiB tiles; dst: ntiles KiB. The folded words go to
// sink[global thread id] as in the read probe.
__global__ __launch_bounds__(256) void stream_read_write_kernel(const u32x4_t* __restrict__ src, int64_t ntiles,
                                                                u32x4_t* __restrict__ dst,
                                                                uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  uint32_t acc = 0;
  for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < ntiles; t += nw) {
    const u32x4_t* p = src + t * 512 + lane;
    u32x4_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_nontemporal_load(p + j * 64);
    u32x4_t r = v[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) r ^= v[j];
    acc += r[0] ^ r[3];
    __builtin_nontemporal_store(r, dst + t * 64 + lane);
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace tka_probe

extern "C" int tka_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int grid, void* stream) {
  if (!src || !sink || bytes < 16 || (bytes & 15) || grid < 1) return 1;
  hipLaunchKernelGGL(tka_probe::stream_read_kernel, dim3((unsigned)grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const tka_probe::u32x4_t*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// src: `bytes` to read (a multiple of 8 KiB); dst: bytes / 8 written; sink: grid * 256 words.
extern "C" int tka_probe_stream_read_write(const void* src, int64_t bytes, void* dst, uint32_t* sink, int grid,
                                           void* stream) {
  if (!src || !dst || !sink || bytes < 8192 || (bytes % 8192) || grid < 1) return 1;
  hipLaunchKernelGGL(tka_probe::stream_read_write_kernel, dim3((unsigned)grid), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const tka_probe::u32x4_t*>(src),
                     bytes / 8192, reinterpret_cast<tka_probe::u32x4_t*>(dst), sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
