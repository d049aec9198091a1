// Streaming-read probe: reads a buffer once with 16-byte loads and nothing
// else, the plain memory-bound kernel a weight-streaming matmul of the same
// size is compared against. It gives the HBM read rate the chip reaches for
// a transfer of that size, launch and drain included (the "achievable"
// figure beside the 8 TB/s peak).

#include "common.hpp"

namespace w4 {

// PER 16-byte loads per lane, all issued before the first is used; the lanes
// of a block cover 256 * PER consecutive 16-byte pieces, piece i of lane t at
// (block * PER + i) * 256 + t, so every wave instruction reads 1 KiB
// contiguous. The XOR of everything read decides a store that is taken only
// when it equals a fixed constant, which keeps the loads live.
template <int PER>
__global__ __launch_bounds__(256) void k_read_probe(const u4* __restrict__ src, size_t pieces,
                                                    unsigned* sink) {
  const size_t base = (size_t)blockIdx.x * 256 * PER + threadIdx.x;
  u4 v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const size_t idx = base + (size_t)i * 256;
    v[i] = idx < pieces ? src[idx] : u4{0u, 0u, 0u, 0u};
  }
  unsigned x = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) x ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
  if (x == 0x9E3779B9u) sink[blockIdx.x & 1023] = x;
}

}  // namespace w4

using namespace w4;

extern "C" int w4_read_probe(const void* buf, size_t bytes, int per, uint32_t* sink,
                             hipStream_t stream) {
  if (!buf || !sink) return W4_ERR_NULL;
  if (bytes == 0 || bytes % 16) return W4_ERR_SHAPE;
  if (per != 1 && per != 2 && per != 4 && per != 8) return W4_ERR_ARG;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return W4_ERR_ALIGN;
  const size_t pieces = bytes / 16;
  const size_t blocks = (pieces + 256 * (size_t)per - 1) / (256 * (size_t)per);
  if (blocks > 0x7fffffffu) return W4_ERR_SHAPE;
  const dim3 grid((unsigned)blocks), block(256);
  const u4* src = reinterpret_cast<const u4*>(buf);
  switch (per) {
    case 1: hipLaunchKernelGGL(k_read_probe<1>, grid, block, 0, stream, src, pieces, sink); break;
    case 2: hipLaunchKernelGGL(k_read_probe<2>, grid, block, 0, stream, src, pieces, sink); break;
    case 4: hipLaunchKernelGGL(k_read_probe<4>, grid, block, 0, stream, src, pieces, sink); break;
    default: hipLaunchKernelGGL(k_read_probe<8>, grid, block, 0, stream, src, pieces, sink); break;
  }
  return launch_status();
}
