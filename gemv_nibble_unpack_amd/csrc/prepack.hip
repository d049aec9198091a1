// Offline re-ordering of packed weights into the tile order the matmul
// kernels stream ("compressed format" advice on the BitBLAS practical-guide
// page: transform the weight once, ahead of time, so the run-time path does
// no layout work). Byte-exact and invertible; unprepack_w is the inverse.
//
// Inside each 4-byte word (8 INT4 codes or 16 INT2 codes of consecutive k)
// the codes are re-ordered so that the in-register unpack needs only
// AND/OR/shift:
//   W4A8 : byte j holds (k_j, k_{j+4}) in (low, high) nibble. Then
//          (w << 4) & 0xF0F0F0F0 gives k0..k3 and w & 0xF0F0F0F0 gives k4..k7
//          as int8 values 16*q (sign comes for free from the top nibble).
//   W4A16: nibble position p holds k_{(0,2,4,6,1,3,5,7)[p]}. Then
//          (w & 0x000F000F) | 0x64006400 is the fp16 pair (1024+q0, 1024+q1),
//          the 0x00F000F0 mask gives (k2, k3) scaled by 16, and the same two
//          masks on w >> 8 give (k4, k5) and (k6, k7).
//   W2A8 : byte j holds (k_j, k_{j+4}, k_{j+8}, k_{j+12}) in bit pairs 0,2,4,6.
//          Then (w << 6), (w << 4), (w << 2), w masked with 0xC0C0C0C0 give
//          k0..3, k4..7, k8..11, k12..15 as int8 values 64*c.
//   W8A8 : bytes stay in k order (they are the MFMA operand as they are).

#include "common.hpp"

namespace w4 {

__device__ __forceinline__ uint32_t nib(uint32_t w, int i) { return (w >> (4 * i)) & 15u; }
__device__ __forceinline__ uint32_t crumb(uint32_t w, int i) { return (w >> (2 * i)) & 3u; }

// canonical word -> tile word
__device__ __forceinline__ uint32_t shuffle_word(int layout, uint32_t w) {
  uint32_t o = 0;
  if (layout == W4_LAYOUT_W4A8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) o |= (nib(w, j) | (nib(w, j + 4) << 4)) << (8 * j);
  } else if (layout == W4_LAYOUT_W4A16) {
    constexpr int perm[8] = {0, 2, 4, 6, 1, 3, 5, 7};
#pragma unroll
    for (int p = 0; p < 8; ++p) o |= nib(w, perm[p]) << (4 * p);
  } else if (layout == W4_LAYOUT_W2A8) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o |= (crumb(w, j) | (crumb(w, j + 4) << 2) | (crumb(w, j + 8) << 4) |
            (crumb(w, j + 12) << 6))
           << (8 * j);
  } else {
    o = w;
  }
  return o;
}

// tile word -> canonical word
__device__ __forceinline__ uint32_t unshuffle_word(int layout, uint32_t o) {
  uint32_t w = 0;
  if (layout == W4_LAYOUT_W4A8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t b = (o >> (8 * j)) & 0xFFu;
      w |= (b & 15u) << (4 * j);
      w |= (b >> 4) << (4 * (j + 4));
    }
  } else if (layout == W4_LAYOUT_W4A16) {
    constexpr int perm[8] = {0, 2, 4, 6, 1, 3, 5, 7};
#pragma unroll
    for (int p = 0; p < 8; ++p) w |= nib(o, p) << (4 * perm[p]);
  } else if (layout == W4_LAYOUT_W2A8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t b = (o >> (8 * j)) & 0xFFu;
#pragma unroll
      for (int i = 0; i < 4; ++i) w |= ((b >> (2 * i)) & 3u) << (2 * (j + 4 * i));
    }
  } else {
    w = o;
  }
  return w;
}

// One thread per 16-byte lane chunk of the code section.
__global__ __launch_bounds__(256) void k_prepack_codes(int layout, const uint8_t* __restrict__ Wq,
                                                        int N, int rowbytes, int KT,
                                                        size_t nchunks, uint8_t* __restrict__ Wp) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= nchunks) return;
  const int lane = (int)(idx & 63);
  const size_t tile = idx >> 6;
  const int kt = (int)(tile % KT);
  const int t = (int)(tile / KT);
  const int n = t * TILE_N + (lane & 15);
  const int byte0 = 64 * kt + 16 * (lane >> 4);
  uint32_t words[4];
#pragma unroll
  for (int wi = 0; wi < 4; ++wi) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = byte0 + 4 * wi + i;
      const uint32_t b = (n < N && c < rowbytes) ? Wq[(size_t)n * rowbytes + c] : 0u;
      w |= b << (8 * i);
    }
    words[wi] = shuffle_word(layout, w);
  }
  *reinterpret_cast<u4*>(Wp + idx * 16) = u4{words[0], words[1], words[2], words[3]};
}

__global__ __launch_bounds__(256) void k_unprepack_codes(int layout, const uint8_t* __restrict__ Wp,
                                                          int N, int rowbytes, int KT,
                                                          size_t nchunks, uint8_t* __restrict__ Wq) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= nchunks) return;
  const int lane = (int)(idx & 63);
  const size_t tile = idx >> 6;
  const int kt = (int)(tile % KT);
  const int t = (int)(tile / KT);
  const int n = t * TILE_N + (lane & 15);
  if (n >= N) return;
  const int byte0 = 64 * kt + 16 * (lane >> 4);
  const u4 v = *reinterpret_cast<const u4*>(Wp + idx * 16);
#pragma unroll
  for (int wi = 0; wi < 4; ++wi) {
    const uint32_t w = unshuffle_word(layout, v[wi]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = byte0 + 4 * wi + i;
      if (c < rowbytes) Wq[(size_t)n * rowbytes + c] = (uint8_t)(w >> (8 * i));
    }
  }
}

// Group scales/zeros of the W4A16 layout: one thread per (n tile, k quad, row).
__global__ __launch_bounds__(256) void k_prepack_meta(const uint16_t* __restrict__ scales,
                                                       const uint8_t* __restrict__ zeros, int N,
                                                       int G, int NT, int KQ,
                                                       uint16_t* __restrict__ St,
                                                       uint8_t* __restrict__ Zt) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)NT * KQ * TILE_N) return;
  const int r = (int)(idx % TILE_N);
  const size_t tq = idx / TILE_N;
  const int q = (int)(tq % KQ);
  const int t = (int)(tq / KQ);
  const int n = t * TILE_N + r;
  uint16_t s[4];
  uint32_t z = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = 4 * q + i;
    const bool ok = n < N && g < G;
    s[i] = ok ? scales[(size_t)n * G + g] : (uint16_t)0;
    z |= (ok ? (uint32_t)zeros[(size_t)n * G + g] : 0u) << (8 * i);
  }
  *reinterpret_cast<u2*>(St + idx * 4) =
      u2{(uint32_t)s[0] | ((uint32_t)s[1] << 16), (uint32_t)s[2] | ((uint32_t)s[3] << 16)};
  reinterpret_cast<uint32_t*>(Zt)[idx] = z;
}

__global__ __launch_bounds__(256) void k_unprepack_meta(const uint16_t* __restrict__ St,
                                                         const uint8_t* __restrict__ Zt, int N,
                                                         int G, int NT, int KQ,
                                                         uint16_t* __restrict__ scales,
                                                         uint8_t* __restrict__ zeros) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)NT * KQ * TILE_N) return;
  const int r = (int)(idx % TILE_N);
  const size_t tq = idx / TILE_N;
  const int q = (int)(tq % KQ);
  const int t = (int)(tq / KQ);
  const int n = t * TILE_N + r;
  if (n >= N) return;
  const uint32_t z = reinterpret_cast<const uint32_t*>(Zt)[idx];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = 4 * q + i;
    if (g < G) {
      scales[(size_t)n * G + g] = St[idx * 4 + i];
      zeros[(size_t)n * G + g] = (uint8_t)(z >> (8 * i));
    }
  }
}

// canonical bytes per weight row
inline int code_row_bytes(int layout, int K) {
  return layout == W4_LAYOUT_W2A8 ? K / 4 : layout == W4_LAYOUT_W8A8 ? K : K / 2;
}

inline int check_layout_shape(int layout, int N, int K) {
  if (layout != W4_LAYOUT_W4A8 && layout != W4_LAYOUT_W4A16 && layout != W4_LAYOUT_W2A8 &&
      layout != W4_LAYOUT_W8A8)
    return W4_ERR_ARG;
  if (N < 1 || K < 16 || K > W4_MAX_K || K % 16) return W4_ERR_SHAPE;
  if (layout == W4_LAYOUT_W4A16 && K % W4_GROUP_SIZE) return W4_ERR_SHAPE;
  return W4_OK;
}

}  // namespace w4

using namespace w4;

extern "C" size_t prepack_bytes(int layout, int N, int K) {
  if (check_layout_shape(layout, N, K) != W4_OK) return 0;
  return geometry(layout, N, K).total;
}

extern "C" int prepack_w(int layout, const uint8_t* Wq, const void* scales, const uint8_t* zeros,
                         int N, int K, uint8_t* Wp, hipStream_t stream) {
  const int st = check_layout_shape(layout, N, K);
  if (st != W4_OK) return st;
  if (!Wq || !Wp) return W4_ERR_NULL;
  if (layout == W4_LAYOUT_W4A16 && (!scales || !zeros)) return W4_ERR_NULL;
  if (!aligned(Wq, 16) || !aligned(Wp, 16) || (scales && !aligned(scales, 2)))
    return W4_ERR_ALIGN;
  const Geometry g = geometry(layout, N, K);
  const int rowbytes = code_row_bytes(layout, K);
  const size_t nchunks = (size_t)g.NT * g.KT * 64;
  hipLaunchKernelGGL(k_prepack_codes, dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0,
                     stream, layout, Wq, N, rowbytes, g.KT, nchunks, Wp);
  if (layout == W4_LAYOUT_W4A16) {
    const size_t nm = (size_t)g.NT * g.KQ * TILE_N;
    hipLaunchKernelGGL(k_prepack_meta, dim3((unsigned)((nm + 255) / 256)), dim3(256), 0, stream,
                       (const uint16_t*)scales, zeros, N, K / W4_GROUP_SIZE, g.NT, g.KQ,
                       (uint16_t*)(Wp + g.s_off), Wp + g.z_off);
  }
  return launch_status();
}

extern "C" int unprepack_w(int layout, const uint8_t* Wp, int N, int K, uint8_t* Wq, void* scales,
                           uint8_t* zeros, hipStream_t stream) {
  const int st = check_layout_shape(layout, N, K);
  if (st != W4_OK) return st;
  if (!Wq || !Wp) return W4_ERR_NULL;
  if (layout == W4_LAYOUT_W4A16 && (!scales || !zeros)) return W4_ERR_NULL;
  if (!aligned(Wq, 16) || !aligned(Wp, 16) || (scales && !aligned(scales, 2)))
    return W4_ERR_ALIGN;
  const Geometry g = geometry(layout, N, K);
  const int rowbytes = code_row_bytes(layout, K);
  const size_t nchunks = (size_t)g.NT * g.KT * 64;
  hipLaunchKernelGGL(k_unprepack_codes, dim3((unsigned)((nchunks + 255) / 256)), dim3(256), 0,
                     stream, layout, Wp, N, rowbytes, g.KT, nchunks, Wq);
  if (layout == W4_LAYOUT_W4A16) {
    const size_t nm = (size_t)g.NT * g.KQ * TILE_N;
    hipLaunchKernelGGL(k_unprepack_meta, dim3((unsigned)((nm + 255) / 256)), dim3(256), 0,
                       stream, (const uint16_t*)(Wp + g.s_off), Wp + g.z_off, N,
                       K / W4_GROUP_SIZE, g.NT, g.KQ, (uint16_t*)scales, zeros);
  }
  return launch_status();
}
