// Decode-side kernel: C[M,N] = A[M,K] x W[N,K]^T for M <= 16 (one 16-row MFMA
// fragment of activations), streaming the prepacked low-bit weights once.
//
// Dataflow (INT4 quantization page, Part 1 step 3, re-targeted to gfx950):
// packed weight tiles are loaded with one global_load_dwordx4 per lane (a
// 1 KiB tile per wave instruction, fully coalesced), unpacked in registers
// with a few bit operations, and fed to the matrix cores:
//   * INT8 activations: 4-bit (2-bit) codes become int8 values 16*q (64*c)
//     and go to v_mfma_i32_16x16x64_i8; the INT32 sum is exact and shifted
//     back by 4 (6) bits before the epilogue.
//   * fp16 activations: codes become fp16 (q - z) exactly via the 0x6400
//     exponent trick (1024 + q) and one packed add/fma, go to
//     v_mfma_f32_16x16x32_f16, and each 128-k group's partial sum is scaled
//     by its fp16 group scale in float32 (BitBLAS page, "Advanced features 2").
// Reduction over k: inside a wave the matrix core sums the four 16-lane
// k quarters; across the waves of a block through LDS; across blocks
// (split-K) through a float32/int32 workspace that the last-arriving block
// sums in a fixed order, so results are deterministic.
// Epilogue (INT4 page, Part 1 step 4): acc * w_scale * a_scale (+ bias).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace w4 {

enum Kind { KIND_W4A8 = 0, KIND_W4A16 = 1, KIND_W2A8 = 2 };

struct MMParams {
  const void* A;               // int8 [M,K] (A8) or fp16 [M,K] (A16)
  const float* a_scale;        // [M] (A8)
  const uint8_t* Wt;           // prepacked code section
  const uint16_t* St;          // W4A16 scale section
  const uint8_t* Zt;           // W4A16 zero section
  const float* w_scale;        // W4A8 per-row scales [N]
  const uint16_t* w_scale16;   // W2A8 per-tensor scale [1]
  const uint16_t* bias;        // [N] or NULL
  void* C;
  int out_dtype;
  int M, N, K, NT, KT, KQ;
  int ksplit, kts;             // split-K factor and k tiles per split
  unsigned* counters;          // [mtiles * ngroups]  (split-K only)
  void* partials;              // [mtiles][ksplit][ngroups][TN*256] 4-byte
};

// ---- unpack helpers (word layouts are fixed by prepack) --------------------
// W4A16: one 32-bit word (8 codes) -> 8 fp16 values (q - z), slots in k order.
__device__ __forceinline__ h8 unpack_w4_f16(uint32_t w, h2 zlo, h2 zhi) {
  const uint32_t w8 = w >> 8;
  const h2 p0 = __builtin_bit_cast(h2, (w & 0x000F000Fu) | 0x64006400u);   // 1024+q
  const h2 p1 = __builtin_bit_cast(h2, (w & 0x00F000F0u) | 0x64006400u);   // 1024+16q
  const h2 p2 = __builtin_bit_cast(h2, (w8 & 0x000F000Fu) | 0x64006400u);
  const h2 p3 = __builtin_bit_cast(h2, (w8 & 0x00F000F0u) | 0x64006400u);
  const h2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const h2 d0 = p0 + zlo;                                       // q - z
  const h2 d1 = __builtin_elementwise_fma(p1, sixteenth, zhi);  // 64+q-(64+z)
  const h2 d2 = p2 + zlo;
  const h2 d3 = __builtin_elementwise_fma(p3, sixteenth, zhi);
  return h8{d0[0], d0[1], d1[0], d1[1], d2[0], d2[1], d3[0], d3[1]};
}

// W4A8: two words (16 codes) -> one i8 MFMA operand of values 16*q.
__device__ __forceinline__ i4 unpack_w4_i8(uint32_t w0, uint32_t w1) {
  return i4{(int)((w0 << 4) & 0xF0F0F0F0u), (int)(w0 & 0xF0F0F0F0u),
            (int)((w1 << 4) & 0xF0F0F0F0u), (int)(w1 & 0xF0F0F0F0u)};
}

// W2A8: one word (16 codes) -> one i8 MFMA operand of values 64*c.
__device__ __forceinline__ i4 unpack_w2_i8(uint32_t w) {
  return i4{(int)((w << 6) & 0xC0C0C0C0u), (int)((w << 4) & 0xC0C0C0C0u),
            (int)((w << 2) & 0xC0C0C0C0u), (int)(w & 0xC0C0C0C0u)};
}

template <int KIND>
struct KindTraits;
template <>
struct KindTraits<KIND_W4A8> {
  static constexpr int TILE_K = 128, A_CHUNKS = 2, SHIFT = 4;  // 16-B A loads per lane per tile
};
template <>
struct KindTraits<KIND_W4A16> {
  static constexpr int TILE_K = 128, A_CHUNKS = 4, SHIFT = 0;
};
template <>
struct KindTraits<KIND_W2A8> {
  static constexpr int TILE_K = 256, A_CHUNKS = 4, SHIFT = 6;
};

// Epilogue for one output element.
template <int KIND>
__device__ __forceinline__ void store_out(const MMParams& p, int m, int n, float facc, int iacc) {
  if constexpr (KIND == KIND_W4A16) {
    float v = facc;
    if (p.bias) v += h2f(p.bias[n]);
    reinterpret_cast<uint16_t*>(p.C)[(size_t)m * p.N + n] = f2h(v);
  } else {
    const int acc = iacc >> KindTraits<KIND>::SHIFT;  // exact: the sum is a multiple of 2^SHIFT
    if (p.out_dtype == W4_OUT_I32) {
      reinterpret_cast<int32_t*>(p.C)[(size_t)m * p.N + n] = acc;
      return;
    }
    const float ws = KIND == KIND_W4A8 ? p.w_scale[n] : h2f(p.w_scale16[0]);
    float v = (float)acc * ws * p.a_scale[m];
    if (p.out_dtype == W4_OUT_F32) {
      reinterpret_cast<float*>(p.C)[(size_t)m * p.N + n] = v;
    } else {
      if (p.bias) v += h2f(p.bias[n]);
      reinterpret_cast<uint16_t*>(p.C)[(size_t)m * p.N + n] = f2h(v);
    }
  }
}

// Grid: x = group of TN n tiles, y = k split, z = 16-row m tile.
template <int KIND, int WAVES, int TN, int U>
__global__ __launch_bounds__(WAVES * 64) void k_gemv(const MMParams p) {
  using Tr = KindTraits<KIND>;
  constexpr bool A16 = KIND == KIND_W4A16;
  typedef typename std::conditional<A16, f4, i4>::type Acc;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;   // A row within the m tile / W row within an n tile
  const int b = lane >> 4;   // k quarter of a tile
  const int mtile = blockIdx.z;
  const int m = mtile * 16 + r;
  const bool mval = m < p.M;
  const int t0 = blockIdx.x * TN;
  const int kt_begin = blockIdx.y * p.kts;
  const int kt_end = min(p.KT, kt_begin + p.kts);

  Acc acc[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) acc[t] = Acc{};

  const size_t a_row = (size_t)m * p.K;

  for (int kt0 = kt_begin + wave; kt0 < kt_end; kt0 += WAVES * U) {
    // ---- issue every load of this step first ------------------------------
    u4 wv[U][TN];
    u4 av[U][Tr::A_CHUNKS];
    uint16_t sv[U][TN];
    uint32_t zv[U][TN];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kt = kt0 + u * WAVES;
      const bool kval = kt < kt_end;
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int tile = t0 + t;
        if (kval && tile < p.NT) {
          wv[u][t] = __builtin_nontemporal_load(reinterpret_cast<const u4*>(
              p.Wt + ((size_t)tile * p.KT + kt) * TILE_BYTES + lane * 16));
          if constexpr (A16) {
            const size_t mi = ((size_t)tile * p.KQ + (kt >> 2)) * TILE_N + r;
            sv[u][t] = p.St[mi * 4 + (kt & 3)];
            zv[u][t] = p.Zt[mi * 4 + (kt & 3)];
          }
        } else {
          wv[u][t] = u4{0u, 0u, 0u, 0u};
          if constexpr (A16) {
            sv[u][t] = 0;
            zv[u][t] = 0;
          }
        }
      }
      const int kbase = kt * Tr::TILE_K + b * (Tr::TILE_K / 4);
#pragma unroll
      for (int j = 0; j < Tr::A_CHUNKS; ++j) {
        if constexpr (A16) {
          av[u][j] = (kval && mval)
                         ? *reinterpret_cast<const u4*>(
                               reinterpret_cast<const uint16_t*>(p.A) + a_row + kbase + 8 * j)
                         : u4{0u, 0u, 0u, 0u};
        } else {
          const int k0 = kbase + 16 * j;
          av[u][j] = (kval && mval && k0 < p.K)
                         ? *reinterpret_cast<const u4*>(
                               reinterpret_cast<const int8_t*>(p.A) + a_row + k0)
                         : u4{0u, 0u, 0u, 0u};
        }
      }
    }
    // ---- unpack + matrix-core products ------------------------------------
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        if constexpr (A16) {
          const _Float16 z = (_Float16)(float)zv[u][t];
          const _Float16 zl = -((_Float16)1024.0f + z);
          const _Float16 zh = -((_Float16)64.0f + z);
          const h2 zlo = {zl, zl}, zhi = {zh, zh};
          f4 part = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const h8 bf = unpack_w4_f16(wv[u][t][j], zlo, zhi);
            const h8 af = __builtin_bit_cast(h8, av[u][j]);
            part = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, part, 0, 0, 0);
          }
          const float s = h2f(sv[u][t]);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[t][e] = fmaf(part[e], s, acc[t][e]);
        } else if constexpr (KIND == KIND_W4A8) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const i4 bf = unpack_w4_i8(wv[u][t][2 * j], wv[u][t][2 * j + 1]);
            const i4 af = __builtin_bit_cast(i4, av[u][j]);
            acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf, acc[t], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const i4 bf = unpack_w2_i8(wv[u][t][j]);
            const i4 af = __builtin_bit_cast(i4, av[u][j]);
            acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf, acc[t], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- cross-wave reduction through LDS ---------------------------------
  // MFMA 16x16 output: lane holds column (lane & 15), rows 4*(lane >> 4) + e.
  __shared__ float red[WAVES][TN][16][16];
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // copy the element to a scalar first: __builtin_bit_cast applied to an
      // ext-vector element reads element 0 with this compiler
      const auto v = acc[t][e];
      red[wave][t][4 * b + e][r] = __builtin_bit_cast(float, v);
    }
  __syncthreads();

  const int rows = min(16, p.M - mtile * 16);
  const int nout = TN * 16 * 16;
  const int ngroups = gridDim.x;
  const size_t slot = (size_t)mtile * ngroups + blockIdx.x;

  if (p.ksplit == 1) {
    for (int idx = threadIdx.x; idx < nout; idx += WAVES * 64) {
      const int t = idx >> 8, row = (idx >> 4) & 15, col = idx & 15;
      const int n = (t0 + t) * 16 + col;
      if (row >= rows || n >= p.N) continue;
      float fs = 0.f;
      int is = 0;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        if constexpr (A16) fs += red[w][t][row][col];
        else is += __builtin_bit_cast(int, red[w][t][row][col]);
      }
      store_out<KIND>(p, mtile * 16 + row, n, fs, is);
    }
    return;
  }

  // ---- split-K: publish this block's partial, last block finishes -------
  uint32_t* part = reinterpret_cast<uint32_t*>(p.partials) +
                   ((size_t)mtile * p.ksplit + blockIdx.y) * ngroups * nout +
                   (size_t)blockIdx.x * nout;
  for (int idx = threadIdx.x; idx < nout; idx += WAVES * 64) {
    const int t = idx >> 8, row = (idx >> 4) & 15, col = idx & 15;
    float fs = 0.f;
    int is = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      if constexpr (A16) fs += red[w][t][row][col];
      else is += __builtin_bit_cast(int, red[w][t][row][col]);
    }
    part[idx] = A16 ? __builtin_bit_cast(uint32_t, fs) : (uint32_t)is;
  }
  __threadfence();
  __syncthreads();
  __shared__ int last;
  if (threadIdx.x == 0) last = atomicAdd(&p.counters[slot], 1u) == (unsigned)(p.ksplit - 1);
  __syncthreads();
  if (!last) return;
  __threadfence();
  const uint32_t* base = reinterpret_cast<const uint32_t*>(p.partials) +
                         (size_t)mtile * p.ksplit * ngroups * nout + (size_t)blockIdx.x * nout;
  for (int idx = threadIdx.x; idx < nout; idx += WAVES * 64) {
    const int t = idx >> 8, row = (idx >> 4) & 15, col = idx & 15;
    const int n = (t0 + t) * 16 + col;
    if (row >= rows || n >= p.N) continue;
    float fs = 0.f;
    int is = 0;
    for (int s = 0; s < p.ksplit; ++s) {
      const uint32_t v = base[(size_t)s * ngroups * nout + idx];
      if constexpr (A16) fs += __builtin_bit_cast(float, v);
      else is += (int)v;
    }
    store_out<KIND>(p, mtile * 16 + row, n, fs, is);
  }
  if (threadIdx.x == 0) p.counters[slot] = 0u;  // leave the workspace zeroed
}

}  // namespace w4
