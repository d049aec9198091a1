// Shared helpers for the gfx950 kernels and the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gemv_nibble_unpack.h"

namespace w4 {

// ---------------------------------------------------------------------------
// vector types used by the MFMA builtins and 16-byte memory operations
// ---------------------------------------------------------------------------
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef int i4 __attribute__((ext_vector_type(4)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef unsigned u2 __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// prepacked layout geometry
//
// Weights are cut into tiles of 16 output rows (n) x TILE_K reduction
// elements (k). Every tile is 1 KiB: 64 lanes x 16 bytes, so one
// global_load_dwordx4 per lane of a wave moves one whole tile. Lane l of a
// tile holds row n = 16*t + (l & 15) and the (l >> 4)-th quarter of the
// tile's k range, i.e. 16 consecutive bytes of that row in the canonical
// packed order, re-ordered inside each 4-byte word so that the unpack in
// registers is a handful of AND/OR/shift operations (see the unpack_*
// helpers). Tiles are stored n-tile-major: tile (t, kt) at (t*KT + kt) KiB.
//
// The W4A16 layout appends the group scales (fp16) and zeros (uint8) in the
// same n-tile order, four consecutive groups per (tile row, quad) so a lane
// fetches its row's four scales with one 8-byte load and its four zeros
// with one 4-byte load.
// ---------------------------------------------------------------------------
constexpr int TILE_N = 16;
constexpr int TILE_BYTES = 1024;

// Workspace layout shared by every plan that splits K across blocks: the
// first WS_COUNTERS bytes hold only the per-output-tile arrival counters,
// which each call leaves zero again; the partial sums start right after and
// are written before they are read. Any mix of shapes and plans can therefore
// reuse one workspace (zero-filled once) on one stream: a call's counters never
// land on bytes an earlier call used as scratch.
constexpr size_t WS_COUNTERS = 16 * 1024;
// Split-K arrival counters (one per output tile of a split launch); the last
// KiB of the area is left unused.
constexpr int WS_COUNTER_SLOTS = 3840;

struct Geometry {
  int NT;          // n tiles
  int KT;          // k tiles
  int KQ;          // k quads (groups of four k tiles)
  int tile_k;      // k extent of one tile
  size_t w_bytes;  // bytes of the code section
  size_t s_off;    // byte offset of the scale section (W4A16)
  size_t z_off;    // byte offset of the zero section (W4A16)
  size_t total;    // prepacked bytes
};

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

__host__ __device__ inline Geometry geometry(int layout, int N, int K) {
  Geometry g{};
  g.tile_k = layout == W4_LAYOUT_W2A8 ? 256 : layout == W4_LAYOUT_W8A8 ? 64 : 128;
  g.NT = ceil_div(N, TILE_N);
  g.KT = ceil_div(K, g.tile_k);
  g.KQ = ceil_div(g.KT, 4);
  g.w_bytes = (size_t)g.NT * g.KT * TILE_BYTES;
  g.s_off = g.w_bytes;
  g.z_off = g.w_bytes;
  g.total = g.w_bytes;
  if (layout == W4_LAYOUT_W4A16) {
    g.z_off = g.s_off + (size_t)g.NT * g.KQ * TILE_N * 4 * sizeof(uint16_t);
    g.total = g.z_off + (size_t)g.NT * g.KQ * TILE_N * 4;
  }
  return g;
}

// ---------------------------------------------------------------------------
// host-side validation helpers
// ---------------------------------------------------------------------------
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Kernels that take more than 64 KiB of dynamic LDS must say so once.
inline void allow_smem(const void* kernel, size_t bytes) {
  if (bytes > 65536) (void)hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                (int)bytes);
}

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? W4_OK : W4_ERR_HIP;
}

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
// Wave-wide reductions (64 lanes) through cross-lane shuffles.
// c / d for 0 <= c < 2^20 and 1 <= d < 2^24 without an integer division
// sequence: x = (c + 1/2) / d lies at least 1/(2d) from an integer, while the
// reciprocal (within 1 ulp) and the product leave an error below x * 2^-22 =
// (c + 1/2) / d * 2^-22 < 1/(2d), so truncating x gives the exact quotient.
__device__ __forceinline__ int small_div(int c, int d) {
  return (int)(((float)c + 0.5f) * __builtin_amdgcn_rcpf((float)d));
}

// Wave max with the row-local steps on DPP (quad swaps, then the 8- and
// 16-lane mirrors; each lane of a row of 16 ends with the row's max) and the
// four row maxima read into scalars: a handful of VALU cycles instead of a
// chain of six LDS crossbar permutes. A max does not depend on the order it is
// taken in, so the result is the same value as a shuffle tree's. Every lane
// of the wave must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));                      // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_f<0x4E>(v));                      // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp_f<0x141>(v));                     // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));                     // row_mirror
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}
// Sum over each row of 16 lanes, left in every lane of the row (the same
// DPP steps; a float sum in this fixed order, every lane of a row holding the
// identical value). Every lane active.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return v;
}

// The same for an integer sum (exact in any order). Every lane active.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int wave_sum_i(int v) {
  v += dpp_i<0xB1>(v);                               // quad_perm [1, 0, 3, 2]
  v += dpp_i<0x4E>(v);                               // quad_perm [2, 3, 0, 1]
  v += dpp_i<0x141>(v);                              // row_half_mirror
  v += dpp_i<0x140>(v);                              // row_mirror
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// The code decision rint(fl(w / s)), clipped to [-lim, lim] (0 for s == 0),
// with the correctly rounded float32 division.
__device__ __forceinline__ int sym_code_div(float w, float s, float lim) {
  return s > 0.f ? (int)fminf(fmaxf(rintf(w / s), -lim), lim) : 0;
}

// The code decision rint(fl(w / s)) of a division by a scale, for
// |w / s| <= 128, with a multiply by rs = fl(1 / s) (correctly rounded)
// instead of a division per element.
// y = fl(w * rs) differs from w / s by at most 128 * (2^-24 + 2^-24) = 2^-16,
// and fl(w / s) differs from w / s by at most 2^-17, so rint(y) and
// rint(fl(w / s)) can differ only if y lies within 2^-15 of a half integer.
// Lanes within 2^-14 of one take the correctly rounded division. rs must be
// finite: below s = 2^-128 (subnormal) it overflows, and the caller divides
// instead. A subnormal s with a finite reciprocal carries a relative error of
// at most 2^-21, so |w / s| stays below 127.001 and the bound above holds.
__device__ __forceinline__ int sym_code_rcp(float w, float s, float rs, float lim) {
  if (!(s > 0.f)) return 0;
  const float y = w * rs;
  float q = rintf(y);
  if (__builtin_expect(fabsf(y - floorf(y) - 0.5f) < 0x1p-14f, 0)) q = rintf(w / s);
  return (int)fminf(fmaxf(q, -lim), lim);
}

// Eight per-token INT8 codes of one chunk, packed little-endian into (lo, hi),
// and their sum added to `sum`: code = rint(fl(x / s)) clipped to [-127, 127],
// 0 for s == 0, with s = max|x| / 127 of the row and rs = fl(1 / s) (0 when
// s == 0). y = fl(x * rs) is rounded to an integer by adding 1.5 * 2^23: for
// |y| < 2^22 the sum lies in [2^23, 2^24), where the floats are the integers,
// so the addition itself rounds y to nearest even, and the sum's bits are
// 0x4B400000 + code, whose low byte is the code in two's complement. A normal
// s keeps |y| below 127.5, so the clip never acts on this path. A chunk with
// any y within 2^-14 of a half integer (where y and fl(x / s) may round
// apart, see sym_code_rcp), or with a subnormal s (whose own rounding error
// can carry |x / s| past the clip), takes the correctly rounded division.
__device__ __forceinline__ void codes8_i8(const float (&x)[8], float s, float rs, uint32_t& lo,
                                          uint32_t& hi, int& sum) {
#pragma clang fp contract(off)
  constexpr float R = 12582912.0f;                   // 1.5 * 2^23
  constexpr uint32_t RB = 0x4B400000u;               // bits of R
  uint32_t b[8];
  float dev = 0.f;                                   // largest |rint(y) - y|, exact
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float y = x[e] * rs;
    const float t = y + R;
    dev = fmaxf(dev, fabsf((t - R) - y));
    b[e] = __builtin_bit_cast(uint32_t, t);
  }
  if (__builtin_expect(dev > 0.5f - 0x1p-14f || (s > 0.f && s < 0x1p-126f), 0)) {
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = RB + (uint32_t)sym_code_div(x[e], s, 127.f);
  }
  // low bytes of b[0..3] and b[4..7]
  lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u),
                             __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u), 0x05040100u);
  hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[7], b[6], 0x0c0c0400u),
                             __builtin_amdgcn_perm(b[5], b[4], 0x0c0c0400u), 0x05040100u);
  sum += (int)(b[0] + b[1] + b[2] + b[3] + b[4] + b[5] + b[6] + b[7] - 8u * RB);
}

// Cross-block exchange of split-K partial sums through the workspace, at
// device scope. A device-scope fence writes back and invalidates the whole
// L2 of the XCD (costly once per block); instead the partial sums themselves
// are stored and loaded at device scope (written through to, and read from,
// the level all XCDs share), so the only ordering a block needs is that its
// stores have completed before it counts itself in (stores_done, then a
// barrier, then the device-scope arrival count).
__device__ __forceinline__ void dev_store(uint32_t* a, uint32_t v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t dev_load(const uint32_t* a) {
  return __hip_atomic_load(const_cast<uint32_t*>(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// the same for two consecutive 32-bit values (8-byte aligned)
__device__ __forceinline__ void dev_store2(uint32_t* a, uint32_t lo, uint32_t hi) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(a), (uint64_t)lo | ((uint64_t)hi << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t dev_load2(const uint32_t* a) {
  return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<uint32_t*>(a)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned dev_arrive(unsigned* c) {
  return __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// wait until this wave's stores are acknowledged; the clobber keeps the
// compiler from moving memory accesses across the wait
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Sum of `count` partial values `stride` apart, read at device scope and
// added in index order (float32 or int32 bits). The loads are issued 8 at a
// time before any is added: each is a round trip to the level all XCDs share,
// and loaded one per loop turn they would be waited for one after another.
template <bool FLOAT>
__device__ __forceinline__ void dev_sum(const uint32_t* base, size_t stride, int count, float& fs,
                                        int& is) {
  for (int z0 = 0; z0 < count; z0 += 8) {
    uint32_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = dev_load(base + (size_t)min(z0 + j, count - 1) * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (z0 + j < count) {
        if constexpr (FLOAT) fs += __builtin_bit_cast(float, v[j]);
        else is += (int)v[j];
      }
    }
  }
}

// fp16 bit pattern <-> float
__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ uint16_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);  // round to nearest even
}

}  // namespace w4
